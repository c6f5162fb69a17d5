// ring.h -- device helpers shared by the kernels that stage operands through
// an LDS ring filled by direct global -> LDS loads (internal).
#pragma once

#include "device.h"

namespace moe {

typedef __attribute__((address_space(3))) const void lvoid_t;

// Scalar (wave-uniform) load through the constant address space.
__device__ __forceinline__ int32_t sload(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding and its LDS reads are done, then meet the other waves.
template <int N>
__device__ __forceinline__ void ring_wait() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ u32x4 lds16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// A wave-uniform pointer, made visible as such.
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | (uint64_t)lo);
}

// 8-byte store to global memory (a global, not flat, store: flat stores would
// also count against the LDS counter the ring waits on).  Plain stores: the
// streaming (nontemporal) kind measured much slower for the down outputs.
__device__ __forceinline__ void store8(uint16_t* p, u32x2 v) {
  *(__attribute__((address_space(1))) u32x2*)p = v;
}

// W_down slices (64 rows k x 512 B): 16-byte chunk c of row r sits at chunk
// c ^ wd_swz(r).  The transpose reads of one instruction cover 16 rows
// (8 q + c, q, c = 0..3) at one 32-byte column window; the XOR spreads them
// over the 8 windows of a 256-byte bank line, two rows each.
__device__ __forceinline__ int wd_swz(int r) { return 2 * ((r & 3) + 4 * ((r >> 3) & 1)); }

// LDS transpose read: within each group of 16 lanes, lane i receives element
// (i & 3) of the 4 x 16-bit values addressed by lane 4 c + (i >> 2), for
// c = 0..3.  So if lane 4 c + m of a group points at row c, columns 4 m..4 m + 3
// of a [k][column] block, lane i gets column i at rows 0..3.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_tr16(const uint8_t* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(__attribute__((address_space(3))) uint8_t*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Row slices (rows of 128 B): 16-byte chunk c of row r sits at
// r * 128 + 16 (c ^ ((r >> 1) & 7)), so that 16 consecutive rows read at one
// chunk index cover all 64 banks.  A DMA load (1 KiB) covering rows
// 8 j + lane / 8 (j = the load's 8-row group) has lane l at slot l & 7, i.e.
// logical chunk rs_chunk(j, lane).
__device__ __forceinline__ int rs_addr(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }
__device__ __forceinline__ int rs_chunk(int j, int lane) { return (lane & 7) ^ ((4 * j + (lane >> 4)) & 7); }

}  // namespace moe
