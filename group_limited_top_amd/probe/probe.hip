// probe.hip -- measurement kernels of libmoe_probe (include/moe_probe.h).
#include "moe_probe.h"

#include <hip/hip_runtime.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Streaming read through direct global -> LDS loads (global_load_lds_dwordx4,
// the load the layer's weight-streaming kernels use): each wave brings 4 KiB
// a round into its own LDS slot (4 loads of 1 KiB; M0 holds the LDS address,
// saved and restored, with the one wait state an LDS DMA needs after a scalar
// write of M0).  Nothing reads the slot, so rounds may overwrite it in any
// order; the wave waits for all its loads before it ends.
__global__ __launch_bounds__(256) void k_probe_read(const uint8_t* __restrict__ buf, size_t nround,
                                                    uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t slot[4][4096];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)slot[w])));
  const uint32_t off = 16u * (threadIdx.x & 63);
  for (size_t r = (size_t)blockIdx.x * 4 + w; r < nround; r += (size_t)gridDim.x * 4) {
    const uint64_t b = reinterpret_cast<uint64_t>(buf + r * 4096);
    const uint32_t blo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t bhi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const void* base = reinterpret_cast<const void*>(((uint64_t)bhi << 32) | (uint64_t)blo);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\ts_add_u32 m0, m0, 1024\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 offset:1024\n\ts_add_u32 m0, m0, 1024\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 offset:2048\n\ts_add_u32 m0, m0, 1024\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 offset:3072\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(base), "s"(lds)
        : "memory", "scc");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (threadIdx.x == 0 && nround == 0) sink[0] = 0;
}

__global__ __launch_bounds__(256) void k_probe_mfma(float* out, int iters) {
  const int tid = threadIdx.x;
  // operands: bf16 1.0 and 2^-12, so the sums stay small and finite
  const s16x8 a = {0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80};
  const s16x8 b = {0x3980, 0x3980, 0x3980, 0x3980, 0x3980, 0x3980, 0x3980, (short)(0x3980 + (tid & 1))};
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  // inline asm with each accumulator tied to itself in AGPRs: the compiler's
  // own loop kept copying the accumulators between registers every round
  for (int it = 0; it < iters; ++it) {
    asm volatile(
        "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
        "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
        "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
        "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
        "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7"
        : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3), "+a"(c4), "+a"(c5), "+a"(c6), "+a"(c7)
        : "v"(a), "v"(b));
  }
  // the accumulators are read only after the loop: wait out the last MFMAs
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  const f32x4 s4 = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  out[(size_t)blockIdx.x * 256 + tid] = s4[0] + s4[1] + s4[2] + s4[3];
}

}  // namespace

extern "C" {

int moe_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                          hipStream_t stream) {
  if (!buf || !sink || bytes == 0 || bytes % 4096 != 0 || ((uintptr_t)buf & 15u) || blocks <= 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_probe_read, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint8_t*>(buf), bytes / 4096, sink);
  return (int)hipGetLastError();
}

int moe_probe_mfma_bf16(float* out, int blocks, int iters, hipStream_t stream) {
  if (!out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_probe_mfma, dim3((unsigned)blocks), dim3(256), 0, stream, out, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
