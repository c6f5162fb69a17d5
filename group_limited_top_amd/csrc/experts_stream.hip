// experts_stream.hip -- gate/up + SwiGLU for few rows per expert (a small
// batch of tokens), bf16.
//
// [Routing §四]: every expert is down(silu(gate x) * up x) over stacked
// [E][I][H] weights; [Routing §五]: the shared expert is one more bucket (all T
// tokens).  With tiles of kTileRows = 32 token rows (about 16 rows per expert
// at 512 tokens) the projection is bound by reading each expert's weights
// once, so the kernel is built around streaming them.
//
// Block = one 32-row tile x 64 features (16 per wave, of both gate and up).
// Every stage is a 128-deep K slice of 160 rows x 256 bytes (40 KiB): 64 gate
// rows, 64 up rows and the 32 token rows, so every load instruction covers
// whole 256-byte row segments.  Four stages (160 KiB, all of the CU's LDS)
// form a ring filled by direct global -> LDS loads (global_load_lds_dwordx4:
// each wave instruction writes 1 KiB, lane l at +16 l): three stages are in
// flight while one is computed.  Each of the 4 waves issues 10 loads per
// stage; before computing stage c a wave waits until at most the 20 loads of
// stages c+1, c+2 are outstanding, then all waves meet at a barrier.
#include "device.h"
#include "expert_tiles.h"
#include "kernels.h"

namespace moe {

constexpr int kStageB = 40960;  // bytes per stage

typedef __attribute__((address_space(3))) const void lvoid_t;

// One stage's loads of this wave: load g (0..9) brings the lane's 16 bytes
// from base[g] + off[g] (a wave-uniform 64-bit base plus a 32-bit per-lane
// byte offset) into LDS lds + 4096 g + 16 * lane (global_load_lds_dwordx4,
// M0 = the wave's LDS destination).  Written as inline asm so that the
// compiler does not treat the ring's later LDS reads as dependent on every
// load in flight; the ring orders them itself (ring_sync).  The memory clobber
// keeps LDS reads from moving across it.  M0 is saved and restored around the
// loads (the compiler owns it), and every write of M0 is followed by the one
// wait state that an LDS DMA reading M0 needs after a scalar write of it.
__device__ __forceinline__ void dma_stage(const void* const (&base)[10], const uint32_t (&off)[10],
                                          uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %21\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %11\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %12\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %13\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %14\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %5, %15\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %6, %16\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %7, %17\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %8, %18\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %9, %19\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %10, %20\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "v"(off[4]), "v"(off[5]), "v"(off[6]),
        "v"(off[7]), "v"(off[8]), "v"(off[9]), "s"(base[0]), "s"(base[1]), "s"(base[2]),
        "s"(base[3]), "s"(base[4]), "s"(base[5]), "s"(base[6]), "s"(base[7]), "s"(base[8]),
        "s"(base[9]), "s"(lds)
      : "memory", "scc");
}

// LDS byte address of wave w's first 1 KiB slot in a stage buffer.
__device__ __forceinline__ uint32_t wave_slot(const uint8_t* stage, int wave) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lvoid_t*)stage)) + 1024u * wave);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// and all its LDS operations are done, then meet the other waves.
template <int N>
__device__ __forceinline__ void ring_sync() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ u32x4 lds16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// The ring.  Stages are loaded in order (dma(buf) issues this wave's
// loads of the next stage into buf).  A stage's operands are read from LDS
// into one of two register sets (read(buf, set)) while the MFMAs of the
// previous stage are still being issued: mfma(set, half) runs half of a
// stage's MFMAs, and the barrier of stage c + 1 sits between the two halves
// of stage c, so the LDS latency of stage c + 1 hides behind the second half.
// Stage c + 4 goes into stage c's buffer once all waves have read stage c
// (ring_sync waits for this wave's LDS reads before the barrier).
// nk (stages) must be a positive multiple of 4; kLoads = loads per wave per stage.
template <int kLoads, class Dma, class Read, class Mfma>
__device__ __forceinline__ void run_ring(int nk, uint8_t* s0, uint8_t* s1, uint8_t* s2, uint8_t* s3,
                                         Dma&& dma, Read&& read, Mfma&& mfma) {
  constexpr int kTwo = 2 * kLoads;
  dma(s0);
  dma(s1);
  dma(s2);
  ring_sync<kTwo>();  // stage 0 landed (stages 1, 2 may be in flight)
  dma(s3);
  read(s0, 0);
  // steady state: stages c .. c+3; stage c + k + 4 goes into stage c + k's buffer
  for (int c = 0; c < nk - 4; c += 4) {
    mfma(0, 0); ring_sync<kTwo>(); dma(s0); read(s1, 1); mfma(0, 1);
    mfma(1, 0); ring_sync<kTwo>(); dma(s1); read(s2, 0); mfma(1, 1);
    mfma(0, 0); ring_sync<kTwo>(); dma(s2); read(s3, 1); mfma(0, 1);
    mfma(1, 0); ring_sync<kTwo>(); dma(s3); read(s0, 0); mfma(1, 1);
  }
  // last four stages: nothing more to load
  mfma(0, 0); ring_sync<kTwo>(); read(s1, 1); mfma(0, 1);
  mfma(1, 0); ring_sync<kLoads>(); read(s2, 0); mfma(1, 1);
  mfma(0, 0); ring_sync<0>(); read(s3, 1); mfma(0, 1);
  mfma(1, 0); mfma(1, 1);
}

constexpr int kSBK = 128;    // K depth of a stage
constexpr int kSRowB = 256;  // bytes per staged row

// Swizzled position of 16-byte chunk c of a 256-byte staged row r (16 chunks;
// the XOR with the row's low 4 bits spreads 16 consecutive rows read at one
// chunk index over all banks).
__device__ __forceinline__ int sswz(int r, int c) { return r * kSRowB + ((c ^ (r & 15)) << 4); }

// gate/up: block = one 32-row tile x 64 features; wave w = features 16 w..16 w+15
// of gate and up.  Stage rows 0..63 gate rows i0.., 64..127 up rows, 128..159
// token rows; load j of wave w covers stage rows 16 j + 4 w .. + 3.
__global__ __launch_bounds__(256, 1) void k_gateup_stream(const ExpertArgs a, int nslices) {
  __shared__ __attribute__((aligned(1024))) uint8_t s0[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t s2[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t s3[kStageB];
  const int slice = blockIdx.x % nslices;
  TileInfo ti;
  if (!decode_tile(a, blockIdx.x / nslices, ti)) return;
  const int I = ti.shared ? a.Is : a.I;
  const int i0 = slice * 64;
  if (i0 >= I) return;
  const int H = a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;

  const size_t ebase = ti.shared ? 0 : (size_t)ti.e * a.I * H;
  uint32_t off[10];
#pragma unroll
  for (int j = 0; j < 10; ++j) {
    const int r = 16 * j + 4 * wave + (lane >> 4);  // stage row
    const int c = (lane & 15) ^ (r & 15);           // logical chunk held at this lane's slot
    if (j < 8) {
      off[j] = (uint32_t)(((size_t)(i0 + (r & 63)) * H + c * 8) * 2);
    } else {
      int tr = r - 128;
      if (tr >= ti.nrows) tr = 0;  // padding rows load row 0; their outputs are not stored
      const int tok = ti.shared ? ti.row0 + tr : a.sorted_pair[ti.row0 + tr] / a.K;
      off[j] = (uint32_t)(((size_t)tok * H + c * 8) * 2);
    }
  }
  const uint16_t* gp = reinterpret_cast<const uint16_t*>(ti.shared ? a.ws_gate : a.w_gate) + ebase;
  const uint16_t* up = reinterpret_cast<const uint16_t*>(ti.shared ? a.ws_up : a.w_up) + ebase;
  const uint16_t* xp = reinterpret_cast<const uint16_t*>(a.x);
  auto dma = [&](uint8_t* st) {
    const void* base[10] = {gp, gp, gp, gp, up, up, up, up, xp, xp};
    dma_stage(base, off, wave_slot(st, wave));
    gp += kSBK;
    up += kSBK;
    xp += kSBK;
  };

  const int nsub = (ti.nrows + 15) >> 4;  // 1 or 2
  f32x4 accg[2], accu[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    accg[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    accu[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  u32x4 Ag[2][4], Au[2][4], B[2][4][2];  // [set][32-deep substep s][token sub-tile n]
  auto read = [&](const uint8_t* st, int set) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t != set) continue;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        Ag[t][u] = lds16(st + sswz(16 * wave + r16, 4 * u + q));
        Au[t][u] = lds16(st + sswz(64 + 16 * wave + r16, 4 * u + q));
#pragma unroll
        for (int n = 0; n < 2; ++n)
          if (n < nsub) B[t][u][n] = lds16(st + sswz(128 + 16 * n + r16, 4 * u + q));
      }
    }
  };
  auto mfma = [&](int set, int half) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t != set) continue;
#pragma unroll
      for (int u = 2 * half; u < 2 * half + 2; ++u)
#pragma unroll
        for (int n = 0; n < 2; ++n)
          if (n < nsub) {
            accg[n] = mfma16x16x32(Ag[t][u], B[t][u][n], accg[n]);
            accu[n] = mfma16x16x32(Au[t][u], B[t][u][n], accu[n]);
          }
    }
  };
  run_ring<10>(H / kSBK, s0, s1, s2, s3, dma, read, mfma);

  // epilogue: lane holds features i0 + 16 w + 4q + 0..3 of token row 16 n + r16
  uint16_t* hbase = reinterpret_cast<uint16_t*>(ti.shared ? a.h_shared : a.h_routed);
  const int ib = i0 + 16 * wave + 4 * q;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int row = 16 * n + r16;
    if (n < nsub && row < ti.nrows) {
      float hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[i] = silu_f32(accg[n][i]) * accu[n][i];
      u32x2 pk;
      pk.x = pack_bf16x2(hv[0], hv[1]);
      pk.y = pack_bf16x2(hv[2], hv[3]);
      *reinterpret_cast<u32x2*>(hbase + (size_t)(ti.row0 + row) * I + ib) = pk;
    }
  }
}

bool stream_ring_ok(const ExpertArgs& a) {
  // the ring takes a multiple of 4 stages of kSBK; lane offsets are 32-bit
  const int64_t imax = a.I > a.Is ? a.I : a.Is;
  return a.H % (4 * kSBK) == 0 && (int64_t)a.T * a.H * 2 < (int64_t(1) << 32) &&
         imax * a.H * 2 < (int64_t(1) << 32);
}

hipError_t launch_gateup_stream_bf16(const ExpertArgs& a, int64_t tiles, hipStream_t s,
                                     const StageTimer* tm) {
  const int imax = a.I > a.Is ? a.I : a.Is;
  const int slices = imax / 64;
  stage_begin(tm, kGateUp, s);
  hipLaunchKernelGGL(k_gateup_stream, dim3((unsigned)(tiles * slices)), dim3(256), 0, s, a, slices);
  stage_end(tm, kGateUp, s);
  return hipGetLastError();
}

}  // namespace moe
