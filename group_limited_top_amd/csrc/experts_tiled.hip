// experts_tiled.hip -- MFMA grouped GEMMs for experts with many rows (a large
// batch of tokens).
//
// [Routing §四]: every expert is down(silu(gate x) * up x) over stacked
// [E][I][H] weights; [Routing §五]: the shared expert is one more bucket (all T
// tokens).  Rows are the expert-sorted pairs; a tile is kTiledRows rows of one
// expert.
//
// Data flow.  A block is 8 waves (two per SIMD) over one 128-row token tile.
// Each weight element is used by exactly one wave, so weights go from global
// memory straight into registers in MFMA operand layout (no LDS round trip);
// the token tile, which all 8 waves use, is staged in LDS in 64-deep K slices
// (two stages, one barrier per stage).  16x16x32 bf16 MFMAs take the weights
// as the A operand and the token rows as B, so that each lane ends holding
// consecutive output features of one token (wide stores).
//
//   gate/up: block = 128 tokens x 256 features; wave w = 32 features of both
//            gate and up x 128 tokens (2 x 2 x 8 MFMA tiles); epilogue
//            h = silu(g) * u in registers.
//   down:    block = 128 tokens x 512 output columns; wave w = 64 columns.
//            W_down[e] is [I][H] (H contiguous): each lane loads 4
//            consecutive h at 8 consecutive i and transposes the 8x4 block in
//            registers, giving 4 MFMA tiles whose row m maps to h = h0 + 4m + j.
//
// Blocks are launched in a multiple of 8 and mapped so that each XCD (blocks
// b with equal b mod 8) works on consecutive tiles, i.e. on the same experts,
// sharing their weights in its L2.
#include "device.h"
#include "expert_tiles.h"
#include "kernels.h"

namespace moe {

// Pipeline.  Every stage is a 32-deep K slice of 640 rows x 64 bytes
// (40 KiB): 512 weight rows (gate/up) or 32 W_down rows of 1 KiB (down), plus
// the 128 token rows.  Four stages (160 KiB, all of the CU's LDS) form a ring
// filled by direct global -> LDS loads (global_load_lds_dwordx4: each wave
// instruction writes 1 KiB, lane l at +16 l), so three stages are in flight
// while one is computed, without holding any of it in registers.  Each of the
// 4 waves issues 10 such loads per stage; before computing stage c a wave
// waits until at most the 20 loads of stages c+1, c+2 are outstanding, then
// all waves meet at a barrier.
constexpr int kTBK = 32;                 // K depth of one stage
constexpr int kRowB = kTBK * 2;          // bytes per staged token / gate-up weight row
constexpr int kStageB = 40960;           // bytes per stage
constexpr int kTokOff = 32768;           // token rows start here in a stage
constexpr int kDmaPerWave = 10;          // 1 KiB loads per wave per stage
constexpr int kGuFeat = 256;             // features per gate/up block (64 per wave)
constexpr int kDnCols = 512;             // output columns per down block (128 per wave)

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

// Swizzled position of 16-byte chunk c of a 64-byte staged row r: the chunk
// index is XORed with bits 2..3 of the row, so that 16 consecutive rows read
// at one chunk index fall on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int r, int c) { return r * kRowB + ((c ^ ((r >> 2) & 3)) << 4); }

__device__ __forceinline__ int xcd_logical(int b, int n) {  // n: a multiple of 8
  return (b & 7) * (n >> 3) + (b >> 3);
}

__device__ __forceinline__ u32x4 lds16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// The ring.  Stages are loaded in order (dma(buf) issues this wave's 10
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

// Source of this lane's token-row chunk in load j (8 or 9) of wave w: token
// row 64 (j - 8) + 16 w + lane / 4, logical chunk (lane & 3) ^ ((lane >> 4) & 3).
__device__ __forceinline__ int token_row_of(int j, int wave, int lane) {
  return 64 * (j - 8) + 16 * wave + (lane >> 2);
}
__device__ __forceinline__ int chunk_of(int lane) { return (lane & 3) ^ ((lane >> 4) & 3); }

// ----------------------------------------------------------------------------
// gate/up: block = 128 tokens x 256 features; wave w = 64 features (64 gate +
// 64 up rows) x 128 tokens, 8 x 8 MFMA tiles.  Stage rows 0..255 are gate rows
// i0.., 256..511 up rows, 512..639 tokens.  FULL: all 128 token rows present.
template <bool FULL>
__device__ __forceinline__ void gateup_tile(const ExpertArgs& a, const TileInfo& ti, int slice,
                                            uint8_t* s0, uint8_t* s1, uint8_t* s2, uint8_t* s3) {
  const int I = ti.shared ? a.Is : a.I;
  const int i0 = slice * kGuFeat;
  const int H = a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int f0 = i0 + 64 * wave;
  const bool wact = f0 < I;  // wave-uniform; idle waves still load and sync

  // load g < 8: weight rows i0 + 64 (g & 3) + 16 w + lane / 4 of gate (g < 4) or
  // up, clamped into range; loads 8, 9: token rows.  Byte offsets are fixed,
  // the wave-uniform bases advance by one stage per dma().
  const size_t ebase = ti.shared ? 0 : (size_t)ti.e * a.I * H;
  const int ck = chunk_of(lane);
  const int wr = i0 + 16 * wave + (lane >> 2);
  uint32_t off[kDmaPerWave];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    off[j] = (uint32_t)(((size_t)min(wr + 64 * j, I - 1) * H + ck * 8) * 2);
    off[4 + j] = off[j];
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int row = token_row_of(8 + j, wave, lane);
    if (row >= ti.nrows) row = 0;  // padding rows load row 0; their outputs are not stored
    const int tok = ti.shared ? ti.row0 + row : a.sorted_pair[ti.row0 + row] / a.K;
    off[8 + j] = (uint32_t)(((size_t)tok * H + ck * 8) * 2);
  }
  const uint16_t* gp = reinterpret_cast<const uint16_t*>(ti.shared ? a.ws_gate : a.w_gate) + ebase;
  const uint16_t* up = reinterpret_cast<const uint16_t*>(ti.shared ? a.ws_up : a.w_up) + ebase;
  const uint16_t* xp = reinterpret_cast<const uint16_t*>(a.x);
  auto dma = [&](uint8_t* st) {
    const void* base[kDmaPerWave] = {gp, gp, gp, gp, up, up, up, up, xp, xp};
    dma_stage(base, off, wave_slot(st, wave));
    gp += kTBK;
    up += kTBK;
    xp += kTBK;
  };

  f32x4 acc[8][8];  // [gate s = 0..3, up s = 4..7][token sub-tile n]
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[s][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nsub = (ti.nrows + 15) >> 4;

  u32x4 A[2][8], B[2][8];  // two operand sets: [set][gate s = 0..3, up s = 4..7], [set][n]
  auto read = [&](const uint8_t* st, int set) {
    if (!wact) return;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t != set) continue;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        A[t][u] = lds16(st + swz(64 * wave + 16 * u + r16, q));
        A[t][4 + u] = lds16(st + swz(256 + 64 * wave + 16 * u + r16, q));
      }
#pragma unroll
      for (int n = 0; n < 8; ++n)
        if (FULL || n < nsub) B[t][n] = lds16(st + swz(512 + 16 * n + r16, q));
    }
  };
  auto mfma = [&](int set, int half) {
    if (!wact) return;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t != set) continue;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h != half) continue;
#pragma unroll
        for (int n = 4 * h; n < 4 * h + 4; ++n) {
          if (FULL || n < nsub) {
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[u][n] = mfma16x16x32(A[t][u], B[t][n], acc[u][n]);
          }
        }
      }
    }
  };

  run_ring<kDmaPerWave>(H / kTBK, s0, s1, s2, s3, dma, read, mfma);
  if (!wact) return;

  // epilogue: lane holds features f0 + 16 s + 4q + 0..3 of token row 16 n + r16
  uint16_t* hbase = reinterpret_cast<uint16_t*>(ti.shared ? a.h_shared : a.h_routed);
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int row = 16 * n + r16;
    if (row < ti.nrows) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = silu_f32(acc[s][n][i]) * acc[4 + s][n][i];
        u32x2 pk;
        pk.x = pack_bf16x2(hv[0], hv[1]);
        pk.y = pack_bf16x2(hv[2], hv[3]);
        *reinterpret_cast<u32x2*>(hbase + (size_t)(ti.row0 + row) * I + f0 + 16 * s + 4 * q) = pk;
      }
    }
  }
}

__global__ __launch_bounds__(256, 1) void k_gateup_tiled(const ExpertArgs a, int nslices,
                                                          int nblocks) {
  __shared__ __attribute__((aligned(1024))) uint8_t s0[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t s2[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t s3[kStageB];
  const int lb = xcd_logical(blockIdx.x, nblocks);
  const int slice = lb % nslices;
  TileInfo ti;
  if (!decode_tile(a, lb / nslices, ti)) return;
  if (slice * kGuFeat >= (ti.shared ? a.Is : a.I)) return;
  if (ti.nrows == kTiledRows) gateup_tile<true>(a, ti, slice, s0, s1, s2, s3);
  else gateup_tile<false>(a, ti, slice, s0, s1, s2, s3);
}

// ----------------------------------------------------------------------------
// v[r] holds W[k = r][h = 0..7]; a[j] gets W[k = 0..7][h = j] as four k-pairs,
// i.e. the A-operand row of column h = j.
__device__ __forceinline__ void transpose8x8(const u32x4 (&v)[8], u32x4 (&a)[8]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t x0 = v[2 * c][jj], x1 = v[2 * c + 1][jj];
      a[2 * jj][c] = (x0 & 0xffffu) | (x1 << 16);
      a[2 * jj + 1][c] = (x0 >> 16) | (x1 & 0xffff0000u);
    }
  }
}

// down: block = 128 tokens x 512 output columns; wave w = 128 columns x 128
// tokens.  Stage: 32 W_down rows i (1 KiB = 512 columns each) then the 128
// hidden rows.  Lane (r16, q) reads 8 consecutive h at the 8 rows 8q..8q+7
// and transposes the 8x8 block in registers: virtual tile j has row m at
// h = 128 w + 8 m + j.
template <bool FULL>
__device__ __forceinline__ void down_tile(const ExpertArgs& a, const TileInfo& ti, int slice,
                                          uint8_t* s0, uint8_t* s1, uint8_t* s2, uint8_t* s3) {
  const int I = ti.shared ? a.Is : a.I;
  const int H = a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int hb = slice * kDnCols;       // first column of the block
  const int h0 = hb + 128 * wave;       // first column of this wave
  const bool wact = h0 < H;

  // load g < 8: W_down row k0 + 4 g + w, columns hb + 8 lane .. + 7 (clamped);
  // loads 8, 9: hidden rows.  Byte offsets are fixed, the bases advance.
  const size_t ebase = ti.shared ? 0 : (size_t)ti.e * a.I * H;
  const int ck = chunk_of(lane);
  const int hcol = min(hb + 8 * lane, H - 8);
  uint32_t off[kDmaPerWave];
#pragma unroll
  for (int j = 0; j < 8; ++j) off[j] = (uint32_t)(((size_t)(4 * j + wave) * H + hcol) * 2);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int row = token_row_of(8 + j, wave, lane);
    if (row >= ti.nrows) row = 0;
    off[8 + j] = (uint32_t)(((size_t)(ti.row0 + row) * I + ck * 8) * 2);
  }
  const uint16_t* wp = reinterpret_cast<const uint16_t*>(ti.shared ? a.ws_down : a.w_down) + ebase;
  const uint16_t* hp = reinterpret_cast<const uint16_t*>(ti.shared ? a.h_shared : a.h_routed);
  auto dma = [&](uint8_t* st) {
    const void* base[kDmaPerWave] = {wp, wp, wp, wp, wp, wp, wp, wp, hp, hp};
    dma_stage(base, off, wave_slot(st, wave));
    wp += (size_t)kTBK * H;
    hp += kTBK;
  };

  f32x4 acc[8][8];  // [virtual tile j][token sub-tile n]
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nsub = (ti.nrows + 15) >> 4;

  // W row 4 j + w of the stage sits at LDS row 4 j + w, i.e. row i at i * 1 KiB.
  // read() fetches the raw 8x8 blocks; the first half of mfma() transposes them.
  u32x4 V[2][8], B[2][8], am[8];
  auto read = [&](const uint8_t* st, int set) {
    if (!wact) return;
    const uint8_t* wb = st + 256 * wave + 16 * r16;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t != set) continue;
#pragma unroll
      for (int r = 0; r < 8; ++r) V[t][r] = lds16(wb + (8 * q + r) * 1024);
#pragma unroll
      for (int n = 0; n < 8; ++n)
        if (FULL || n < nsub) B[t][n] = lds16(st + kTokOff + swz(16 * n + r16, q));
    }
  };
  auto mfma = [&](int set, int half) {
    if (!wact) return;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t != set) continue;
      if (half == 0) transpose8x8(V[t], am);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h != half) continue;
#pragma unroll
        for (int n = 4 * h; n < 4 * h + 4; ++n) {
          if (FULL || n < nsub) {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j][n] = mfma16x16x32(am[j], B[t][n], acc[j][n]);
          }
        }
      }
    }
  };

  run_ring<kDmaPerWave>(I / kTBK, s0, s1, s2, s3, dma, read, mfma);
  if (!wact) return;

  // epilogue: tile j, C row 4q + i -> h = h0 + 8 (4q + i) + j: 8 consecutive h
  uint16_t* obase = reinterpret_cast<uint16_t*>(ti.shared ? a.o_shared : a.o_routed);
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int row = 16 * n + r16;
    if (row < ti.nrows) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 pk;
        pk.x = pack_bf16x2(acc[0][n][i], acc[1][n][i]);
        pk.y = pack_bf16x2(acc[2][n][i], acc[3][n][i]);
        pk.z = pack_bf16x2(acc[4][n][i], acc[5][n][i]);
        pk.w = pack_bf16x2(acc[6][n][i], acc[7][n][i]);
        st16(obase + (size_t)(ti.row0 + row) * H + h0 + 8 * (4 * q + i), pk);
      }
    }
  }
}

__global__ __launch_bounds__(256, 1) void k_down_tiled(const ExpertArgs a, int nslices,
                                                        int nblocks) {
  __shared__ __attribute__((aligned(1024))) uint8_t s0[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t s2[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t s3[kStageB];
  const int lb = xcd_logical(blockIdx.x, nblocks);
  const int slice = lb % nslices;
  TileInfo ti;
  if (!decode_tile(a, lb / nslices, ti)) return;
  if (slice * kDnCols >= a.H) return;
  if (ti.nrows == kTiledRows) down_tile<true>(a, ti, slice, s0, s1, s2, s3);
  else down_tile<false>(a, ti, slice, s0, s1, s2, s3);
}

// ----------------------------------------------------------------------------
// gate/up weight streaming through the ring: few rows per expert (tiles of
// kTileRows = 32 token rows), so the projection is bound by reading each
// expert's weights once.  The same 4-stage ring as above, with stages that
// favour HBM: every load instruction covers whole 256-byte row segments.
constexpr int kSBK = 128;    // K depth of a gate/up streaming stage
constexpr int kSRowB = 256;  // bytes per staged row in gate/up streaming

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

hipError_t launch_experts_tiled_bf16(const ExpertArgs& a, hipStream_t s, const StageTimer* tm) {
  if (!a.tiles_ready) {
    stage_begin(tm, kTiles, s);
    const hipError_t e = launch_tiles(a, s);
    stage_end(tm, kTiles, s);
    if (e != hipSuccess) return e;
  }
  // the ring runs whole groups of four 32-deep stages
  if (a.H % (4 * kTBK) != 0 || a.I % (4 * kTBK) != 0 || a.Is % (4 * kTBK) != 0 || a.H < 8)
    return hipErrorInvalidValue;
  const int64_t tiles = max_expert_tiles(a.T, a.K, a.E, a.Is, a.tile_rows);
  const int imax = a.I > a.Is ? a.I : a.Is;
  const int gu_slices = (imax + kGuFeat - 1) / kGuFeat;
  int64_t nb = tiles * gu_slices;
  nb = (nb + 7) / 8 * 8;
  stage_begin(tm, kGateUp, s);
  hipLaunchKernelGGL(k_gateup_tiled, dim3((unsigned)nb), dim3(256), 0, s, a, gu_slices,
                     (int)nb);
  stage_end(tm, kGateUp, s);
  const int dn_slices = (a.H + kDnCols - 1) / kDnCols;
  nb = tiles * dn_slices;
  nb = (nb + 7) / 8 * 8;
  stage_begin(tm, kDown, s);
  hipLaunchKernelGGL(k_down_tiled, dim3((unsigned)nb), dim3(256), 0, s, a, dn_slices,
                     (int)nb);
  stage_end(tm, kDown, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine_bf16(a, s, tm);
}

}  // namespace moe
