// experts_tiled.hip -- LDS-tiled MFMA grouped GEMMs for experts with many
// rows (a large batch of tokens).
//
// [Routing §四]: every expert is down(silu(gate x) * up x) over stacked
// [E][I][H] weights; [Routing §五]: the shared expert is one more bucket (all T
// tokens).  Rows are the expert-sorted pairs; a tile is kTiledRows rows of one
// expert.  Both kernels stage 32-deep K slices of both operands in LDS (two
// stages, one barrier per stage) and run 16x16x32 bf16 MFMAs with the weights
// as the A operand and the token rows as B, so that each lane ends holding
// consecutive output features of one token (wide stores).
//
//   gate/up: block = 128 tokens x 128 features (256 weight rows: 128 gate +
//            128 up); wave (wi, wt) = 64 features of both gate and up x 64
//            tokens (8 x 4 MFMA tiles); epilogue h = silu(g) * u in registers.
//   down:    block = 256 output columns x 128 tokens; W_down[e] is [I][H] (H
//            contiguous), staged as [i][h] rows; each lane reads 8 consecutive
//            h at 8 consecutive i and transposes the 8x8 block in registers,
//            giving 8 MFMA tiles whose row m maps to h = h0 + 8m + j.
//
// Blocks are launched in a multiple of 8 and mapped so that each XCD (blocks
// b with equal b mod 8) works on consecutive tiles, i.e. on the same experts,
// sharing their weights in its L2.
#include "device.h"
#include "expert_tiles.h"
#include "kernels.h"

namespace moe {

constexpr int kTBK = 32;                       // K depth of one LDS stage
constexpr int kTRow = kTBK * 2;                // bytes per staged row (four 16-byte chunks)
constexpr int kGuWRows = 256;                  // weight rows per gate/up block
constexpr int kGuRows = kGuWRows + kTiledRows;  // staged rows per gate/up stage
constexpr int kDnCols = 256;                   // output columns per down block
constexpr int kDnWRow = kDnCols * 2 + 32;      // bytes per staged W_down row (+32: bank spread)

// LDS position of 16-byte chunk c of staged row r.  Rows are 64 bytes; the
// chunk index is XORed with bits 2..3 of the row so that the 16 (or 32) lanes
// one ds_read_b128 serves at a time -- 16 consecutive rows at one chunk, or
// two chunks -- fall on disjoint banks with either 64 or 128 four-byte banks.
__device__ __forceinline__ int swz(int r, int c) { return r * kTRow + ((c ^ ((r >> 2) & 3)) << 4); }

__device__ __forceinline__ int xcd_logical(int b, int n) {  // n: a multiple of 8
  return (b & 7) * (n >> 3) + (b >> 3);
}

__device__ __forceinline__ u32x4 lds16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void k_gateup_tiled(const ExpertArgs a, int nslices,
                                                          int nblocks) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kGuRows * kTRow];
  const int lb = xcd_logical(blockIdx.x, nblocks);
  const int slice = lb % nslices;
  TileInfo ti;
  if (!decode_tile(a, lb / nslices, ti)) return;
  const int I = ti.shared ? a.Is : a.I;
  const int i0 = slice * 128;
  if (i0 >= I) return;
  const int H = a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int wi = wave & 1, wt = wave >> 1;

  // staging role: row rr (+64 u), 16-byte column c16 of the 64-byte slice row
  const int rr = tid >> 2, c16 = tid & 3;
  const size_t ebase = ti.shared ? 0 : (size_t)ti.e * a.I * H;
  const uint16_t* wg = reinterpret_cast<const uint16_t*>(ti.shared ? a.ws_gate : a.w_gate) + ebase +
                       (size_t)(i0 + rr) * H + c16 * 8;
  const uint16_t* wu = reinterpret_cast<const uint16_t*>(ti.shared ? a.ws_up : a.w_up) + ebase +
                       (size_t)(i0 + rr) * H + c16 * 8;
  const uint16_t* xp[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = u * 64 + rr;
    xp[u] = nullptr;
    if (row < ti.nrows) {
      const int tok = ti.shared ? ti.row0 + row : a.sorted_pair[ti.row0 + row] / a.K;
      xp[u] = reinterpret_cast<const uint16_t*>(a.x) + (size_t)tok * H + c16 * 8;
    }
  }
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  u32x4 sa[6], sb[6];  // global loads of two future stages in flight
  auto gload = [&](u32x4 (&st)[6], int k0) {
    st[0] = ld16(wg + k0);
    st[1] = ld16(wg + (size_t)64 * H + k0);
    st[2] = ld16(wu + k0);
    st[3] = ld16(wu + (size_t)64 * H + k0);
    st[4] = xp[0] ? ld16(xp[0] + k0) : zero4;
    st[5] = xp[1] ? ld16(xp[1] + k0) : zero4;
  };
  auto sstore = [&](const u32x4 (&st)[6], int stage) {
    uint8_t* base = lds[stage];
#pragma unroll
    for (int u = 0; u < 6; ++u) st16(base + swz(64 * u + rr, c16), st[u]);
  };
  // tokens of this wave that exist (wave-uniform)
  const int wrows = ti.nrows - wt * 64;
  f32x4 acc[8][4];
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[s][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int stage) {
    const uint8_t* base = lds[stage];
    u32x4 A[8], B[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      A[s] = lds16(base + swz(wi * 64 + s * 16 + r16, q));
      A[4 + s] = lds16(base + swz(128 + wi * 64 + s * 16 + r16, q));
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) B[n] = lds16(base + swz(256 + wt * 64 + n * 16 + r16, q));
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      if (n * 16 < wrows) {
#pragma unroll
        for (int s = 0; s < 8; ++s) acc[s][n] = mfma16x16x32(A[s], B[n], acc[s][n]);
      }
    }
  };

  // stage c is computed from LDS buffer c & 1 while the global loads of
  // stages c + 1 and c + 2 are in flight (register sets alternate)
  const int nk = H / kTBK;
  gload(sa, 0);
  if (nk > 1) gload(sb, kTBK);
  sstore(sa, 0);
  __syncthreads();
  for (int c = 0; c < nk; c += 2) {
    if (c + 2 < nk) gload(sa, (c + 2) * kTBK);
    compute(0);
    if (c + 1 < nk) sstore(sb, 1);
    __syncthreads();
    if (c + 1 >= nk) break;
    if (c + 3 < nk) gload(sb, (c + 3) * kTBK);
    compute(1);
    if (c + 2 < nk) sstore(sa, 0);
    __syncthreads();
  }

  // epilogue: lane holds features i0 + 64 wi + 16 s + 4q + 0..3 of token row 64 wt + 16 n + r16
  uint16_t* hbase = reinterpret_cast<uint16_t*>(ti.shared ? a.h_shared : a.h_routed);
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int row = wt * 64 + n * 16 + r16;
    if (row < ti.nrows) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = silu_f32(acc[s][n][i]) * acc[4 + s][n][i];
        u32x2 pk;
        pk.x = pack_bf16x2(hv[0], hv[1]);
        pk.y = pack_bf16x2(hv[2], hv[3]);
        *reinterpret_cast<u32x2*>(hbase + (size_t)(ti.row0 + row) * I + i0 + wi * 64 + s * 16 +
                                  4 * q) = pk;
      }
    }
  }
}

// ----------------------------------------------------------------------------
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

__global__ __launch_bounds__(256, 2) void k_down_tiled(const ExpertArgs a, int nslices,
                                                        int nblocks) {
  __shared__ __attribute__((aligned(16))) uint8_t ldw[2][kTBK * kDnWRow];
  __shared__ __attribute__((aligned(16))) uint8_t ldh[2][kTiledRows * kTRow];
  const int lb = xcd_logical(blockIdx.x, nblocks);
  const int slice = lb % nslices;
  TileInfo ti;
  if (!decode_tile(a, lb / nslices, ti)) return;
  const int I = ti.shared ? a.Is : a.I;
  const int H = a.H;
  const int h0 = slice * kDnCols;
  if (h0 >= H) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int wh = wave & 1, wt = wave >> 1;

  // W_down staging: row (i) tid >> 3 of the 32-deep slice, 16-byte columns (tid & 7) + 8u
  const int wr = tid >> 3, wc = tid & 7;
  const size_t ebase = ti.shared ? 0 : (size_t)ti.e * a.I * H;
  const uint16_t* wd = reinterpret_cast<const uint16_t*>(ti.shared ? a.ws_down : a.w_down) + ebase +
                       (size_t)wr * H + h0 + wc * 8;
  // hidden-row staging: rows (tid >> 2) + 64u, 16-byte column tid & 3
  const int hr = tid >> 2, hc = tid & 3;
  const uint16_t* hsrc = reinterpret_cast<const uint16_t*>(ti.shared ? a.h_shared : a.h_routed);
  const uint16_t* hp[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = u * 64 + hr;
    hp[u] = row < ti.nrows ? hsrc + (size_t)(ti.row0 + row) * I + hc * 8 : nullptr;
  }
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  u32x4 sa[6], sb[6];
  auto gload = [&](u32x4 (&st)[6], int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) st[u] = ld16(wd + (size_t)k0 * H + u * 64);
    st[4] = hp[0] ? ld16(hp[0] + k0) : zero4;
    st[5] = hp[1] ? ld16(hp[1] + k0) : zero4;
  };
  auto sstore = [&](const u32x4 (&st)[6], int stage) {
#pragma unroll
    for (int u = 0; u < 4; ++u) st16(ldw[stage] + wr * kDnWRow + (wc + 8 * u) * 16, st[u]);
    st16(ldh[stage] + swz(hr, hc), st[4]);
    st16(ldh[stage] + swz(64 + hr, hc), st[5]);
  };
  const int wrows = ti.nrows - wt * 64;
  f32x4 acc[8][4];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int stage) {
    u32x4 v[8], am[8], B[4];
    const uint8_t* wb = ldw[stage] + (wh * 128 + 8 * r16) * 2;
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = lds16(wb + (q * 8 + r) * kDnWRow);
#pragma unroll
    for (int n = 0; n < 4; ++n) B[n] = lds16(ldh[stage] + swz(wt * 64 + n * 16 + r16, q));
    transpose8x8(v, am);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      if (n * 16 < wrows) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j][n] = mfma16x16x32(am[j], B[n], acc[j][n]);
      }
    }
  };

  const int nk = I / kTBK;
  gload(sa, 0);
  if (nk > 1) gload(sb, kTBK);
  sstore(sa, 0);
  __syncthreads();
  for (int c = 0; c < nk; c += 2) {
    if (c + 2 < nk) gload(sa, (c + 2) * kTBK);
    compute(0);
    if (c + 1 < nk) sstore(sb, 1);
    __syncthreads();
    if (c + 1 >= nk) break;
    if (c + 3 < nk) gload(sb, (c + 3) * kTBK);
    compute(1);
    if (c + 2 < nk) sstore(sa, 0);
    __syncthreads();
  }

  // epilogue: tile j, C row 4q+i -> h = h0 + 128 wh + 8 (4q + i) + j
  uint16_t* obase = reinterpret_cast<uint16_t*>(ti.shared ? a.o_shared : a.o_routed);
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int row = wt * 64 + n * 16 + r16;
    if (row < ti.nrows) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 pk;
        pk.x = pack_bf16x2(acc[0][n][i], acc[1][n][i]);
        pk.y = pack_bf16x2(acc[2][n][i], acc[3][n][i]);
        pk.z = pack_bf16x2(acc[4][n][i], acc[5][n][i]);
        pk.w = pack_bf16x2(acc[6][n][i], acc[7][n][i]);
        st16(obase + (size_t)(ti.row0 + row) * H + h0 + wh * 128 + 8 * (4 * q + i), pk);
      }
    }
  }
}

hipError_t launch_experts_tiled_bf16(const ExpertArgs& a, hipStream_t s, const StageTimer* tm) {
  if (!a.tiles_ready) {
    stage_begin(tm, kTiles, s);
    const hipError_t e = launch_tiles(a, s);
    stage_end(tm, kTiles, s);
    if (e != hipSuccess) return e;
  }
  const int64_t tiles = max_expert_tiles(a.T, a.K, a.E, a.Is, a.tile_rows);
  const int imax = a.I > a.Is ? a.I : a.Is;
  const int gu_slices = (imax + 127) / 128;
  int64_t nb = tiles * gu_slices;
  nb = (nb + 7) / 8 * 8;
  stage_begin(tm, kGateUp, s);
  hipLaunchKernelGGL(k_gateup_tiled, dim3((unsigned)nb), dim3(256), 0, s, a, gu_slices, (int)nb);
  stage_end(tm, kGateUp, s);
  const int dn_slices = (a.H + kDnCols - 1) / kDnCols;
  nb = tiles * dn_slices;
  nb = (nb + 7) / 8 * 8;
  stage_begin(tm, kDown, s);
  hipLaunchKernelGGL(k_down_tiled, dim3((unsigned)nb), dim3(256), 0, s, a, dn_slices, (int)nb);
  stage_end(tm, kDown, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine_bf16(a, s, tm);
}

}  // namespace moe
