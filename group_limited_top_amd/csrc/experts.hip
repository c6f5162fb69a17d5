// experts.hip -- grouped SwiGLU experts, shared expert and weighted combine.
//
// [Routing §四]: gate_proj, up_proj and down_proj are each one stacked
// [E][I][H] tensor; every expert is down(silu(gate x) * up x).  [Routing §五]:
// the shared expert has the same form, runs on every token and is added to the
// weighted routed sum with no weight.
//
// Row space.  The T*K pairs are processed in expert-sorted order (row q of
// expert e is pair sorted_pair[q], q in [offsets[e], offsets[e+1])); the shared
// expert is handled as one more "expert" E whose rows are the T tokens.  Work
// is cut into tiles of kTileRows rows of one expert; the tile list is built on
// the device from offsets (no host synchronisation), and the launch grid is
// sized for the worst case (blocks past the last tile exit at once).
//
// Weight-streaming kernels (bf16).  With few rows per expert the projections
// are bound by reading the 1.5 GB of stacked weights once.  Each block owns a
// slice of one expert's weights and streams it straight from HBM into
// registers in MFMA operand layout, while the (few) token rows sit in LDS:
//   gate/up: A = weight rows (I index) with K = H contiguous, B = token rows;
//   down:    A = W_down^T; W_down[e] is [I][H] (H contiguous), so each lane
//            loads 8 consecutive h of 8 consecutive i and transposes the 8x8
//            bf16 block in registers, giving 8 MFMA tiles whose row m maps to
//            h = h0 + 8m + j.
#include "device.h"
#include "expert_tiles.h"
#include "kernels.h"

namespace moe {

int64_t max_expert_tiles(int64_t T, int64_t K, int E, int Is, int tile_rows) {
  const int64_t P = T * K;
  int64_t n = (P + tile_rows - 1) / tile_rows + E;
  if (Is > 0) n += (T + tile_rows - 1) / tile_rows;
  return n;
}

// Few rows per expert (on average fewer than kGRows / 2): stream each
// expert's weights once past its rows; otherwise run the LDS-pipelined MFMA
// GEMMs (bf16, shapes with gemm_shape_ok).
int expert_tile_rows(int64_t T, int K, int E, int I, int Is, int H, bool bf16) {
  return (bf16 && gemm_shape_ok(T, K, I, Is, H) && (T * K) / E >= kGRows / 2) ? kGRows : kTileRows;
}

// tile_off[g] = number of tiles of "experts" 0..g-1 (E + 1 of them, the last
// is the shared expert with T rows when Is > 0); tile_off[E + 1] = total;
// tile_tab = one entry per tile (write_tile_entry).
__global__ __launch_bounds__(1024) void k_tiles(const int32_t* __restrict__ offsets, int E, int T,
                                                 int Is, int tile_rows,
                                                 int32_t* __restrict__ tile_off,
                                                 int32_t* __restrict__ tile_tab) {
  __shared__ int32_t sc[1024];
  const int g = threadIdx.x;
  int32_t n = 0, rows = 0, first = 0;
  if (g < E) {
    first = offsets[g];
    rows = offsets[g + 1] - first;
    n = (rows + tile_rows - 1) / tile_rows;
  } else if (g == E && Is > 0) {
    rows = T;
    n = (T + tile_rows - 1) / tile_rows;
  }
  sc[g] = n;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int32_t add = (g >= d) ? sc[g - d] : 0;
    __syncthreads();
    sc[g] += add;
    __syncthreads();
  }
  if (g <= E) tile_off[g] = sc[g] - n;
  if (g == E) tile_off[E + 1] = sc[g];
  for (int32_t m = 0; m < n; ++m) write_tile_entry(tile_tab, sc[g] - n + m, g, first, rows, m, tile_rows);
}

hipError_t launch_tiles(const ExpertArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_tiles, dim3(1), dim3(1024), 0, s, a.offsets, a.E, a.T, a.Is, a.tile_rows,
                     a.tile_off, a.tile_tab);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// gate/up + SwiGLU, bf16.  Block: 4 waves, one tile of rows, 64 consecutive
// intermediate rows i (16 per wave) of both gate and up.  K = H is streamed in
// chunks of 256: weights go global -> registers (double-buffered), token rows
// global -> LDS (double-buffered).
// ----------------------------------------------------------------------------
constexpr int kGuChunk = 256;
constexpr int kGuRowU4 = kGuChunk / 8 + 1;  // 16-byte units per LDS row (+1: bank spread)
constexpr int kSub = kTileRows / 16;       // 16-row MFMA sub-tiles per tile

__global__ __launch_bounds__(256, 2) void k_gateup_bf16(const ExpertArgs a, int slices) {
  __shared__ u32x4 xs[2][kTileRows][kGuRowU4];
  const int slice = blockIdx.x % slices;
  TileInfo ti;
  if (!decode_tile(a, blockIdx.x / slices, ti)) return;
  const int I = ti.shared ? a.Is : a.I;
  const int i0 = slice * 64;
  if (i0 >= I) return;
  const int H = a.H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, r16 = lane & 15;

  // token-row staging: thread -> (row, 4 x 16 B of the chunk)
  const int sr = threadIdx.x >> 3, sc = (threadIdx.x & 7) * 4;
  const uint16_t* xrow = nullptr;
  if (sr < ti.nrows) {
    const int tok = ti.shared ? ti.row0 + sr : a.sorted_pair[ti.row0 + sr] / a.K;
    xrow = reinterpret_cast<const uint16_t*>(a.x) + (size_t)tok * H;
  }
  // weight rows of this lane
  const size_t ebase = ti.shared ? 0 : (size_t)ti.e * a.I * H;
  const int wrow = i0 + wave * 16 + r16;
  const uint16_t* wg = reinterpret_cast<const uint16_t*>(ti.shared ? a.ws_gate : a.w_gate) + ebase +
                       (size_t)wrow * H + q * 8;
  const uint16_t* wu = reinterpret_cast<const uint16_t*>(ti.shared ? a.ws_up : a.w_up) + ebase +
                       (size_t)wrow * H + q * 8;

  const int nchunks = H / kGuChunk;
  const int nsub = (ti.nrows + 15) >> 4;
  u32x4 ga[8], ua[8], gb[8], ub[8], xst[4];
  f32x4 accg[kSub], accu[kSub];
#pragma unroll
  for (int n = 0; n < kSub; ++n) {
    accg[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    accu[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  auto load_w = [&](u32x4* g, u32x4* u, int c) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      g[s] = ld16(wg + c * kGuChunk + s * 32);
      u[s] = ld16(wu + c * kGuChunk + s * 32);
    }
  };
  auto load_x = [&](int c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) xst[i] = xrow ? ld16(xrow + c * kGuChunk + (sc + i) * 8) : zero4;
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) xs[buf][sr][sc + i] = xst[i];
  };
  auto compute = [&](const u32x4* g, const u32x4* u, int buf) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int n = 0; n < kSub; ++n) {
        if (n < nsub) {
          const u32x4 b = xs[buf][n * 16 + r16][s * 4 + q];
          accg[n] = mfma16x16x32(g[s], b, accg[n]);
          accu[n] = mfma16x16x32(u[s], b, accu[n]);
        }
      }
    }
  };

  load_w(ga, ua, 0);
  load_x(0);
  store_x(0);
  __syncthreads();
  for (int c = 0; c < nchunks; c += 2) {
    if (c + 1 < nchunks) {
      load_w(gb, ub, c + 1);
      load_x(c + 1);
    }
    compute(ga, ua, 0);
    if (c + 1 < nchunks) store_x(1);
    __syncthreads();
    if (c + 1 >= nchunks) break;
    if (c + 2 < nchunks) {
      load_w(ga, ua, c + 2);
      load_x(c + 2);
    }
    compute(gb, ub, 1);
    if (c + 2 < nchunks) store_x(0);
    __syncthreads();
  }

  // epilogue: lane holds rows i = i0 + 16*wave + 4q + 0..3 of token row n*16 + r16
  uint16_t* hbase = reinterpret_cast<uint16_t*>(ti.shared ? a.h_shared : a.h_routed);
  const int ib = i0 + wave * 16 + 4 * q;
#pragma unroll
  for (int n = 0; n < kSub; ++n) {
    const int row = n * 16 + r16;
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

// ----------------------------------------------------------------------------
// down, bf16.  Block: 4 waves, one tile of rows, 512 output columns (128 per
// wave).  The tile's hidden rows h [rows][I] sit in LDS; W_down streams from
// HBM 8 x 16 B per lane per 32-deep k step and is transposed in registers.
// ----------------------------------------------------------------------------
__device__ __forceinline__ void transpose8x8_bf16(const u32x4 (&v)[8], u32x4 (&a)[8]) {
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

__global__ __launch_bounds__(256) void k_down_bf16(const ExpertArgs a, int hslices) {
  extern __shared__ u32x4 hs[];  // [kTileRows][I/8 + 1]
  const int hslice = blockIdx.x % hslices;
  TileInfo ti;
  if (!decode_tile(a, blockIdx.x / hslices, ti)) return;
  const int I = ti.shared ? a.Is : a.I;
  const int H = a.H;
  const int RS = I / 8 + 1;
  const uint16_t* hsrc = reinterpret_cast<const uint16_t*>(ti.shared ? a.h_shared : a.h_routed);
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  for (int v = threadIdx.x; v < kTileRows * (I / 8); v += 256) {
    const int r = v / (I / 8), c = v % (I / 8);
    hs[r * RS + c] = (r < ti.nrows) ? ld16(hsrc + (size_t)(ti.row0 + r) * I + c * 8) : zero4;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int h0 = hslice * 512 + wave * 128;
  if (h0 >= H) return;  // no barrier below
  const size_t ebase = ti.shared ? 0 : (size_t)ti.e * a.I * H;
  const uint16_t* wd = reinterpret_cast<const uint16_t*>(ti.shared ? a.ws_down : a.w_down) + ebase +
                       (size_t)(q * 8) * H + h0 + 8 * r16;
  const int nsub = (ti.nrows + 15) >> 4;
  f32x4 acc[8][kSub];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int n = 0; n < kSub; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 va[8], vb[8], vc[8], am[8];
  auto load = [&](u32x4 (&v)[8], int k0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = ld16_stream(wd + (size_t)(k0 + r) * H);
  };
  auto step = [&](const u32x4 (&v)[8], int k0) {
    transpose8x8_bf16(v, am);
#pragma unroll
    for (int n = 0; n < kSub; ++n) {
      if (n < nsub) {
        const u32x4 b = hs[(n * 16 + r16) * RS + k0 / 8 + q];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j][n] = mfma16x16x32(am[j], b, acc[j][n]);
      }
    }
  };
  // three 32-deep batches rotate: two are in flight while one is used
  load(va, 0);
  if (32 < I) load(vb, 32);
  for (int k0 = 0; k0 < I; k0 += 96) {
    if (k0 + 64 < I) load(vc, k0 + 64);
    step(va, k0);
    if (k0 + 32 >= I) break;
    if (k0 + 96 < I) load(va, k0 + 96);
    step(vb, k0 + 32);
    if (k0 + 64 >= I) break;
    if (k0 + 128 < I) load(vb, k0 + 128);
    step(vc, k0 + 64);
  }

  // epilogue: tile j, C row 4q+i -> h = h0 + 8*(4q+i) + j; 8 consecutive h per (n, i)
  uint16_t* obase = reinterpret_cast<uint16_t*>(ti.shared ? a.o_shared : a.o_routed);
#pragma unroll
  for (int n = 0; n < kSub; ++n) {
    const int row = n * 16 + r16;
    if (n < nsub && row < ti.nrows) {
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

// ----------------------------------------------------------------------------
// combine, bf16: y[t] = o_shared[t] + sum_j w[t][j] * o_routed[pair_slot[t*K+j]]
// in j order, fp32, one rounding.  [Routing §四] (weighted sum), §五 (shared
// output added as is).
// ----------------------------------------------------------------------------
// KT > 0: top_k == KT known at compile time (fewer registers: more waves in
// flight); KT == 0: any top_k <= 16.  A block takes NT consecutive tokens;
// each thread one 16-byte chunk of all their rows, every row load issued
// before any arithmetic.  The rows are read once: nontemporal loads (138.7 ->
// 112.6 us at 16384 tokens, 4.9 -> 6.0 TB/s).
template <int KT, int NT>
__global__ __launch_bounds__(256) void k_combine_bf16(const ExpertArgs a) {
  constexpr int kMaxK = KT > 0 ? KT : 16;  // top_k <= 16 (the supported envelope)
  const int K = KT > 0 ? KT : a.K;
  const int H = a.H, T = a.T;
  const int t0 = blockIdx.x * NT;
  const uint16_t* osh = reinterpret_cast<const uint16_t*>(a.o_shared);
  const uint16_t* orr = reinterpret_cast<const uint16_t*>(a.o_routed);
  uint16_t* y = reinterpret_cast<uint16_t*>(a.y);
  int32_t slot[NT][kMaxK];
  float wj[NT][kMaxK];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int t = min(t0 + u, T - 1);  // a token past the end repeats the last (not stored)
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      slot[u][j] = j < K ? a.pair_slot[(size_t)t * K + j] : -1;
      wj[u][j] = j < K ? a.topk_w[(size_t)t * K + j] : 0.0f;
    }
  }
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  for (int c = threadIdx.x; c < H / 8; c += blockDim.x) {
    u32x4 vs[NT], v[NT][kMaxK];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int t = min(t0 + u, T - 1);
      vs[u] = a.Is > 0 ? ld16_stream(osh + (size_t)t * H + c * 8) : zero4;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        v[u][j] = slot[u][j] >= 0 ? ld16_stream(orr + (size_t)slot[u][j] * H + c * 8) : zero4;
    }
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      if (t0 + u >= T) break;  // block-uniform
      float acc[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = bf16_lo(vs[u][i]);
        acc[2 * i + 1] = bf16_hi(vs[u][i]);
      }
      // j order, one product and one sum per term, as specified
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (slot[u][j] < 0) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = acc[2 * i] + wj[u][j] * bf16_lo(v[u][j][i]);
          acc[2 * i + 1] = acc[2 * i + 1] + wj[u][j] * bf16_hi(v[u][j][i]);
        }
      }
      u32x4 pk;
      pk.x = pack_bf16x2(acc[0], acc[1]);
      pk.y = pack_bf16x2(acc[2], acc[3]);
      pk.z = pack_bf16x2(acc[4], acc[5]);
      pk.w = pack_bf16x2(acc[6], acc[7]);
      st16(y + (size_t)(t0 + u) * H + c * 8, pk);
    }
  }
}

hipError_t launch_experts_bf16(const ExpertArgs& a, hipStream_t s, const StageTimer* tm) {
  if (a.tile_rows == kGRows) return launch_experts_gemm_bf16(a, s, tm);
  // the down kernel's LDS tile can exceed the 64 KiB default for I > 960
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(k_down_bf16), hipFuncAttributeMaxDynamicSharedMemorySize,
      kTileRows * (1024 / 8 + 1) * 16);
  if (attr != hipSuccess) return attr;
  if (!a.tiles_ready) {
    stage_begin(tm, kTiles, s);
    (void)launch_tiles(a, s);
    stage_end(tm, kTiles, s);
  }
  const int64_t tiles = max_expert_tiles(a.T, a.K, a.E, a.Is, a.tile_rows);
  const int imax = a.I > a.Is ? a.I : a.Is;
  if (stream_ring_ok(a)) {
    const hipError_t e = launch_gateup_stream_bf16(a, tiles, s, tm);
    if (e != hipSuccess) return e;
  } else {
    const int slices = imax / 64;
    stage_begin(tm, kGateUp, s);
    hipLaunchKernelGGL(k_gateup_bf16, dim3((unsigned)(tiles * slices)), dim3(256), 0, s, a, slices);
    stage_end(tm, kGateUp, s);
  }
  if (down_stream_ok(a)) {
    const hipError_t e = launch_down_stream_bf16(a, tiles, s, tm);
    if (e != hipSuccess) return e;
  } else {
    const int hslices = (a.H + 511) / 512;
    const size_t lds = (size_t)kTileRows * (imax / 8 + 1) * 16;
    stage_begin(tm, kDown, s);
    hipLaunchKernelGGL(k_down_bf16, dim3((unsigned)(tiles * hslices)), dim3(256), lds, s, a,
                       hslices);
    stage_end(tm, kDown, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_combine_bf16(a, s, tm);
}

const char* expert_stage_kernel(int stage, int64_t T, int K, int E, int I, int Is, int H,
                                bool bf16) {
  const bool tiled = expert_tile_rows(T, K, E, I, Is, H, bf16) == kGRows;
  ExpertArgs a{};
  a.T = (int)T;
  a.H = H;
  a.E = E;
  a.K = K;
  a.I = I;
  a.Is = Is;
  switch (stage) {
    case kGateUp:
      if (!bf16) return stream_f32_ok(a) ? "k_gateup_stream_f32" : "k_gateup_f32";
      if (tiled) return "k_expert_gemm<0>";
      return stream_ring_ok(a) ? "k_gateup_stream" : "k_gateup_bf16";
    case kDown:
      if (!bf16) return stream_f32_ok(a) ? "k_down_stream_f32" : "k_down_f32";
      if (tiled) return "k_expert_gemm<1>";
      return down_stream_ok(a) ? "k_down_stream" : "k_down_bf16";
    case kCombine: return bf16 ? "k_combine_bf16" : "k_combine_f32";
    default: return nullptr;
  }
}

#ifndef MOE_COMBINE_NT
#define MOE_COMBINE_NT 1
#endif
hipError_t launch_combine_bf16(const ExpertArgs& a, hipStream_t s, const StageTimer* tm) {
  stage_begin(tm, kCombine, s);
  if (a.K == 8) {
    constexpr int NT = MOE_COMBINE_NT;
    hipLaunchKernelGGL((k_combine_bf16<8, NT>), dim3((unsigned)((a.T + NT - 1) / NT)), dim3(256), 0,
                       s, a);
  } else {
    hipLaunchKernelGGL((k_combine_bf16<0, 1>), dim3((unsigned)a.T), dim3(256), 0, s, a);
  }
  stage_end(tm, kCombine, s);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// fp32 variants (small fp32 layers): weight streams on fp32 FMA.  The
// weights are read once, in 16-byte pieces with eight in flight per thread;
// only the tile's real rows are computed (a tile of a small layer holds a
// few rows of its expert), their activations broadcast from LDS.
// ----------------------------------------------------------------------------
constexpr int kF32KC = 256;  // K chunk of x staged in LDS (floats)
constexpr int kF32IC = 256;  // I chunk of h staged in LDS (floats)

// gate/up: block (256 threads) = one tile x 64 features; wave v streams the
// gate (v even) or up (v odd) rows i0 + lane over the first (v < 2) or second
// half of the K chunks, so that each wave's chain of dependent loads is half
// as long; the four partial sums meet in LDS (half 0 + half 1, in that order)
// for silu(g) u.
__global__ __launch_bounds__(256) void k_gateup_f32(const ExpertArgs a, int slices) {
  __shared__ __attribute__((aligned(16))) float xs[2][kTileRows][kF32KC];  // 64 KiB
  __shared__ int toks[kTileRows];  // the token of each row of the tile
  const int slice = blockIdx.x % slices;
  TileInfo ti;
  if (!decode_tile(a, blockIdx.x / slices, ti)) return;
  const int I = ti.shared ? a.Is : a.I;
  const int i0 = slice * 64;
  if (i0 >= I) return;  // block-uniform
  const int H = a.H, tid = threadIdx.x;
  const int f = tid & 63, wv = tid >> 6, half = wv >> 1, t128 = tid & 127;
  const bool up = (wv & 1) != 0;
  const bool has_row = i0 + f < I;
  const float* x = reinterpret_cast<const float*>(a.x);
  const size_t ebase = ti.shared ? 0 : (size_t)ti.e * a.I * H;
  const float* W = reinterpret_cast<const float*>(up ? (ti.shared ? a.ws_up : a.w_up)
                                                     : (ti.shared ? a.ws_gate : a.w_gate)) +
                   ebase + (size_t)min(i0 + f, I - 1) * H;
  const int nrows = ti.nrows;
  if (tid < nrows) toks[tid] = ti.shared ? ti.row0 + tid : a.sorted_pair[ti.row0 + tid] / a.K;
  __syncthreads();
  // K chunks [0, nh0) to half 0, [nh0, nch) to half 1; both halves take
  // nh0 rounds of barriers
  const int nch = (H + kF32KC - 1) / kF32KC, nh0 = (nch + 1) / 2;
  float (*xh)[kF32KC] = xs[half];
  // consecutive FMAs go to different rows: independent chains (with few
  // waves per SIMD nothing else hides a dependent FMA's latency)
  float acc[kTileRows];
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) acc[r] = 0.0f;
  for (int it = 0; it < nh0; ++it) {
    const int ch = half == 0 ? it : nh0 + it;
    const bool mine = ch < nch;  // wave-uniform
    const int k0 = ch * kF32KC;
    const int kc = mine ? min(kF32KC, H - k0) : 0;  // a multiple of 64
    // this half's x rows of the chunk, 16 bytes a piece: every load issued
    // before any LDS store (a piece past the end re-reads the last one,
    // stored nowhere)
    if (mine) {
      const int n = nrows * (kc / 4);
      constexpr int kPer = kTileRows * (kF32KC / 4) / 128;
      f32x4 tmp[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int v = min(t128 + 128 * j, n - 1);
        const int r = v / (kc / 4), c = v % (kc / 4);
        tmp[j] = *reinterpret_cast<const f32x4*>(x + (size_t)toks[r] * H + k0 + 4 * c);
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int v = t128 + 128 * j;
        if (v < n) *reinterpret_cast<f32x4*>(&xh[v / (kc / 4)][4 * (v % (kc / 4))]) = tmp[j];
      }
    }
    __syncthreads();
    if (mine && has_row) {
      // 32 floats a batch; the next batch's loads are in flight while this
      // one is used (kc is a multiple of 64: batches come in pairs)
      f32x4 wa[8], wb[8];
      auto fetch = [&](f32x4 (&w)[8], int k) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 8; ++u) w[u] = *reinterpret_cast<const f32x4*>(W + k0 + k + 4 * u);
      };
      // rows in groups of 8, one (uniform) test a group: rows past the
      // tile's end compute on LDS contents nobody stores
      auto use = [&](const f32x4 (&w)[8], int k) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < kTileRows; g += 8) {
          if (g >= nrows) continue;  // (not break: the loop must unroll, acc stays in registers)
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            f32x4 xv[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) xv[r] = *reinterpret_cast<const f32x4*>(&xh[g + r][k + 4 * u]);
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
              for (int r = 0; r < 8; ++r) acc[g + r] = __builtin_fmaf(w[u][c], xv[r][c], acc[g + r]);
          }
        }
      };
      fetch(wa, 0);
      for (int k = 0; k < kc; k += 64) {
        fetch(wb, k + 32);
        use(wa, k);
        if (k + 64 < kc) fetch(wa, k + 64);
        use(wb, k + 32);
      }
    }
    __syncthreads();
  }
  // partial sums to LDS (xs is free after the last barrier): ps[v][r][f]
  float (*ps)[kTileRows][64] = reinterpret_cast<float (*)[kTileRows][64]>(&xs[0][0][0]);
  if (wv != 0) {
#pragma unroll
    for (int r = 0; r < kTileRows; ++r)
      if (r < nrows) ps[wv][r][f] = acc[r];
  }
  __syncthreads();
  if (wv == 0 && has_row) {
    float* h = reinterpret_cast<float*>(ti.shared ? a.h_shared : a.h_routed);
#pragma unroll
    for (int r = 0; r < kTileRows; ++r)
      if (r < nrows) {
        const float g = acc[r] + ps[2][r][f];
        const float u = ps[1][r][f] + ps[3][r][f];
        h[(size_t)(ti.row0 + r) * I + i0 + f] = silu_f32(g) * u;
      }
  }
}

// down: block (4 waves) = one tile x 512 output columns; thread t mod 128 =
// 4 consecutive columns, streaming W_down's rows (coalesced 16-byte loads);
// the first two waves take the first half of each I chunk, the other two the
// second half, so that each wave's chain of dependent loads is half as long.
// The halves' sums meet in LDS (half 0 + half 1).
__global__ __launch_bounds__(256) void k_down_f32(const ExpertArgs a, int hslices) {
  __shared__ __attribute__((aligned(16))) float hsm[kTileRows][kF32IC];  // 32 KiB
  const int hslice = blockIdx.x % hslices;
  TileInfo ti;
  if (!decode_tile(a, blockIdx.x / hslices, ti)) return;
  const int I = ti.shared ? a.Is : a.I;
  const int H = a.H, tid = threadIdx.x, t128 = tid & 127, half = tid >> 7;
  const int c0 = hslice * 512 + 4 * t128;
  const bool has_col = c0 < H;  // H is a multiple of 64
  const float* hsrc = reinterpret_cast<const float*>(ti.shared ? a.h_shared : a.h_routed);
  const size_t ebase = ti.shared ? 0 : (size_t)ti.e * a.I * H;
  const float* Wd = reinterpret_cast<const float*>(ti.shared ? a.ws_down : a.w_down) + ebase +
                    min(c0, H - 4);
  const int nrows = ti.nrows;
  f32x4 acc[kTileRows];
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < I; k0 += kF32IC) {
    const int kc = min(kF32IC, I - k0);  // a multiple of 64
    {  // every load issued before any LDS store (as in k_gateup_f32)
      const int n = nrows * (kc / 4);
      constexpr int kPer = kTileRows * (kF32IC / 4) / 256;
      f32x4 tmp[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int v = min(tid + 256 * j, n - 1);
        tmp[j] = *reinterpret_cast<const f32x4*>(hsrc + (size_t)(ti.row0 + v / (kc / 4)) * I + k0 +
                                                 4 * (v % (kc / 4)));
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int v = tid + 256 * j;
        if (v < n) *reinterpret_cast<f32x4*>(&hsm[v / (kc / 4)][4 * (v % (kc / 4))]) = tmp[j];
      }
    }
    __syncthreads();
    if (has_col) {
      const int kb = half * (kc / 2), ke = kb + kc / 2;  // this half's k range (multiples of 32)
      for (int k = kb; k < ke; k += 8) {
        f32x4 w[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) w[u] = *reinterpret_cast<const f32x4*>(Wd + (size_t)(k0 + k + u) * H);
        // consecutive FMAs on different rows (independent chains), rows in
        // groups of 8 with one uniform test a group (as in k_gateup_f32)
#pragma unroll
        for (int g = 0; g < kTileRows; g += 8) {
          if (g >= nrows) continue;
#pragma unroll
          for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int r = g; r < g + 8; ++r) {
              const float hv = hsm[r][k + u];
#pragma unroll
              for (int c = 0; c < 4; ++c) acc[r][c] = __builtin_fmaf(hv, w[u][c], acc[r][c]);
            }
        }
      }
    }
    __syncthreads();
  }
  // the halves meet, 16 rows a round through hsm (free after the last barrier)
  f32x4 (*red)[128] = reinterpret_cast<f32x4 (*)[128]>(&hsm[0][0]);  // [16][128]
  float* o = reinterpret_cast<float*>(ti.shared ? a.o_shared : a.o_routed);
#pragma unroll
  for (int g = 0; g < kTileRows; g += 16) {
    if (g >= nrows) break;  // block-uniform
    if (half == 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (g + r < nrows) red[r][t128] = acc[g + r];
    }
    __syncthreads();
    if (half == 0 && has_col) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (g + r < nrows) {
          const f32x4 b = red[r][t128];
          f32x4 v;
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = acc[g + r][c] + b[c];
          *reinterpret_cast<f32x4*>(o + (size_t)(ti.row0 + g + r) * H + c0) = v;
        }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_combine_f32(const ExpertArgs a) {
  constexpr int kMaxK = 16;  // top_k <= 16 (the supported envelope)
  const int t = blockIdx.x;
  const int H = a.H, K = a.K;
  const float* osh = reinterpret_cast<const float*>(a.o_shared);
  const float* orr = reinterpret_cast<const float*>(a.o_routed);
  float* y = reinterpret_cast<float*>(a.y);
  // the token's pair slots and weights, then every row load before any use,
  // so that the K + 1 loads are in flight together (as in k_combine_bf16)
  int32_t slot[kMaxK];
  float wj[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    slot[j] = j < K ? a.pair_slot[(size_t)t * K + j] : -1;
    wj[j] = j < K ? a.topk_w[(size_t)t * K + j] : 0.0f;
  }
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  for (int c = threadIdx.x; c < H / 4; c += blockDim.x) {
    const f32x4 vs = a.Is > 0 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(osh + (size_t)t * H + 4 * c)) : zero4;
    f32x4 v[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      v[j] = slot[j] >= 0 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(orr + (size_t)slot[j] * H + 4 * c)) : zero4;
    // j order, one product and one sum per term, as specified
    f32x4 acc = vs;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (slot[j] < 0) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = acc[i] + wj[j] * v[j][i];
    }
    *reinterpret_cast<f32x4*>(y + (size_t)t * H + 4 * c) = acc;
  }
}

hipError_t launch_experts_f32(const ExpertArgs& a, hipStream_t s, const StageTimer* tm) {
  if (!a.tiles_ready) {
    stage_begin(tm, kTiles, s);
    (void)launch_tiles(a, s);
    stage_end(tm, kTiles, s);
  }
  const int64_t tiles = max_expert_tiles(a.T, a.K, a.E, a.Is, a.tile_rows);
  if (stream_f32_ok(a)) {
    const hipError_t e = launch_stream_f32(a, tiles, s, tm);
    if (e != hipSuccess) return e;
  } else {
    const int imax = a.I > a.Is ? a.I : a.Is;
    const int slices = imax / 64;
    stage_begin(tm, kGateUp, s);
    hipLaunchKernelGGL(k_gateup_f32, dim3((unsigned)(tiles * slices)), dim3(256), 0, s, a, slices);
    stage_end(tm, kGateUp, s);
    const int hslices = (a.H + 511) / 512;
    stage_begin(tm, kDown, s);
    hipLaunchKernelGGL(k_down_f32, dim3((unsigned)(tiles * hslices)), dim3(256), 0, s, a, hslices);
    stage_end(tm, kDown, s);
  }
  stage_begin(tm, kCombine, s);
  hipLaunchKernelGGL(k_combine_f32, dim3((unsigned)a.T), dim3(256), 0, s, a);
  stage_end(tm, kCombine, s);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// residual + RMSNorm (for stacking layers; gamma = 1), one block per row
// ----------------------------------------------------------------------------
// Rows too wide to keep in registers (bf16 beyond 32768 features): two passes,
// the second reading x_out back.
template <bool BF16>
__global__ __launch_bounds__(256) void k_residual_rmsnorm(const void* x_in, const void* y,
                                                           void* x_out, void* r_out, int H,
                                                           float eps) {
  __shared__ float red[256];
  const int t = blockIdx.x;
  float ss = 0.0f;
  // pass 1: x_out = RN(x + y), sum of squares of the rounded values
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    const size_t i = (size_t)t * H + h;
    float v;
    if (BF16) {
      v = bf16_to_f32(reinterpret_cast<const uint16_t*>(x_in)[i]);
      if (y) v = v + bf16_to_f32(reinterpret_cast<const uint16_t*>(y)[i]);
      const uint32_t b = f32_to_bf16_bits(v);
      reinterpret_cast<uint16_t*>(x_out)[i] = (uint16_t)b;
      v = bf16_to_f32((uint16_t)b);
    } else {
      v = reinterpret_cast<const float*>(x_in)[i];
      if (y) v = v + reinterpret_cast<const float*>(y)[i];
      reinterpret_cast<float*>(x_out)[i] = v;
    }
    ss = __builtin_fmaf(v, v, ss);
  }
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int d = 128; d > 0; d >>= 1) {
    if (threadIdx.x < d) red[threadIdx.x] += red[threadIdx.x + d];
    __syncthreads();
  }
  const float inv = 1.0f / sqrtf(red[0] / (float)H + eps);
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    const size_t i = (size_t)t * H + h;
    if (BF16) {
      const float v = bf16_to_f32(reinterpret_cast<const uint16_t*>(x_out)[i]);
      reinterpret_cast<uint16_t*>(r_out)[i] = (uint16_t)f32_to_bf16_bits(v * inv);
    } else {
      const float v = reinterpret_cast<const float*>(x_out)[i];
      reinterpret_cast<float*>(r_out)[i] = v * inv;
    }
  }
}

// The same with the row in registers: thread i holds 16-byte chunks i, i + 256,
// ... (NC of them), so x_out is written once and never read back; sums: each
// thread's elements in order, then the wave (butterfly), then the 4 waves in
// order.
template <bool BF16, int NC>
__global__ __launch_bounds__(256) void k_residual_rmsnorm_reg(const void* x_in, const void* y,
                                                               void* x_out, void* r_out, int H,
                                                               float eps) {
  constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int nch = H / EPC;
  const size_t row = (size_t)t * nch;  // chunk index of the row's start
  const u32x4* xi = reinterpret_cast<const u32x4*>(x_in) + row;
  const u32x4* yi = y ? reinterpret_cast<const u32x4*>(y) + row : nullptr;
  u32x4* xo = reinterpret_cast<u32x4*>(x_out) + row;
  u32x4* ro = reinterpret_cast<u32x4*>(r_out) + row;
  float v[NC][EPC];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c = tid + 256 * j;
    if (c >= nch) continue;
    const u32x4 a = xi[c];
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    const u32x4 b = yi ? yi[c] : zero4;
    u32x4 out;
    if (BF16) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float lo = bf16_lo(a[k]), hi = bf16_hi(a[k]);
        if (yi) {
          lo = lo + bf16_lo(b[k]);
          hi = hi + bf16_hi(b[k]);
        }
        out[k] = pack_bf16x2(lo, hi);
        v[j][2 * k] = bf16_lo(out[k]);
        v[j][2 * k + 1] = bf16_hi(out[k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float f = __uint_as_float(a[k]);
        if (yi) f = f + __uint_as_float(b[k]);
        v[j][k] = f;
        out[k] = __float_as_uint(f);
      }
    }
    xo[c] = out;
#pragma unroll
    for (int k = 0; k < EPC; ++k) ss = __builtin_fmaf(v[j][k], v[j][k], ss);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) ss += __shfl_xor(ss, o, 64);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float tot = ((red[0] + red[1]) + red[2]) + red[3];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c = tid + 256 * j;
    if (c >= nch) continue;
    u32x4 out;
    if (BF16) {
#pragma unroll
      for (int k = 0; k < 4; ++k) out[k] = pack_bf16x2(v[j][2 * k] * inv, v[j][2 * k + 1] * inv);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) out[k] = __float_as_uint(v[j][k] * inv);
    }
    ro[c] = out;
  }
}

hipError_t launch_residual_rmsnorm(bool bf16, const void* x_in, const void* y, void* x_out,
                                   void* r_out, int T, int H, float eps, hipStream_t s) {
  const int nch = H / (bf16 ? 8 : 4);
  const int per = (nch + 255) / 256;  // chunks per thread
  const dim3 g((unsigned)T), b(256);
#define MOE_RMS(B, N) hipLaunchKernelGGL((k_residual_rmsnorm_reg<B, N>), g, b, 0, s, x_in, y, x_out, r_out, H, eps)
  if (bf16) {
    if (per <= 1) MOE_RMS(true, 1);
    else if (per <= 2) MOE_RMS(true, 2);
    else if (per <= 4) MOE_RMS(true, 4);
    else if (per <= 8) MOE_RMS(true, 8);
    else if (per <= 16) MOE_RMS(true, 16);
    else hipLaunchKernelGGL(k_residual_rmsnorm<true>, g, b, 0, s, x_in, y, x_out, r_out, H, eps);
  } else {
    if (per <= 1) MOE_RMS(false, 1);
    else if (per <= 2) MOE_RMS(false, 2);
    else if (per <= 4) MOE_RMS(false, 4);
    else if (per <= 8) MOE_RMS(false, 8);
    else if (per <= 16) MOE_RMS(false, 16);
    else hipLaunchKernelGGL(k_residual_rmsnorm<false>, g, b, 0, s, x_in, y, x_out, r_out, H, eps);
  }
#undef MOE_RMS
  return hipGetLastError();
}

}  // namespace moe
