// backward.hip -- backward of the MoE layer for the routing the forward chose.
//
// The layer ([Routing §二 steps 1-3, §四, §五]) with the chosen experts held
// fixed (the choice is piecewise constant and carries no gradient; the expert
// bias only enters the choice):
//   s = sigmoid(lam), w_j = scale * s_j / (sum_k s_k + 1e-20) over the chosen
//   experts, y = shared(x) + sum_j w_j * down(silu(gate x) * up x).
// For an upstream gradient dy, with r = dy . W_down^T (per pair):
//   dL/dw_j = <dy, expert_j(x)> = <a_j, r_j>  (a = silu(g) * u), d_a = w_j r_j,
//   d_g = d_a * u * silu'(g), d_u = d_a * silu(g),
//   dx   = sum over pairs of d_g . W_gate + d_u . W_up   (+ the shared expert)
//          + sum_j dlam_j * W_r[e_j],
//   dW_gate[e] = sum over e's pairs of d_g^T x, dW_up likewise with d_u,
//   dW_down[e] = sum over e's pairs of (w_j a_j)^T dy,
//   dlam_m = scale / D * (dL/dw_m - sum_j dL/dw_j s_j / D) * s_m (1 - s_m),
//   dW_r[e] = sum over e's pairs of dlam * x.
// Rows are the expert-sorted pairs (then the T shared rows), as in the forward.
//
// Steps: permute (the forward's kernels) -> k_bwd_gemm<kRowsNT> (g = x W_g^T,
// u = x W_u^T, r = dy W_d^T, fp32) -> k_bwd_act (per row: a, dL/dw, d_g, d_u,
// w a in bf16) -> k_bwd_router (per token: dlam) -> k_bwd_gemm<kRowsNN>
// (per-row dx = d_g W_g + d_u W_u, bf16) ->
// k_bwd_wgrad<2, 64> (dW_gate, dW_up) and k_bwd_wgrad<1, *> (dW_down) per
// expert, fp32, summed over the expert's rows in order ->
// k_bwd_router_wgrad + k_bwd_router_reduce
// (dW_r = dlogit^T x over token chunks, then the chunks in order) ->
// k_bwd_combine (dx per token: shared row, then the K pair rows in j order,
// then the router's share sum_j dlam_j W_r[e_j] in j order, fp32, one
// rounding).  Every sum has a fixed order: the results are bit-reproducible.
// With many rows per expert (bwd_tile_rows == kGRows) the two row products
// run on the forward's persistent DMA-ring expert GEMM instead (k_expert_gemm
// modes 2-4, 256-row tiles; launch_bwd_gur_gemm, launch_bwd_dx_gemm).
//
// Block order: the row-tile GEMMs give each XCD a contiguous run of (row
// tile, column tile) items, expert by expert and column-major within one, so
// the tiles of one expert run together on one XCD and those sharing a weight
// slab start together (they read it once into that XCD's L2); the
// weight-gradient kernels start the shared expert's long tiles first (spread
// over the XCDs) and then give each XCD a contiguous run of routed experts.
//
// The GEMM tile: 64 x BN outputs (BN = 256, or 64 where a width is not a
// multiple of 256), 4 waves each owning all 64 rows x BN / 4 columns (4 x
// BN / 64 MFMA 16x16x32 tiles), operands staged in LDS through registers
// (double buffer).  An operand whose rows are K-contiguous in memory ("KC") is
// staged as [row][k] and read with ds_read_b128; one stored [k][row] ("RC") is
// staged as is and read with the gfx950 transpose read, which hands each lane
// 4 consecutive k of one row.  K steps are 64 deep in the g/u/r GEMM, whose
// operands are both KC, so every staged row is a whole 128-byte line (half
// lines halve what the load path delivers); 32 deep in the other two, whose
// wide operand is RC with 512-byte rows (there the smaller LDS footprint,
// more blocks per CU, measured faster).
#include <algorithm>

#include "backward.h"
#include "device.h"
#include "expert_tiles.h"
#include "kernels.h"
#include "ring.h"

namespace moe {

namespace {

constexpr int kBM = 64;
constexpr int kBT = 256;  // threads per GEMM block

enum BwdGemm { kRowsNT = 0, kRowsNN = 1 };

// KC staging: row r, 16-byte chunk c.  64-deep steps (8 chunks, one 128-byte
// line a row): chunk XOR (r / 2) % 8 puts the 16 rows one read covers at one
// logical chunk on 16 distinct 4-bank groups (row parity x 8 positions).
// 32-deep steps (4 chunks): chunk XOR (r / 4) % 4 does the same for 64-byte
// rows.
template <int BK>
__device__ __forceinline__ int kc_off(int r, int c) {
  return BK == 64 ? r * 128 + ((c ^ ((r >> 1) & 7)) << 4) : r * 64 + ((c ^ ((r >> 2) & 3)) << 4);
}
// RC staging: k row (of 32), 16-byte chunk c (of 8); the XOR spreads the 16 k
// rows one transpose read covers over 4 chunk pairs (2 rows each).
__device__ __forceinline__ int rc_swz(int k) { return 2 * (((k >> 1) & 1) | (((k >> 3) & 1) << 1)); }
__device__ __forceinline__ int rc_off(int k, int c) { return k * 128 + ((c ^ rc_swz(k)) << 4); }
// RC staging of a 256-wide operand (rows of 512 bytes, 32 chunks): the 16 k
// rows of one transpose read start on the same bank, so the XOR spreads them
// over 8 chunk pairs (rows 8 q + c and 8 (q + 2) + c share one).
__device__ __forceinline__ int rcw_swz(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }
__device__ __forceinline__ int rcw_off(int k, int c) { return k * 512 + ((c ^ rcw_swz(k)) << 4); }

__device__ __forceinline__ float sigm(float z) { return 1.0f / (1.0f + __expf(-z)); }

// Block b of a grid of n blocks (n a multiple of 8) -> work item: blocks are
// dealt to the 8 XCDs in turn, so XCD b % 8 gets items (b % 8) n / 8 + b / 8,
// a contiguous run.
__device__ __forceinline__ int xcd_item(int b, int n) { return (b & 7) * (n >> 3) + (b >> 3); }

struct BwdArgs {
  int T, H, E, K, I, P;  // P = T * K routed rows
  int rtiles;            // row tiles the grids cover (a bound on the real count)
  float scale;
  const uint16_t* x;     // [T][H]
  const uint16_t* dy;    // [T][H]
  const float* logits;   // [T][E]
  const int32_t* idx;    // [T][K]
  const float* w_router; // [E][H]
  const uint16_t *wg, *wu, *wd;     // [E][I][H]
  const uint16_t *swg, *swu, *swd;  // [I][H] (shared) or null
  // permute
  const int32_t* offsets;      // [E+1]
  const int32_t* sorted_pair;  // [P]
  const int32_t* pair_slot;    // [P]
  const int32_t* tile_off;     // [E+2]
  const int32_t* tile_tab;     // row tiles {e | nrows << 16, row0}
  // intermediates (rows: P routed in sorted order, then T shared)
  float *g, *u, *r;            // [P+T][I]
  uint16_t *dg, *du, *aw;      // [P+T][I] bf16
  float* gw;                   // [P] dL/dw per pair id
  float* dlam;                 // [P] dL/dlam per pair id
  uint16_t* dxp;               // [P+T][H] bf16
  // outputs
  uint16_t* dx;                // [T][H]
  float* dw_router;            // [E][H]
  float *dwg, *dwu, *dwd;      // [E][I][H]
  float *dswg, *dswu, *dswd;   // [I][H] or null
};

__device__ __forceinline__ void decode_row_tile(const BwdArgs& a, int t, int& e, int& row0,
                                                int& nrows, int& orow) {
  const int32_t v = a.tile_tab[2 * t];
  e = v & 0xffff;
  nrows = v >> 16;
  row0 = a.tile_tab[2 * t + 1];
  orow = e < a.E ? row0 : a.P + row0;  // row in the intermediates
}

// Fragment reads (lane (q, i) = (lane / 16, lane % 16)); KC: half h of the
// 64-deep step is chunks 4 h .. 4 h + 3.
template <int BK>
__device__ __forceinline__ u32x4 read_kc(const uint8_t* buf, int r0, int h, int lane) {
  const int q = lane >> 4, i = lane & 15;
  return lds16(buf + kc_off<BK>(r0 + i, 4 * h + q));
}
// RC operand of width W (64: 128-byte rows, 256: 512-byte rows)
template <int W>
__device__ __forceinline__ u32x4 read_rc(const uint8_t* buf, int r0, int lane) {
  // lane 4 c + m of group q points at k row 8 q + c, rows r0 + 4 m .. + 3
  const int q = lane >> 4, i = lane & 15, c = i >> 2, m = i & 3;
  const int k = 8 * q + c;
  const int col = r0 + 4 * m;
  const int sw = W == 64 ? rc_swz(k) : rcw_swz(k);
  const uint8_t* p = buf + k * (2 * W) + (((col >> 3) ^ sw) << 4) + ((col & 4) << 1);
  const u32x2 lo = lds_tr16(p), hi = lds_tr16(p + 4 * 2 * W);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

}  // namespace

// One 64 x BN output tile.  MODE:
//   kRowsNT: blockIdx.x = row tile, blockIdx.y = column tile over 3 I-wide
//            segments: (x, W_g) -> g, (x, W_u) -> u, (dy, W_d) -> r; fp32 out.
//            A rows gathered (token of each pair), B = weight rows; both KC.
//   kRowsNN: blockIdx.x = row tile, blockIdx.y = column tile over H;
//            K = 2 I: (d_g, W_g) then (d_u, W_u); A KC, B RC (weights
//            [k][column]); bf16 out (per-row dx).
template <int MODE, int BN>
__global__ __launch_bounds__(kBT, 2) void k_bwd_gemm(const BwdArgs a) {
  constexpr int TN = BN / 64;                  // MFMA column tiles per wave
  constexpr int BK = MODE == kRowsNT ? 64 : 32;  // K depth of a step
  constexpr int NH = BK / 32;                  // MFMA k blocks per step
  constexpr int NA = BK / 32;                  // A chunks staged per thread
  constexpr int NB = BN * BK / 2048;           // B chunks staged per thread
  __shared__ __attribute__((aligned(16))) uint8_t sa[2][kBM * BK * 2];
  __shared__ __attribute__((aligned(16))) uint8_t sb[2][BN * BK * 2];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, I = a.I, K = a.K, E = a.E;

  int e = 0, row0 = 0, nrows = 0, orow = 0, n0 = 0, seg = 0, kdim = 0;
  {
    // items expert by expert; within an expert column-major, so the row
    // tiles that share a weight slab are consecutive: they start together and
    // read the slab's K window from L2 (row-major, they started up to most of
    // a tile's run apart and the expert's slabs did not fit the XCD's L2)
    const int ncol = MODE == kRowsNT ? 3 * I / BN : H / BN;
    const int w = xcd_item(blockIdx.x, gridDim.x);
    if (w >= a.tile_off[E + 1] * ncol) return;  // past the real tile count
    const int g = upper_bound_i32(a.tile_off, E + 2, w / ncol) - 1;
    const int t0 = a.tile_off[g], nt = a.tile_off[g + 1] - t0;
    const int local = w - t0 * ncol;
    const int t = t0 + local % nt, ct = local / nt;
    decode_row_tile(a, t, e, row0, nrows, orow);
    if (MODE == kRowsNT) {
      const int per = I / BN;
      seg = ct / per;
      n0 = (ct % per) * BN;
      kdim = H;
    } else {
      n0 = ct * BN;
      kdim = 2 * I;
    }
  }
  const bool sh = e >= E;
  const size_t ebase = sh ? 0 : (size_t)e * I * H;

  // Staging (chunk = 16 bytes):
  //   KC (CA = BK / 8 chunks a row): A rows tid / CA + (256 / CA) u, chunk
  //     tid % CA; kRowsNT B rows likewise.
  //   kRowsNN B (RC, BK k rows of BN / 8 chunks): k row n / (BN / 8), chunk
  //     n % (BN / 8) for n = tid + 256 u.
  constexpr int CA = BK / 8, RS = 256 / CA;
  const int kr = tid / CA, kc = tid % CA;
  const uint16_t* a_row[NA] = {};
  const uint16_t* a_row2[NA] = {};  // kRowsNN: d_u rows
  const uint16_t* b_row[NB] = {};   // kRowsNT: weight rows
  if (MODE == kRowsNT) {
#pragma unroll
    for (int u = 0; u < NA; ++u) {
      const int m = min(kr + RS * u, nrows - 1);
      const int tok = sh ? row0 + m : a.sorted_pair[row0 + m] / K;
      a_row[u] = (seg < 2 ? a.x : a.dy) + (size_t)tok * H + 8 * kc;
    }
    const uint16_t* wsrc = seg == 0 ? (sh ? a.swg : a.wg) : seg == 1 ? (sh ? a.swu : a.wu)
                                                                      : (sh ? a.swd : a.wd);
#pragma unroll
    for (int u = 0; u < NB; ++u) b_row[u] = wsrc + ebase + (size_t)(n0 + kr + RS * u) * H + 8 * kc;
  } else if (MODE == kRowsNN) {
#pragma unroll
    for (int u = 0; u < NA; ++u) {
      const int m = min(kr + RS * u, nrows - 1);
      a_row[u] = a.dg + (size_t)(orow + m) * I + 8 * kc;
      a_row2[u] = a.du + (size_t)(orow + m) * I + 8 * kc;
    }
  }
  constexpr int CPR = BN / 8;  // kRowsNN B: chunks per k row

  auto load = [&](int k0, u32x4 (&va)[NA], u32x4 (&vb)[NB]) __attribute__((always_inline)) {
    if (MODE == kRowsNT) {
#pragma unroll
      for (int u = 0; u < NA; ++u) va[u] = ld16(a_row[u] + k0);
#pragma unroll
      for (int u = 0; u < NB; ++u) vb[u] = ld16(b_row[u] + k0);
    } else if (MODE == kRowsNN) {
      const bool second = k0 >= I;
      const int kk = second ? k0 - I : k0;
#pragma unroll
      for (int u = 0; u < NA; ++u) va[u] = ld16((second ? a_row2[u] : a_row[u]) + kk);
      const uint16_t* w = (second ? (sh ? a.swu : a.wu) : (sh ? a.swg : a.wg)) + ebase +
                          (size_t)kk * H + n0;
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int n = tid + 256 * u;
        vb[u] = ld16(w + (size_t)(n / CPR) * H + 8 * (n % CPR));
      }
    }
  };
  auto stage = [&](int buf, const u32x4 (&va)[NA], const u32x4 (&vb)[NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NA; ++u) st16(sa[buf] + kc_off<BK>(kr + RS * u, kc), va[u]);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (MODE == kRowsNT) {
        st16(sb[buf] + kc_off<BK>(kr + RS * u, kc), vb[u]);
      } else {
        const int n = tid + 256 * u;
        if (BN == 64) st16(sb[buf] + rc_off(n / CPR, n % CPR), vb[u]);
        else st16(sb[buf] + rcw_off(n / CPR, n % CPR), vb[u]);
      }
    }
  };

  f32x4 acc[4][TN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (kdim + BK - 1) / BK;
  auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      u32x4 fa[4], fb[TN];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        fa[t] = read_kc<BK>(sa[buf], 16 * t, h, lane);
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int rb = wv * (BN / 4) + 16 * t;
        fb[t] = MODE == kRowsNT ? read_kc<BK>(sb[buf], rb, h, lane)
                                : read_rc<BN>(sb[buf] + h * 32 * 2 * BN, rb, lane);
      }
      // the column side as the MFMA's row operand: each lane ends with 4
      // consecutive output columns of one row (one wide store)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x32(fb[j], fa[i], acc[i][j]);
    }
  };
  // Loads run two steps ahead of the MFMAs and LDS stores one: at step s the
  // register set staged at the end of step s - 1 takes step s + 2's loads,
  // and the set loaded at step s - 1 is staged for step s + 1.  The step count
  // is even (H / 64 and 2 I / 32) and nothing in the loop is conditional
  // (loads past the last step repeat it, stores past it go to the free
  // buffer), so the compiler's load waits count only the older set.
  u32x4 va0[NA], vb0[NB], va1[NA], vb1[NB];
  auto step = [&](int s, u32x4 (&fa)[NA], u32x4 (&fb)[NB], const u32x4 (&la)[NA],
                  const u32x4 (&lb)[NB]) __attribute__((always_inline)) {
    load(min(s + 2, nk - 1) * BK, fa, fb);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
    compute(s & 1);
    stage((s + 1) & 1, la, lb);
    __syncthreads();
  };
  load(0, va0, vb0);
  stage(0, va0, vb0);
  load(min(1, nk - 1) * BK, va1, vb1);
  __syncthreads();
  for (int s = 0; s < nk; s += 2) {
    step(s, va0, vb0, va1, vb1);
    step(s + 1, va1, vb1, va0, vb0);
  }

  // acc[i][j][c] = C[A row 16 i + r16][B row wv * BN / 4 + 16 j + 4 q + c]
  const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ar = 16 * i + r16;  // A row in the tile
    if (ar >= nrows) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int bc = wv * (BN / 4) + 16 * j + 4 * q;  // first of 4 B rows in the tile
      if (MODE == kRowsNT) {
        float* out = seg == 0 ? a.g : seg == 1 ? a.u : a.r;
        *reinterpret_cast<f32x4*>(out + (size_t)(orow + ar) * I + n0 + bc) = acc[i][j];
      } else {
        u32x2 pk;
        pk.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        pk.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<u32x2*>(a.dxp + (size_t)(orow + ar) * H + n0 + bc) = pk;
      }
    }
  }
}

// Weight gradients, K = the expert's rows (32 a step).  NSEG = 2: dW_gate and
// dW_up from d_g, d_u against the same x rows (x staged once for both), AW =
// 64 features; NSEG = 1: dW_down from w a against dy rows, AW = 128 (or 64).
// Tile: NSEG x AW features x 256 h; wave w owns h 64 w .. + 63 of every
// feature.  The MFMA takes the h side as its row operand, so each lane ends
// with 4 consecutive h of one feature: one 16-byte store.  All operands are
// RC (rows of the expert), staged as is and read with the transpose read.
// Items: the shared expert's first (its K is T; blocks dealt round the
// XCDs), then the routed experts', each XCD a contiguous run of them.
template <int NSEG, int AW>
__global__ __launch_bounds__(256, 2) void k_bwd_wgrad(const BwdArgs a) {
  constexpr int NT = AW / 16;               // feature tiles per segment
  constexpr int NAC = AW / 64;              // A chunks staged per thread per segment
  __shared__ __attribute__((aligned(16))) uint8_t sa[2][NSEG][32 * AW * 2];
  __shared__ __attribute__((aligned(16))) uint8_t sb[2][32 * 512];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, I = a.I, K = a.K, E = a.E;
  const int nh = H / 256, per = (I / AW) * nh;
  const int ns = a.swg ? per : 0, ns8 = (ns + 7) & ~7;
  int e, w;
  const int b = blockIdx.x;
  if (b < ns8) {
    if (b >= ns) return;
    e = E;
    w = b;
  } else {
    const int wi = xcd_item(b - ns8, (int)gridDim.x - ns8);
    if (wi >= E * per) return;
    e = wi / per;
    w = wi % per;
  }
  const int i0 = (w / nh) * AW, h0 = (w % nh) * 256;
  const bool sh = e >= E;
  const int orow = sh ? a.P : a.offsets[e];
  const int kdim = sh ? a.T : a.offsets[e + 1] - orow;
  const uint16_t* asrc[NSEG];
  if (NSEG == 2) {
    asrc[0] = a.dg;
    asrc[NSEG - 1] = a.du;
  } else {
    asrc[0] = a.aw;
  }
  const uint16_t* bsrc = NSEG == 2 ? a.x : a.dy;

  // staging: A k row tid / (AW / 8) (+ 256 / (AW / 8) u), chunk tid % (AW / 8);
  // B k row tid / 8, chunks tid % 8 + 8 u (one gathered row per thread)
  constexpr int ACR = AW / 8;
  const int br = tid >> 3, bc = tid & 7;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  // Rows past the expert's end are loaded from its last row (always a valid
  // address, no branch) and zeroed when staged.  The sorted pair of this
  // lane's B row k0 + br comes from a vector load issued first in the step
  // two steps before its rows' loads, so waiting for it leaves the newer data
  // loads in flight (a scalar load here was waited for, a whole L2 round trip,
  // at every step's barrier).  The shared expert's rows are the tokens
  // themselves; its pair load is a dummy.
  auto pair_of = [&](int k0) -> int { return a.sorted_pair[sh ? 0 : orow + min(k0 + br, kdim - 1)]; };
  auto load = [&](int k0, int pair, u32x4 (&va)[NSEG][NAC], u32x4 (&vb)[4]) __attribute__((always_inline)) {
    const int tok = sh ? min(k0 + br, kdim - 1) : pair / K;
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg)
#pragma unroll
      for (int u = 0; u < NAC; ++u) {
        const int n = tid + 256 * u;
        const int m = min(k0 + n / ACR, kdim - 1);
        va[sg][u] = ld16(asrc[sg] + (size_t)(orow + m) * I + i0 + 8 * (n % ACR));
      }
    const uint16_t* bp = bsrc + (size_t)tok * H + h0 + 8 * bc;
#pragma unroll
    for (int u = 0; u < 4; ++u) vb[u] = ld16(bp + 64 * u);
  };
  auto stage = [&](int buf, int k0, const u32x4 (&va)[NSEG][NAC], const u32x4 (&vb)[4])
      __attribute__((always_inline)) {
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg)
#pragma unroll
      for (int u = 0; u < NAC; ++u) {
        const int n = tid + 256 * u;
        const u32x4 v = k0 + n / ACR < kdim ? va[sg][u] : z4;
        if (AW == 64) st16(sa[buf][sg] + rc_off(n / ACR, n % ACR), v);
        else st16(sa[buf][sg] + (n / ACR) * 256 + (((n % ACR) ^ rcw_swz(n / ACR)) << 4), v);
      }
    const bool bok = k0 + br < kdim;
#pragma unroll
    for (int u = 0; u < 4; ++u) st16(sb[buf] + rcw_off(br, bc + 8 * u), bok ? vb[u] : z4);
  };

  f32x4 acc[NSEG * NT][4];
#pragma unroll
  for (int i = 0; i < NSEG * NT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nk = (kdim + 31) / 32;  // steps of 32 rows
  if (nk == 0) {                    // no rows: the gradients are zero
    const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg) {
      float* out = NSEG == 2 ? (sg == 0 ? a.dwg : a.dwu) : a.dwd;
      out += (size_t)e * I * H;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4*>(out + (size_t)(i0 + 16 * t + r16) * H + h0 + 64 * wv + 16 * j + 4 * q) =
              f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  auto compute = [&](int buf) __attribute__((always_inline)) {
    u32x4 fh[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) fh[j] = read_rc<256>(sb[buf], 64 * wv + 16 * j, lane);
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        u32x4 fi;
        if (AW == 64) {
          fi = read_rc<64>(sa[buf][sg], 16 * t, lane);
        } else {
          // 256-byte rows: the same transpose read with the 16-chunk swizzle
          const int q = lane >> 4, i = lane & 15, c = i >> 2, m = i & 3;
          const int k = 8 * q + c;
          const int col = 16 * t + 4 * m;
          const uint8_t* p = sa[buf][sg] + k * 256 + (((col >> 3) ^ rcw_swz(k)) << 4) + ((col & 4) << 1);
          const u32x2 lo = lds_tr16(p), hi = lds_tr16(p + 4 * 256);
          fi = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[sg * NT + t][j] = mfma16x16x32(fh[j], fi, acc[sg * NT + t][j]);
      }
  };
  // Loads two steps ahead of the MFMAs, LDS stores one, nothing in the loop
  // conditional (as in k_bwd_gemm); step s first loads the pair ids of step
  // s + 3's rows, then step s + 2's data.
  u32x4 va0[NSEG][NAC], vb0[4], va1[NSEG][NAC], vb1[4];
  auto step = [&](int st, int p_use, int& p_next, u32x4 (&fa)[NSEG][NAC], u32x4 (&fb)[4],
                  const u32x4 (&la)[NSEG][NAC], const u32x4 (&lb)[4]) __attribute__((always_inline)) {
    p_next = pair_of(32 * (st + 3));
    load(32 * (st + 2), p_use, fa, fb);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
    // the compute of a step past the end (an odd count) is skipped; it issues
    // no memory loads, so the loads' waits are the same either way
    if (st < nk) compute(st & 1);
    stage((st + 1) & 1, 32 * (st + 1), la, lb);
    __syncthreads();
  };
  load(0, pair_of(0), va0, vb0);
  stage(0, 0, va0, vb0);
  load(32, pair_of(32), va1, vb1);
  int pa = pair_of(64), pb = 0;
  __syncthreads();
  for (int st = 0; st < nk; st += 2) {
    step(st, pa, pb, va0, vb0, va1, vb1);
    step(st + 1, pb, pa, va1, vb1, va0, vb0);
  }
  // lane: feature i0 + 16 t + r16, h h0 + 64 wv + 16 j + 4 q .. + 3
  const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int sg = 0; sg < NSEG; ++sg) {
    float* out;
    if (NSEG == 2) out = sg == 0 ? (sh ? a.dswg : a.dwg) : (sh ? a.dswu : a.dwu);
    else out = sh ? a.dswd : a.dwd;
    if (!sh) out += (size_t)e * I * H;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(out + (size_t)(i0 + 16 * t + r16) * H + h0 + 64 * wv + 16 * j + 4 * q) =
            acc[sg * NT + t][j];
  }
}

// Per row (one wave): a = silu(g) u, dL/dw = <a, r> (routed rows), d_a = w r,
// d_g = d_a u silu'(g), d_u = d_a silu(g), w a; w = 1 for the shared rows.
__global__ __launch_bounds__(256) void k_bwd_act(const BwdArgs a, int nrows_total) {
  const int lane = threadIdx.x & 63;
  const int row = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nrows_total) return;
  const int I = a.I, K = a.K, E = a.E;
  // routed rows past offsets[E] exist only for pairs the permute skipped (an
  // index outside [0, E)): nothing to compute there
  if (row < a.P && row >= a.offsets[E]) return;
  float w = 1.0f;
  int p = -1;
  if (row < a.P) {
    p = a.sorted_pair[row];
    const int t = p / K, j = p - (p / K) * K;
    // the token's routing weights from its chosen experts' logits (every
    // load issued before the sums), summed in j order
    int ix[16];
    float lg[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) ix[k] = min(max(a.idx[(size_t)t * K + min(k, K - 1)], 0), E - 1);
#pragma unroll
    for (int k = 0; k < 16; ++k) lg[k] = a.logits[(size_t)t * E + ix[k]];
    float S = 0.0f, sj = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k >= K) continue;
      const float sk = sigm(lg[k]);
      S += sk;
      sj = k == j ? sk : sj;
    }
    w = a.scale * (sj / (S + 1e-20f));
  }
  const size_t base = (size_t)row * I;
  float dot = 0.0f;
  for (int i0 = 8 * lane; i0 < I; i0 += 512) {  // 8 consecutive features a lane
    f32x4 gv[2], uv[2], rv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      gv[h] = *reinterpret_cast<const f32x4*>(a.g + base + i0 + 4 * h);
      uv[h] = *reinterpret_cast<const f32x4*>(a.u + base + i0 + 4 * h);
      rv[h] = *reinterpret_cast<const f32x4*>(a.r + base + i0 + 4 * h);
    }
    float dg[8], du[8], aw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float g = gv[k >> 2][k & 3], u = uv[k >> 2][k & 3], r = rv[k >> 2][k & 3];
      const float sg = sigm(g);
      const float silu = g * sg;
      const float act = silu * u;
      dot += act * r;
      const float da = w * r;
      dg[k] = da * u * (sg * (1.0f + g * (1.0f - sg)));
      du[k] = da * silu;
      aw[k] = w * act;
    }
    u32x4 pg, pu, pa;
    pg.x = pack_bf16x2(dg[0], dg[1]); pg.y = pack_bf16x2(dg[2], dg[3]);
    pg.z = pack_bf16x2(dg[4], dg[5]); pg.w = pack_bf16x2(dg[6], dg[7]);
    pu.x = pack_bf16x2(du[0], du[1]); pu.y = pack_bf16x2(du[2], du[3]);
    pu.z = pack_bf16x2(du[4], du[5]); pu.w = pack_bf16x2(du[6], du[7]);
    pa.x = pack_bf16x2(aw[0], aw[1]); pa.y = pack_bf16x2(aw[2], aw[3]);
    pa.z = pack_bf16x2(aw[4], aw[5]); pa.w = pack_bf16x2(aw[6], aw[7]);
    st16(a.dg + base + i0, pg);
    st16(a.du + base + i0, pu);
    st16(a.aw + base + i0, pa);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) dot += __shfl_xor(dot, o, 64);
  if (p >= 0 && lane == 0) a.gw[p] = dot;
}

// Per token: dlam of its K chosen experts (quotient rule, then the sigmoid's slope).
__global__ __launch_bounds__(256) void k_bwd_router(const BwdArgs a) {
  const int t = (int)blockIdx.x * 256 + threadIdx.x;
  if (t >= a.T) return;
  const int K = a.K, E = a.E;
  float s[16], S = 0.0f, sgs = 0.0f;
  for (int j = 0; j < K; ++j) {
    s[j] = sigm(a.logits[(size_t)t * E + min(max(a.idx[(size_t)t * K + j], 0), E - 1)]);
    S += s[j];
  }
  const float D = S + 1e-20f;
  for (int j = 0; j < K; ++j) sgs += a.gw[(size_t)t * K + j] * s[j];
  for (int j = 0; j < K; ++j) {
    const float ds = a.scale / D * (a.gw[(size_t)t * K + j] - sgs / D);
    a.dlam[(size_t)t * K + j] = ds * s[j] * (1.0f - s[j]);
  }
}

// dW_r = dlogit^T x, dlogit[t][e] = dlam of the pair (t, j) with idx[t][j] = e,
// else 0, never stored: each 32-token step scatters its tokens' K values into
// an LDS tile that is otherwise zero (the thread that owns a token slot first
// clears the values it wrote there two steps before).  Each value v enters the
// bf16 MFMA as two planes, hi = bf16(v) and lo = bf16(v - hi), against the
// same x rows, so the product keeps 16 bits of v; x is bf16 already.  Tile:
// 256 experts x 64 h, 4 waves of 64 experts x 64 h.  blockIdx.z = token chunk;
// its sums go to part[z][e][h], summed in chunk order after.
constexpr int kRwChunkMax = 16;
constexpr int kRwStep = 32;  // tokens per step
__global__ __launch_bounds__(256) void k_bwd_router_wgrad(const BwdArgs a, int chunk, float* part) {
  __shared__ __attribute__((aligned(16))) uint8_t sa[2][2][kRwStep * 512];  // [buf][hi/lo][token][expert]
  __shared__ __attribute__((aligned(16))) uint8_t sb[2][kRwStep * 128];     // [buf][token][h]
  __shared__ int16_t sprev[2][kRwStep][16];  // expert (- e0) each slot wrote, or -1
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, E = a.E, K = a.K;
  const int h0 = blockIdx.x * 64, e0 = blockIdx.y * 256;
  const int ehi = min(E - e0, 256);  // experts of this tile
  const int t0 = blockIdx.z * chunk, t1 = min(a.T, t0 + chunk);
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  for (int i = tid; i < 2 * 2 * kRwStep * 512 / 16; i += 256) st16(&sa[0][0][0] + 16 * i, z4);
  for (int i = tid; i < 2 * kRwStep * 16; i += 256) (&sprev[0][0][0])[i] = -1;
  __syncthreads();

  // token-slot threads (tid < 32) load the token's K (expert, dlam); every
  // thread loads one 16-byte piece of x: token tid / 8, h chunk tid % 8
  const int br = tid >> 3, bc = tid & 7;
  auto load = [&](int tb, int32_t (&ix)[16], float (&dl)[16], u32x4& vb) __attribute__((always_inline)) {
    const int t = tb + tid;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool ok = tid < kRwStep && t < t1 && j < K;
      ix[j] = ok ? a.idx[(size_t)t * K + j] - e0 : -1;
      dl[j] = ok ? a.dlam[(size_t)t * K + j] : 0.0f;
    }
    const int tx = tb + br;
    vb = tx < t1 ? ld16(a.x + (size_t)tx * H + h0 + 8 * bc) : z4;
  };
  auto lds_b16 = [](uint8_t* base, int k, int el) -> uint16_t* {
    return reinterpret_cast<uint16_t*>(base + rcw_off(k, el >> 3) + 2 * (el & 7));
  };
  auto stage = [&](int buf, const int32_t (&ix)[16], const float (&dl)[16], const u32x4& vb)
      __attribute__((always_inline)) {
    if (tid < kRwStep) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {  // clear what this slot wrote two steps ago
        const int el = sprev[buf][tid][j];
        if (el >= 0) {
          *lds_b16(sa[buf][0], tid, el) = 0;
          *lds_b16(sa[buf][1], tid, el) = 0;
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const bool in = ix[j] >= 0 && ix[j] < ehi;
        if (in) {
          const uint32_t hb = f32_to_bf16_bits(dl[j]);
          const float r = dl[j] - __uint_as_float(hb << 16);
          *lds_b16(sa[buf][0], tid, ix[j]) = (uint16_t)hb;
          *lds_b16(sa[buf][1], tid, ix[j]) = (uint16_t)f32_to_bf16_bits(r);
        }
        sprev[buf][tid][j] = in ? (int16_t)ix[j] : (int16_t)-1;
      }
    }
    st16(sb[buf] + rc_off(br, bc), vb);
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nk = t1 > t0 ? (t1 - t0 + kRwStep - 1) / kRwStep : 0;
  int32_t ix[16];
  float dl[16];
  u32x4 vb;
  if (nk > 0) {
    load(t0, ix, dl, vb);
    stage(0, ix, dl, vb);
  }
  __syncthreads();
  for (int st = 0; st < nk; ++st) {
    const int buf = st & 1;
    if (st + 1 < nk) load(t0 + kRwStep * (st + 1), ix, dl, vb);
    u32x4 fb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = read_rc<64>(sb[buf], 16 * j, lane);
#pragma unroll
    for (int pl = 0; pl < 2; ++pl) {
      u32x4 fa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = read_rc<256>(sa[buf][pl], 64 * wv + 16 * i, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(fa[i], fb[j], acc[i][j]);
    }
    if (st + 1 < nk) stage(buf ^ 1, ix, dl, vb);
    __syncthreads();
  }
  const int q = lane >> 4, r16 = lane & 15;
  float* out = part + (size_t)blockIdx.z * E * H;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ee = e0 + 64 * wv + 16 * i + 4 * q + c;
      if (ee < E)
#pragma unroll
        for (int j = 0; j < 4; ++j) out[(size_t)ee * H + h0 + 16 * j + r16] = acc[i][j][c];
    }
}

// dW_r = sum of the chunks' partial sums, in chunk order; 4 values per thread.
__global__ __launch_bounds__(256) void k_bwd_router_reduce(const BwdArgs a, int nchunk,
                                                           const float* part) {
  const size_t n = (size_t)a.E * a.H;
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(part + i);
  for (int c = 1; c < nchunk; ++c) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(part + (size_t)c * n + i);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += v[k];
  }
  *reinterpret_cast<f32x4*>(a.dw_router + i) = acc;
}

// dx[t] = shared row + the pair rows in j order + the router's share
// sum_j dlam_j W_r[e_j] in j order (fp32, one rounding); each thread 8
// consecutive h, every pair row's load in flight before the sums.
__global__ __launch_bounds__(256) void k_bwd_combine(const BwdArgs a) {
  constexpr int kMaxK = 16;
  const int t = blockIdx.x;
  const int H = a.H, K = a.K;
  int32_t slot[kMaxK], eix[kMaxK];
  float dl[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    slot[j] = j < K ? a.pair_slot[(size_t)t * K + j] : -1;  // -1: skipped
    eix[j] = j < K ? a.idx[(size_t)t * K + j] : 0;
    dl[j] = j < K ? a.dlam[(size_t)t * K + j] : 0.0f;
  }
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  for (int h0 = threadIdx.x * 8; h0 < H; h0 += 256 * 8) {
    // every row is read once: nontemporal loads (as in the forward combine)
    const u32x4 vs = a.swg ? ld16_stream(a.dxp + (size_t)(a.P + t) * H + h0) : zero4;
    u32x4 v[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      v[j] = slot[j] >= 0 ? ld16_stream(a.dxp + (size_t)slot[j] * H + h0) : zero4;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = bf16_lo(vs[i]);
      acc[2 * i + 1] = bf16_hi(vs[i]);
    }
    // (skip, not break: a break lets the compiler sink each row's load into
    // its iteration, one load in flight at a time)
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (slot[j] < 0) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += bf16_lo(v[j][i]);
        acc[2 * i + 1] += bf16_hi(v[j][i]);
      }
    }
    // the router's share: dlam_j W_r[e_j] in j order, 4 pairs' W_r pieces in
    // flight at a time (W_r, 4 bytes an element, stays in L2)
#pragma unroll
    for (int j0 = 0; j0 < kMaxK; j0 += 4) {
      if (j0 >= K) break;  // block-uniform
      f32x4 wr[4][2];
#pragma unroll
      for (int j = j0; j < j0 + 4; ++j) {
        const float* row = a.w_router + (size_t)(slot[j] >= 0 ? eix[j] : 0) * H + h0;
        wr[j - j0][0] = slot[j] >= 0 ? *reinterpret_cast<const f32x4*>(row) : f32x4{0.f, 0.f, 0.f, 0.f};
        wr[j - j0][1] = slot[j] >= 0 ? *reinterpret_cast<const f32x4*>(row + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = j0; j < j0 + 4; ++j) {
        if (slot[j] < 0) continue;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[c] += dl[j] * wr[j - j0][0][c];
          acc[4 + c] += dl[j] * wr[j - j0][1][c];
        }
      }
    }
    u32x4 pk;
    pk.x = pack_bf16x2(acc[0], acc[1]);
    pk.y = pack_bf16x2(acc[2], acc[3]);
    pk.z = pack_bf16x2(acc[4], acc[5]);
    pk.w = pack_bf16x2(acc[6], acc[7]);
    st16(a.dx + (size_t)t * H + h0, pk);
  }
}

// ---------------------------------------------------------------------------

// Token chunks of the router weight gradient: enough for (H / 64) x chunks to
// fill the chip at any batch (up to kRwChunkMax chunks of >= one step).
static int router_chunks(int64_t T) {
  return (int)std::min<int64_t>(kRwChunkMax, std::max<int64_t>(1, (T + kRwStep - 1) / kRwStep));
}

int bwd_tile_rows(int64_t T, int K, int E, int I, int Is, int H) {
  return expert_tile_rows(T, K, E, I, Is, H, true) == kGRows && bwd_gemm_ok(T, K, I, Is, H)
             ? kGRows
             : kBwdTileRows;
}

// The trash area of the expert GEMM's backward modes (8 KiB per XCD slot).
constexpr size_t kBwdTrashBytes = 65536;

size_t bwd_intermediate_bytes(int64_t T, int K, int E, int I, int H, bool shared) {
  const size_t rows = (size_t)(T * K + (shared ? T : 0));
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  // d_g and d_u carry kGRows rows of padding: the expert GEMM reads whole
  // 256-row tiles of them
  return 3 * al(rows * I * 4) + 2 * al((rows + kGRows) * I * 2) + al(rows * I * 2) +
         2 * al((size_t)T * K * 4) + al(rows * H * 2) + al((size_t)router_chunks(T) * E * H * 4) +
         al(kBwdTrashBytes);
}

hipError_t launch_backward(const BwdInputs& in, hipStream_t s) {
  BwdArgs a;
  a.T = in.T;
  a.H = in.H;
  a.E = in.E;
  a.K = in.K;
  a.I = in.I;
  a.P = in.T * in.K;
  a.scale = in.scale;
  a.x = in.x;
  a.dy = in.dy;
  a.logits = in.logits;
  a.idx = in.idx;
  a.w_router = in.w_router;
  a.wg = in.wg;
  a.wu = in.wu;
  a.wd = in.wd;
  a.swg = in.swg;
  a.swu = in.swu;
  a.swd = in.swd;
  a.offsets = in.offsets;
  a.sorted_pair = in.sorted_pair;
  a.pair_slot = in.pair_slot;
  a.tile_off = in.tile_off;
  a.tile_tab = in.tile_tab;
  a.dx = in.dx;
  a.dw_router = in.dw_router;
  a.dwg = in.dwg;
  a.dwu = in.dwu;
  a.dwd = in.dwd;
  a.dswg = in.dswg;
  a.dswu = in.dswu;
  a.dswd = in.dswd;
  const bool shared = in.swg != nullptr;
  const int64_t rows = (int64_t)a.P + (shared ? a.T : 0);
  uint8_t* p = reinterpret_cast<uint8_t*>(in.scratch);
  auto take = [&](size_t bytes) {
    uint8_t* q = p;
    p += (bytes + 255) / 256 * 256;
    return q;
  };
  a.g = reinterpret_cast<float*>(take((size_t)rows * a.I * 4));
  a.u = reinterpret_cast<float*>(take((size_t)rows * a.I * 4));
  a.r = reinterpret_cast<float*>(take((size_t)rows * a.I * 4));
  a.dg = reinterpret_cast<uint16_t*>(take((size_t)(rows + kGRows) * a.I * 2));
  a.du = reinterpret_cast<uint16_t*>(take((size_t)(rows + kGRows) * a.I * 2));
  a.aw = reinterpret_cast<uint16_t*>(take((size_t)rows * a.I * 2));
  a.gw = reinterpret_cast<float*>(take((size_t)a.P * 4));
  a.dlam = reinterpret_cast<float*>(take((size_t)a.P * 4));
  a.dxp = reinterpret_cast<uint16_t*>(take((size_t)rows * a.H * 2));
  const int nchunk = router_chunks(a.T);
  float* rpart = reinterpret_cast<float*>(take((size_t)nchunk * a.E * a.H * 4));
  void* trash = take(kBwdTrashBytes);
  const int chunk = (int)(((a.T + nchunk - 1) / nchunk + kRwStep - 1) / kRwStep * kRwStep);

  // row tiles: a host upper bound; blocks past the count the permute wrote exit
  const int64_t rtiles = max_expert_tiles(a.T, a.K, a.E, shared ? a.I : 0, in.tile_rows);
  a.rtiles = (int)rtiles;
  auto grid8 = [](int64_t n) { return dim3((unsigned)((n + 7) / 8 * 8)); };
  // many rows per expert: the row products on the forward's expert GEMM
  const bool gemm = in.tile_rows == kGRows;
  ExpertArgs ea{};
  if (gemm) {
    ea.T = a.T;
    ea.H = a.H;
    ea.E = a.E;
    ea.K = a.K;
    ea.I = a.I;
    ea.Is = shared ? a.I : 0;
    ea.x = a.x;
    ea.sorted_pair = a.sorted_pair;
    ea.w_gate = a.wg;
    ea.w_up = a.wu;
    ea.w_down = a.wd;
    ea.ws_gate = a.swg;
    ea.ws_up = a.swu;
    ea.ws_down = a.swd;
    ea.tile_off = const_cast<int32_t*>(a.tile_off);
    ea.tile_tab = const_cast<int32_t*>(a.tile_tab);
    ea.tile_rows = kGRows;
    ea.tiles_ready = true;
    ea.dy = a.dy;
    ea.bwd_g = a.g;
    ea.bwd_u = a.u;
    ea.bwd_r = a.r;
    ea.bwd_dg = a.dg;
    ea.bwd_du = a.du;
    ea.bwd_dx = a.dxp;
    ea.trash = trash;
    const hipError_t e = launch_bwd_gur_gemm(ea, s);
    if (e != hipSuccess) return e;
  } else if (a.I % 256 == 0) {
    hipLaunchKernelGGL((k_bwd_gemm<kRowsNT, 256>), grid8(rtiles * (3 * a.I / 256)), dim3(kBT), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_bwd_gemm<kRowsNT, 64>), grid8(rtiles * (3 * a.I / 64)), dim3(kBT), 0, s, a);
  }
  hipLaunchKernelGGL(k_bwd_act, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a, (int)rows);
  hipLaunchKernelGGL(k_bwd_router, dim3((unsigned)((a.T + 255) / 256)), dim3(256), 0, s, a);
  if (gemm) {
    const hipError_t e = launch_bwd_dx_gemm(ea, s);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL((k_bwd_gemm<kRowsNN, 256>), grid8(rtiles * (a.H / 256)), dim3(kBT), 0, s, a);
  }
  {
    auto grid_w = [&](int aw) {
      const int64_t per = (a.I / aw) * (a.H / 256);
      const int64_t ns8 = shared ? (per + 7) / 8 * 8 : 0;
      return dim3((unsigned)(ns8 + (a.E * per + 7) / 8 * 8));
    };
    hipLaunchKernelGGL((k_bwd_wgrad<2, 64>), grid_w(64), dim3(256), 0, s, a);
    if (a.I % 128 == 0)
      hipLaunchKernelGGL((k_bwd_wgrad<1, 128>), grid_w(128), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_bwd_wgrad<1, 64>), grid_w(64), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(k_bwd_router_wgrad, dim3((unsigned)(a.H / 64), (unsigned)((a.E + 255) / 256),
                                              (unsigned)nchunk), dim3(256), 0, s, a, chunk, rpart);
  hipLaunchKernelGGL(k_bwd_router_reduce, dim3((unsigned)(((size_t)a.E * a.H / 4 + 255) / 256)),
                     dim3(256), 0, s, a, nchunk, (const float*)rpart);
  hipLaunchKernelGGL(k_bwd_combine, dim3((unsigned)a.T), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
