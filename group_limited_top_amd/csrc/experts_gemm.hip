// experts_gemm.hip -- MFMA grouped GEMMs of the experts for many rows per
// expert (a large batch of tokens).
//
// [Routing §四]: every expert is down(silu(gate x) * up x) over stacked
// [E][I][H] weights; [Routing §五]: the shared expert is one more bucket (all T
// tokens).  Rows are the expert-sorted pairs; a row tile is kGRows rows of one
// expert (the tile table, see write_tile_entry).
//
// Block: 8 waves (two per SIMD), a 256 x 256 output tile; wave w = (wm, wn)
// = (w / 2, w % 2) owns 64 token rows (64 wm..) x 128 columns, 8 x 4 MFMA
// 16x16x32 tiles (128 accumulators per lane).  The two waves of a SIMD
// (w, w + 4) have different rows, so a tile with at most 128 rows still
// keeps every SIMD busy.
//   gate/up: columns = 128 gate + 128 up weight rows (features i0..i0+127);
//            wave (wm, wn) owns features 64 wn.. of both gate and up, so
//            h = silu(g) * u is formed in registers.  K = H.
//   down:    rows = h rows (contiguous), columns = 256 outputs; W_down[e] is
//            [I][H] (H contiguous), and the LDS transpose read
//            (ds_read_b64_tr_b16) turns its staged [k][column] rows into the
//            MFMA operand (4 consecutive k of one column per lane).  K = I.
// The layer backward's row products run on the same kernel: g, u (the
// gate/up products kept apart, fp32), r = dy W_down^T (a gate-shaped product:
// dy rows against W_down's rows, 256 features a tile, fp32), and dx per row =
// d_g W_gate + d_u W_up (a down-shaped product with K = 2 I: the d_g rows
// against W_gate, then the d_u rows against W_up; bf16).
//
// Data path.  A step is 64 deep in K, so every staged row is one whole
// 128-byte line (half lines halve what the load path delivers per CU).  The
// operands of a step are two 32 KiB slices (tokens, weights) staged by direct
// global -> LDS loads (global_load_lds_dwordx4: 1 KiB per wave instruction);
// five slice buffers (160 KiB, all of the CU's LDS) form a ring, so while a
// step is computed the next one and a half steps are in flight.  Operands go
// from LDS to registers in two 32-deep halves a step: the first half's after
// the step's barrier, the second half's between the first half's MFMAs.
//
// Blocks are persistent (one per CU) and walk a static list of tiles, the
// ring running on from one tile into the next.  Tiles are ordered expert by
// expert; XCD x (blocks b with b mod 8 = x) takes the x-th eighth of the list
// and its blocks interleave over it, so the blocks of one XCD work on the same
// few experts at a time and share their weights and token rows in its L2.
#include "device.h"
#include "expert_tiles.h"
#include "kernels.h"
#include "ring.h"

namespace moe {

constexpr int kGK = 64;           // K depth of a step
constexpr int kSliceB = 32768;    // bytes of one staged slice
constexpr int kRingN = 5;         // slice buffers in the ring
constexpr int kGuFeat = 128;      // h features per gate/up tile
constexpr int kDnOut = 256;       // output columns per down tile

// One slice's 4 loads of this wave: load j brings the lane's 16 bytes from
// base + off[j] into LDS lds + 1 KiB j + 16 lane.  M0 (the LDS destination) is
// saved and restored around the loads, and every write of M0 is followed by
// the one wait state an LDS DMA reading M0 needs after a scalar write of it.
// Inline asm keeps the compiler from tying later LDS reads to these loads; the
// ring orders them (ring_wait).  The memory clobber keeps LDS accesses in
// place around it.
__device__ __forceinline__ void dma4(const void* base_, const uint32_t (&off)[4], uint32_t lds) {
  // the base is wave-uniform; readfirstlane makes that visible (its result
  // is a signed int: widen each half as unsigned)
  const uint64_t b = reinterpret_cast<uint64_t>(base_);
  const uint32_t blo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t bhi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const void* base = reinterpret_cast<const void*>(((uint64_t)bhi << 32) | (uint64_t)blo);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %6\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %5\n\ts_add_u32 m0, m0, 1024\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %5\n\ts_add_u32 m0, m0, 1024\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %5\n\ts_add_u32 m0, m0, 1024\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %5\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(base), "s"(lds)
      : "memory", "scc");
}

struct GTile {
  int e, row0, nrows, s;  // expert (E = shared), first row, rows, column slice
};

// Tile t of the list: row tile t / S, column slice t % S.  Everything here is
// wave-uniform; readfirstlane keeps it in scalar registers, so the table is
// read with scalar loads (a vector load would make the compiler wait for all
// vector-memory operations in flight, the ring's loads included).
__device__ __forceinline__ GTile gtile(const int32_t* tab, int t, int S) {
  t = __builtin_amdgcn_readfirstlane(t);
  const int rt = t / S;
  GTile g;
  const int32_t v = __builtin_amdgcn_readfirstlane(sload(tab + 2 * rt));
  g.e = v & 0xffff;
  g.nrows = v >> 16;
  g.row0 = __builtin_amdgcn_readfirstlane(sload(tab + 2 * rt + 1));
  g.s = t - rt * S;
  return g;
}

// MODE 0: gate/up + SwiGLU; MODE 1: down; the backward's MODE 2: g, u;
// MODE 3: r; MODE 4: dx.
template <int MODE>
__global__ __launch_bounds__(512, 1) void k_expert_gemm(const ExpertArgs a, int S) {
  // modes 0, 2, 3: K = H, gathered token rows against K-contiguous weight rows;
  // modes 1, 4: contiguous h rows against N-contiguous weights
  constexpr bool kGU = MODE == 0 || MODE == 2 || MODE == 3;
  // epilogue stores per wave: 8 bytes each (mode 0), 16 (modes 1, 4), 16-byte
  // fp32 pieces (modes 2, 3)
  constexpr int kStores = (MODE == 2 || MODE == 3) ? 32 : 16;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRingN * kSliceB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int q = lane >> 4, r16 = lane & 15;
  const int H = a.H, I = a.I, E = a.E;
  // the operand arrays, read once from the kernel arguments into scalar
  // registers (selecting among struct fields later would otherwise become a
  // vector load of the argument block)
  const uint8_t* const x_p = uniform_ptr(reinterpret_cast<const uint8_t*>(MODE == 3 ? a.dy : a.x));
  const uint8_t* const hr_p =
      uniform_ptr(reinterpret_cast<const uint8_t*>(MODE == 4 ? a.bwd_dg : a.h_routed));
  const uint8_t* const hs_p = uniform_ptr(reinterpret_cast<const uint8_t*>(a.h_shared));
  const uint8_t* const hu_p = uniform_ptr(reinterpret_cast<const uint8_t*>(a.bwd_du));  // mode 4
  const uint16_t* const wg_p = uniform_ptr(reinterpret_cast<const uint16_t*>(a.w_gate));
  const uint16_t* const wu_p = uniform_ptr(reinterpret_cast<const uint16_t*>(a.w_up));
  const uint16_t* const wd_p = uniform_ptr(reinterpret_cast<const uint16_t*>(a.w_down));
  const uint16_t* const sg_p = uniform_ptr(reinterpret_cast<const uint16_t*>(a.ws_gate));
  const uint16_t* const su_p = uniform_ptr(reinterpret_cast<const uint16_t*>(a.ws_up));
  const uint16_t* const sd_p = uniform_ptr(reinterpret_cast<const uint16_t*>(a.ws_down));
  const int32_t* const sp_p = uniform_ptr(a.sorted_pair);
  uint16_t* const hrw_p = uniform_ptr(reinterpret_cast<uint16_t*>(a.h_routed));
  uint16_t* const orw_p = uniform_ptr(reinterpret_cast<uint16_t*>(MODE == 4 ? a.bwd_dx : a.o_routed));
  uint16_t* const osw_p = MODE == 4 ? orw_p + (size_t)a.T * a.K * a.H
                                    : uniform_ptr(reinterpret_cast<uint16_t*>(a.o_shared));
  float* const bo_p = uniform_ptr(MODE == 2 ? a.bwd_g : a.bwd_r);  // modes 2, 3
  float* const bu_p = uniform_ptr(a.bwd_u);                          // mode 2
  uint16_t* const btr_p = uniform_ptr(reinterpret_cast<uint16_t*>(a.trash));
  const int T = a.T, K = a.K;
  const int32_t* const tab_p = uniform_ptr(a.tile_tab);
  const int32_t* const toff_p = uniform_ptr(a.tile_off);
  // (the argument block is not touched below: a use after one of the inline
  // asm statements, which clobber memory, would keep a private copy of it)
  // Shared-expert arrays as offsets from the routed ones: the lambdas below
  // then pick with an integer select (a select between two captured pointers
  // would become a load through a select of their addresses, which keeps
  // them in private memory).
  // this wave's gate or up rows (mode 3: W_down's, both halves of the tile)
  const uint16_t* const wgu_p = MODE == 3 ? wd_p : w < 4 ? wg_p : wu_p;
  const ptrdiff_t sh_wgu = (MODE == 3 ? sd_p : w < 4 ? sg_p : su_p) - wgu_p;  // shared minus routed
  const ptrdiff_t sh_wd = sd_p - wd_p;
  const ptrdiff_t sh_wg = sg_p - wg_p, sh_wu = su_p - wu_p;  // mode 4
  // mode 4: the shared rows follow the P routed rows of d_g and d_u
  const ptrdiff_t sh_h = MODE == 4 ? (ptrdiff_t)a.T * a.K * a.I * 2 : hs_p - hr_p;  // bytes
  const ptrdiff_t sh_hw = sh_h / 2;      // bf16 elements (both arrays are 256-byte aligned)
  const ptrdiff_t sh_o = osw_p - orw_p;

  // this block's tiles: first + m * nbx, m = 0 .. count - 1
  const int ntiles = sload(toff_p + E + 1) * S;
  const int nbx = (int)(gridDim.x >> 3);
  const int x8 = (int)(blockIdx.x & 7);
  const int lo = (int)((int64_t)ntiles * x8 / 8), hi = (int)((int64_t)ntiles * (x8 + 1) / 8);
  const int first = lo + (int)(blockIdx.x >> 3);
  if (first >= hi) return;
  const int count = (hi - first + nbx - 1) / nbx;
  const int nI = I / kGK;  // mode 4: steps against W_gate, then as many against W_up
  const int nsteps = kGU ? H / kGK : MODE == 4 ? 2 * nI : nI;
  const int total = count * nsteps;  // steps of this block
  const int nslices = 2 * total;     // slice 2s: token rows of step s, 2s + 1: weights
  const uint32_t ring0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lvoid_t*)ring)));

  // ---- DMA ---------------------------------------------------------------
  // token rows: this wave's loads j cover slice rows 32 w + 8 j + lane / 8
  int xm = -1, xk = 0;          // tile (m) and step of the next token slice
  const uint8_t* xb = nullptr;  // wave-uniform base of the current tile
  uint32_t xo[4];               // lane offsets of the current tile
  int32_t ptok[4];              // gate/up: sorted pairs of the next tile's rows
  int pe = 0, prow0 = 0;
  // weights
  int wmi = -1, wk = 0;
  const uint8_t* wb = nullptr;
  const uint8_t* wb2 = nullptr;  // mode 4: W_up
  const uint8_t* xb2 = nullptr;  // mode 4: the d_u rows
  uint32_t wo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (kGU) {
      // gate (w < 4) or up rows 32 (w & 3) + 8 j + lane / 8 of the tile's features
      wo[j] = (uint32_t)((8 * j + (lane >> 3)) * H * 2 + rs_chunk(j, lane) * 16);
    } else {
      // W_down row r = 2 (4 w + j) + lane / 32 of the step; LDS slot lane & 31
      // holds logical chunk (lane & 31) ^ wd_swz(r)
      const int r = 2 * (4 * w + j) + (lane >> 5);
      wo[j] = (uint32_t)(r * H * 2 + (((lane & 31) ^ wd_swz(r)) * 16));
    }
    // down: h rows of the tile are contiguous (the buffers are padded by a
    // whole tile, so rows past the tile's end are readable)
    xo[j] = (uint32_t)((32 * w + 8 * j + (lane >> 3)) * I * 2 + rs_chunk(j, lane) * 16);
  }
  // The sorted pairs of a tile's rows 32 w + 8 j + lane / 8 (rows past the
  // tile's end repeat its last row), read with scalar loads: they wait on
  // lgkmcnt, never on the ring's vmcnt, and arrive in registers the compiler
  // knows about.  Each lane then picks its row's value.
  auto fetch_rows = [&](int t) __attribute__((always_inline)) {
    const GTile g = gtile(tab_p, t, S);
    pe = g.e;
    prow0 = g.row0;
    if (kGU && g.e < E) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int32_t v = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int32_t sv = sload(sp_p + g.row0 + min(32 * w + 8 * j + k, g.nrows - 1));
          v = (lane >> 3) == k ? sv : v;
        }
        ptok[j] = v;
      }
    }
  };
  fetch_rows(first);
  auto issue_x = [&](uint32_t lds) __attribute__((always_inline)) {
    if (xk == 0) {
      ++xm;
      if (kGU) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tok = pe < E ? ptok[j] / K : prow0 + 32 * w + 8 * j + (lane >> 3);
          xo[j] = (uint32_t)(min(tok, T - 1) * H * 2 + rs_chunk(j, lane) * 16);
        }
        xb = x_p;
      } else {
        xb = uniform_ptr(hr_p + (pe < E ? 0 : sh_h) + (size_t)prow0 * I * 2);
        if (MODE == 4) xb2 = uniform_ptr(hu_p + (pe < E ? 0 : sh_h) + (size_t)prow0 * I * 2);
      }
      if (xm + 1 < count) fetch_rows(first + (xm + 1) * nbx);
    }
    if (MODE == 4 && xk >= nI) dma4(xb2 + (xk - nI) * 128, xo, lds);
    else dma4(xb + xk * 128, xo, lds);
    if (++xk == nsteps) xk = 0;
  };
  auto issue_w = [&](uint32_t lds) __attribute__((always_inline)) {
    if (wk == 0) {
      ++wmi;
      const GTile g = gtile(tab_p, first + wmi * nbx, S);
      const bool sh = g.e >= E;
      const size_t ebase = sh ? 0 : (size_t)g.e * I * H;
      if (kGU) {
        const uint16_t* src = wgu_p + (sh ? sh_wgu : 0);
        // mode 3: 256 W_down rows a tile, waves 4..7 the second 128
        const int row = MODE == 3 ? g.s * 2 * kGuFeat + kGuFeat * (w >> 2) + 32 * (w & 3)
                                  : g.s * kGuFeat + 32 * (w & 3);
        wb = uniform_ptr(reinterpret_cast<const uint8_t*>(src + ebase + (size_t)row * H));
      } else if (MODE == 4) {
        wb = uniform_ptr(reinterpret_cast<const uint8_t*>(wg_p + (sh ? sh_wg : 0) + ebase +
                                                          (size_t)g.s * kDnOut));
        wb2 = uniform_ptr(reinterpret_cast<const uint8_t*>(wu_p + (sh ? sh_wu : 0) + ebase +
                                                           (size_t)g.s * kDnOut));
      } else {
        const uint16_t* src = wd_p + (sh ? sh_wd : 0);
        wb = uniform_ptr(reinterpret_cast<const uint8_t*>(src + ebase + (size_t)g.s * kDnOut));
      }
    }
    const size_t step_bytes = kGU ? 128 : (size_t)kGK * H * 2;
    if (MODE == 4 && wk >= nI) dma4(wb2 + (wk - nI) * step_bytes, wo, lds);
    else dma4(wb + wk * step_bytes, wo, lds);
    if (++wk == nsteps) wk = 0;
  };
  // Slice sigma goes to buffer sigma % 5; slice 2 s holds the token rows of
  // step s, slice 2 s + 1 its weights.  The prologue issues slices 0..4; step
  // g then issues slice 2 g + 3 (weights of step g + 1) and 2 g + 4 (tokens of
  // step g + 2), each cursor from one place.
  auto slot = [&](int sigma) __attribute__((always_inline)) {
    return ring0 + (uint32_t)((sigma % kRingN) * kSliceB) + 4096u * w;
  };

  // ---- compute -------------------------------------------------------------
  f32x4 acc[8][4];  // [column tile i][row tile n]
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[i][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // lane parts of the LDS addresses of half step h; 16-row groups of a row
  // slice are whole 2 KiB apart (the swizzle only sees a row's low bits)
  // down: lane 4 c + m of group q reads row 32 h + 8 q + c (+ 4 for the
  // second read) at columns 128 wn + 32 (t / 2) + 8 m + 4 (t % 2) .. + 3 for
  // A tile t, i.e. 16-byte chunk 16 wn + 4 (t / 2) + m, half t % 2.  So tile
  // t's MFMA row 4 q + c is column 128 wn + 32 (t / 2) + 8 q + 4 (t % 2) + c,
  // and tiles 2 u, 2 u + 1 give each lane 8 consecutive columns (one 16-byte
  // store).  Rows 32 h + 8 q + c and + 4 share their swizzle, so a lane's
  // chunk for tile t is 16 wn + (dn_v ^ 4 (t / 2)).
  int lane_b[2], lane_a[2];
  int dn_v = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    lane_b[h] = rs_addr(64 * wm + r16, 4 * h + q);
    if (kGU) {
      lane_a[h] = rs_addr(64 * wn + r16, 4 * h + q);
    } else {
      const int r = 32 * h + 8 * q + (r16 >> 2);
      lane_a[h] = r * 512 + 256 * wn;
      dn_v = (r16 & 3) ^ wd_swz(r);
    }
  }
  // A step: the operands of its first 32-deep half (B0, A), then that half's
  // MFMAs with the LDS reads of the second half between them (B1 first; A[i]
  // is refilled as soon as its four MFMAs are issued), then the second half's
  // MFMAs.  The second half's reads are thus hidden behind MFMAs; 64 operand
  // registers where two full sets would need 96.
  auto read_a = [&](const uint8_t* bw, int i) __attribute__((always_inline)) {
    if (kGU) {
      return lds16(bw + (i < 4 ? 2048 * i : 16384 + 2048 * (i - 4)));
    } else {
      const uint8_t* p = bw + 8 * (i & 1) + ((dn_v ^ (4 * (i >> 1))) << 4);
      const u32x2 lo = lds_tr16(p), hi = lds_tr16(p + 4 * 512);
      return u32x4{lo.x, lo.y, hi.x, hi.y};
    }
  };
  auto full_step = [&](int g) __attribute__((always_inline)) {
    const uint8_t* bx = ring + ((2 * g) % kRingN) * kSliceB;
    const uint8_t* bw = ring + ((2 * g + 1) % kRingN) * kSliceB;
    u32x4 A[8], B0[4], B1[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) B0[n] = lds16(bx + lane_b[0] + 2048 * n);
#pragma unroll
    for (int i = 0; i < 8; ++i) A[i] = read_a(bw + lane_a[0], i);
#pragma unroll
    for (int n = 0; n < 4; ++n) B1[n] = lds16(bx + lane_b[1] + 2048 * n);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[i][n] = mfma16x16x32(A[i], B0[n], acc[i][n]);
      A[i] = read_a(bw + lane_a[1], i);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[i][n] = mfma16x16x32(A[i], B1[n], acc[i][n]);
    // keep that order (the scheduler would otherwise gather the reads)
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, kGU ? 1 : 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 32, 0);
  };
  // Every epilogue issues the same number of stores per wave (kStores), rows
  // past the tile's end going to trash (the padding rows of h_routed, whose
  // contents are never used), so that the ring's waits can count them.
  // Each lane has its own 16 bytes of trash (blocks spread over the padding
  // rows), so the dropped stores do not all hit one line.
  uint16_t* const trash = (MODE >= 2 ? btr_p : hrw_p + (size_t)T * K * I) +
                         (size_t)(blockIdx.x & 7) * 4096 + 8 * tid;
  auto epilogue = [&](int m) __attribute__((always_inline)) {
    const GTile g = gtile(tab_p, first + m * nbx, S);
    const bool sh = g.e >= E;
    const int rr = 64 * wm + r16;
    if (MODE == 0) {
      const int Iw = I;  // I == Is on this path
      uint16_t* hb = hrw_p + (sh ? sh_hw : 0) +
                     (size_t)(g.row0 + rr) * Iw + g.s * kGuFeat + 64 * wn + 4 * q;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const bool ok = rr + 16 * n < g.nrows;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float hv[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) hv[c] = silu_f32(acc[i][n][c]) * acc[4 + i][n][c];
          u32x2 pk;
          pk.x = pack_bf16x2(hv[0], hv[1]);
          pk.y = pack_bf16x2(hv[2], hv[3]);
          uint16_t* dst = ok ? hb + (size_t)16 * n * Iw + 16 * i : trash;
          store8(dst, pk);
        }
      }
    } else if (MODE == 2 || MODE == 3) {
      // fp32 rows: a routed tile's at its sorted rows, a shared one's after
      // the P routed rows.  The lane holds 4 consecutive features of each
      // column tile i: mode 2 g (i < 4) and u (i >= 4) of features 64 wn +
      // 16 (i % 4) + 4 q of the slice; mode 3 r of features 64 wn + 16 i +
      // 4 q (i < 4) and 128 + 64 wn + 16 (i - 4) + 4 q.
      const size_t orow = (sh ? (size_t)T * K : 0) + (size_t)(g.row0 + rr);
      const int f0 = g.s * (MODE == 2 ? kGuFeat : 2 * kGuFeat) + 64 * wn + 4 * q;
      float* const ob = bo_p + orow * I + f0;
      float* const ub = bu_p + orow * I + f0;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const bool ok = rr + 16 * n < g.nrows;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float* dst;
          if (MODE == 2) dst = (i < 4 ? ob : ub) + (size_t)16 * n * I + 16 * (i & 3);
          else dst = ob + (size_t)16 * n * I + (i < 4 ? 16 * i : kGuFeat + 16 * (i - 4));
          *(__attribute__((address_space(1))) f32x4*)(ok ? dst : reinterpret_cast<float*>(trash)) =
              acc[i][n];
        }
      }
    } else {
      // tiles 2 u, 2 u + 1: lane holds columns 128 wn + 32 u + 8 q + 0..7
      uint16_t* ob = orw_p + (sh ? sh_o : 0) +
                     (size_t)(g.row0 + rr) * H + g.s * kDnOut + 128 * wn + 8 * q;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const bool ok = rr + 16 * n < g.nrows;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          u32x4 pk;
          pk.x = pack_bf16x2(acc[2 * u][n][0], acc[2 * u][n][1]);
          pk.y = pack_bf16x2(acc[2 * u][n][2], acc[2 * u][n][3]);
          pk.z = pack_bf16x2(acc[2 * u + 1][n][0], acc[2 * u + 1][n][1]);
          pk.w = pack_bf16x2(acc[2 * u + 1][n][2], acc[2 * u + 1][n][3]);
          uint16_t* dst = ok ? ob + (size_t)16 * n * H + 32 * u : trash;
          *(__attribute__((address_space(1))) u32x4*)dst = pk;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[i][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // Step g: wait until slices 2g, 2g + 1 have landed and every wave is done
  // with step g - 1, refill step g - 1's buffers (slices up to 2g + 4), then
  // compute.  Loads per wave per slice: 4.  A tile's epilogue runs in the next
  // step, after that step's loads are issued: its stores are then younger than
  // the slices the following wait needs (that wait lets them stay
  // outstanding) and have until the wait after it to complete.
  for (int sg = 0; sg < 2 && sg < total; ++sg) {
    issue_x(slot(2 * sg));
    issue_w(slot(2 * sg + 1));
  }
  if (2 < total) issue_x(slot(4));
  int g = 0;
  bool stored = false;  // the previous step issued an epilogue's stores
  for (int cm = 0; cm < count; ++cm) {
    const bool wact = 64 * wm < gtile(tab_p, first + cm * nbx, S).nrows;  // this wave has rows
    for (int ck = 0; ck < nsteps; ++ck, ++g) {
      // slices issued so far: min(2 total, max(5, 2 g + 3)); those after the
      // two this step needs (2 g, 2 g + 1):
      const int ahead = min(nslices, max(kRingN, 2 * g + 3)) - (2 * g + 2);
      if (stored) {
        if (ahead >= 1) ring_wait<4 + kStores>();
        else ring_wait<kStores>();
      } else {
        if (ahead >= 3) ring_wait<12>();
        else if (ahead == 2) ring_wait<8>();
        else if (ahead == 1) ring_wait<4>();
        else ring_wait<0>();
      }
      if (g >= 1 && g + 1 < total) issue_w(slot(2 * g + 3));
      if (g >= 1 && g + 2 < total) issue_x(slot(2 * g + 4));
      stored = ck == 0 && cm > 0;
      if (stored) epilogue(cm - 1);
      if (wact) full_step(g);
    }
  }
  epilogue(count - 1);
}

bool gemm_shape_ok(int64_t T, int K, int I, int Is, int H) {
  // 128-feature gate/up and 256-column down slices, whole 64-deep steps, lane
  // byte offsets below 2^31
  return I == Is && I % kGuFeat == 0 && I % kGK == 0 && H % kDnOut == 0 && H % kGK == 0 &&
         T * H * 2 < (int64_t(1) << 31) && T * K * I * 2 < (int64_t(1) << 31) &&
         (int64_t)H * 2 * kGK < (int64_t(1) << 31);
}

static int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

// One persistent block per CU (a multiple of 8, so that every XCD has as
// many), fewer when there are fewer tiles.
static dim3 gemm_grid(int64_t tiles) {
  const int cus = cu_count() / 8 * 8;
  const int64_t g = tiles < cus ? (tiles + 7) / 8 * 8 : cus;
  return dim3((unsigned)(g > 0 ? g : 8));
}

hipError_t launch_experts_gemm_bf16(const ExpertArgs& a, hipStream_t s, const StageTimer* tm) {
  if (a.tile_rows != kGRows || !gemm_shape_ok(a.T, a.K, a.I, a.Is, a.H)) return hipErrorInvalidValue;
  if (!a.tiles_ready) {
    stage_begin(tm, kTiles, s);
    const hipError_t e = launch_tiles(a, s);
    stage_end(tm, kTiles, s);
    if (e != hipSuccess) return e;
  }
  const int64_t rtiles = max_expert_tiles(a.T, a.K, a.E, a.Is, a.tile_rows);
  const int gu_slices = a.I / kGuFeat, dn_slices = a.H / kDnOut;
  stage_begin(tm, kGateUp, s);
  hipLaunchKernelGGL(k_expert_gemm<0>, gemm_grid(rtiles * gu_slices), dim3(512), 0, s, a, gu_slices);
  stage_end(tm, kGateUp, s);
  stage_begin(tm, kDown, s);
  hipLaunchKernelGGL(k_expert_gemm<1>, gemm_grid(rtiles * dn_slices), dim3(512), 0, s, a, dn_slices);
  stage_end(tm, kDown, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine_bf16(a, s, tm);
}

bool bwd_gemm_ok(int64_t T, int K, int I, int Is, int H) {
  // r's tiles are 256 features wide
  return gemm_shape_ok(T, K, I, Is, H) && I % (2 * kGuFeat) == 0;
}

hipError_t launch_bwd_gur_gemm(const ExpertArgs& a, hipStream_t s) {
  if (a.tile_rows != kGRows || !bwd_gemm_ok(a.T, a.K, a.I, a.Is, a.H) || !a.trash)
    return hipErrorInvalidValue;
  const int64_t rtiles = max_expert_tiles(a.T, a.K, a.E, a.Is, a.tile_rows);
  const int gu = a.I / kGuFeat, rs = a.I / (2 * kGuFeat);
  hipLaunchKernelGGL(k_expert_gemm<2>, gemm_grid(rtiles * gu), dim3(512), 0, s, a, gu);
  hipLaunchKernelGGL(k_expert_gemm<3>, gemm_grid(rtiles * rs), dim3(512), 0, s, a, rs);
  return hipGetLastError();
}

hipError_t launch_bwd_dx_gemm(const ExpertArgs& a, hipStream_t s) {
  if (a.tile_rows != kGRows || !bwd_gemm_ok(a.T, a.K, a.I, a.Is, a.H) || !a.trash)
    return hipErrorInvalidValue;
  const int64_t rtiles = max_expert_tiles(a.T, a.K, a.E, a.Is, a.tile_rows);
  const int dn = a.H / kDnOut;
  hipLaunchKernelGGL(k_expert_gemm<4>, gemm_grid(rtiles * dn), dim3(512), 0, s, a, dn);
  return hipGetLastError();
}

}  // namespace moe
