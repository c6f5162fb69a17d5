// experts_stream.hip -- the expert projections for few rows per expert (a
// small batch of tokens), bf16.
//
// [Routing §四]: every expert is down(silu(gate x) * up x) over stacked
// [E][I][H] weights; [Routing §五]: the shared expert is one more bucket (all T
// tokens).  With tiles of kTileRows = 32 token rows (about 16 rows per expert
// at 512 tokens) both projections are bound by reading each expert's weights
// once, so the kernel is built around streaming them.
//
// One kernel, two modes; a work item is one 32-row tile x a slice of the
// output features, and every stage is a 128-deep K slice of 160 rows x 256
// bytes (40 KiB): 128 weight rows and the 32 token rows, so every load
// instruction covers whole 256-byte row segments.
//   gate/up (MODE 0): 64 features a slice (16 per wave, of both gate and up);
//            weight rows 0..63 are gate rows, 64..127 up rows (K = H
//            contiguous), token rows are the gathered x rows; h = silu(g) u
//            is formed in registers.
//   down (MODE 1): 256 output columns a slice (64 per wave), stages 64
//            deep: W_down[e] is [I][H], so a stage holds 64 consecutive k
//            rows of the slice's columns (512 bytes each), and the LDS
//            transpose read turns them into the MFMA operand (4 consecutive k
//            of one column per lane); the token rows are the tile's h rows
//            (contiguous, no gather), 128 bytes each, so they are 1/8 of a
//            stage's 36 KiB.  K = I.  (A layout of 128 columns and 128-deep
//            stages, h rows 1/4 of the bytes and items of half as many
//            stages, ran at 106 us against 98 at 512 tokens.)
// Four stage buffers (160 KiB, all of the CU's LDS) form a ring filled by
// direct global -> LDS loads (global_load_lds_dwordx4: each wave instruction
// writes 1 KiB, lane l at +16 l), three stages in flight while one is
// computed.  Blocks are persistent (one per CU) and the ring runs on from one
// item into the next, so no block pays a ring fill or leaves a CU idle at the
// end of the grid.

#include <type_traits>

#include "device.h"
#include "expert_tiles.h"
#include "kernels.h"
#include "ring.h"

namespace moe {

constexpr int kStageB = 40960;  // bytes per stage
constexpr int kSBK = 128;       // K depth of a stage
constexpr int kSRowB = 256;     // bytes per staged row
constexpr int kSFeat = 64;      // gate/up features per item
constexpr int kSOut = 256;      // bf16 down output columns per item
constexpr int kSOutF32 = 128;   // fp32 down output columns per item

// One stage's loads of this wave: load g (0..9) brings the lane's 16 bytes
// from base[g] + off[g] (a wave-uniform 64-bit base plus a 32-bit per-lane
// byte offset) into LDS lds + 4096 g + 16 * lane (global_load_lds_dwordx4,
// M0 = the wave's LDS destination).  Written as inline asm so that the
// compiler does not treat the ring's later LDS reads as dependent on every
// load in flight; the ring orders them itself (ring_wait).  The memory
// clobber keeps LDS reads from moving across it.  M0 is saved and restored
// around the loads (the compiler owns it), and every write of M0 is followed
// by the one wait state that an LDS DMA reading M0 needs after a scalar write
// of it.  The weight loads (g < 8) carry the nontemporal hint: every weight
// byte is read once per item and cached copies only evict the token rows,
// which the item's neighbours (the other feature slices of its tile) read
// again; measured, the hint lifts the stream from 5.7 to 6.3 TB/s.
__device__ __forceinline__ void dma_stage(const void* const (&base)[10], const uint32_t (&off)[10],
                                          uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %21\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %11 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %12 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %13 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %14 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %5, %15 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %6, %16 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %7, %17 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %8, %18 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
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

// The first nine of dma_stage's loads (a stage of 64 rows of 512 bytes and
// 32 rows of 128 bytes: 36 KiB).
__device__ __forceinline__ void dma_stage9(const void* const (&base)[10], const uint32_t (&off)[10],
                                           uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %19\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %10 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %11 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %12 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %13 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %5, %14 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %6, %15 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %7, %16 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %8, %17 nt\n\ts_add_u32 m0, m0, 4096\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %9, %18\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "v"(off[4]), "v"(off[5]), "v"(off[6]),
        "v"(off[7]), "v"(off[8]), "s"(base[0]), "s"(base[1]), "s"(base[2]), "s"(base[3]),
        "s"(base[4]), "s"(base[5]), "s"(base[6]), "s"(base[7]), "s"(base[8]), "s"(lds)
      : "memory", "scc");
}

struct GItem {
  int e, row0, nrows, i0;  // expert (E = shared), first row, rows, first feature / column
};

// LDS byte address of wave w's first 1 KiB slot in stage buffer b.
__device__ __forceinline__ uint32_t ring0_of(const uint8_t* ring, int b, int w) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lvoid_t*)ring)) + kStageB * b +
      1024u * w);
}

// Swizzled position of 16-byte chunk c of a 256-byte staged row r (16 chunks;
// the XOR with the row's low 4 bits spreads 16 consecutive rows read at one
// chunk index over all banks).
__device__ __forceinline__ int sswz(int r, int c) { return r * kSRowB + ((c ^ (r & 15)) << 4); }

// 16-byte store to global memory (a global, not flat, store: see store8).
__device__ __forceinline__ void store16(uint16_t* p, u32x4 v) {
  *(__attribute__((address_space(1))) u32x4*)p = v;
}

// fp32 down stages: W_down k-row r (512 bytes: 128 output columns) keeps
// 16-byte chunk c at r * 512 + 16 (c ^ 4 ((r >> 2) & 3)), so the four k-rows
// that one per-element operand read covers (4 apart) meet four different
// 64-byte bank groups.
__device__ __forceinline__ int f32d_chunk(int r, int c) { return c ^ (((r >> 2) & 3) << 2); }

// Item t = tile t / S, slice t % S.  A stage is 160 KiB / 4 = 40 KiB: 32 KiB
// of weight rows, then 32 token rows of 256 bytes (stage rows 128..159, chunk
// c at sswz(128 + n, c)); loads 0..7 of each wave bring weights, 8 and 9
// token rows (load j of wave w fills stage bytes 4096 j + 1024 w + 16 lane).
//   MODE 0 (gate/up, bf16): weight row r < 64 is gate row i0 + r, r >= 64 up
//     row i0 + r - 64, K columns 128 s .. of stage s (256 bytes); chunk c at
//     sswz(r, c).
//   MODE 1 (down, bf16): weight row r (of 64) is W_down row 64 s + r at
//     columns i0 .. i0 + 255 (512 bytes), chunk c at r * 512 + 16
//     (c ^ wd_swz(r)) (the layout of k_expert_gemm's down slices: the
//     transpose reads of 16 rows at one 32-byte window meet two to a
//     window); the 32 token rows (128 bytes, K columns 64 s ..) follow at
//     32 KiB, chunk c of row n at rs_addr(n, c); one token load a wave
//     (9 loads a stage).
//   MODE 2 (gate/up, fp32): as MODE 0 with fp32 rows: K columns 64 s .. (256
//     bytes), 64 features an item.
//   MODE 3 (down, fp32): weight row r (of 64) is W_down row 64 s + r at
//     columns i0 .. i0 + 127 (512 bytes), chunk c at r * 512 + 16
//     f32d_chunk(r, c); token rows carry K columns 64 s ...
template <int MODE>
__device__ __forceinline__ void stream_body(const ExpertArgs& a, int S) {
  constexpr bool kDown = MODE == 1 || MODE == 3;
  constexpr bool kF32 = MODE == 2 || MODE == 3;
  constexpr bool kWide = MODE == 1;  // bf16 down: 512-byte weight rows, 128-byte token rows
  typedef typename std::conditional<kF32, float, uint16_t>::type elt_t;
  constexpr int kEl = sizeof(elt_t);
  constexpr int kSK = (kF32 || kWide) ? 64 : kSBK;  // K depth of a stage
  constexpr int kCols = MODE == 1 ? kSOut : MODE == 3 ? kSOutF32 : kSFeat;  // output columns an item
  constexpr int kLoads = kWide ? 9 : 10;  // loads per wave per stage
  constexpr int kStores = (MODE == 3 || kWide) ? 4 : 2;  // epilogue stores per wave
  constexpr int kAT = kWide ? 4 : 2;  // accumulator tiles a token tile
  // with at least 4 stages an item the epilogue's item is one of the last two
  // the issue cursor started (fp32 down items may have fewer: re-read)
  constexpr bool kKeepItems = MODE != 3;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * kStageB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int H = a.H, I = a.I, E = a.E, T = a.T, K = a.K;
  // everything from the argument block is read here, before the first asm
  // statement (see k_expert_gemm)
  const uint8_t* const x_p = uniform_ptr(reinterpret_cast<const uint8_t*>(a.x));
  const elt_t* const wg_p = uniform_ptr(reinterpret_cast<const elt_t*>(a.w_gate));
  const elt_t* const wu_p = uniform_ptr(reinterpret_cast<const elt_t*>(a.w_up));
  const ptrdiff_t sh_g = uniform_ptr(reinterpret_cast<const elt_t*>(a.ws_gate)) - wg_p;
  const ptrdiff_t sh_u = uniform_ptr(reinterpret_cast<const elt_t*>(a.ws_up)) - wu_p;
  const elt_t* const wd_p = uniform_ptr(reinterpret_cast<const elt_t*>(a.w_down));
  const ptrdiff_t sh_d = uniform_ptr(reinterpret_cast<const elt_t*>(a.ws_down)) - wd_p;
  const int32_t* const sp_p = uniform_ptr(a.sorted_pair);
  elt_t* const hr_p = uniform_ptr(reinterpret_cast<elt_t*>(a.h_routed));
  const ptrdiff_t sh_h = uniform_ptr(reinterpret_cast<elt_t*>(a.h_shared)) - hr_p;
  elt_t* const or_p = uniform_ptr(reinterpret_cast<elt_t*>(a.o_routed));
  const ptrdiff_t sh_o = uniform_ptr(reinterpret_cast<elt_t*>(a.o_shared)) - or_p;
  const int32_t* const tab_p = uniform_ptr(a.tile_tab);
  const int32_t* const toff_p = uniform_ptr(a.tile_off);
  // dropped stores (rows past a tile's end) go to the padding rows of
  // h_routed, which nothing reads: 8 (MODE 0) or 16 bytes a lane, at most
  // 32 KiB past the last row (the padding holds kGRows rows of I >= 64)
  elt_t* const trash = hr_p + (size_t)T * K * I +
                       (kF32 ? (size_t)(blockIdx.x & 7) * 1024 + 4 * tid
                             : (size_t)(blockIdx.x & 7) * 2048 + (MODE == 0 ? 4 : 8) * tid);

  // this block's items: first + m * nbx, m = 0 .. count - 1 (XCD x, i.e.
  // blocks b with b mod 8 = x, takes the x-th eighth of the list, so the
  // slices of a tile run on one XCD and share its token rows)
  const int nitems = sload(toff_p + E + 1) * S;
  const int nbx = (int)(gridDim.x >> 3);
  const int x8 = (int)(blockIdx.x & 7);
  const int lo = (int)((int64_t)nitems * x8 / 8), hi = (int)((int64_t)nitems * (x8 + 1) / 8);
  const int first = lo + (int)(blockIdx.x >> 3);
  if (first >= hi) return;
  const int count = (hi - first + nbx - 1) / nbx;
  const int nst = (kDown ? I : H) / kSK;  // stages per item
  const int total = count * nst;          // stages of this block
  auto item = [&](int m) __attribute__((always_inline)) {
    const int t = __builtin_amdgcn_readfirstlane(first + m * nbx);
    const int rt = t / S;
    GItem it;
    const int32_t v = __builtin_amdgcn_readfirstlane(sload(tab_p + 2 * rt));
    it.e = v & 0xffff;
    it.nrows = v >> 16;
    it.row0 = __builtin_amdgcn_readfirstlane(sload(tab_p + 2 * rt + 1));
    it.i0 = (t - rt * S) * kCols;
    return it;
  };
  // lane offsets of the weight loads (fixed; gate/up: row (r & 63) of the
  // item's 64 of gate or up; down: row r of the stage) and of the token
  // loads (per item)
  uint32_t off[10];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (MODE == 3) {
      const int r = 8 * j + 2 * w + (lane >> 5);
      off[j] = (uint32_t)(r * H * 4 + (f32d_chunk(r, lane & 31) << 4));
    } else if (kWide) {
      const int r = 8 * j + 2 * w + (lane >> 5);
      off[j] = (uint32_t)(r * H * 2 + (((lane & 31) ^ wd_swz(r)) << 4));
    } else {
      const int r = 16 * j + 4 * w + (lane >> 4);
      off[j] = (uint32_t)((r & 63) * H * kEl + (((lane & 15) ^ (r & 15)) << 4));
    }
  }
  int32_t ptok[2];  // gate/up: sorted pairs of the token rows of the next item (gathered)
  int pe = 0;
  auto fetch_rows = [&](int m) __attribute__((always_inline)) {
    const GItem it = item(m);
    pe = it.e;
    // token rows 16 j + 4 w + lane / 16 of the item (rows past its end repeat
    // its last row): scalar loads, which wait on lgkmcnt and never on the
    // ring's vmcnt; each lane picks its row's value
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int32_t v = 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int tr = min(16 * j + 4 * w + m, it.nrows - 1);
        const int32_t sv = it.e < E ? sload(sp_p + it.row0 + tr) : it.row0 + tr;
        v = (lane >> 4) == m ? sv : v;
      }
      ptok[j] = v;
    }
  };
  if (!kDown) fetch_rows(0);

  // stage cursor: item sm, stage sk of it; prev and cur are the last two
  // items started (the epilogue's, kept so that it reads no table entry)
  int sm = -1, sk = 0;
  GItem prev{}, cur{};
  // rows of the item of the stage in ring slot b, byte b (a tile holds at
  // most 32 rows): compute skips the second 16-row token tile when the item
  // has at most 16 rows (its accumulators stay zero; the epilogue sends those
  // rows to trash)
  uint32_t ring_rows = 0;
  const uint8_t *gb = nullptr, *ub = nullptr, *tb = nullptr;
  auto issue = [&](int c) __attribute__((always_inline)) {
    if (sk == 0) {
      ++sm;
      const GItem it = item(sm);
      prev = cur;
      cur = it;
      const bool sh = it.e >= E;
      if (!kDown) {
        const size_t wofs = (sh ? 0 : (size_t)it.e * I * H) + (size_t)it.i0 * H;
        gb = reinterpret_cast<const uint8_t*>(uniform_ptr(wg_p + (sh ? sh_g : 0) + wofs));
        ub = reinterpret_cast<const uint8_t*>(uniform_ptr(wu_p + (sh ? sh_u : 0) + wofs));
        tb = x_p;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = 16 * (8 + j) + 4 * w + (lane >> 4);
          const int tok = pe < E ? ptok[j] / K : ptok[j];
          off[8 + j] = (uint32_t)(min(tok, T - 1) * H * kEl + (((lane & 15) ^ (r & 15)) << 4));
        }
        if (sm + 1 < count) fetch_rows(sm + 1);
      } else {
        const size_t wofs = (sh ? 0 : (size_t)it.e * I * H) + (size_t)it.i0;
        gb = reinterpret_cast<const uint8_t*>(uniform_ptr(wd_p + (sh ? sh_d : 0) + wofs));
        ub = gb;
        tb = reinterpret_cast<const uint8_t*>(
            uniform_ptr(hr_p + (sh ? sh_h : 0) + (size_t)it.row0 * I));
        if (kWide) {
          // one load: token rows 8 w + lane / 8, 128 bytes (64 k) each
          const int r = 8 * w + (lane >> 3);
          const int tr = min(r, it.nrows - 1);
          off[8] = (uint32_t)(tr * I * 2 + (((lane & 7) ^ ((r >> 1) & 7)) << 4));
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int r = 16 * (8 + j) + 4 * w + (lane >> 4);
            const int tr = min(r - 128, it.nrows - 1);
            off[8 + j] = (uint32_t)(tr * I * kEl + (((lane & 15) ^ (r & 15)) << 4));
          }
        }
      }
    }
    const void* base[10] = {gb, gb, gb, gb, ub, ub, ub, ub, tb, tb};
    const uint32_t lds = ring0_of(ring, c & 3, w);
    ring_rows = (ring_rows & ~(0xffu << (8 * (c & 3)))) | ((uint32_t)cur.nrows << (8 * (c & 3)));
    // stage advance: gate/up weights and all token rows move 256 bytes along
    // K; down weights move kSK rows
    const size_t kw = kDown ? (size_t)sk * kSK * H * kEl : (size_t)sk * kSRowB;
    const int kt = sk * kSK * kEl;
    const void* bk[10];
#pragma unroll
    for (int j = 0; j < 10; ++j)
      bk[j] = reinterpret_cast<const uint8_t*>(base[j]) + (j < 8 ? kw : (size_t)kt);
    if (kWide) dma_stage9(bk, off, lds);
    else dma_stage(bk, off, lds);
    if (++sk == nst) sk = 0;
  };

  // acc[t][n]: gate/up: t = 0 gate, 1 up, features 16 w + (MFMA row) of
  // token tile n; down: column tile t (see below), token tile n
  f32x4 acc[kAT][2];
#pragma unroll
  for (int t = 0; t < kAT; ++t)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // fp32 (16x16x4 MFMA, one element of A and of B a lane): K block b of 16
  // is read as 16-byte chunks 4 b + q (k = 16 b + 4 q .. + 3) and MFMA j of
  // the block takes element j, i.e. k = 16 b + 4 q + j from lane group q.
  // MODE 3's A operand (W_down[k][column]) is read element by element: lane
  // (m, q) takes k row 16 b + 4 q + j at column 32 w + 16 t + m.
  // MODE 1 transpose reads: lane 4 c + m of group q points at k row
  // 32 u + 8 q + c (+ 4 for the second read, which shares the row's swizzle)
  // and columns 64 w + 32 (t / 2) + 8 m + 4 (t % 2) .. + 3 (chunk
  // 8 w + 4 (t / 2) + m, half t % 2), so column tile t's MFMA row 4 q' + i is
  // column 64 w + 32 (t / 2) + 8 q' + 4 (t % 2) + i and tiles 2 v, 2 v + 1
  // give each lane the 8 columns 64 w + 32 v + 8 q' .. + 7.
  const int wd_row = 8 * q + (r16 >> 2);
  const int wd_lane = wd_row * 512 + ((((8 * w + (r16 & 3)) ^ wd_swz(wd_row))) << 4);
  auto compute_nt = [&](int c, auto ntc) __attribute__((always_inline)) {
    constexpr int NT = decltype(ntc)::value;  // 16-row token tiles computed
    const uint8_t* st = ring + (c & 3) * kStageB;
    if (kWide) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 A[4], B[2] = {};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          // chunk 8 w + 4 (t / 2) + m: the XOR with wd_swz (even, < 16) keeps
          // bit 2 of the chunk, so 4 (t / 2) moves the swizzled chunk by 4
          const uint8_t* p =
              st + 32 * u * 512 + (wd_lane ^ ((4 * (t >> 1)) << 4)) + 8 * (t & 1);
          const u32x2 lo = lds_tr16(p), hi = lds_tr16(p + 4 * 512);
          A[t] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) B[n] = lds16(st + 32768 + rs_addr(16 * n + r16, 4 * u + q));
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[t][n] = mfma16x16x32(A[t], B[n], acc[t][n]);
      }
    } else if (!kF32) {
      u32x4 A0[4], A1[4], B[4][2] = {};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        A0[u] = lds16(st + sswz(16 * w + r16, 4 * u + q));
        A1[u] = lds16(st + sswz(64 + 16 * w + r16, 4 * u + q));
#pragma unroll
        for (int n = 0; n < NT; ++n) B[u][n] = lds16(st + sswz(128 + 16 * n + r16, 4 * u + q));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          acc[0][n] = mfma16x16x32(A0[u], B[u][n], acc[0][n]);
          acc[1][n] = mfma16x16x32(A1[u], B[u][n], acc[1][n]);
        }
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        f32x4 B[2] = {};
        float A[2][4];  // [t][j]: the A element of MFMA j of operand t
#pragma unroll
        for (int n = 0; n < NT; ++n)
          B[n] = __builtin_bit_cast(f32x4, lds16(st + sswz(128 + 16 * n + r16, 4 * b + q)));
        if (!kDown) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const f32x4 v =
                __builtin_bit_cast(f32x4, lds16(st + sswz(64 * t + 16 * w + r16, 4 * b + q)));
#pragma unroll
            for (int j = 0; j < 4; ++j) A[t][j] = v[j];
          }
        } else {
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r = 16 * b + 4 * q + j, col = 32 * w + 16 * t + r16;
              A[t][j] = *reinterpret_cast<const float*>(
                  st + r * 512 + (f32d_chunk(r, col >> 2) << 4) + 4 * (col & 3));
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int t = 0; t < 2; ++t)
              acc[t][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[t][j], B[n][j], acc[t][n], 0, 0, 0);
      }
    }
  };
  auto compute = [&](int c) __attribute__((always_inline)) {
    if (((ring_rows >> (8 * (c & 3))) & 0xffu) > 16u)
      compute_nt(c, std::integral_constant<int, 2>());
    else
      compute_nt(c, std::integral_constant<int, 1>());
  };

  // epilogue: exactly kStores stores per wave (rows past the tile end go to
  // trash).  MODE 0: lane holds features i0 + 16 w + 4 q + 0..3 of token row
  // 16 n + r16 (bf16, 8 bytes); MODE 1: columns i0 + 64 w + 32 v + 8 q + 0..7
  // for v = 0, 1 (two 16-byte stores); MODE 2: features i0 + 16 w + 4 q +
  // 0..3 (fp32, 16 bytes); MODE 3: columns i0 + 32 w + 16 t + 4 q + 0..3 of
  // column tile t (fp32, 16 bytes).
  auto epilogue = [&](const GItem& it) __attribute__((always_inline)) {
    const bool sh = it.e >= E;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int row = 16 * n + r16;
      const bool ok = row < it.nrows;
      if (MODE == 0 || MODE == 2) {
        elt_t* hb = hr_p + (sh ? sh_h : 0) + (size_t)it.row0 * I + it.i0 + 16 * w + 4 * q;
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = silu_f32(acc[0][n][i]) * acc[1][n][i];
        if (MODE == 0) {
          u32x2 pk;
          pk.x = pack_bf16x2(hv[0], hv[1]);
          pk.y = pack_bf16x2(hv[2], hv[3]);
          store8(reinterpret_cast<uint16_t*>(ok ? hb + (size_t)row * I : trash), pk);
        } else {
          const u32x4 pk = {__float_as_uint(hv[0]), __float_as_uint(hv[1]),
                            __float_as_uint(hv[2]), __float_as_uint(hv[3])};
          store16(reinterpret_cast<uint16_t*>(ok ? hb + (size_t)row * I : trash), pk);
        }
      } else if (kWide) {
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          elt_t* ob = or_p + (sh ? sh_o : 0) + (size_t)it.row0 * H + it.i0 + 64 * w + 32 * v + 8 * q;
          u32x4 pk;
          pk.x = pack_bf16x2(acc[2 * v][n][0], acc[2 * v][n][1]);
          pk.y = pack_bf16x2(acc[2 * v][n][2], acc[2 * v][n][3]);
          pk.z = pack_bf16x2(acc[2 * v + 1][n][0], acc[2 * v + 1][n][1]);
          pk.w = pack_bf16x2(acc[2 * v + 1][n][2], acc[2 * v + 1][n][3]);
          store16(reinterpret_cast<uint16_t*>(ok ? ob + (size_t)row * H : trash), pk);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          elt_t* ob = or_p + (sh ? sh_o : 0) + (size_t)it.row0 * H + it.i0 + 32 * w + 16 * t + 4 * q;
          const u32x4 pk = {__float_as_uint(acc[t][n][0]), __float_as_uint(acc[t][n][1]),
                            __float_as_uint(acc[t][n][2]), __float_as_uint(acc[t][n][3])};
          store16(reinterpret_cast<uint16_t*>(ok ? ob + (size_t)row * H : trash), pk);
        }
      }
#pragma unroll
      for (int t = 0; t < kAT; ++t) acc[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // Stage c: wait until it has landed and every wave is done with stage c - 1,
  // load stage c + 3 into c - 1's buffer, run the epilogue of the previous item
  // when c starts a new one (its stores are then younger than stage c + 3's
  // loads: the waits of stages c + 1 .. c + 3 leave them outstanding), compute.
  // (A wait that may have two epilogues' stores outstanding, with fewer than
  // 4 stages an item, counts one: it waits for more than it needs.)
  for (int c = 0; c < 3 && c < total; ++c) issue(c);
  int epi = -8;  // stage at which the last epilogue ran
  for (int c = 0; c < total; ++c) {
    const int ahead = min(total, max(3, c + 3)) - (c + 1);  // stages issued after c
    const bool st = c <= epi + 3;
    if (ahead >= 2) { if (st) ring_wait<2 * kLoads + kStores>(); else ring_wait<2 * kLoads>(); }
    else if (ahead == 1) { if (st) ring_wait<kLoads + kStores>(); else ring_wait<kLoads>(); }
    else { if (st) ring_wait<kStores>(); else ring_wait<0>(); }
    if (c + 3 < total) issue(c + 3);
    // (with nst >= 4 stages an item, issue(c + 3) has not started another
    // item yet: prev is item c / nst - 1)
    if (c > 0 && c % nst == 0) {
      if (kKeepItems) epilogue(prev);
      else epilogue(item(c / nst - 1));
      epi = c;
    }
    compute(c);
  }
  if (kKeepItems) epilogue(cur);
  else epilogue(item(count - 1));
}

__global__ __launch_bounds__(256, 1) void k_gateup_stream(const ExpertArgs a, int S) {
  stream_body<0>(a, S);
}
__global__ __launch_bounds__(256, 1) void k_down_stream(const ExpertArgs a, int S) {
  stream_body<1>(a, S);
}
__global__ __launch_bounds__(256, 1) void k_gateup_stream_f32(const ExpertArgs a, int S) {
  stream_body<2>(a, S);
}
__global__ __launch_bounds__(256, 1) void k_down_stream_f32(const ExpertArgs a, int S) {
  stream_body<3>(a, S);
}

bool stream_ring_ok(const ExpertArgs& a) {
  // whole stages, at least 4 an item; routed and shared experts of one
  // width; lane offsets 32-bit
  return a.H % kSBK == 0 && a.H / kSBK >= 4 && (a.Is == 0 || a.Is == a.I) &&
         a.I % kSFeat == 0 && (int64_t)a.T * a.H * 2 < (int64_t(1) << 31) &&
         (int64_t)a.I * a.H * 2 < (int64_t(1) << 31) &&
         ((int64_t)a.T * a.K + kGRows) * a.I * 2 < (int64_t(1) << 31);
}

bool down_stream_ok(const ExpertArgs& a) {
  // 256-column items of whole 64-deep stages, at least 4 an item; weight lane
  // offsets (64 rows) 32-bit
  return stream_ring_ok(a) && a.H % kSOut == 0 && a.I % 64 == 0 && a.I / 64 >= 4 &&
         (int64_t)64 * a.H * 2 < (int64_t(1) << 31);
}

static dim3 stream_grid(int64_t items) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  int64_t g = items < cus ? (items + 7) / 8 * 8 : cus / 8 * 8;
  return dim3((unsigned)(g > 0 ? g : 8));
}

hipError_t launch_gateup_stream_bf16(const ExpertArgs& a, int64_t tiles, hipStream_t s,
                                     const StageTimer* tm) {
  const int slices = a.I / kSFeat;
  stage_begin(tm, kGateUp, s);
  hipLaunchKernelGGL(k_gateup_stream, stream_grid(tiles * slices), dim3(256), 0, s, a, slices);
  stage_end(tm, kGateUp, s);
  return hipGetLastError();
}

bool stream_f32_ok(const ExpertArgs& a) {
  // whole 64-deep stages, at least 4 an item for gate/up; 64-feature and
  // 128-column slices; routed and shared experts of one width; lane offsets
  // 32-bit
  return a.H % 128 == 0 && a.H / 64 >= 4 && a.I % 64 == 0 && (a.Is == 0 || a.Is == a.I) &&
         (int64_t)a.T * a.H * 4 < (int64_t(1) << 31) &&
         (int64_t)64 * a.H * 4 < (int64_t(1) << 31) && (int64_t)kTileRows * a.I * 4 < (int64_t(1) << 31);
}

hipError_t launch_stream_f32(const ExpertArgs& a, int64_t tiles, hipStream_t s,
                             const StageTimer* tm) {
  const int gslices = a.I / kSFeat, dslices = a.H / kSOutF32;
  stage_begin(tm, kGateUp, s);
  hipLaunchKernelGGL(k_gateup_stream_f32, stream_grid(tiles * gslices), dim3(256), 0, s, a,
                     gslices);
  stage_end(tm, kGateUp, s);
  stage_begin(tm, kDown, s);
  hipLaunchKernelGGL(k_down_stream_f32, stream_grid(tiles * dslices), dim3(256), 0, s, a, dslices);
  stage_end(tm, kDown, s);
  return hipGetLastError();
}

hipError_t launch_down_stream_bf16(const ExpertArgs& a, int64_t tiles, hipStream_t s,
                                   const StageTimer* tm) {
  stage_begin(tm, kDown, s);
  const int slices = a.H / kSOut;
  hipLaunchKernelGGL(k_down_stream, stream_grid(tiles * slices), dim3(256), 0, s, a, slices);
  stage_end(tm, kDown, s);
  return hipGetLastError();
}

}  // namespace moe
