// experts_stream.hip -- gate/up + SwiGLU for few rows per expert (a small
// batch of tokens), bf16.
//
// [Routing §四]: every expert is down(silu(gate x) * up x) over stacked
// [E][I][H] weights; [Routing §五]: the shared expert is one more bucket (all T
// tokens).  With tiles of kTileRows = 32 token rows (about 16 rows per expert
// at 512 tokens) the projection is bound by reading each expert's weights
// once, so the kernel is built around streaming them.
//
// gate/up: work item = one 32-row tile x 64 features (16 per wave, of both
// gate and up).  Every stage is a 128-deep K slice of 160 rows x 256 bytes (40 KiB):
// 64 gate rows, 64 up rows and the 32 token rows, so every load instruction
// covers whole 256-byte row segments.  Four stage buffers (160 KiB, all of the
// CU's LDS) form a ring filled by direct global -> LDS loads
// (global_load_lds_dwordx4: each wave instruction writes 1 KiB, lane l at
// +16 l), three stages in flight while one is computed.  Blocks are persistent
// (one per CU) and the ring runs on from one item into the next, so no block
// pays a ring fill or leaves a CU idle at the end of the grid.

#include "device.h"
#include "expert_tiles.h"
#include "kernels.h"
#include "ring.h"

namespace moe {

constexpr int kStageB = 40960;  // bytes per stage
constexpr int kSBK = 128;       // K depth of a stage
constexpr int kSRowB = 256;     // bytes per staged row
constexpr int kSFeat = 64;      // features per item

// One stage's loads of this wave: load g (0..9) brings the lane's 16 bytes
// from base[g] + off[g] (a wave-uniform 64-bit base plus a 32-bit per-lane
// byte offset) into LDS lds + 4096 g + 16 * lane (global_load_lds_dwordx4,
// M0 = the wave's LDS destination).  Written as inline asm so that the
// compiler does not treat the ring's later LDS reads as dependent on every
// load in flight; the ring orders them itself (ring_wait).  The memory
// clobber keeps LDS reads from moving across it.  M0 is saved and restored
// around the loads (the compiler owns it), and every write of M0 is followed
// by the one wait state that an LDS DMA reading M0 needs after a scalar write
// of it.
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

struct GItem {
  int e, row0, nrows, i0;  // expert (E = shared), first row, rows, first feature
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

// Item t = tile t / S, feature slice t % S.  Stage rows 0..63: gate rows
// i0 + r, 64..127: up rows, 128..159: token rows; load j of wave w covers
// stage rows 16 j + 4 w .. + 3 (16 lanes per 256-byte row).
__global__ __launch_bounds__(256, 1) void k_gateup_stream(const ExpertArgs a, int S) {
  constexpr int kLoads = 10;   // loads per wave per stage
  constexpr int kStores = 2;   // epilogue stores per wave
  __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * kStageB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int H = a.H, I = a.I, E = a.E, T = a.T, K = a.K;
  // everything from the argument block is read here, before the first asm
  // statement (see k_expert_gemm)
  const uint8_t* const x_p = uniform_ptr(reinterpret_cast<const uint8_t*>(a.x));
  const uint16_t* const wg_p = uniform_ptr(reinterpret_cast<const uint16_t*>(a.w_gate));
  const uint16_t* const wu_p = uniform_ptr(reinterpret_cast<const uint16_t*>(a.w_up));
  const ptrdiff_t sh_g = uniform_ptr(reinterpret_cast<const uint16_t*>(a.ws_gate)) - wg_p;
  const ptrdiff_t sh_u = uniform_ptr(reinterpret_cast<const uint16_t*>(a.ws_up)) - wu_p;
  const int32_t* const sp_p = uniform_ptr(a.sorted_pair);
  uint16_t* const hr_p = uniform_ptr(reinterpret_cast<uint16_t*>(a.h_routed));
  const ptrdiff_t sh_h = uniform_ptr(reinterpret_cast<uint16_t*>(a.h_shared)) - hr_p;
  const int32_t* const tab_p = uniform_ptr(a.tile_tab);
  const int32_t* const toff_p = uniform_ptr(a.tile_off);
  uint16_t* const trash = hr_p + (size_t)T * K * I + (size_t)(blockIdx.x & 7) * 2048 + 4 * tid;

  // this block's items: first + m * nbx, m = 0 .. count - 1 (XCD x, i.e.
  // blocks b with b mod 8 = x, takes the x-th eighth of the list, so the 16
  // feature slices of a tile run on one XCD and share its token rows)
  const int nitems = sload(toff_p + E + 1) * S;
  const int nbx = (int)(gridDim.x >> 3);
  const int x8 = (int)(blockIdx.x & 7);
  const int lo = (int)((int64_t)nitems * x8 / 8), hi = (int)((int64_t)nitems * (x8 + 1) / 8);
  const int first = lo + (int)(blockIdx.x >> 3);
  if (first >= hi) return;
  const int count = (hi - first + nbx - 1) / nbx;
  const int nst = H / kSBK;        // stages per item
  const int total = count * nst;   // stages of this block
  auto item = [&](int m) __attribute__((always_inline)) {
    const int t = __builtin_amdgcn_readfirstlane(first + m * nbx);
    const int rt = t / S;
    GItem it;
    const int32_t v = __builtin_amdgcn_readfirstlane(sload(tab_p + 2 * rt));
    it.e = v & 0xffff;
    it.nrows = v >> 16;
    it.row0 = __builtin_amdgcn_readfirstlane(sload(tab_p + 2 * rt + 1));
    it.i0 = (t - rt * S) * kSFeat;
    return it;
  };

  // lane offsets: weights fixed (row (r & 63) of the item's 64), tokens per item
  uint32_t off[10];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 16 * j + 4 * w + (lane >> 4);
    off[j] = (uint32_t)((r & 63) * H * 2 + (((lane & 15) ^ (r & 15)) << 4));
  }
  int32_t ptok[2];  // sorted pairs of the token rows of the next item (gathered)
  int pe = 0, prow0 = 0;
  auto fetch_rows = [&](int m) __attribute__((always_inline)) {
    const GItem it = item(m);
    pe = it.e;
    prow0 = it.row0;
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
  fetch_rows(0);

  // stage cursor: item m, stage kk of it
  int sm = -1, sk = 0;
  const uint8_t *gb = nullptr, *ub = nullptr;
  auto issue = [&](int c) __attribute__((always_inline)) {
    if (sk == 0) {
      ++sm;
      const GItem it = item(sm);
      const bool sh = it.e >= E;
      const size_t wofs = (sh ? 0 : (size_t)it.e * I * H) + (size_t)it.i0 * H;
      gb = reinterpret_cast<const uint8_t*>(uniform_ptr(wg_p + (sh ? sh_g : 0) + wofs));
      ub = reinterpret_cast<const uint8_t*>(uniform_ptr(wu_p + (sh ? sh_u : 0) + wofs));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 16 * (8 + j) + 4 * w + (lane >> 4);
        const int tok = pe < E ? ptok[j] / K : ptok[j];
        off[8 + j] = (uint32_t)(min(tok, T - 1) * H * 2 + (((lane & 15) ^ (r & 15)) << 4));
      }
      if (sm + 1 < count) fetch_rows(sm + 1);
    }
    const void* base[10] = {gb, gb, gb, gb, ub, ub, ub, ub, x_p, x_p};
    const uint32_t lds = ring0_of(ring, c & 3, w);
    const int kb = sk * kSRowB;
    const void* bk[10];
#pragma unroll
    for (int j = 0; j < 10; ++j) bk[j] = reinterpret_cast<const uint8_t*>(base[j]) + kb;
    dma_stage(bk, off, lds);
    if (++sk == nst) sk = 0;
  };

  f32x4 accg[2], accu[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) accg[n] = accu[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int c) __attribute__((always_inline)) {
    const uint8_t* st = ring + (c & 3) * kStageB;
    u32x4 Ag[4], Au[4], B[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      Ag[u] = lds16(st + sswz(16 * w + r16, 4 * u + q));
      Au[u] = lds16(st + sswz(64 + 16 * w + r16, 4 * u + q));
#pragma unroll
      for (int n = 0; n < 2; ++n) B[u][n] = lds16(st + sswz(128 + 16 * n + r16, 4 * u + q));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        accg[n] = mfma16x16x32(Ag[u], B[u][n], accg[n]);
        accu[n] = mfma16x16x32(Au[u], B[u][n], accu[n]);
      }
  };
  // epilogue: lane holds features i0 + 16 w + 4 q + 0..3 of token row 16 n + r16;
  // exactly kStores stores per wave (rows past the tile end go to trash)
  auto epilogue = [&](int m) __attribute__((always_inline)) {
    const GItem it = item(m);
    uint16_t* hb = hr_p + (it.e >= E ? sh_h : 0) + (size_t)it.row0 * I + it.i0 + 16 * w + 4 * q;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int row = 16 * n + r16;
      float hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[i] = silu_f32(accg[n][i]) * accu[n][i];
      u32x2 pk;
      pk.x = pack_bf16x2(hv[0], hv[1]);
      pk.y = pack_bf16x2(hv[2], hv[3]);
      store8(row < it.nrows ? hb + (size_t)row * I : trash, pk);
      accg[n] = accu[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // Stage c: wait until it has landed and every wave is done with stage c - 1,
  // load stage c + 3 into c - 1's buffer, run the epilogue of the previous item
  // when c starts a new one (its stores are then younger than stage c + 3's
  // loads: the waits of stages c + 1 .. c + 3 leave them outstanding), compute.
  for (int c = 0; c < 3 && c < total; ++c) issue(c);
  int epi = -8;  // stage at which the last epilogue ran
  for (int c = 0; c < total; ++c) {
    const int ahead = min(total, max(3, c + 3)) - (c + 1);  // stages issued after c
    const bool st = c <= epi + 3;
    if (ahead >= 2) { if (st) ring_wait<2 * kLoads + kStores>(); else ring_wait<2 * kLoads>(); }
    else if (ahead == 1) { if (st) ring_wait<kLoads + kStores>(); else ring_wait<kLoads>(); }
    else { if (st) ring_wait<kStores>(); else ring_wait<0>(); }
    if (c + 3 < total) issue(c + 3);
    if (c > 0 && c % nst == 0) {
      epilogue(c / nst - 1);
      epi = c;
    }
    compute(c);
  }
  epilogue(count - 1);
}

bool stream_ring_ok(const ExpertArgs& a) {
  // whole stages; routed and shared experts of one width; lane offsets 32-bit
  return a.H % kSBK == 0 && a.H / kSBK >= 4 && (a.Is == 0 || a.Is == a.I) &&
         a.I % kSFeat == 0 && (int64_t)a.T * a.H * 2 < (int64_t(1) << 31) &&
         (int64_t)a.I * a.H * 2 < (int64_t(1) << 31) &&
         ((int64_t)a.T * a.K + kGRows) * a.I * 2 < (int64_t(1) << 31);
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

}  // namespace moe
