// permute.hip -- per-expert counts and a stable bucket order of the pairs.
//
// [Routing §六]: per-expert hit counts are a bincount of the chosen indices;
// [Routing §四]: the eager inference path sorts tokens into one bucket per
// expert before running each bucket.  The T*K (token, slot) pairs
// p = t*K + j are counting-sorted by expert keeping ascending p inside each
// bucket.  Ranks are computed without atomics on the data path: a wave takes 64
// consecutive pairs at a time, finds the lanes holding the same expert with
// ballots over the index bits, and ranks each lane among the lower lanes of
// its group; per-wave running counts live in LDS.  Everything is integer
// arithmetic in a fixed order, so results are deterministic.
//
// The same kernels also build the expert-tile list (tile_off, tile_rows rows
// per tile; the shared expert is "expert" E with T rows) used by the expert
// kernels.
//
// An index outside [0, E) is skipped (not counted, pair_slot = -1) and sets
// status bit 2.
#include "device.h"
#include "expert_tiles.h"
#include "kernels.h"

namespace moe {

constexpr int kPermMaxE = 512;

// Ballot-based match: `same` = lanes holding the same valid expert as this one.
__device__ __forceinline__ uint64_t match_lanes(int32_t e, bool valid, int nbits) {
  uint64_t same = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t ones = __ballot(valid && bit);
    same &= bit ? ones : ~ones;
  }
  return same;
}

// Inclusive scan of v over the block's 1024 threads: shuffle scan inside each
// wave, then the 16 wave totals.
__device__ __forceinline__ int32_t block_scan_1024(int32_t v, int32_t* sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  if (lane == 63) sc[w] = v;
  __syncthreads();
  if (w == 0) {
    int32_t t = lane < 16 ? sc[lane] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int32_t o = __shfl_up(t, d);
      if (lane >= d) t += o;
    }
    if (lane < 16) sc[16 + lane] = t;
  }
  __syncthreads();
  const int32_t r = v + (w > 0 ? sc[16 + w - 1] : 0);
  __syncthreads();
  return r;
}

// LDS a finish_counts call needs: the block scan's 1024 ints and, per expert
// (and the shared expert), its first tile, first row and rows.
struct FinishLds {
  int32_t sc[1024];
  int32_t toff[kPermMaxE + 2];
  int32_t first[kPermMaxE + 1];
  int32_t rows[kPermMaxE + 1];
};

// counts/offsets/tracking/tile_off/tile_tab from per-expert totals held by
// thread e (and the exclusive expert offsets in offs_lds when given).  With
// write false (block-uniform) only offs_lds is filled.  The tile entries are
// written by all threads, tile t by thread t mod 1024 (its expert found by a
// binary search of the tile offsets): one expert may own hundreds of tiles.
__device__ __forceinline__ void finish_counts(int32_t total, int E, int T, int Is, int tile_rows,
                                              FinishLds& fl,
                                              int32_t* counts, int32_t* offsets,
                                              int32_t* offs_lds, int64_t* tracking,
                                              int32_t* tile_off, int32_t* tile_tab,
                                              bool write = true) {
  int32_t* const sc = fl.sc;
  const int e = threadIdx.x;
  const int32_t incl = block_scan_1024(e < E ? total : 0, sc);
  if (e < E && offs_lds) offs_lds[e] = incl - total;
  if (!write) return;
  if (e < E) {
    counts[e] = total;
    offsets[e] = incl - total;
    if (tracking) tracking[e] += (int64_t)total;
  }
  if (e == E - 1) offsets[E] = incl;
  // tiles of tile_rows rows per expert, the shared expert last
  int32_t n = 0;
  if (e < E) n = (total + tile_rows - 1) / tile_rows;
  else if (e == E && Is > 0) n = (T + tile_rows - 1) / tile_rows;
  const int32_t tin = block_scan_1024(n, sc);
  if (e <= E) {
    tile_off[e] = tin - n;
    fl.toff[e] = tin - n;
    fl.first[e] = e < E ? incl - total : 0;
    fl.rows[e] = e < E ? total : T;
  }
  if (e == E) {
    tile_off[E + 1] = tin;
    fl.toff[E + 1] = tin;
  }
  __syncthreads();
  const int32_t ntiles = fl.toff[E + 1];
  for (int32_t t = threadIdx.x; t < ntiles; t += 1024) {
    // the largest expert x with toff[x] <= t (experts without tiles share
    // their successor's offset and lose to it)
    int lo = 0, hi = E;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (fl.toff[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    write_tile_entry(tile_tab, t, lo, fl.first[lo], fl.rows[lo], t - fl.toff[lo], tile_rows);
  }
}

// ----------------------------------------------------------------------------
// Small P (<= 16 waves x 16 batches x 64 = 16384 pairs): one block does it all.
// ----------------------------------------------------------------------------
constexpr int kSmallWaves = 16, kSmallBatches = 16;
constexpr int kSmallMaxP = kSmallWaves * kSmallBatches * 64;

__global__ __launch_bounds__(1024) void k_permute_small(
    const int32_t* __restrict__ idx, int P, int E, int T, int Is, int tile_rows,
    int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_slot, int64_t* __restrict__ tracking,
    int32_t* __restrict__ tile_off, int32_t* __restrict__ tile_tab,
    uint32_t* __restrict__ status) {
  __shared__ int32_t cnt[kSmallWaves][kPermMaxE];  // 32 KB
  __shared__ FinishLds fl;
  __shared__ int32_t offs[kPermMaxE];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kSmallWaves * kPermMaxE; i += 1024) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int nbits = 32 - __clz(E - 1);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int per = ((P + kSmallWaves * 64 - 1) / (kSmallWaves * 64)) * 64;  // pairs per wave
  const int p0 = w * per;
  // every index load first, straight-line (clamped: a pair past the end
  // re-reads the last one, unused), so that they are in flight together
  int32_t raw[kSmallBatches];
#pragma unroll
  for (int b = 0; b < kSmallBatches; ++b) raw[b] = idx[min(p0 + b * 64 + lane, P - 1)];
  int32_t rank[kSmallBatches], ev[kSmallBatches];
  int bad = 0;
#pragma unroll
  for (int b = 0; b < kSmallBatches; ++b) {
    rank[b] = -1;
    ev[b] = -1;
    if (b * 64 < per) {  // block-uniform
      const int p = p0 + b * 64 + lane;
      const bool active = p < P && b * 64 + lane < per;
      const int32_t e = active ? raw[b] : 0;
      const bool valid = active && (uint32_t)e < (uint32_t)E;
      bad |= active && !valid;
      const uint64_t same = match_lanes(e, valid, nbits);
      if (valid) {
        const int32_t old = cnt[w][e];
        rank[b] = old + __popcll(same & below);
        ev[b] = e;
        if ((same >> lane) == 1ull) cnt[w][e] = old + __popcll(same);  // last lane of its group
      }
    }
  }
  __syncthreads();
  // exclusive prefix over waves for each expert; totals
  int32_t total = 0;
  if (threadIdx.x < E) {
    for (int ww = 0; ww < kSmallWaves; ++ww) {
      const int32_t c = cnt[ww][threadIdx.x];
      cnt[ww][threadIdx.x] = total;
      total += c;
    }
  }
  finish_counts(total, E, T, Is, tile_rows, fl, counts, offsets, offs, tracking, tile_off, tile_tab);
  __syncthreads();
#pragma unroll
  for (int b = 0; b < kSmallBatches; ++b) {
    if (b * 64 < per) {
      const int p = p0 + b * 64 + lane;
      if (p < P && b * 64 + lane < per) {
        const int32_t e = ev[b];
        int32_t pos = -1;
        if (e >= 0) {
          pos = offs[e] + cnt[w][e] + rank[b];
          sorted_pair[pos] = p;
        }
        pair_slot[p] = pos;
      }
    }
  }
  if (__any(bad) && lane == 0) atomicOr(status, 2u);
}

// ----------------------------------------------------------------------------
// Large P: rank per chunk -> per-expert prefix over the chunks (one wave an
// expert) -> scatter (every block scans the expert totals for the offsets;
// block 0 also writes counts, offsets, tracking and the tile list).
// A chunk of `ch` pairs is split over the 4 waves of a block; ch is a power of
// two >= 512 chosen so that there are at most 256 chunks (one block a CU: a
// wave's ranking runs through its pairs 64 at a time, one LDS count update
// after another, so fewer pairs a wave is what shortens it).
// ----------------------------------------------------------------------------
constexpr int kPermMaxChunks = 256;  // k_perm_scan: at most 4 chunks a lane
int permute_chunk(int64_t P) {
  int64_t ch = 512;
  while ((P + ch - 1) / ch > kPermMaxChunks) ch *= 2;
  return (int)ch;
}

__global__ __launch_bounds__(256) void k_perm_rank(const int32_t* __restrict__ idx, int64_t P,
                                                    int E, int ch, int32_t* __restrict__ prank,
                                                    int32_t* __restrict__ chunk_hist,
                                                    uint32_t* __restrict__ status) {
  __shared__ int32_t cnt[4][kPermMaxE];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * kPermMaxE; i += 256) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int nbits = 32 - __clz(E - 1);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int sub = ch / 4;
  const int64_t q0 = (int64_t)blockIdx.x * ch + (int64_t)w * sub;
  int bad = 0;
  // 8 batches of 64 pairs at a time, their index loads issued together
  // (clamped: a pair past the end re-reads the last one, unused; sub is a
  // multiple of 128, so a wave's last group may use only its first batches)
  for (int b0 = 0; b0 < sub; b0 += 512) {
    int32_t raw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) raw[u] = idx[min(q0 + b0 + 64 * u + lane, P - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (b0 + 64 * u >= sub) continue;  // uniform
      const int64_t p = q0 + b0 + 64 * u + lane;
      const bool active = p < P;
      const int32_t e = active ? raw[u] : 0;
      const bool valid = active && (uint32_t)e < (uint32_t)E;
      bad |= active && !valid;
      const uint64_t same = match_lanes(e, valid, nbits);
      if (valid) {
        const int32_t old = cnt[w][e];
        prank[p] = old + __popcll(same & below);
        if ((same >> lane) == 1ull) cnt[w][e] = old + __popcll(same);
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    int32_t run = 0;
    for (int ww = 0; ww < 4; ++ww) {
      const int32_t c = cnt[ww][e];
      cnt[ww][e] = run;
      run += c;
    }
    chunk_hist[(size_t)blockIdx.x * E + e] = run;
  }
  __syncthreads();
  // add the wave's prefix inside the chunk
  for (int b = 0; b < sub; b += 64) {
    const int64_t p = q0 + b + lane;
    if (p < P) {
      const int32_t e = idx[p];
      if ((uint32_t)e < (uint32_t)E) prank[p] += cnt[w][e];
    }
  }
  if (__any(bad) && lane == 0) atomicOr(status, 2u);
}

// Per expert, the exclusive prefix of its chunk counts over the chunks (its
// pairs in the chunks before each one) and its total: one wave an expert,
// lane l taking chunks l cpl .. l cpl + cpl - 1 (cpl <= 4).
__global__ __launch_bounds__(256) void k_perm_scan(const int32_t* __restrict__ chunk_hist,
                                                    int nchunks, int E,
                                                    int32_t* __restrict__ chunk_base,
                                                    int32_t* __restrict__ etotal) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;  // wave-uniform; no barrier in this kernel
  const int cpl = (nchunks + 63) / 64;
  int32_t v[4], part = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane * cpl + i;
    v[i] = (i < cpl && c < nchunks) ? chunk_hist[(size_t)c * E + e] : 0;
    part += v[i];
  }
  int32_t incl = part;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  int32_t run = incl - part;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane * cpl + i;
    if (i < cpl && c < nchunks) chunk_base[(size_t)c * E + e] = run;
    run += v[i];
  }
  if (lane == 63) etotal[e] = incl;
}

// Every block scans the expert totals for the expert offsets (block 0 also
// writes counts, offsets, tracking and the tile list), then places its
// 1024 ppt pairs (ppt <= kScatterPPT a thread, so that the scan is paid by
// few blocks): offset of the expert + pairs of the expert in earlier chunks
// + rank inside the chunk.
constexpr int kScatterPPT = 4;
__global__ __launch_bounds__(1024) void k_perm_scatter(const int32_t* __restrict__ idx, int64_t P,
                                                        int ppt, int E, int T, int Is, int tile_rows,
                                                        int ch,
                                                        const int32_t* __restrict__ prank,
                                                        const int32_t* __restrict__ chunk_base,
                                                        const int32_t* __restrict__ etotal,
                                                        int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets,
                                                        int64_t* __restrict__ tracking,
                                                        int32_t* __restrict__ tile_off,
                                                        int32_t* __restrict__ tile_tab,
                                                        int32_t* __restrict__ sorted_pair,
                                                        int32_t* __restrict__ pair_slot) {
  __shared__ FinishLds fl;
  __shared__ int32_t offs[kPermMaxE];
  const int64_t p0 = (int64_t)blockIdx.x * 1024 * ppt + threadIdx.x;
  // the pairs' indices, ranks and chunk bases are loaded before the scan's
  // waits (a pair past the end is not loaded)
  int32_t e[kScatterPPT], base[kScatterPPT], rk[kScatterPPT];
#pragma unroll
  for (int k = 0; k < kScatterPPT; ++k) {
    const int64_t p = p0 + (int64_t)k * 1024;
    e[k] = (k < ppt && p < P) ? idx[p] : -1;
  }
#pragma unroll
  for (int k = 0; k < kScatterPPT; ++k) {
    const int64_t p = p0 + (int64_t)k * 1024;
    const bool v = (uint32_t)e[k] < (uint32_t)E;
    base[k] = v ? chunk_base[(size_t)(p / ch) * E + e[k]] : 0;
    rk[k] = v ? prank[p] : 0;
  }
  const int32_t total = (int)threadIdx.x < E ? etotal[threadIdx.x] : 0;
  finish_counts(total, E, T, Is, tile_rows, fl, counts, offsets, offs, tracking, tile_off,
                tile_tab, blockIdx.x == 0);
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kScatterPPT; ++k) {
    const int64_t p = p0 + (int64_t)k * 1024;
    if (k >= ppt || p >= P) break;
    int32_t pos = -1;
    if ((uint32_t)e[k] < (uint32_t)E) {
      pos = offs[e[k]] + base[k] + rk[k];
      sorted_pair[pos] = (int32_t)p;
    }
    pair_slot[p] = pos;
  }
}

size_t permute_scratch_ints(int64_t P, int E) {
  if (P <= kSmallMaxP) return 0;
  const int64_t nch = (P + permute_chunk(P) - 1) / permute_chunk(P);
  return (size_t)P + 2 * (size_t)nch * E + E;  // prank, chunk_hist, chunk_base, etotal
}

hipError_t launch_permute(const int32_t* idx, int64_t P, int E, int T, int Is, int tile_rows,
                          int32_t* scratch, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_slot, int64_t* tracking,
                          int32_t* tile_off, int32_t* tile_tab, uint32_t* status,
                          hipStream_t s, const StageTimer* tm) {
  if (P <= kSmallMaxP) {
    stage_begin(tm, kHist, s);
    hipLaunchKernelGGL(k_permute_small, dim3(1), dim3(1024), 0, s, idx, (int)P, E, T, Is,
                       tile_rows, counts, offsets, sorted_pair, pair_slot, tracking, tile_off,
                       tile_tab, status);
    stage_end(tm, kHist, s);
    return hipGetLastError();
  }
  const int ch = permute_chunk(P);
  const int nch = (int)((P + ch - 1) / ch);
  int32_t* prank = scratch;
  int32_t* chunk_hist = scratch + P;
  int32_t* chunk_base = chunk_hist + (size_t)nch * E;
  int32_t* etotal = chunk_base + (size_t)nch * E;
  stage_begin(tm, kHist, s);
  hipLaunchKernelGGL(k_perm_rank, dim3((unsigned)nch), dim3(256), 0, s, idx, P, E, ch, prank,
                     chunk_hist, status);
  stage_end(tm, kHist, s);
  stage_begin(tm, kScan, s);
  hipLaunchKernelGGL(k_perm_scan, dim3((unsigned)((E + 3) / 4)), dim3(256), 0, s, chunk_hist, nch,
                     E, chunk_base, etotal);
  stage_end(tm, kScan, s);
  stage_begin(tm, kScatter, s);
  // about 128 blocks once there are enough pairs
  const int ppt = (int)std::min<int64_t>(kScatterPPT, std::max<int64_t>(1, P / (1024 * 128)));
  const int64_t per_block = 1024 * (int64_t)ppt;
  hipLaunchKernelGGL(k_perm_scatter, dim3((unsigned)((P + per_block - 1) / per_block)), dim3(1024),
                     0, s, idx, P, ppt, E, T, Is, tile_rows, ch, prank, chunk_base, etotal, counts,
                     offsets, tracking, tile_off, tile_tab, sorted_pair, pair_slot);
  stage_end(tm, kScatter, s);
  return hipGetLastError();
}

}  // namespace moe
