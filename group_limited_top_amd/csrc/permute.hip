// permute.hip -- per-expert counts and a stable bucket order of the pairs.
//
// [Routing §六]: per-expert hit counts are a bincount of the chosen indices;
// [Routing §四]: the eager inference path sorts tokens into one bucket per
// expert before running each bucket.  Here the T*K (token, slot) pairs,
// p = t*K + j, are counting-sorted by expert, keeping ascending p inside each
// bucket, in three deterministic kernels (integer LDS atomics only):
//   1. per-chunk histograms (chunks of kPermuteChunk consecutive pairs);
//   2. one block: per-expert scan over chunks, counts, exclusive offsets,
//      tracking += counts;
//   3. per chunk, one wave walks its pairs in order and scatters them, ranking
//      equal experts inside each 64-pair step with ballots.
// An index outside [0, E) is skipped (not counted, pair_slot = -1) and raises
// status bit 2 in the workspace status word.
#include "device.h"
#include "kernels.h"

namespace moe {

constexpr int kPermMaxE = 512;

__global__ __launch_bounds__(256) void k_chunk_hist(const int32_t* __restrict__ idx, int64_t P,
                                                     int E, int32_t* __restrict__ chunk_hist) {
  __shared__ int32_t hist[kPermMaxE];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * kPermuteChunk;
  const int64_t p1 = min(P, p0 + kPermuteChunk);
  for (int64_t p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    const int32_t e = idx[p];
    if ((uint32_t)e < (uint32_t)E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    chunk_hist[(size_t)blockIdx.x * E + e] = hist[e];
}

// One block of kPermMaxE threads (thread e owns expert e).
__global__ __launch_bounds__(kPermMaxE) void k_count_scan(int32_t* __restrict__ chunk_hist,
                                                          int nchunks, int E, int64_t P,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int64_t* __restrict__ tracking) {
  __shared__ int32_t scan[kPermMaxE];
  const int e = threadIdx.x;
  int32_t total = 0;
  if (e < E) {
    for (int c = 0; c < nchunks; ++c) {
      const int32_t v = chunk_hist[(size_t)c * E + e];
      chunk_hist[(size_t)c * E + e] = total;  // exclusive prefix over chunks
      total += v;
    }
  }
  scan[e] = total;
  __syncthreads();
  // inclusive Hillis-Steele scan over experts
  for (int d = 1; d < kPermMaxE; d <<= 1) {
    const int32_t add = (e >= d) ? scan[e - d] : 0;
    __syncthreads();
    scan[e] += add;
    __syncthreads();
  }
  const int32_t excl = scan[e] - total;
  if (e < E) {
    counts[e] = total;
    offsets[e] = excl;
    if (tracking) tracking[e] += (int64_t)total;
    for (int c = 0; c < nchunks; ++c) chunk_hist[(size_t)c * E + e] += excl;
  }
  if (e == E - 1) offsets[E] = excl + total;
}

__global__ __launch_bounds__(64) void k_scatter(const int32_t* __restrict__ idx, int64_t P, int E,
                                                const int32_t* __restrict__ chunk_base,
                                                int32_t* __restrict__ sorted_pair,
                                                int32_t* __restrict__ pair_slot,
                                                uint32_t* __restrict__ status) {
  __shared__ int32_t cursor[kPermMaxE];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) cursor[e] = chunk_base[(size_t)blockIdx.x * E + e];
  __syncthreads();
  const int nbits = 32 - __clz(E - 1);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t p0 = (int64_t)blockIdx.x * kPermuteChunk;
  const int64_t p1 = min(P, p0 + kPermuteChunk);
  int bad = 0;
  for (int64_t base = p0; base < p1; base += 64) {
    const int64_t p = base + lane;
    const bool active = p < p1;
    const int32_t e = active ? idx[p] : 0;
    const bool valid = active && (uint32_t)e < (uint32_t)E;
    bad |= active && !valid;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t ones = __ballot(valid && ((e >> b) & 1));
      same &= ((e >> b) & 1) ? ones : ~ones;
    }
    int32_t pos = -1;
    if (valid) pos = cursor[e] + __popcll(same & below);
    __syncthreads();  // every lane has read its cursor before any update
    if (valid && (same >> lane) == 1ull) cursor[e] += __popcll(same);  // last lane of its group
    if (valid) sorted_pair[pos] = (int32_t)p;
    if (active) pair_slot[p] = pos;
    __syncthreads();
  }
  if (__any(bad) && lane == 0) atomicOr(status, 2u);
}

hipError_t launch_permute(const int32_t* idx, int64_t P, int E, int32_t* chunk_hist,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                          int32_t* pair_slot, int64_t* tracking, uint32_t* status,
                          hipStream_t s, const StageTimer* tm) {
  const int nchunks = (int)((P + kPermuteChunk - 1) / kPermuteChunk);
  if (nchunks > 0) {
    stage_begin(tm, kHist, s);
    hipLaunchKernelGGL(k_chunk_hist, dim3((unsigned)nchunks), dim3(256), 0, s, idx, P, E,
                       chunk_hist);
    stage_end(tm, kHist, s);
  }
  stage_begin(tm, kScan, s);
  hipLaunchKernelGGL(k_count_scan, dim3(1), dim3(kPermMaxE), 0, s, chunk_hist, nchunks, E, P,
                     counts, offsets, tracking);
  stage_end(tm, kScan, s);
  if (nchunks > 0) {
    stage_begin(tm, kScatter, s);
    hipLaunchKernelGGL(k_scatter, dim3((unsigned)nchunks), dim3(64), 0, s, idx, P, E, chunk_hist,
                       sorted_pair, pair_slot, status);
    stage_end(tm, kScatter, s);
  }
  return hipGetLastError();
}

}  // namespace moe
