// kernels.h -- host-side launchers of the libmoe kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Optional event pair around one kernel stage (see moe_layer_forward_timed).
struct StageTimer {
  int stage = -1;
  hipEvent_t start = nullptr, stop = nullptr;
};
inline void stage_begin(const StageTimer* t, int stage, hipStream_t s) {
  if (t && t->stage == stage) (void)hipEventRecord(t->start, s);
}
inline void stage_end(const StageTimer* t, int stage, hipStream_t s) {
  if (t && t->stage == stage) (void)hipEventRecord(t->stop, s);
}
enum Stage { kSplit = 0, kLogits, kSelect, kHist, kScan, kScatter, kTiles, kGateUp, kDown, kCombine };

// Router ----------------------------------------------------------------------
hipError_t launch_split_router(const float* w, uint16_t* split, int E, int H, hipStream_t s,
                               const StageTimer* tm = nullptr);
hipError_t launch_logits_bf16(const uint16_t* x, const uint16_t* split, float* logits, int T, int H,
                              int E, hipStream_t s, const StageTimer* tm = nullptr);
hipError_t launch_logits_f32(const float* x, const float* w, float* logits, int T, int H, int E,
                             hipStream_t s, const StageTimer* tm = nullptr);
hipError_t launch_select(const float* logits, const float* bias, int32_t* idx, float* w,
                         uint32_t* status, int T, int E, int n_group, int topk_group, int K,
                         float scale, bool record_nonfinite, hipStream_t s,
                         const StageTimer* tm = nullptr);
hipError_t launch_sigmoid32(const float* z, float* out, int64_t n, hipStream_t s);

// Permute ---------------------------------------------------------------------
constexpr int kPermuteChunk = 1024;  // pairs per histogram / scatter block
hipError_t launch_permute(const int32_t* idx, int64_t P, int E, int32_t* chunk_hist,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                          int32_t* pair_slot, int64_t* tracking, uint32_t* status,
                          hipStream_t s, const StageTimer* tm = nullptr);

// Experts ---------------------------------------------------------------------
constexpr int kTileRows = 32;  // token rows per expert tile

struct ExpertArgs {
  int T, H, E, K, I, Is;
  const void* x;
  const float* topk_w;
  const int32_t* offsets;      // [E+1]
  const int32_t* sorted_pair;  // [P]
  const int32_t* pair_slot;    // [P]
  const void *w_gate, *w_up, *w_down;
  const void *ws_gate, *ws_up, *ws_down;
  void* y;
  // workspace
  int32_t* tile_off;  // [E+2]
  void* h_routed;     // [P][I]
  void* h_shared;     // [T][Is]
  void* o_routed;     // [P][H]
  void* o_shared;     // [T][H]
};
int64_t max_expert_tiles(int64_t T, int64_t K, int E, int Is);
hipError_t launch_experts_bf16(const ExpertArgs& a, hipStream_t s, const StageTimer* tm = nullptr);
hipError_t launch_experts_f32(const ExpertArgs& a, hipStream_t s, const StageTimer* tm = nullptr);

// Residual + RMSNorm ----------------------------------------------------------
hipError_t launch_residual_rmsnorm(bool bf16, const void* x_in, const void* y, void* x_out,
                                   void* r_out, int T, int H, float eps, hipStream_t s);

}  // namespace moe
