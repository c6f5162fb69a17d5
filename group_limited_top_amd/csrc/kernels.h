// kernels.h -- host-side launchers of the libmoe kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kTileRows = 32;    // token rows per tile of the weight-streaming kernels
constexpr int kGRows = 256;      // token rows per tile of the LDS-pipelined GEMMs
// Rows per expert tile for a layer: many rows per expert -> LDS-pipelined GEMMs.
int expert_tile_rows(int64_t T, int K, int E, int I, int Is, int H, bool bf16);

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
// K-split factor of the bf16 logits kernel (partials [ks][T][E] are summed by
// the selection kernel) and whether it splits the router weight itself.
int logits_ksplit(int T, int H, int E);
bool logits_split_in_kernel(int T);
hipError_t launch_logits_bf16(const uint16_t* x, const float* w32, const uint16_t* wsplit,
                              float* out, int T, int H, int E, int ks, hipStream_t s,
                              const StageTimer* tm = nullptr);
hipError_t launch_logits_f32(const float* x, const float* w, float* logits, int T, int H, int E,
                             hipStream_t s, const StageTimer* tm = nullptr);
int select_epl(int E);  // experts per lane of the selection kernel (power of two)
hipError_t launch_select(const float* part, int ks, float* logits_out, const float* bias,
                         int32_t* idx, float* w, uint32_t* status, int T, int E, int n_group,
                         int topk_group, int K, float scale, bool record_nonfinite, hipStream_t s,
                         const StageTimer* tm = nullptr);
hipError_t launch_sigmoid32(const float* z, float* out, int64_t n, hipStream_t s);

// Permute ---------------------------------------------------------------------
size_t permute_scratch_ints(int64_t P, int E);
hipError_t launch_permute(const int32_t* idx, int64_t P, int E, int T, int Is, int tile_rows,
                          int32_t* scratch, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_slot, int64_t* tracking,
                          int32_t* tile_off, int32_t* tile_tab, uint32_t* status,
                          hipStream_t s, const StageTimer* tm = nullptr);

// Experts ---------------------------------------------------------------------

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
  int32_t* tile_tab;  // [max_expert_tiles][2] (see write_tile_entry)
  int tile_rows;      // token rows per tile (kTileRows or kGRows)
  bool tiles_ready;   // tile_off already built (by the permute kernels)
  void* h_routed;     // [P][I]
  void* h_shared;     // [T][Is]
  void* o_routed;     // [P][H]
  void* o_shared;     // [T][H]
  // the backward's row products (k_expert_gemm modes 2-4); their rows are
  // the sorted pairs, then the T shared rows
  const void* dy;          // [T][H] upstream gradient (mode 3's token rows)
  float *bwd_g, *bwd_u;    // [P + T][I] fp32 (mode 2)
  float* bwd_r;            // [P + T][I] fp32 (mode 3)
  const void *bwd_dg, *bwd_du;  // [P + T + kGRows][I] bf16 (mode 4's rows)
  void* bwd_dx;            // [P + T][H] bf16 (mode 4)
  void* trash;             // >= 64 KiB: modes 2-4 send stores of rows past a tile's end here
};
int64_t max_expert_tiles(int64_t T, int64_t K, int E, int Is, int tile_rows);
// LDS-pipelined MFMA GEMMs (tile_rows == kGRows); shapes with gemm_shape_ok.
bool gemm_shape_ok(int64_t T, int K, int I, int Is, int H);
hipError_t launch_experts_gemm_bf16(const ExpertArgs& a, hipStream_t s, const StageTimer* tm);
// The backward's row products on the same GEMM (256-row tiles already built):
// g, u = x W_g^T, x W_u^T and r = dy W_d^T (fp32), then dx per row =
// d_g W_g + d_u W_u (bf16).  Usable when bwd_gemm_ok.
bool bwd_gemm_ok(int64_t T, int K, int I, int Is, int H);
hipError_t launch_bwd_gur_gemm(const ExpertArgs& a, hipStream_t s);
hipError_t launch_bwd_dx_gemm(const ExpertArgs& a, hipStream_t s);
// gate/up weight streaming through the LDS ring (32-row tiles); usable when
// stream_ring_ok.
bool stream_ring_ok(const ExpertArgs& a);
hipError_t launch_gateup_stream_bf16(const ExpertArgs& a, int64_t tiles, hipStream_t s,
                                     const StageTimer* tm);
// down weight streaming through the same ring; usable when down_stream_ok.
bool down_stream_ok(const ExpertArgs& a);
// fp32 gate/up and down weight streaming through the same ring; usable when
// stream_f32_ok.
bool stream_f32_ok(const ExpertArgs& a);
hipError_t launch_stream_f32(const ExpertArgs& a, int64_t tiles, hipStream_t s,
                             const StageTimer* tm);
hipError_t launch_down_stream_bf16(const ExpertArgs& a, int64_t tiles, hipStream_t s,
                                   const StageTimer* tm);
hipError_t launch_combine_bf16(const ExpertArgs& a, hipStream_t s, const StageTimer* tm);
hipError_t launch_experts_bf16(const ExpertArgs& a, hipStream_t s, const StageTimer* tm = nullptr);
hipError_t launch_experts_f32(const ExpertArgs& a, hipStream_t s, const StageTimer* tm = nullptr);
// Name of the kernel an expert stage (kGateUp, kDown, kCombine) launches for
// this shape; nullptr for other stages.
const char* expert_stage_kernel(int stage, int64_t T, int K, int E, int I, int Is, int H, bool bf16);

// Load balancing --------------------------------------------------------------
constexpr int kNStat = 8;  // summary values per layer (moe_expert_stats)
hipError_t launch_expert_stats(const int64_t* tracking, float* load, double* summary, int L, int E,
                               int n_group, hipStream_t s);
hipError_t launch_bias_update(const int32_t* counts, const float* bias_in, float* bias_out, int E,
                              double rate, hipStream_t s);
size_t aux_workspace_bytes(int T, int E);
hipError_t launch_aux_loss(const float* logits, const int32_t* counts, double* f, double* P,
                           double* loss, double* part, int T, int E, hipStream_t s);

// Residual + RMSNorm ----------------------------------------------------------
hipError_t launch_residual_rmsnorm(bool bf16, const void* x_in, const void* y, void* x_out,
                                   void* r_out, int T, int H, float eps, hipStream_t s);

}  // namespace moe
