// backward.h -- launch interface of the layer backward (internal).
#pragma once

#include "kernels.h"

namespace moe {

// Backward --------------------------------------------------------------------
constexpr int kBwdTileRows = 64;  // row tiles of the backward's own grouped GEMMs
// Rows per tile the backward's permute builds: kGRows when the row products
// run on the forward's expert GEMM (many rows per expert, bwd_gemm_ok),
// kBwdTileRows for the backward's own row GEMMs otherwise.
int bwd_tile_rows(int64_t T, int K, int E, int I, int Is, int H);
struct BwdInputs {
  int T, H, E, K, I;  // I: routed = shared intermediate size (or no shared expert)
  float scale;
  const uint16_t *x, *dy;       // [T][H] bf16
  const float* logits;          // [T][E]
  const int32_t* idx;           // [T][K]
  const float* w_router;        // [E][H]
  const uint16_t *wg, *wu, *wd;    // [E][I][H]
  const uint16_t *swg, *swu, *swd; // [I][H] or null
  const int32_t *offsets, *sorted_pair, *pair_slot, *tile_off, *tile_tab;  // permute output
  int tile_rows;                // the tiles' rows (bwd_tile_rows)
  void* scratch;                // bwd_intermediate_bytes
  uint16_t* dx;                 // [T][H]
  float* dw_router;             // [E][H]
  float *dwg, *dwu, *dwd;       // [E][I][H]
  float *dswg, *dswu, *dswd;    // [I][H] or null
};
size_t bwd_intermediate_bytes(int64_t T, int K, int E, int I, int H, bool shared);
hipError_t launch_backward(const BwdInputs& in, hipStream_t s);

}  // namespace moe
