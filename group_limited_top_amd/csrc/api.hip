// api.hip -- the C ABI of libmoe (include/moe.h): validation, workspace
// layout and launch sequencing.  Everything here runs on the host; nothing
// touches device memory before validation has passed.
#include "moe.h"

#include <math.h>
#include <string.h>

#include "backward.h"
#include "kernels.h"
#include "layer_check.h"

namespace {

constexpr size_t kAlign = 256;
// Token counts stay below 2^30 so that every token index and launch-size
// expression (token + block size, token + loop stride) fits an int.
constexpr int32_t kMaxTokens = 1 << 30;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace regions (byte offsets from ws).  One layout serves every entry
// point; regions an entry point does not use are simply left alone.
struct Layout {
  size_t status;       // uint32 status word (first 256 bytes)
  size_t split;        // bf16 [3][E][H] router weight parts (bf16 path, large T)
  size_t logits;       // fp32 [ks][T][E] logits (K-split partials when ks > 1)
  size_t idx;          // int32 [T][K]
  size_t w;            // fp32 [T][K]
  size_t counts;       // int32 [E]
  size_t offsets;      // int32 [E+1]
  size_t sorted_pair;  // int32 [P]
  size_t pair_slot;    // int32 [P]
  size_t perm;         // int32 permute scratch (large P only)
  size_t tile_off;     // int32 [E+2]
  size_t tile_tab;     // int32 [max tiles][2]
  size_t h_routed;     // dtype [P][I]
  size_t h_shared;     // dtype [T][Is]
  size_t o_routed;     // dtype [P][H]
  size_t o_shared;     // dtype [T][H]
  size_t total;
};

Layout make_layout(const moe_desc_t& d) {
  const size_t T = (size_t)d.T, H = (size_t)d.H, E = (size_t)d.E, K = (size_t)d.top_k;
  const size_t P = T * K;
  const size_t elt = d.dtype == MOE_BF16 ? 2 : 4;
  const bool bf16 = d.dtype == MOE_BF16;
  const size_t ks = bf16 ? (size_t)moe::logits_ksplit(d.T, d.H, d.E) : 1;
  const size_t Is = (size_t)d.I_shared;
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.status = take(kAlign);
  L.split = take(bf16 && !moe::logits_split_in_kernel(d.T) ? 3 * E * H * 2 : 0);
  L.logits = take(ks * T * E * 4);
  L.idx = take(P * 4);
  L.w = take(P * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.sorted_pair = take(P * 4);
  L.pair_slot = take(P * 4);
  L.perm = take(moe::permute_scratch_ints((int64_t)P, d.E) * 4);
  L.tile_off = take((E + 2) * 4);
  L.tile_tab = take((size_t)moe::max_expert_tiles(d.T, d.top_k, d.E, d.I_shared,
                                                  moe::expert_tile_rows(d.T, d.top_k, d.E, d.I,
                                                                        d.I_shared, d.H, bf16)) *
                    8);
  // h rows are padded by one GEMM row tile (its loads may run past the last row)
  L.h_routed = take((P + moe::kGRows) * (size_t)d.I * elt);
  L.h_shared = take((T + moe::kGRows) * Is * elt);
  L.o_routed = take(P * H * elt);
  L.o_shared = take(Is > 0 ? T * H * elt : 0);
  L.total = o;
  return L;
}

int validate(const moe_desc_t* d) {
  if (!d) return MOE_ERR_INVALID;
  if (d->T < 0 || d->H <= 0 || d->E <= 0 || d->n_group <= 0 || d->topk_group <= 0 ||
      d->top_k <= 0 || d->I <= 0 || d->I_shared < 0)
    return MOE_ERR_INVALID;
  if (d->E % d->n_group != 0) return MOE_ERR_INVALID;
  const int gsize = d->E / d->n_group;
  if (gsize < 2) return MOE_ERR_INVALID;
  if (d->topk_group > d->n_group) return MOE_ERR_INVALID;
  if ((int64_t)d->top_k > (int64_t)d->topk_group * gsize) return MOE_ERR_INVALID;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (!isfinite(d->routed_scaling_factor)) return MOE_ERR_INVALID;
  if (d->flags & ~(MOE_F_WRITE_LOGITS | MOE_F_CHECK_FINITE)) return MOE_ERR_INVALID;
  // kernel envelope
  if (d->E > 512 || d->n_group > 64 || d->top_k > 16) return MOE_ERR_UNSUPPORTED;
  {  // the selection kernel maps a group onto a power-of-two run of lanes
    const int epl = moe::select_epl(d->E);
    const int lpg = gsize / epl;
    if (gsize % epl != 0 || (lpg & (lpg - 1)) != 0) return MOE_ERR_UNSUPPORTED;
  }
  if (d->dtype == MOE_BF16 && d->H % 256 != 0) return MOE_ERR_UNSUPPORTED;
  if (d->dtype == MOE_F32 && (d->H % 64 != 0 || d->H > 16384)) return MOE_ERR_UNSUPPORTED;
  if (d->I % 64 != 0 || d->I > 1024) return MOE_ERR_UNSUPPORTED;
  if (d->I_shared % 64 != 0 || d->I_shared > 1024) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)d->T * d->top_k >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if (d->T >= kMaxTokens) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

bool misaligned(const void* p) { return p && ((uintptr_t)p & 15u) != 0; }

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}

int check_ws(const moe_desc_t& d, void* ws, size_t ws_bytes) {
  if (!ws || ws_bytes < make_layout(d).total) return MOE_ERR_WORKSPACE;
  if (misaligned(ws)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

int tile_rows(const moe_desc_t& d) {
  return moe::expert_tile_rows(d.T, d.top_k, d.E, d.I, d.I_shared, d.H, d.dtype == MOE_BF16);
}

// route into (idx, w); logits_user (nullable) receives the fp32 logits
int run_route(const moe_desc_t& d, const void* x, const float* w_router, const float* bias,
              float* logits_user, int32_t* idx, float* w, void* ws, hipStream_t s,
              const moe::StageTimer* tm = nullptr) {
  const Layout L = make_layout(d);
  float* part = at<float>(ws, L.logits);
  int ks = 1;
  hipError_t e;
  if (d.dtype == MOE_BF16) {
    ks = moe::logits_ksplit(d.T, d.H, d.E);
    uint16_t* split = nullptr;
    if (!moe::logits_split_in_kernel(d.T)) {
      split = at<uint16_t>(ws, L.split);
      e = moe::launch_split_router(w_router, split, d.E, d.H, s, tm);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    if (ks == 1 && logits_user) part = logits_user;
    e = moe::launch_logits_bf16(reinterpret_cast<const uint16_t*>(x), w_router, split, part, d.T,
                                d.H, d.E, ks, s, tm);
  } else {
    if (logits_user) part = logits_user;
    e = moe::launch_logits_f32(reinterpret_cast<const float*>(x), w_router, part, d.T, d.H, d.E, s,
                               tm);
  }
  if (e != hipSuccess) return MOE_ERR_HIP;
  float* copy_out = (logits_user && part != logits_user) ? logits_user : nullptr;
  e = moe::launch_select(part, ks, copy_out, bias, idx, w, at<uint32_t>(ws, L.status), d.T, d.E,
                         d.n_group, d.topk_group, d.top_k, d.routed_scaling_factor,
                         (d.flags & MOE_F_CHECK_FINITE) != 0, s, tm);
  return hip_rc(e);
}

int run_permute(const moe_desc_t& d, const int32_t* idx, int32_t* counts, int32_t* offsets,
                int32_t* sorted_pair, int32_t* pair_slot, int64_t* tracking, void* ws,
                hipStream_t s, const moe::StageTimer* tm = nullptr) {
  const Layout L = make_layout(d);
  return hip_rc(moe::launch_permute(idx, (int64_t)d.T * d.top_k, d.E, d.T, d.I_shared,
                                    tile_rows(d), at<int32_t>(ws, L.perm), counts, offsets, sorted_pair,
                                    pair_slot, tracking, at<int32_t>(ws, L.tile_off),
                                    at<int32_t>(ws, L.tile_tab), at<uint32_t>(ws, L.status), s, tm));
}

int run_experts(const moe_desc_t& d, const void* x, const float* topk_w, const int32_t* offsets,
                const int32_t* sorted_pair, const int32_t* pair_slot, const moe_weights_t& W,
                void* y, void* ws, hipStream_t s, bool tiles_ready,
                const moe::StageTimer* tm = nullptr) {
  const Layout L = make_layout(d);
  moe::ExpertArgs a;
  a.T = d.T;
  a.H = d.H;
  a.E = d.E;
  a.K = d.top_k;
  a.I = d.I;
  a.Is = d.I_shared;
  a.x = x;
  a.topk_w = topk_w;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.pair_slot = pair_slot;
  a.w_gate = W.w_gate;
  a.w_up = W.w_up;
  a.w_down = W.w_down;
  a.ws_gate = W.ws_gate;
  a.ws_up = W.ws_up;
  a.ws_down = W.ws_down;
  a.y = y;
  a.tile_off = at<int32_t>(ws, L.tile_off);
  a.tile_tab = at<int32_t>(ws, L.tile_tab);
  a.tiles_ready = tiles_ready;
  a.tile_rows = tile_rows(d);
  a.h_routed = at<void>(ws, L.h_routed);
  a.h_shared = at<void>(ws, L.h_shared);
  a.o_routed = at<void>(ws, L.o_routed);
  a.o_shared = at<void>(ws, L.o_shared);
  return hip_rc(d.dtype == MOE_BF16 ? moe::launch_experts_bf16(a, s, tm)
                                    : moe::launch_experts_f32(a, s, tm));
}

int check_weights(const moe_desc_t& d, const moe_weights_t* W, bool need_router) {
  if (!W) return MOE_ERR_INVALID;
  if (need_router && !W->w_router) return MOE_ERR_INVALID;
  if (!W->w_gate || !W->w_up || !W->w_down) return MOE_ERR_INVALID;
  const bool has_shared = W->ws_gate || W->ws_up || W->ws_down;
  if (d.I_shared > 0 && (!W->ws_gate || !W->ws_up || !W->ws_down)) return MOE_ERR_INVALID;
  if (d.I_shared == 0 && has_shared) return MOE_ERR_INVALID;
  const void* ps[] = {W->w_router, W->expert_bias, W->w_gate, W->w_up,
                      W->w_down,   W->ws_gate,     W->ws_up,  W->ws_down};
  for (const void* p : ps)
    if (misaligned(p)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

// Backward workspace regions.
struct BwdLayout {
  size_t status, counts, offsets, sorted_pair, pair_slot, perm, tile_off, tile_tab, inter, total;
};

BwdLayout make_bwd_layout(const moe_desc_t& d) {
  const size_t T = (size_t)d.T, E = (size_t)d.E, P = T * (size_t)d.top_k;
  BwdLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.status = take(kAlign);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.sorted_pair = take(P * 4);
  L.pair_slot = take(P * 4);
  L.perm = take(moe::permute_scratch_ints((int64_t)P, d.E) * 4);
  L.tile_off = take((E + 2) * 4);
  L.tile_tab = take((size_t)moe::max_expert_tiles(d.T, d.top_k, d.E, d.I_shared,
                                                  moe::kBwdTileRows) * 8);
  L.inter = take(moe::bwd_intermediate_bytes(d.T, d.top_k, d.E, d.I, d.H, d.I_shared > 0));
  L.total = o;
  return L;
}

// The backward's envelope on top of the forward's: bf16, the shared expert
// (if any) as wide as the routed ones.
int validate_bwd(const moe_desc_t* d) {
  const int rc = validate(d);
  if (rc) return rc;
  if (d->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d->I_shared != 0 && d->I_shared != d->I) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)(d->T * (int64_t)d->top_k + d->T) * d->H >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_backward_workspace_size(const moe_desc_t* desc) {
  if (validate_bwd(desc) != MOE_OK) return 0;
  return make_bwd_layout(*desc).total;
}

int moe_layer_backward(const moe_desc_t* desc, const void* x, const moe_weights_t* weights,
                       const int32_t* topk_idx, const float* logits, const void* dy, void* dx,
                       float* dw_router, float* dw_gate, float* dw_up, float* dw_down,
                       float* dws_gate, float* dws_up, float* dws_down, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  int rc = validate_bwd(desc);
  if (rc) return rc;
  const moe_desc_t& d = *desc;
  if (d.T == 0) return MOE_OK;
  rc = check_weights(d, weights, true);
  if (rc) return rc;
  if (!x || !topk_idx || !logits || !dy || !dx || !dw_router || !dw_gate || !dw_up || !dw_down)
    return MOE_ERR_INVALID;
  const bool sh = d.I_shared > 0;
  if (sh != (dws_gate != nullptr) || sh != (dws_up != nullptr) || sh != (dws_down != nullptr))
    return MOE_ERR_INVALID;
  if (dx == x || dx == dy) return MOE_ERR_INVALID;
  const void* ps[] = {x, topk_idx, logits, dy, dx, dw_router, dw_gate, dw_up, dw_down,
                      dws_gate, dws_up, dws_down};
  for (const void* p : ps)
    if (misaligned(p)) return MOE_ERR_ALIGN;
  const BwdLayout L = make_bwd_layout(d);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (misaligned(ws)) return MOE_ERR_ALIGN;
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* sorted_pair = at<int32_t>(ws, L.sorted_pair);
  int32_t* pair_slot = at<int32_t>(ws, L.pair_slot);
  int32_t* tile_off = at<int32_t>(ws, L.tile_off);
  int32_t* tile_tab = at<int32_t>(ws, L.tile_tab);
  const int tile_rows = moe::bwd_tile_rows(d.T, d.top_k, d.E, d.I, d.I_shared, d.H);
  rc = hip_rc(moe::launch_permute(topk_idx, (int64_t)d.T * d.top_k, d.E, d.T, d.I_shared,
                                  tile_rows, at<int32_t>(ws, L.perm),
                                  at<int32_t>(ws, L.counts), offsets, sorted_pair, pair_slot,
                                  nullptr, tile_off, tile_tab, at<uint32_t>(ws, L.status),
                                  stream));
  if (rc) return rc;
  moe::BwdInputs in;
  in.T = d.T;
  in.H = d.H;
  in.E = d.E;
  in.K = d.top_k;
  in.I = d.I;
  in.scale = d.routed_scaling_factor;
  in.x = static_cast<const uint16_t*>(x);
  in.dy = static_cast<const uint16_t*>(dy);
  in.logits = logits;
  in.idx = topk_idx;
  in.w_router = weights->w_router;
  in.wg = static_cast<const uint16_t*>(weights->w_gate);
  in.wu = static_cast<const uint16_t*>(weights->w_up);
  in.wd = static_cast<const uint16_t*>(weights->w_down);
  in.swg = static_cast<const uint16_t*>(weights->ws_gate);
  in.swu = static_cast<const uint16_t*>(weights->ws_up);
  in.swd = static_cast<const uint16_t*>(weights->ws_down);
  in.offsets = offsets;
  in.sorted_pair = sorted_pair;
  in.pair_slot = pair_slot;
  in.tile_off = tile_off;
  in.tile_tab = tile_tab;
  in.tile_rows = tile_rows;
  in.scratch = at<void>(ws, L.inter);
  in.dx = static_cast<uint16_t*>(dx);
  in.dw_router = dw_router;
  in.dwg = dw_gate;
  in.dwu = dw_up;
  in.dwd = dw_down;
  in.dswg = dws_gate;
  in.dswu = dws_up;
  in.dswd = dws_down;
  return hip_rc(moe::launch_backward(in, stream));
}


size_t moe_workspace_size(const moe_desc_t* desc) {
  if (validate(desc) != MOE_OK) return 0;
  return make_layout(*desc).total;
}

int moe_route(const moe_desc_t* desc, const void* x, const float* w_router,
              const float* expert_bias, float* logits, int32_t* topk_idx, float* topk_w, void* ws,
              size_t ws_bytes, hipStream_t stream) {
  int rc = validate(desc);
  if (rc) return rc;
  if (desc->T == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_w) return MOE_ERR_INVALID;
  if ((rc = check_ws(*desc, ws, ws_bytes))) return rc;
  const void* ps[] = {x, w_router, expert_bias, logits, topk_idx, topk_w};
  for (const void* p : ps)
    if (misaligned(p)) return MOE_ERR_ALIGN;
  return run_route(*desc, x, w_router, expert_bias, logits, topk_idx, topk_w, ws, stream);
}

int moe_permute(const moe_desc_t* desc, const int32_t* topk_idx, int32_t* counts,
                int32_t* offsets, int32_t* sorted_pair, int32_t* pair_slot, int64_t* tracking,
                void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = validate(desc);
  if (rc) return rc;
  if (desc->T == 0) return MOE_OK;
  if (!topk_idx || !counts || !offsets || !sorted_pair || !pair_slot) return MOE_ERR_INVALID;
  if ((rc = check_ws(*desc, ws, ws_bytes))) return rc;
  const void* ps[] = {topk_idx, counts, offsets, sorted_pair, pair_slot, tracking};
  for (const void* p : ps)
    if (misaligned(p)) return MOE_ERR_ALIGN;
  return run_permute(*desc, topk_idx, counts, offsets, sorted_pair, pair_slot, tracking, ws,
                     stream);
}

int moe_experts(const moe_desc_t* desc, const void* x, const float* topk_w,
                const int32_t* offsets, const int32_t* sorted_pair, const int32_t* pair_slot,
                const moe_weights_t* weights, void* y, void* ws, size_t ws_bytes,
                hipStream_t stream) {
  int rc = validate(desc);
  if (rc) return rc;
  if (desc->T == 0) return MOE_OK;
  if (!x || !topk_w || !offsets || !sorted_pair || !pair_slot || !y) return MOE_ERR_INVALID;
  if (x == y) return MOE_ERR_INVALID;
  if ((rc = check_weights(*desc, weights, false))) return rc;
  if ((rc = check_ws(*desc, ws, ws_bytes))) return rc;
  const void* ps[] = {x, topk_w, offsets, sorted_pair, pair_slot, y};
  for (const void* p : ps)
    if (misaligned(p)) return MOE_ERR_ALIGN;
  return run_experts(*desc, x, topk_w, offsets, sorted_pair, pair_slot, *weights, y, ws, stream,
                     false);
}

}  // extern "C"

namespace moe {

int validate_desc(const moe_desc_t* desc) { return validate(desc); }

int layer_forward_check(const moe_desc_t* desc, const void* x, const moe_weights_t* weights,
                        void* y, int32_t* topk_idx_out, float* topk_w_out, float* logits_out,
                        int32_t* counts_out, int64_t* tracking, void* ws, size_t ws_bytes) {
  int rc = validate(desc);
  if (rc) return rc;
  if (desc->T == 0) return MOE_OK;
  if (!x || !y || x == y) return MOE_ERR_INVALID;
  if ((rc = check_weights(*desc, weights, true))) return rc;
  if ((rc = check_ws(*desc, ws, ws_bytes))) return rc;
  const void* ps[] = {x, y, topk_idx_out, topk_w_out, logits_out, counts_out, tracking};
  for (const void* p : ps)
    if (misaligned(p)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

}  // namespace moe

static int layer_forward(const moe_desc_t* desc, const void* x, const moe_weights_t* weights,
                         void* y, int32_t* topk_idx_out, float* topk_w_out, float* logits_out,
                         int32_t* counts_out, int64_t* tracking, void* ws, size_t ws_bytes,
                         hipStream_t stream, const moe::StageTimer* tm) {
  int rc = moe::layer_forward_check(desc, x, weights, y, topk_idx_out, topk_w_out, logits_out,
                                    counts_out, tracking, ws, ws_bytes);
  if (rc || desc->T == 0) return rc;
  const moe_desc_t& d = *desc;
  const Layout L = make_layout(d);
  float* lg = (d.flags & MOE_F_WRITE_LOGITS) ? logits_out : nullptr;
  int32_t* idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, L.idx);
  float* w = topk_w_out ? topk_w_out : at<float>(ws, L.w);
  int32_t* counts = counts_out ? counts_out : at<int32_t>(ws, L.counts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* sp = at<int32_t>(ws, L.sorted_pair);
  int32_t* ps_ = at<int32_t>(ws, L.pair_slot);
  if ((rc = run_route(d, x, weights->w_router, weights->expert_bias, lg, idx, w, ws, stream, tm)))
    return rc;
  if ((rc = run_permute(d, idx, counts, offsets, sp, ps_, tracking, ws, stream, tm))) return rc;
  return run_experts(d, x, w, offsets, sp, ps_, *weights, y, ws, stream, true, tm);
}

extern "C" {

int moe_layer_forward(const moe_desc_t* desc, const void* x, const moe_weights_t* weights,
                      void* y, int32_t* topk_idx_out, float* topk_w_out, float* logits_out,
                      int32_t* counts_out, int64_t* tracking, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  return layer_forward(desc, x, weights, y, topk_idx_out, topk_w_out, logits_out, counts_out,
                       tracking, ws, ws_bytes, stream, nullptr);
}

int moe_layer_forward_timed(const moe_desc_t* desc, const void* x, const moe_weights_t* weights,
                            void* y, int32_t* topk_idx_out, float* topk_w_out, float* logits_out,
                            int32_t* counts_out, int64_t* tracking, void* ws, size_t ws_bytes,
                            hipStream_t stream, int stage, hipEvent_t start, hipEvent_t stop) {
  if (stage < 0 || stage >= MOE_NUM_STAGES || !start || !stop) return MOE_ERR_INVALID;
  moe::StageTimer tm;
  tm.stage = stage;
  tm.start = start;
  tm.stop = stop;
  return layer_forward(desc, x, weights, y, topk_idx_out, topk_w_out, logits_out, counts_out,
                       tracking, ws, ws_bytes, stream, &tm);
}

const char* moe_stage_kernel(const moe_desc_t* desc, int stage) {
  if (validate(desc) != MOE_OK || desc->T == 0) return nullptr;
  const moe_desc_t& d = *desc;
  return moe::expert_stage_kernel(stage, d.T, d.top_k, d.E, d.I, d.I_shared, d.H,
                                  d.dtype == MOE_BF16);
}

int moe_residual_rmsnorm(const moe_desc_t* desc, const void* x_in, const void* y, void* x_out,
                         void* r_out, float eps, hipStream_t stream) {
  int rc = validate(desc);
  if (rc) return rc;
  if (desc->T == 0) return MOE_OK;
  if (!x_in || !x_out || !r_out || !(eps >= 0.0f)) return MOE_ERR_INVALID;
  const void* ps[] = {x_in, y, x_out, r_out};
  for (const void* p : ps)
    if (misaligned(p)) return MOE_ERR_ALIGN;
  return hip_rc(moe::launch_residual_rmsnorm(desc->dtype == MOE_BF16, x_in, y, x_out, r_out, desc->T,
                                             desc->H, eps, stream));
}

int moe_status(void* ws, size_t ws_bytes, hipStream_t stream, uint32_t* status) {
  if (!ws || !status || ws_bytes < kAlign) return MOE_ERR_INVALID;
  if (hipStreamSynchronize(stream) != hipSuccess) return MOE_ERR_HIP;
  uint32_t v = 0;
  if (hipMemcpy(&v, ws, sizeof v, hipMemcpyDeviceToHost) != hipSuccess) return MOE_ERR_HIP;
  const uint32_t zero = 0;
  if (hipMemcpy(ws, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess) return MOE_ERR_HIP;
  *status = v;
  return MOE_OK;
}

int moe_sigmoid32(const float* z, float* s, int64_t n, hipStream_t stream) {
  if (n < 0) return MOE_ERR_INVALID;
  if (n == 0) return MOE_OK;
  if (!z || !s) return MOE_ERR_INVALID;
  if (misaligned(z) || misaligned(s)) return MOE_ERR_ALIGN;
  return hip_rc(moe::launch_sigmoid32(z, s, n, stream));
}

size_t moe_aux_loss_workspace_size(int32_t T, int32_t E) {
  if (T < 1 || T >= kMaxTokens || E < 2 || E > 1024) return 0;
  return align_up(moe::aux_workspace_bytes(T, E));
}

int moe_expert_stats(int32_t L, int32_t E, int32_t n_group, const int64_t* tracking, float* load,
                     double* summary, hipStream_t stream) {
  if (L < 0 || E < 1 || n_group < 1 || E % n_group != 0) return MOE_ERR_INVALID;
  if (E > 1024 || n_group > 64) return MOE_ERR_UNSUPPORTED;
  if (L == 0) return MOE_OK;
  if (!tracking || !load || !summary) return MOE_ERR_INVALID;
  if (misaligned(tracking) || misaligned(load) || misaligned(summary)) return MOE_ERR_ALIGN;
  return hip_rc(moe::launch_expert_stats(tracking, load, summary, L, E, n_group, stream));
}

int moe_bias_update(int32_t E, const int32_t* counts, const float* bias_in, float* bias_out,
                    double rate, hipStream_t stream) {
  if (E < 1 || !counts || !bias_out || !isfinite(rate)) return MOE_ERR_INVALID;
  if (E > 1024) return MOE_ERR_UNSUPPORTED;
  if (misaligned(counts) || misaligned(bias_in) || misaligned(bias_out)) return MOE_ERR_ALIGN;
  return hip_rc(moe::launch_bias_update(counts, bias_in, bias_out, E, rate, stream));
}

int moe_aux_loss(int32_t T, int32_t E, const float* logits, const int32_t* counts, double* f,
                 double* P, double* loss, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (T < 1 || E < 2 || !logits || !counts || !f || !P || !loss) return MOE_ERR_INVALID;
  if (E > 1024 || T >= kMaxTokens) return MOE_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < moe_aux_loss_workspace_size(T, E)) return MOE_ERR_WORKSPACE;
  const void* ps[] = {logits, counts, f, P, loss, ws};
  for (const void* p : ps)
    if (misaligned(p)) return MOE_ERR_ALIGN;
  return hip_rc(moe::launch_aux_loss(logits, counts, f, P, loss, static_cast<double*>(ws), T, E,
                                     stream));
}

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "success";
    case MOE_ERR_INVALID: return "invalid argument (null pointer, negative size or inconsistent shape)";
    case MOE_ERR_UNSUPPORTED: return "shape outside the kernels' supported envelope";
    case MOE_ERR_WORKSPACE: return "workspace missing or smaller than moe_workspace_size()";
    case MOE_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case MOE_ERR_HIP: return "a HIP launch or runtime call failed";
    case MOE_ERR_SCRATCH:
      return "the layer needs more scratch than the no-allocation entry point's static buffer "
             "holds (MOE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error code";
  }
}

}  // extern "C"
