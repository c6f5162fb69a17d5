// Host sanitizer driver for libmoe's C ABI (built by tests/test_sanitizers.py
// from the library's sources with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code, no device code).  It drives the
// argument validation, workspace sizing and error paths of every entry point
// with valid, boundary and invalid descriptions and pointers; every call here
// fails validation or is host-only, so no kernel is launched and no device is
// needed.  Exits 0 when every call returned the expected code.
#include <limits.h>
#include <stdint.h>
#include <stdio.h>

#include "moe.h"

static int failures = 0;
static void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    fprintf(stderr, "line %d: %s returned %d, expected %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

static moe_desc_t desc(int T, int H, int E = 256, int G = 8, int KG = 4, int K = 8, int I = 512,
                       int Is = 512, int dt = MOE_BF16) {
  moe_desc_t d;
  d.T = T;
  d.H = H;
  d.E = E;
  d.n_group = G;
  d.topk_group = KG;
  d.top_k = K;
  d.I = I;
  d.I_shared = Is;
  d.routed_scaling_factor = 2.5f;
  d.dtype = dt;
  d.flags = 0;
  return d;
}

int main() {
  // sizes: valid descs over the envelope's corners, and invalid ones
  const int Ts[] = {0, 1, 7, 512, 4096, 16384, 65536, (1 << 30) - 1, 1 << 30, INT_MAX};
  const int Hs[] = {256, 2048, 16384, 64, 0, -256, INT_MAX};
  const int Es[] = {2, 8, 256, 512, 1024, 0, -8};
  for (int T : Ts)
    for (int H : Hs)
      for (int E : Es)
        for (int dt : {(int)MOE_BF16, (int)MOE_F32, 7}) {
          moe_desc_t d = desc(T, H, E, E >= 8 ? 8 : 1, E >= 8 ? 4 : 1, E >= 8 ? 8 : 1, 512,
                              512, dt);
          const size_t n = moe_workspace_size(&d);
          const size_t nb = moe_backward_workspace_size(&d);
          for (int s = 0; s < MOE_NUM_STAGES; ++s) (void)moe_stage_kernel(&d, s);
          if (n == 0 && nb != 0) {
            fprintf(stderr, "backward workspace for a desc the forward rejects\n");
            ++failures;
          }
          if (n > MOE_NOALLOC_SCRATCH_BYTES)
            EXPECT(moe_layer_forward_noalloc(&d, nullptr, nullptr, nullptr, nullptr, nullptr,
                                             nullptr, nullptr, nullptr, nullptr),
                   MOE_ERR_SCRATCH);
        }
  EXPECT((int)moe_workspace_size(nullptr), 0);
  moe_desc_t big = desc(INT_MAX, 2048);
  EXPECT((int)(moe_workspace_size(&big) == 0), 1);  // T * top_k >= 2^31
  moe_desc_t many = desc(1 << 30, 256, 2, 1, 1, 1, 64, 0);
  EXPECT((int)(moe_workspace_size(&many) == 0), 1);  // T >= 2^30
  many.T = (1 << 30) - 1;
  EXPECT((int)(moe_workspace_size(&many) > 0), 1);

  moe_desc_t d = desc(512, 2048);
  void* fake = reinterpret_cast<void*>(0x100000);
  void* odd = reinterpret_cast<void*>(0x100004);
  const size_t ws_big = (size_t)1 << 40;
  const float* ff = static_cast<const float*>(fake);
  float* fo = static_cast<float*>(fake);
  int32_t* io = static_cast<int32_t*>(fake);
  moe_weights_t W = {ff, nullptr, fake, fake, fake, fake, fake, fake};
  // moe_route
  EXPECT(moe_route(nullptr, fake, ff, nullptr, nullptr, io, fo, fake, ws_big, nullptr),
         MOE_ERR_INVALID);
  EXPECT(moe_route(&d, nullptr, ff, nullptr, nullptr, io, fo, fake, ws_big, nullptr),
         MOE_ERR_INVALID);
  EXPECT(moe_route(&d, fake, ff, nullptr, nullptr, io, fo, fake, 16, nullptr), MOE_ERR_WORKSPACE);
  EXPECT(moe_route(&d, odd, ff, nullptr, nullptr, io, fo, fake, ws_big, nullptr), MOE_ERR_ALIGN);
  // moe_permute
  EXPECT(moe_permute(&d, nullptr, io, io, io, io, nullptr, fake, ws_big, nullptr),
         MOE_ERR_INVALID);
  EXPECT(moe_permute(&d, io, io, io, io, io, nullptr, nullptr, ws_big, nullptr),
         MOE_ERR_WORKSPACE);
  EXPECT(moe_permute(&d, io, io, io, io, static_cast<int32_t*>(odd), nullptr, fake, ws_big,
                     nullptr),
         MOE_ERR_ALIGN);
  // moe_experts
  EXPECT(moe_experts(&d, fake, ff, io, io, io, &W, fake, fake, ws_big, nullptr),
         MOE_ERR_INVALID);  // y aliases x
  EXPECT(moe_experts(&d, fake, ff, io, io, io, nullptr, odd, fake, ws_big, nullptr),
         MOE_ERR_INVALID);
  // moe_layer_forward and its variants
  EXPECT(moe_layer_forward(&d, fake, &W, fake, nullptr, nullptr, nullptr, nullptr, nullptr, fake,
                           ws_big, nullptr),
         MOE_ERR_INVALID);
  moe_weights_t W2 = {ff, nullptr, fake, fake, fake, nullptr, nullptr, nullptr};
  EXPECT(moe_layer_forward(&d, fake, &W2, reinterpret_cast<void*>(0x200000), nullptr, nullptr,
                           nullptr, nullptr, nullptr, fake, ws_big, nullptr),
         MOE_ERR_INVALID);
  moe_weights_t W3 = {ff, static_cast<const float*>(odd), fake, fake, fake, fake, fake, fake};
  EXPECT(moe_layer_forward(&d, fake, &W3, reinterpret_cast<void*>(0x200000), nullptr, nullptr,
                           nullptr, nullptr, nullptr, fake, ws_big, nullptr),
         MOE_ERR_ALIGN);
  EXPECT(moe_layer_forward_timed(&d, fake, &W, fake, nullptr, nullptr, nullptr, nullptr, nullptr,
                                 fake, ws_big, nullptr, MOE_NUM_STAGES, nullptr, nullptr),
         MOE_ERR_INVALID);
  moe_desc_t chk = desc(512, 2048);
  chk.flags = MOE_F_CHECK_FINITE;
  EXPECT(moe_layer_forward_noalloc(&chk, fake, &W, reinterpret_cast<void*>(0x200000), nullptr,
                                   nullptr, nullptr, nullptr, nullptr, nullptr),
         MOE_ERR_UNSUPPORTED);
  moe_desc_t zero = desc(0, 2048);
  EXPECT(moe_layer_forward_noalloc(&zero, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, nullptr),
         MOE_OK);
  EXPECT(moe_layer_forward(&zero, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, nullptr, 0, nullptr),
         MOE_OK);
  // residual + RMSNorm, status, sigmoid
  EXPECT(moe_residual_rmsnorm(&d, nullptr, nullptr, fake, fake, 1e-6f, nullptr), MOE_ERR_INVALID);
  EXPECT(moe_residual_rmsnorm(&d, fake, nullptr, fake, fake, -1.0f, nullptr), MOE_ERR_INVALID);
  EXPECT(moe_status(nullptr, 0, nullptr, nullptr), MOE_ERR_INVALID);
  EXPECT(moe_sigmoid32(ff, fo, -1, nullptr), MOE_ERR_INVALID);
  EXPECT(moe_sigmoid32(ff, fo, 0, nullptr), MOE_OK);
  EXPECT(moe_sigmoid32(static_cast<const float*>(odd), fo, 5, nullptr), MOE_ERR_ALIGN);
  // load balancing
  EXPECT(moe_expert_stats(-1, 256, 8, nullptr, nullptr, nullptr, nullptr), MOE_ERR_INVALID);
  EXPECT(moe_expert_stats(1, 255, 8, nullptr, nullptr, nullptr, nullptr), MOE_ERR_INVALID);
  EXPECT(moe_expert_stats(1, 2048, 8, nullptr, nullptr, nullptr, nullptr), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_expert_stats(0, 256, 8, nullptr, nullptr, nullptr, nullptr), MOE_OK);
  EXPECT(moe_bias_update(0, io, nullptr, fo, 0.1, nullptr), MOE_ERR_INVALID);
  EXPECT(moe_bias_update(256, io, nullptr, fo, 1.0 / 0.0, nullptr), MOE_ERR_INVALID);
  EXPECT(moe_bias_update(4096, io, nullptr, fo, 0.1, nullptr), MOE_ERR_UNSUPPORTED);
  EXPECT((int)moe_aux_loss_workspace_size(0, 256), 0);
  EXPECT((int)(moe_aux_loss_workspace_size((1 << 30) - 1, 1024) > 0), 1);
  EXPECT((int)moe_aux_loss_workspace_size(1 << 30, 2), 0);
  EXPECT(moe_aux_loss(1 << 30, 256, ff, io, static_cast<double*>(fake),
                      static_cast<double*>(fake), static_cast<double*>(fake), fake, ws_big,
                      nullptr),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_aux_loss(16, 256, ff, io, nullptr, nullptr, nullptr, fake, ws_big, nullptr),
         MOE_ERR_INVALID);
  EXPECT(moe_aux_loss(16, 256, ff, io, static_cast<double*>(fake), static_cast<double*>(fake),
                      static_cast<double*>(fake), fake, 8, nullptr),
         MOE_ERR_WORKSPACE);
  // backward
  moe_desc_t f32 = desc(512, 2048, 256, 8, 4, 8, 512, 512, MOE_F32);
  EXPECT((int)moe_backward_workspace_size(&f32), 0);
  EXPECT(moe_layer_backward(&f32, fake, &W, io, ff, fake, fake, fo, fo, fo, fo, fo, fo, fo, fake,
                            ws_big, nullptr),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_layer_backward(&d, fake, &W, io, ff, fake, fake, fo, fo, fo, fo, fo, fo, fo, fake,
                            ws_big, nullptr),
         MOE_ERR_INVALID);  // dx aliases x
  EXPECT(moe_layer_backward(&d, fake, &W, io, ff, fake, reinterpret_cast<void*>(0x200000), fo, fo,
                            fo, fo, nullptr, fo, fo, fake, ws_big, nullptr),
         MOE_ERR_INVALID);  // shared-expert gradients must match I_shared
  for (int c = -7; c <= 1; ++c) (void)moe_strerror(c);
  if (failures) return 1;
  printf("abi sanitizer driver ok\n");
  return 0;
}
