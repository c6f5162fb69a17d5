// router.hip -- router logits, sigma32 and group-limited top-k selection.
//
// Method: page "InternLumina-U2中256个专家的路由秘密：分组受限Top-K、Expert Bias与
// Fused MoE详解" ([Routing §n] below), §二 steps 1-3 and §三.
#include "device.h"
#include "kernels.h"

#include <math.h>

namespace moe {

// ----------------------------------------------------------------------------
// sigma32: the router sigmoid, specified in include/moe.h.  All operations are
// IEEE fp64 (v_fma_f64, v_rndne_f64, v_div_* correctly rounded division) and
// the final conversion rounds to nearest even, so the value is reproducible
// bit for bit by any IEEE implementation of the same steps.
// ----------------------------------------------------------------------------
// The Taylor coefficients RN(1/i!), i = 13 .. 2, of exp on the reduced
// argument.  They are read from memory (scalar loads into SGPRs) rather than
// written as literals: each Horner step is then one fma with an SGPR-pair
// operand, where a literal would first be moved into VGPRs for every
// evaluation.  Nothing writes this table.
__device__ double kExpTaylor[12] = {
    0x1.6124613a86d09p-33,  // 1/13!
    0x1.1eed8eff8d898p-29,  // 1/12!
    0x1.ae64567f544e4p-26,  // 1/11!
    0x1.27e4fb7789f5cp-22,  // 1/10!
    0x1.71de3a556c734p-19,  // 1/9!
    0x1.a01a01a01a01ap-16,  // 1/8!
    0x1.a01a01a01a01ap-13,  // 1/7!
    0x1.6c16c16c16c17p-10,  // 1/6!
    0x1.1111111111111p-7,   // 1/5!
    0x1.5555555555555p-5,   // 1/4!
    0x1.5555555555555p-3,   // 1/3!
    0x1.0p-1,               // 1/2!
};

__device__ __forceinline__ float sigmoid32(float z) {
  if (!(z == z)) return z;
  const double t = -(double)z;
  if (t > 104.0) return 0.0f;  // below 2^-150: rounds to +0
  if (t < -40.0) return 1.0f;  // exp(t) < 2^-54: 1 + exp(t) rounds to 1
  // Cody-Waite reduction t = n ln2 + r with ln2 = L1 + L2
  const double n = __builtin_rint(t * 0x1.71547652b82fep+0);
  double r = __builtin_fma(-n, 0x1.62e42fefa39efp-1, t);
  r = __builtin_fma(-n, 0x1.abc9e3b39803fp-56, r);
  // exp(r) by the degree-13 Taylor polynomial, coefficients RN(1/i!), Horner
  double p = kExpTaylor[0];
#pragma unroll
  for (int i = 1; i < 12; ++i) p = __builtin_fma(p, r, kExpTaylor[i]);
  p = __builtin_fma(p, r, 1.0);                    // 1/1!
  p = __builtin_fma(p, r, 1.0);                    // 1/0!
  // 2^n is exact: -58 <= n <= 151 here
  const double two_n = __longlong_as_double((long long)((int)n + 1023) << 52);
  const double e = p * two_n;
  const double den = 1.0 + e;
  return (float)(1.0 / den);
}

__global__ void k_sigmoid32(const float* __restrict__ z, float* __restrict__ out, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) out[i] = sigmoid32(z[i]);
}

hipError_t launch_sigmoid32(const float* z, float* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_sigmoid32, dim3((unsigned)blocks), dim3(256), 0, s, z, out, n);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Router weight split: w = hi + mid + lo exactly, each part bf16.
// Each step subtracts the nearest bf16 of what is left; the remainder of an
// fp32 after removing its top 8 significant bits, twice, has at most 8
// significant bits, so the three parts represent w exactly.  With bf16 x every
// product x*part is then exact in fp32 and only the accumulation rounds.
// Layout: split[p][e][h], p = 0 (hi), 1 (mid), 2 (lo).
// ----------------------------------------------------------------------------
__global__ void k_split_router(const float* __restrict__ w, uint16_t* __restrict__ split,
                               int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) {
    const float v = w[i];
    const uint32_t hi = f32_to_bf16_bits(v);
    const float r1 = v - bf16_to_f32((uint16_t)hi);
    const uint32_t mid = f32_to_bf16_bits(r1);
    const float r2 = r1 - bf16_to_f32((uint16_t)mid);
    const uint32_t lo = f32_to_bf16_bits(r2);
    split[i] = (uint16_t)hi;
    split[n + i] = (uint16_t)mid;
    split[2 * n + i] = (uint16_t)lo;
  }
}

hipError_t launch_split_router(const float* w, uint16_t* split, int E, int H, hipStream_t s,
                               const StageTimer* tm) {
  const int64_t n = (int64_t)E * H;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  stage_begin(tm, kSplit, s);
  hipLaunchKernelGGL(k_split_router, dim3((unsigned)blocks), dim3(256), 0, s, w, split, n);
  stage_end(tm, kSplit, s);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Logits, bf16 activations: logits[t][e] = sum_h x[t][h] * w[e][h] on MFMA with
// w = hi + mid + lo (three bf16 parts), fp32 accumulation.  [Routing §二 step
// 1]: a linear layer in fp32 with no bias term.
//
// Block: 4 waves, tile 64 MT tokens (16 MT per wave, MT MFMA M-tiles) x 64
// experts (4 MFMA N-tiles), K range [z*KR, (z+1)*KR) with z = blockIdx.z (a K
// split; the partial sums are added in fixed order by the selection kernel).
// The weight tile of each 64-deep K chunk is staged in LDS as three bf16
// planes, split from fp32 inside the kernel (SPLIT, small T: each element is
// split by at most a few blocks) or copied from the pre-split planes (large
// T).  x rows go straight from global memory into the A operands.  Each
// staged weight operand feeds MT x 3 MFMAs, so large T uses MT = 4 (the LDS
// reads per MFMA are a quarter of MT = 1's).
// ----------------------------------------------------------------------------
constexpr int kLgBN = 64, kLgKC = 64, kLgRow = kLgKC;
constexpr int kLgMTSmall = 1, kLgMTLarge = 4;  // SPLIT (small T) / pre-split (large T)

// LDS element offset of 16-byte chunk c (8 bf16) of staged weight row r: the
// chunk index is XORed with bits 1..3 of the row, so that 16 consecutive rows
// at one chunk (or two chunks) land on disjoint banks with 64 or 128 banks.
__device__ __forceinline__ int lg_swz(int r, int c) { return r * kLgRow + ((c ^ ((r >> 1) & 7)) << 3); }
constexpr int kMaxKSplit = 16;

__device__ __forceinline__ void split3(float v, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f32_to_bf16_bits(v);
  const float r1 = v - bf16_to_f32((uint16_t)hi);
  mid = f32_to_bf16_bits(r1);
  const float r2 = r1 - bf16_to_f32((uint16_t)mid);
  lo = f32_to_bf16_bits(r2);
}

template <bool SPLIT, int MT>
__global__ __launch_bounds__(256) void k_logits_bf16(const uint16_t* __restrict__ x,
                                                      const float* __restrict__ w32,
                                                      const uint16_t* __restrict__ wsplit,
                                                      float* __restrict__ out, int T, int H,
                                                      int E, int KR) {
  __shared__ uint16_t wl[2][3][kLgBN][kLgRow];  // 48 KiB
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * (64 * MT) + wave * (16 * MT), e0 = blockIdx.y * kLgBN;
  const int kbeg = blockIdx.z * KR;
  // staging role: expert row er, 16 consecutive k at ks16
  const int er = threadIdx.x >> 2, ks16 = (threadIdx.x & 3) * 16;
  const int erc = min(e0 + er, E - 1);
  const float* wsrc32 = SPLIT ? w32 + (size_t)erc * H + kbeg + ks16 : nullptr;
  const uint16_t* wsrc16 = SPLIT ? nullptr : wsplit + (size_t)erc * H + kbeg + ks16;
  const size_t plane = (size_t)E * H;
  const uint16_t* xa[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
    xa[m] = x + (size_t)min(t0 + 16 * m + r, T - 1) * H + kbeg + q * 8;

  u32x4 st[6];  // staged global data: 16 fp32 (SPLIT) or 3 x 16 bf16
  auto load_w = [&](int c) {
    if (SPLIT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) st[i] = ld16(wsrc32 + c * kLgKC + 4 * i);
    } else {
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        st[2 * p] = ld16(wsrc16 + p * plane + c * kLgKC);
        st[2 * p + 1] = ld16(wsrc16 + p * plane + c * kLgKC + 8);
      }
    }
  };
  auto store_w = [&](int buf) {
    u32x4 o[6];
    if (SPLIT) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {  // 8 pairs of fp32 -> 3 packed bf16 pairs
        const float a = __uint_as_float(st[i >> 1][(i & 1) * 2]);
        const float b = __uint_as_float(st[i >> 1][(i & 1) * 2 + 1]);
        uint32_t ah, am, al, bh, bm, bl;
        split3(a, ah, am, al);
        split3(b, bh, bm, bl);
        o[0 + (i >> 2)][i & 3] = ah | (bh << 16);
        o[2 + (i >> 2)][i & 3] = am | (bm << 16);
        o[4 + (i >> 2)][i & 3] = al | (bl << 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 6; ++i) o[i] = st[i];
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      st16(&wl[buf][p][0][0] + lg_swz(er, ks16 / 8), o[2 * p]);
      st16(&wl[buf][p][0][0] + lg_swz(er, ks16 / 8 + 1), o[2 * p + 1]);
    }
  };

  f32x4 acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nchunks = KR / kLgKC;
  u32x4 a_cur[MT][2], a_nxt[MT][2];
  load_w(0);
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int s = 0; s < 2; ++s) a_cur[m][s] = ld16(xa[m] + s * 32);
  store_w(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nchunks;
    if (more) {
      load_w(c + 1);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int s = 0; s < 2; ++s) a_nxt[m][s] = ld16(xa[m] + (c + 1) * kLgKC + s * 32);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          const u32x4 b =
              *reinterpret_cast<const u32x4*>(&wl[buf][p][0][0] + lg_swz(n * 16 + r, s * 4 + q));
#pragma unroll
          for (int m = 0; m < MT; ++m) acc[m][n] = mfma16x16x32(a_cur[m][s], b, acc[m][n]);
        }
      }
    }
    if (more) {
      store_w(buf ^ 1);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        a_cur[m][0] = a_nxt[m][0];
        a_cur[m][1] = a_nxt[m][1];
      }
    }
    __syncthreads();
  }
  // lane holds C[token 4q + i][expert r] of M-tile m, N-tile n
  float* o = out + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int e = e0 + n * 16 + r;
    if (e < E) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 16 * m + 4 * q + i;
          if (t < T) o[(size_t)t * E + e] = acc[m][n][i];
        }
    }
  }
}

bool logits_split_in_kernel(int T) { return T <= 1024; }

static int logits_bm(int T) { return 64 * (logits_split_in_kernel(T) ? kLgMTSmall : kLgMTLarge); }

int logits_ksplit(int T, int H, int E) {
  const int64_t bm = logits_bm(T);
  const int64_t tiles = ((T + bm - 1) / bm) * ((E + kLgBN - 1) / kLgBN);
  int ks = 1;
  while (ks < kMaxKSplit && tiles * ks * 2 <= 512 && (H / kLgKC) % (ks * 2) == 0) ks *= 2;
  return ks;
}

hipError_t launch_logits_bf16(const uint16_t* x, const float* w32, const uint16_t* wsplit,
                              float* out, int T, int H, int E, int ks, hipStream_t s,
                              const StageTimer* tm) {
  const int64_t bm = logits_bm(T);
  dim3 grid((unsigned)((T + bm - 1) / bm), (unsigned)((E + kLgBN - 1) / kLgBN), (unsigned)ks);
  const int KR = H / ks;
  stage_begin(tm, kLogits, s);
  if (logits_split_in_kernel(T))
    hipLaunchKernelGGL((k_logits_bf16<true, kLgMTSmall>), grid, dim3(256), 0, s, x, w32, wsplit,
                       out, T, H, E, KR);
  else
    hipLaunchKernelGGL((k_logits_bf16<false, kLgMTLarge>), grid, dim3(256), 0, s, x, w32, wsplit,
                       out, T, H, E, KR);
  stage_end(tm, kLogits, s);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Logits, fp32 activations (small fp32 layers).  [Routing §二 step 1]:
// logit = x . W_r row, fp32.  Block: 4 waves x 8 experts (32 experts), 8
// tokens.  Lane l of wave v takes expert e0 + 8 v + l / 8 and, of each
// 512-float chunk of the row, the 16-byte pieces 32 j + 4 (l mod 8) (j < 16):
// one wave load instruction reads 8 whole 128-byte lines.  The chunk of W
// sits in registers, the tokens' chunk of x in LDS; each lane sums its
// products per token (fp32 fma), then the expert's 8 lanes add their sums by
// an xor butterfly (IEEE addition commutes, so every lane holds the same
// bits) and lane l stores token l mod 8.
// ----------------------------------------------------------------------------
constexpr int kLfTok = 8;      // tokens per block
constexpr int kLfChunk = 512;  // floats of a row per chunk

__global__ __launch_bounds__(256) void k_logits_f32(const float* __restrict__ x,
                                                     const float* __restrict__ w,
                                                     float* __restrict__ logits, int T, int H, int E) {
  __shared__ __attribute__((aligned(16))) float xs[kLfTok][kLfChunk];  // 16 KiB
  const int tid = threadIdx.x, lane = tid & 63;
  const int t0 = blockIdx.y * kLfTok;
  const int e = blockIdx.x * 32 + (tid >> 3);  // 8 lanes an expert
  const int part = lane & 7;
  const float* wr = w + (size_t)min(e, E - 1) * H + 4 * part;
  float acc[kLfTok];
#pragma unroll
  for (int t = 0; t < kLfTok; ++t) acc[t] = 0.0f;
  for (int k0 = 0; k0 < H; k0 += kLfChunk) {
    const int np = min(kLfChunk, H - k0) / 32;  // pieces in this chunk (H % 64 == 0: >= 2)
    // the chunk of W (pieces past the chunk's end re-read its last piece)
    f32x4 wv[kLfChunk / 32];
#pragma unroll
    for (int j = 0; j < kLfChunk / 32; ++j)
      wv[j] = *reinterpret_cast<const f32x4*>(wr + k0 + 32 * min(j, np - 1));
    // the tokens' chunk of x (tokens past T re-read the last token)
    __syncthreads();  // the previous chunk's readers are done
#pragma unroll
    for (int u = 0; u < kLfTok * kLfChunk / 4 / 256; ++u) {
      const int v = tid + 256 * u;
      const int t = v / (kLfChunk / 4), c = v % (kLfChunk / 4);
      if (4 * c < 32 * np)
        *reinterpret_cast<f32x4*>(&xs[t][4 * c]) =
            *reinterpret_cast<const f32x4*>(x + (size_t)min(t0 + t, T - 1) * H + k0 + 4 * c);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kLfChunk / 32; ++j) {
      if (j >= np) continue;  // uniform
      f32x4 xv[kLfTok];
#pragma unroll
      for (int t = 0; t < kLfTok; ++t) xv[t] = *reinterpret_cast<const f32x4*>(&xs[t][32 * j + 4 * part]);
      // consecutive FMAs on different tokens: independent chains
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int t = 0; t < kLfTok; ++t) acc[t] = __builtin_fmaf(wv[j][c], xv[t][c], acc[t]);
    }
  }
  float mine = 0.0f;
#pragma unroll
  for (int t = 0; t < kLfTok; ++t) {
    float v = acc[t];
    v = v + __shfl_xor(v, 1, 8);
    v = v + __shfl_xor(v, 2, 8);
    v = v + __shfl_xor(v, 4, 8);
    mine = part == t ? v : mine;
  }
  if (e < E && t0 + part < T) logits[(size_t)(t0 + part) * E + e] = mine;
}

hipError_t launch_logits_f32(const float* x, const float* w, float* logits, int T, int H, int E,
                             hipStream_t s, const StageTimer* tm) {
  stage_begin(tm, kLogits, s);
  const dim3 grid((unsigned)((E + 31) / 32), (unsigned)((T + kLfTok - 1) / kLfTok));
  hipLaunchKernelGGL(k_logits_f32, grid, dim3(256), 0, s, x, w, logits, T, H, E);
  stage_end(tm, kLogits, s);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Selection.  One wave per token (4 tokens per block); lane l holds the EPL
// consecutive experts l*EPL .. l*EPL+EPL-1, so a group of E/n_group experts is
// LPG = E/(n_group*EPL) consecutive lanes.
//   [Routing §二 step 1]  s = sigma32(logit) (logit = the K-split partials added
//                         in split order)
//   [Routing §三]         sb = s + bias, used for selection only
//   [Routing §二 step 2]  group score = sum of the group's two largest sb
//                         (xor butterfly over the group's lanes); a group is
//                         kept when fewer than topk_group groups rank before
//                         it (higher score, or equal score and lower index);
//                         the others are masked to -inf; then top_k rounds of
//                         a wave-wide maximum of 64-bit keys (orderable sb,
//                         then the complement of the expert index, so that
//                         ties go to the lower index): each lane's best key,
//                         the 32-bit maximum of their score halves (DPP
//                         within 16-lane rows, readlane across rows), and the
//                         lowest lane holding it
//   [Routing §二 step 3]  S = fp32 sum of the chosen unbiased scores in choice
//                         order, w_j = RN(RN(s_j / RN(S + 1e-20)) * scale)
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint32_t orderable(float v) {
  const uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide maximum of a 32-bit unsigned value (DPP within 16-lane rows,
// readlane across rows), returned to every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, true));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xf, 0xf, true));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, true));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, true));  // row_mirror
  const uint32_t m01 = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t m23 = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return max(m01, m23);
}

__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

template <int EPL, int KSM>
__global__ __launch_bounds__(256) void k_select(const float* __restrict__ part, int KS,
                                                 float* __restrict__ logits_out,
                                                 const float* __restrict__ bias,
                                                 int32_t* __restrict__ idx, float* __restrict__ wout,
                                                 uint32_t* __restrict__ status, int T, int E,
                                                 int n_group, int topk_group, int K, float scale,
                                                 int record) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform; no barrier in this kernel
  float z[EPL], s[EPL], sb[EPL];
  bool valid[EPL];
  int bad = 0;
  // issue every partial-sum load first (straight-line over KSM >= KS splits,
  // KSM fixed at compile time: a split past KS re-reads split 0, an element
  // past E re-reads element E - 1; both are masked below), then add them in
  // split order.  When every lane's EPL elements exist (E a multiple of
  // 64 EPL: a wave-uniform test) they are read as 16-byte pieces.
  float pv[KSM][EPL];
  if (EPL % 4 == 0 && E % (64 * EPL) == 0) {
#pragma unroll
    for (int k = 0; k < KSM; ++k) {
      const float* row = part + ((size_t)(k < KS ? k : 0) * T + t) * E + lane * EPL;
#pragma unroll
      for (int i = 0; i < EPL; i += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(row + i);
        pv[k][i] = v[0];
        pv[k][i + 1] = v[1];
        pv[k][i + 2] = v[2];
        pv[k][i + 3] = v[3];
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < KSM; ++k) {
      const float* row = part + ((size_t)(k < KS ? k : 0) * T + t) * E;
#pragma unroll
      for (int i = 0; i < EPL; ++i) pv[k][i] = row[min(lane * EPL + i, E - 1)];
    }
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    valid[i] = lane * EPL + i < E;
    float acc = pv[0][i];
#pragma unroll
    for (int k = 1; k < KSM; ++k)
      if (k < KS) acc = acc + pv[k][i];
    z[i] = valid[i] ? acc : 0.0f;
  }
  if (logits_out) {
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (valid[i]) logits_out[(size_t)t * E + lane * EPL + i] = z[i];
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    s[i] = sigmoid32(z[i]);
    sb[i] = s[i] + ((bias && valid[i]) ? bias[lane * EPL + i] : 0.0f);
    bad |= valid[i] && !(__builtin_isfinite(z[i]) && __builtin_isfinite(sb[i]));
  }
  if (__any(bad)) {
    if (lane < K) {
      idx[(size_t)t * K + lane] = lane;
      wout[(size_t)t * K + lane] = 0.0f;
    }
    if (lane == 0 && record) atomicOr(status, 1u);
    return;
  }
  // group scores
  const int lpg = E / (n_group * EPL);
  float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const float v = valid[i] ? sb[i] : -INFINITY;
    if (v > m1) {
      m2 = m1;
      m1 = v;
    } else if (v > m2) {
      m2 = v;
    }
  }
  for (int off = 1; off < lpg; off <<= 1) {
    const float o1 = __shfl_xor(m1, off), o2 = __shfl_xor(m2, off);
    const float hi = fmaxf(m1, o1), lo1 = fminf(m1, o1), lo2 = fmaxf(m2, o2);
    m1 = hi;
    m2 = fmaxf(lo1, lo2);
  }
  const float gs = m1 + m2;
  const int my_g = lane / lpg;
  int rank = 0;
  for (int o = 0; o < n_group; ++o) {
    const float go = readlane_f32(gs, o * lpg);
    rank += (go > gs) || (go == gs && o < my_g);
  }
  const bool keep = (lane * EPL < E) && rank < topk_group;
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane * EPL + i;
    key[i] = valid[i] ? (((uint64_t)orderable(keep ? sb[i] : -INFINITY) << 32) |
                         (uint64_t)(0xffffffffu - (uint32_t)e))
                      : 0ull;
  }
  uint32_t taken = 0;
  float S = 0.0f;
  int my_e = 0;
  float my_s = 0.0f;
  for (int j = 0; j < K; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (!((taken >> i) & 1u) && key[i] > best) best = key[i];
    // the wave's largest key: its score half by a 32-bit maximum, then the
    // lowest lane holding that score (lane l holds experts l EPL .. l EPL +
    // EPL - 1, and a lane's best already prefers its lower index on a tie),
    // which is the 64-bit maximum of (score, complemented index)
    const uint32_t hi = (uint32_t)(best >> 32);
    const uint32_t mhi = wave_max_u32(hi);
    const int owner = (int)__builtin_ctzll(__ballot(hi == mhi));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)best, owner);
    const int e = (int)(0xffffffffu - lo);
    const int slot = e % EPL;
    float sv = s[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i)
      if (slot == i) sv = s[i];
    const float ss = readlane_f32(sv, owner);
    if (lane == owner) taken |= 1u << slot;
    S = (j == 0) ? ss : S + ss;
    if (lane == j) {
      my_e = e;
      my_s = ss;
    }
  }
  if (lane < K) {
    const float d = S + 1e-20f;
    const float qv = my_s / d;
    idx[(size_t)t * K + lane] = my_e;
    wout[(size_t)t * K + lane] = qv * scale;
  }
}

int select_epl(int E) {
  const int need = (E + 63) / 64;
  int epl = 1;
  while (epl < need) epl *= 2;
  return epl;
}

template <int EPL>
static void launch_select_epl(dim3 grid, hipStream_t s, const float* part, int ks,
                              float* logits_out, const float* bias, int32_t* idx, float* w,
                              uint32_t* status, int T, int E, int n_group, int topk_group, int K,
                              float scale, int rec) {
  // the K split is a power of two up to kMaxKSplit (logits_ksplit)
  if (ks <= 1)
    hipLaunchKernelGGL((k_select<EPL, 1>), grid, dim3(256), 0, s, part, ks, logits_out, bias, idx,
                       w, status, T, E, n_group, topk_group, K, scale, rec);
  else if (ks <= 2)
    hipLaunchKernelGGL((k_select<EPL, 2>), grid, dim3(256), 0, s, part, ks, logits_out, bias, idx,
                       w, status, T, E, n_group, topk_group, K, scale, rec);
  else if (ks <= 4)
    hipLaunchKernelGGL((k_select<EPL, 4>), grid, dim3(256), 0, s, part, ks, logits_out, bias, idx,
                       w, status, T, E, n_group, topk_group, K, scale, rec);
  else if (ks <= 8)
    hipLaunchKernelGGL((k_select<EPL, 8>), grid, dim3(256), 0, s, part, ks, logits_out, bias, idx,
                       w, status, T, E, n_group, topk_group, K, scale, rec);
  else
    hipLaunchKernelGGL((k_select<EPL, kMaxKSplit>), grid, dim3(256), 0, s, part, ks, logits_out,
                       bias, idx, w, status, T, E, n_group, topk_group, K, scale, rec);
}

hipError_t launch_select(const float* part, int ks, float* logits_out, const float* bias,
                         int32_t* idx, float* w, uint32_t* status, int T, int E, int n_group,
                         int topk_group, int K, float scale, bool record_nonfinite, hipStream_t s,
                         const StageTimer* tm) {
  if (ks < 1 || ks > kMaxKSplit) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((T + 3) / 4));
  const int rec = record_nonfinite ? 1 : 0;
  stage_begin(tm, kSelect, s);
  switch (select_epl(E)) {
    case 1:
      launch_select_epl<1>(grid, s, part, ks, logits_out, bias, idx, w, status, T, E, n_group,
                           topk_group, K, scale, rec);
      break;
    case 2:
      launch_select_epl<2>(grid, s, part, ks, logits_out, bias, idx, w, status, T, E, n_group,
                           topk_group, K, scale, rec);
      break;
    case 4:
      launch_select_epl<4>(grid, s, part, ks, logits_out, bias, idx, w, status, T, E, n_group,
                           topk_group, K, scale, rec);
      break;
    default:
      launch_select_epl<8>(grid, s, part, ks, logits_out, bias, idx, w, status, T, E, n_group,
                           topk_group, K, scale, rec);
      break;
  }
  stage_end(tm, kSelect, s);
  return hipGetLastError();
}

}  // namespace moe
