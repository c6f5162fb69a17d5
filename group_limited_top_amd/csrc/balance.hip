// balance.hip -- load balancing around the routing: statistics of tracked
// expert hits ([Routing §六]), the expert-bias update ([Routing §三]) and the
// auxiliary load-balancing loss E * sum_i f_i * P_i ([Pitfalls, MoE 负载均衡
// Loss 别忘加]).
//
// These are small reductions (E <= 1024 values per layer, or the [T][E]
// logits once).  Every sum runs in a fixed order (per-lane loops in index
// order, then xor-butterfly wave sums and per-wave partials added in wave
// order), so results are bit-reproducible run to run; nothing uses atomics.
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBalThreads = 256;
constexpr int kBalWaves = kBalThreads / 64;

// xor-butterfly reductions: every lane ends with the same value (fp addition
// is commutative, and each lane combines the same pairs).
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide reduction over kBalWaves waves: each wave reduces, wave 0's lane
// values are combined in wave order.  `red` is LDS scratch of kBalWaves
// entries; returns the result in every thread.
template <typename T, typename Op>
__device__ __forceinline__ T block_reduce(T v, T* red, Op op) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = op(v, __shfl_xor(v, o, 64));
  __syncthreads();  // red may still be read by a previous reduction
  if (lane == 0) red[w] = v;
  __syncthreads();
  T r = red[0];
  for (int i = 1; i < kBalWaves; ++i) r = op(r, red[i]);
  return r;
}

// (count, index) pair for arg-max / arg-min with the lower index winning ties.
struct Arg {
  long long v;
  int i;
};
__device__ __forceinline__ Arg shfl_arg(Arg a, int o) {
  return Arg{__shfl_xor(a.v, o, 64), __shfl_xor(a.i, o, 64)};
}
__device__ __forceinline__ Arg arg_max(Arg a, Arg b) {
  return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}
__device__ __forceinline__ Arg arg_min(Arg a, Arg b) {
  return (b.v < a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

}  // namespace

// ----------------------------------------------------------------------------
// Statistics of tracked hits h[e] of one layer (one block per layer):
//   load[e] = RN32(h[e] * E / N), N = sum of h (all 0 when N = 0);
//   summary: N, max load, min load, coefficient of variation
//   sqrt(mean_e (h[e] - N/E)^2) / (N/E), idle experts, most / least hit
//   expert (lower index on ties), largest group load (group hits * n_group / N).
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kBalThreads) void k_expert_stats(const int64_t* __restrict__ tracking,
                                                              float* __restrict__ load,
                                                              double* __restrict__ summary,
                                                              int E, int n_group) {
  __shared__ long long red_i[kBalWaves];
  __shared__ double red_d[kBalWaves];
  __shared__ Arg red_a[kBalWaves];
  __shared__ long long gsum[64];
  const int l = blockIdx.x, tid = threadIdx.x;
  const int64_t* h = tracking + (size_t)l * E;
  float* ld = load + (size_t)l * E;
  double* s = summary + (size_t)l * kNStat;

  long long n = 0, idle = 0;
  Arg hot{-1, 0x7fffffff}, cold{0x7fffffffffffffffLL, 0x7fffffff};
  for (int e = tid; e < E; e += kBalThreads) {
    const long long v = h[e];
    n += v;
    idle += v == 0;
    hot = arg_max(hot, Arg{v, e});
    cold = arg_min(cold, Arg{v, e});
  }
  const long long N = block_reduce(n, red_i, [](long long a, long long b) { return a + b; });
  const long long nidle = block_reduce(idle, red_i, [](long long a, long long b) { return a + b; });
  // arg-max / arg-min: the same butterfly and wave-order steps on pairs
  {
    const int lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      hot = arg_max(hot, shfl_arg(hot, o));
      cold = arg_min(cold, shfl_arg(cold, o));
    }
    __syncthreads();
    if (lane == 0) red_a[w] = hot;
    __syncthreads();
    hot = red_a[0];
    for (int i = 1; i < kBalWaves; ++i) hot = arg_max(hot, red_a[i]);
    __syncthreads();
    if (lane == 0) red_a[w] = cold;
    __syncthreads();
    cold = red_a[0];
    for (int i = 1; i < kBalWaves; ++i) cold = arg_min(cold, red_a[i]);
  }
  // group hit sums: thread g adds its group's experts in index order
  const int gsize = E / n_group;
  if (tid < n_group) {
    long long sg = 0;
    for (int e = tid * gsize; e < (tid + 1) * gsize; ++e) sg += h[e];
    gsum[tid] = sg;
  }
  __syncthreads();
  long long gmax = 0;
  for (int g = 0; g < n_group; ++g) gmax = gsum[g] > gmax ? gsum[g] : gmax;

  const double Nd = (double)N;
  const double mean = Nd / (double)E;
  double ss = 0.0;
  for (int e = tid; e < E; e += kBalThreads) {
    const long long v = h[e];
    ld[e] = N == 0 ? 0.0f : (float)((double)(v * E) / Nd);
    const double dv = (double)v - mean;
    ss += dv * dv;
  }
  ss = block_reduce(ss, red_d, [](double a, double b) { return a + b; });
  if (tid == 0) {
    s[0] = Nd;
    s[4] = (double)nidle;
    s[5] = (double)hot.i;
    s[6] = (double)cold.i;
    if (N == 0) {
      s[1] = s[2] = s[3] = s[7] = 0.0;
    } else {
      s[1] = (double)(hot.v * E) / Nd;
      s[2] = (double)(cold.v * E) / Nd;
      s[3] = sqrt(ss / (double)E) / mean;
      s[7] = (double)(gmax * n_group) / Nd;
    }
  }
}

hipError_t launch_expert_stats(const int64_t* tracking, float* load, double* summary, int L, int E,
                               int n_group, hipStream_t s) {
  if (L <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_expert_stats, dim3((unsigned)L), dim3(kBalThreads), 0, s, tracking, load,
                     summary, E, n_group);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Expert-bias update from one routing's hit counts ([Routing §三]: raise the
// bias of experts that receive few tokens, lower it for those that receive
// many).  In fp64:
//   cbar = sum(counts) / E,  d = max(max_e |counts[e] - cbar|, 1),
//   bias_out[e] = RN32(bias_in[e] + (-rate * (counts[e] - cbar)) / d).
// The maximum is exact in any order, so the result is the same bits as any
// IEEE fp64 evaluation of this formula.  bias_out may equal bias_in.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kBalThreads) void k_bias_update(const int32_t* __restrict__ counts,
                                                             const float* bias_in, float* bias_out,
                                                             int E, double rate) {
  __shared__ long long red_i[kBalWaves];
  __shared__ double red_d[kBalWaves];
  const int tid = threadIdx.x;
  long long n = 0;
  for (int e = tid; e < E; e += kBalThreads) n += counts[e];
  const long long N = block_reduce(n, red_i, [](long long a, long long b) { return a + b; });
  const double cbar = (double)N / (double)E;
  double d = 1.0;
  for (int e = tid; e < E; e += kBalThreads) d = fmax(d, fabs((double)counts[e] - cbar));
  d = block_reduce(d, red_d, [](double a, double b) { return fmax(a, b); });
  __syncthreads();  // every thread has read its counts before any bias is written
  for (int e = tid; e < E; e += kBalThreads) {
    const double b = bias_in ? (double)bias_in[e] : 0.0;
    const double v = (-rate * ((double)counts[e] - cbar)) / d;
    bias_out[e] = (float)(b + v);
  }
}

hipError_t launch_bias_update(const int32_t* counts, const float* bias_in, float* bias_out, int E,
                              double rate, hipStream_t s) {
  hipLaunchKernelGGL(k_bias_update, dim3(1), dim3(kBalThreads), 0, s, counts, bias_in, bias_out,
                     E, rate);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Auxiliary load-balancing loss E * sum_i f_i * P_i, with f_i = counts[i] / T
// (fraction of tokens routed to expert i) and P_i = mean over tokens of
// softmax(logits[t])_i, all in fp64.
//
// Pass 1 (k_aux_partial): block b owns a fixed token range; its NW waves take
// kAuxTok consecutive tokens at a time (wave w the w-th such batch of the
// block, then every NW-th): all of the batch's logits are loaded first (lane
// c holds experts c, c + 64, ...), then per token the max and the sum of
// exp(l - max) by wave butterflies, and each lane adds its experts'
// probabilities to per-lane running sums in token order.  The waves' sums are
// added in wave order into the block's partial row part[b][E].
// Pass 2 (k_aux_reduce, one block per expert): thread i takes partial rows
// i, i + 256, ... in order, then the block reduction; writes P_e, f_e and
// f_e * P_e.  Pass 3 (k_aux_sum, one block): the loss from the f_e * P_e in
// a fixed order.
// ----------------------------------------------------------------------------
constexpr int kAuxTok = 4;          // tokens per wave batch
constexpr int kAuxMaxBlocks = 256;  // partial rows

template <int EPL>
constexpr int aux_waves() {  // waves per pass-1 block: LDS of NW * EPL * 64 doubles
  return EPL <= 4 ? 16 : (EPL <= 8 ? 8 : 4);
}

int aux_blocks(int T, int E) {
  const int epl = (E + 63) / 64;
  const int nw = epl <= 4 ? aux_waves<4>() : (epl <= 8 ? aux_waves<8>() : aux_waves<16>());
  const int64_t b = ((int64_t)T + nw * kAuxTok - 1) / (nw * kAuxTok);
  return b < 1 ? 1 : (b > kAuxMaxBlocks ? kAuxMaxBlocks : (int)b);
}

template <int EPL>
__global__ __launch_bounds__(64 * aux_waves<EPL>()) void k_aux_partial(
    const float* __restrict__ logits, double* __restrict__ part, int T, int E) {
  constexpr int NW = aux_waves<EPL>();
  __shared__ double acc_s[NW][EPL * 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nb = (int)gridDim.x, b = (int)blockIdx.x;
  const int t0 = (int)((int64_t)T * b / nb), t1 = (int)((int64_t)T * (b + 1) / nb);
  double acc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) acc[i] = 0.0;
  for (int tb = t0 + w * kAuxTok; tb < t1; tb += NW * kAuxTok) {
    float v[kAuxTok][EPL];
#pragma unroll
    for (int j = 0; j < kAuxTok; ++j) {
      const int t = tb + j;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        v[j][i] = (t < t1 && e < E) ? logits[(size_t)t * E + e] : 0.0f;
      }
    }
    const int nt = min(kAuxTok, t1 - tb);
    double m[kAuxTok], z[kAuxTok];
#pragma unroll
    for (int j = 0; j < kAuxTok; ++j) {
      m[j] = -INFINITY;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i < E) m[j] = fmax(m[j], (double)v[j][i]);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
#pragma unroll
      for (int j = 0; j < kAuxTok; ++j) m[j] = fmax(m[j], __shfl_xor(m[j], o, 64));
    double p[kAuxTok][EPL];
#pragma unroll
    for (int j = 0; j < kAuxTok; ++j) {
      z[j] = 0.0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        p[j][i] = lane + 64 * i < E ? exp((double)v[j][i] - m[j]) : 0.0;
        z[j] += p[j][i];
      }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
#pragma unroll
      for (int j = 0; j < kAuxTok; ++j) z[j] += __shfl_xor(z[j], o, 64);
#pragma unroll
    for (int j = 0; j < kAuxTok; ++j)
      if (j < nt) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) acc[i] += p[j][i] / z[j];
      }
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) acc_s[w][lane + 64 * i] = acc[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 64 * NW) {
    double r = acc_s[0][e];
    for (int j = 1; j < NW; ++j) r += acc_s[j][e];
    part[(size_t)b * E + e] = r;
  }
}

__global__ __launch_bounds__(kBalThreads) void k_aux_reduce(const double* __restrict__ part,
                                                            int nb,
                                                            const int32_t* __restrict__ counts,
                                                            double* __restrict__ f,
                                                            double* __restrict__ P,
                                                            double* __restrict__ fp, int T,
                                                            int E) {
  __shared__ double red_d[kBalWaves];
  const int e = (int)blockIdx.x;
  double r = 0.0;
  for (int b = threadIdx.x; b < nb; b += kBalThreads) r += part[(size_t)b * E + e];
  r = block_reduce(r, red_d, [](double a, double c) { return a + c; });
  if (threadIdx.x == 0) {
    const double Td = (double)T;
    const double pe = r / Td, fe = (double)counts[e] / Td;
    P[e] = pe;
    f[e] = fe;
    fp[e] = fe * pe;
  }
}

__global__ __launch_bounds__(kBalThreads) void k_aux_sum(const double* __restrict__ fp,
                                                         double* __restrict__ loss, int E) {
  __shared__ double red_d[kBalWaves];
  double s = 0.0;
  for (int e = threadIdx.x; e < E; e += kBalThreads) s += fp[e];
  s = block_reduce(s, red_d, [](double a, double c) { return a + c; });
  if (threadIdx.x == 0) *loss = (double)E * s;
}

size_t aux_workspace_bytes(int T, int E) {
  return ((size_t)aux_blocks(T, E) + 1) * (size_t)E * sizeof(double);
}

hipError_t launch_aux_loss(const float* logits, const int32_t* counts, double* f, double* P,
                           double* loss, double* ws, int T, int E, hipStream_t s) {
  const int nb = aux_blocks(T, E);
  const int epl = (E + 63) / 64;
  double* part = ws;                    // [nb][E]
  double* fp = ws + (size_t)nb * E;     // [E]
  if (epl <= 4)
    hipLaunchKernelGGL(k_aux_partial<4>, dim3(nb), dim3(64 * aux_waves<4>()), 0, s, logits, part,
                       T, E);
  else if (epl <= 8)
    hipLaunchKernelGGL(k_aux_partial<8>, dim3(nb), dim3(64 * aux_waves<8>()), 0, s, logits, part,
                       T, E);
  else
    hipLaunchKernelGGL(k_aux_partial<16>, dim3(nb), dim3(64 * aux_waves<16>()), 0, s, logits,
                       part, T, E);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_aux_reduce, dim3(E), dim3(kBalThreads), 0, s, part, nb, counts, f, P, fp,
                     T, E);
  hipLaunchKernelGGL(k_aux_sum, dim3(1), dim3(kBalThreads), 0, s, fp, loss, E);
  return hipGetLastError();
}

}  // namespace moe
