// Router: fp64 logits GEMV/GEMM, then per-token sigmoid, group-limited top-k
// selection and renormalised weights.
//
// Method: "GLM-5.2 on a 32 GB Mac - native MLX port of the Colibri hierarchy",
// N1 "GLM-5.2 graph" and "G2 implementation status" (biased sigmoid selects,
// lower expert ID wins exact ties, un-biased sigmoid weights, routed scaling);
// colibri README "What's implemented" (DeepSeek-V3-style noaux_tc router);
// "Model support" 4.3 (grouped routing).  Group scoring (sum of the two largest
// keys per contiguous group) and exclusion of experts outside the kept groups
// are the DeepSeek-V3 reading of "grouped routing".
//
// Exactness: a product of two fp32 values is exact in fp64, so the logits are
// accumulated in fp64 (only summation-order rounding of ~1e-16 relative
// remains) and the selection key is fp32(sigmoid(l) + bias) with both steps in
// fp64, matching a plain fp64 evaluation except within ~2^-45 of an fp32
// rounding midpoint.
#include "common.h"

namespace moe {
namespace {

__device__ inline float load_x(const void *x, int bf16, size_t i) {
  if (bf16) {
    uint32_t b = (uint32_t)((const uint16_t *)x)[i] << 16;
    return __uint_as_float(b);
  }
  return ((const float *)x)[i];
}

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ inline unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long u = __shfl_xor(v, o);
    v = u > v ? u : v;
  }
  return v;
}

// Order-preserving map of a finite float onto uint32, combined with an index so
// that the larger key wins and, among equal keys, the lower index wins.
__device__ inline unsigned long long rank_key(float f, int index) {
  uint32_t b = __float_as_uint(f);
  uint32_t s = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)s << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)index);
}
__device__ inline int rank_index(unsigned long long r) { return (int)(0xFFFFFFFFu - (uint32_t)(r & 0xFFFFFFFFu)); }

constexpr int kLogitTokens = 4;  // tokens per block in the logits kernel

// One wave per expert row, kLogitTokens tokens per block: lanes stride over H in
// float4 chunks, fp64 FMA, then a wave reduction.
__global__ __launch_bounds__(256) void k_route_logits(RouteArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + wave;
  const int t0 = blockIdx.y * kLogitTokens;
  if (e >= a.E) return;
  const int nt = min(kLogitTokens, a.S - t0);
  double acc[kLogitTokens];
#pragma unroll
  for (int s = 0; s < kLogitTokens; ++s) acc[s] = 0.0;
  const float *wr = a.W + (size_t)e * a.H;
  for (int c = lane * 4; c < a.H; c += 256) {
    const float4 wv = *(const float4 *)(wr + c);
#pragma unroll
    for (int s = 0; s < kLogitTokens; ++s) {
      if (s < nt) {
        const size_t base = (size_t)(t0 + s) * a.H + c;
        acc[s] = fma((double)wv.x, (double)load_x(a.x, a.x_bf16, base + 0), acc[s]);
        acc[s] = fma((double)wv.y, (double)load_x(a.x, a.x_bf16, base + 1), acc[s]);
        acc[s] = fma((double)wv.z, (double)load_x(a.x, a.x_bf16, base + 2), acc[s]);
        acc[s] = fma((double)wv.w, (double)load_x(a.x, a.x_bf16, base + 3), acc[s]);
      }
    }
  }
#pragma unroll
  for (int s = 0; s < kLogitTokens; ++s) {
    double v = wave_sum_f64(acc[s]);
    if (lane == 0 && s < nt) a.logits[(size_t)(t0 + s) * a.E + e] = v;
  }
}

// One wave per token.
__global__ __launch_bounds__(64) void k_route_select(RouteArgs a) {
  __shared__ float key[kMaxE];
  __shared__ double sg[kMaxE];
  __shared__ int keep[kMaxG];
  const int t = blockIdx.x, lane = threadIdx.x;
  const int E = a.E, G = a.G, per = a.E / a.G;
  const double *l = a.logits + (size_t)t * E;
  for (int e = lane; e < E; e += 64) {
    const double s = 1.0 / (1.0 + exp(-l[e]));
    sg[e] = s;
    key[e] = __double2float_rn(s + (double)a.bias[e]);
  }
  __syncthreads();
  // group scores: lane j scores group j
  unsigned long long gk = 0;
  if (lane < G) {
    float k1 = -INFINITY, k2 = -INFINITY;
    for (int e = lane * per; e < (lane + 1) * per; ++e) {
      const float v = key[e];
      if (v > k1) { k2 = k1; k1 = v; }
      else if (v > k2) { k2 = v; }
    }
    const float score = per == 1 ? k1 : __double2float_rn((double)k1 + (double)k2);
    gk = rank_key(score, lane);
  }
  bool kept = false;
  for (int it = 0; it < a.Gk; ++it) {
    const unsigned long long m = wave_max_u64(kept ? 0ull : gk);
    if (lane < G && gk == m) kept = true;
  }
  if (lane < G) keep[lane] = kept ? 1 : 0;
  __syncthreads();
  // candidate keys, up to kMaxE / 64 per lane
  constexpr int kPer = kMaxE / 64;
  unsigned long long ck[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = lane + 64 * j;
    ck[j] = (e < E && keep[e / per]) ? rank_key(key[e], e) : 0ull;
  }
  int my_idx[kMaxK];
  for (int it = 0; it < a.k; ++it) {
    unsigned long long loc = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) loc = ck[j] > loc ? ck[j] : loc;
    const unsigned long long m = wave_max_u64(loc);
    const int e = rank_index(m);
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (ck[j] == m) ck[j] = 0ull;
    my_idx[it] = e;
  }
  if (lane == 0) {
    double denom = 0.0;
    for (int it = 0; it < a.k; ++it) denom += sg[my_idx[it]];
    for (int it = 0; it < a.k; ++it) {
      const double s = sg[my_idx[it]];
      const double wv = a.norm ? s / denom * (double)a.rsf : s * (double)a.rsf;
      a.idx[(size_t)t * a.k + it] = my_idx[it];
      a.w[(size_t)t * a.k + it] = (float)wv;
    }
  }
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t st) {
  if (a.S == 0) return hipSuccess;
  dim3 grid((a.E + 3) / 4, (a.S + kLogitTokens - 1) / kLogitTokens);
  {
    ProfScope ps("route_logits", st);
    hipLaunchKernelGGL(k_route_logits, grid, dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("route_select", st);
    hipLaunchKernelGGL(k_route_select, dim3(a.S), dim3(64), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace moe
