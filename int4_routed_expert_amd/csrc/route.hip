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

// Few tokens: one workgroup per expert, its 4 waves split H; all loads of a
// lane are issued before the FMAs; partial sums meet in LDS in a fixed order.
constexpr int kFewTokens = 8;
__global__ __launch_bounds__(256) void k_route_logits_few(RouteArgs a) {
  __shared__ double part[4][kFewTokens];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x;
  const int q = a.H / 4;  // each wave's share of H (H is a multiple of 32)
  const float *wr = a.W + (size_t)e * a.H + (size_t)wave * q;
  constexpr int kMaxChunks = 8;  // q / 256 <= 8 for H <= 8192
  const int nch = q / 256;
  float4 wv[kMaxChunks];
#pragma unroll
  for (int m = 0; m < kMaxChunks; ++m)
    if (m < nch) wv[m] = *(const float4 *)(wr + m * 256 + lane * 4);
  double acc[kFewTokens];
#pragma unroll
  for (int s = 0; s < kFewTokens; ++s) {
    acc[s] = 0.0;
    if (s < a.S) {
      float4 xv[kMaxChunks];
#pragma unroll
      for (int m = 0; m < kMaxChunks; ++m) {
        if (m < nch) {
          const size_t base = (size_t)s * a.H + (size_t)wave * q + m * 256 + lane * 4;
          if (a.x_bf16) {
            const uint2 r = *(const uint2 *)((const uint16_t *)a.x + base);
            xv[m] = make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u),
                                __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xFFFF0000u));
          } else {
            xv[m] = *(const float4 *)((const float *)a.x + base);
          }
        }
      }
      double t = 0.0;
#pragma unroll
      for (int m = 0; m < kMaxChunks; ++m) {
        if (m < nch) {
          t = fma((double)wv[m].x, (double)xv[m].x, t);
          t = fma((double)wv[m].y, (double)xv[m].y, t);
          t = fma((double)wv[m].z, (double)xv[m].z, t);
          t = fma((double)wv[m].w, (double)xv[m].w, t);
        }
      }
      acc[s] = t;
    }
  }
  for (int s = 0; s < a.S; ++s) {
    const double v = wave_sum_f64(acc[s]);
    if (lane == 0) part[wave][s] = v;
  }
  __syncthreads();
  if (threadIdx.x < a.S) {
    const int s = threadIdx.x;
    a.logits[(size_t)s * a.E + e] = ((part[0][s] + part[1][s]) + part[2][s]) + part[3][s];
  }
}

// One workgroup per token.  Selection by ranks instead of repeated arg-max:
// an item's rank is the number of items that beat it (larger key, or equal key
// and lower index), which is exactly its position in the tie-broken order.  The
// kept groups' experts are first compacted (in expert order) so every rank is a
// short unrolled scan of LDS.
__global__ __launch_bounds__(256) void k_route_select(RouteArgs a) {
  __shared__ __align__(16) float key[kMaxE];
  __shared__ __align__(16) float ckey[kMaxE];
  __shared__ double sg[kMaxE];
  __shared__ float gsc[kMaxG];
  __shared__ int keep[kMaxG], before[kMaxG];
  __shared__ int sel[kMaxK];
  __shared__ double ssel[kMaxK];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int E = a.E, G = a.G, per = a.E / a.G;
  const double *l = a.logits + (size_t)t * E;
  for (int e = tid; e < E; e += blockDim.x) {
    const double s = 1.0 / (1.0 + exp(-l[e]));
    sg[e] = s;
    key[e] = __double2float_rn(s + (double)a.bias[e]);
  }
  __syncthreads();
  // group score: sum of the group's two largest keys
  for (int j = tid; j < G; j += blockDim.x) {
    float k1 = -INFINITY, k2 = -INFINITY;
    if ((per & 3) == 0) {
      const float4 *p = (const float4 *)(key + j * per);
#pragma unroll 4
      for (int m = 0; m < per / 4; ++m) {
        const float4 v4 = p[m];
        const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float v = vv[c];
          if (v > k1) { k2 = k1; k1 = v; }
          else if (v > k2) { k2 = v; }
        }
      }
    } else {
      for (int e = j * per; e < (j + 1) * per; ++e) {
        const float v = key[e];
        if (v > k1) { k2 = k1; k1 = v; }
        else if (v > k2) { k2 = v; }
      }
    }
    gsc[j] = per == 1 ? k1 : __double2float_rn((double)k1 + (double)k2);
  }
  __syncthreads();
  // keep the topk_group best groups (ties: lower group index)
  for (int j = tid; j < G; j += blockDim.x) {
    const float v = gsc[j];
    int r = 0;
    for (int i = 0; i < G; ++i) r += (gsc[i] > v || (gsc[i] == v && i < j)) ? 1 : 0;
    keep[j] = r < a.Gk;
  }
  __syncthreads();
  for (int j = tid; j < G; j += blockDim.x) {
    int b = 0;
    for (int i = 0; i < j; ++i) b += keep[i];
    before[j] = b;
  }
  __syncthreads();
  // candidates in expert order
  for (int e = tid; e < E; e += blockDim.x) {
    const int j = e / per;
    if (keep[j]) ckey[before[j] * per + (e - j * per)] = key[e];
  }
  const int nc = a.Gk * per;
  for (int p = nc + tid; p < ((nc + 3) & ~3); p += blockDim.x) ckey[p] = -INFINITY;
  __syncthreads();
  // rank of each candidate (ties: lower position = lower expert index)
  for (int p = tid; p < nc; p += blockDim.x) {
    const float v = ckey[p];
    int r = 0;
    const float4 *c4 = (const float4 *)ckey;
#pragma unroll 8
    for (int m = 0; m < (nc + 3) / 4; ++m) {
      const float4 w4 = c4[m];
      const int q = 4 * m;
      r += (w4.x > v || (w4.x == v && q < p)) ? 1 : 0;
      r += (w4.y > v || (w4.y == v && q + 1 < p)) ? 1 : 0;
      r += (w4.z > v || (w4.z == v && q + 2 < p)) ? 1 : 0;
      r += (w4.w > v || (w4.w == v && q + 3 < p)) ? 1 : 0;
    }
    if (r < a.k) {
      // position p -> expert index: p-th candidate in the kept groups, in order
      const int kg = p / per;  // kg-th kept group
      int j = 0;
      for (int c = 0; j < G; ++j)
        if (keep[j] && c++ == kg) break;
      const int e = j * per + (p - kg * per);
      sel[r] = e;
      ssel[r] = sg[e];
    }
  }
  __syncthreads();
  // weights: un-biased sigmoid, renormalised over the selection (summed in rank order), scaled
  if (tid < a.k) {
    double denom = 0.0;
    for (int it = 0; it < a.k; ++it) denom += ssel[it];
    const double s = ssel[tid];
    const double wv = a.norm ? s / denom * (double)a.rsf : s * (double)a.rsf;
    a.idx[(size_t)t * a.k + tid] = sel[tid];
    a.w[(size_t)t * a.k + tid] = (float)wv;
  }
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t st) {
  if (a.S == 0) return hipSuccess;
  {
    ProfScope ps("route_logits", st);
    if (a.S <= kFewTokens && a.H % 1024 == 0) {
      MOE_LAUNCH(k_route_logits_few, dim3(a.E), dim3(256), 0, st, a);
    } else {
      dim3 grid((a.E + 3) / 4, (a.S + kLogitTokens - 1) / kLogitTokens);
      MOE_LAUNCH(k_route_logits, grid, dim3(256), 0, st, a);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("route_select", st);
    MOE_LAUNCH(k_route_select, dim3(a.S), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace moe
