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
#include "route_dev.h"

namespace moe {
namespace {

// Many tokens: one wave per token, 4 per workgroup.  Dynamic LDS: 4 * E * 12 B.
__global__ __launch_bounds__(256) void k_route_select(RouteArgs a) {
  extern __shared__ double sel_lds[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  double *ssg = sel_lds + (size_t)wave * a.E;
  float *skey = (float *)(sel_lds + (size_t)4 * a.E) + (size_t)wave * a.E;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.S) return;
  const double *lt = a.logits + (size_t)t * a.E;
  for (int e = lane; e < a.E; e += 64) score(lt[e], a.bias[e], ssg[e], skey[e]);
  wave_lds_sync();
  select_wave_dispatch(sel_cfg(a), skey, ssg, lane, a.idx + (size_t)t * a.k, a.w + (size_t)t * a.k);
}

// Many tokens: the logits GEMM in fp64 on the matrix cores
// (v_mfma_f64_16x16x4f64: products of fp32 inputs are exact in fp64, sums in
// fp64), one workgroup per 32 tokens x 32 experts (two workgroups per CU).  K
// advances in chunks of 64 staged in LDS as fp32 (bf16 and fp32 inputs both
// widen to fp32 exactly; rows padded to 68 floats so that the fragment reads
// are free of bank conflicts), double-buffered with one barrier per chunk and
// requested two chunks ahead; an H that is an odd multiple of 32 ends with a
// half chunk padded with zeros.  Wave w owns the 16 x 16 block (tokens 16 (w %
// 2), experts 16 (w / 2)) and accumulates it in two chains (k = 0..3 and 4..7
// of every 8), added at the end, so that consecutive MFMAs do not wait for each
// other's results.  Fragment layouts (checked on the GPU): A lane l = (row l%16,
// k l/16), B lane l = (k l/16, column l%16), D lane l value i = (row l/16 + 4i,
// column l%16).
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kLT = 32, kLE = 32, kLK = 64, kLPad = 68;
__global__ __launch_bounds__(256) void k_route_logits_tiled(RouteArgs a) {
  __shared__ __align__(16) float xs[2][kLT][kLPad];
  __shared__ __align__(16) float wsm[2][kLE][kLPad];
  const int t0 = blockIdx.x * kLT, e0 = blockIdx.y * kLE;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int xr = tid >> 3, xc = (tid & 7) * 8;  // loader: x row, 8 columns
  const int wr = tid >> 3, wc = (tid & 7) * 8;  // loader: W row, 8 columns
  const size_t xrow = (size_t)min(t0 + xr, a.S - 1) * a.H;  // rows past S / E are clamped, not stored
  const float *wrow = a.W + (size_t)min(e0 + wr, a.E - 1) * a.H;
  struct Ld { float4 x0, x1, w0, w1; };
  auto load = [&](int k0, Ld &p) {
    if (k0 + xc >= a.H) {  // the last chunk of an H that is an odd multiple of 32: zero columns
      p.x0 = p.x1 = p.w0 = p.w1 = make_float4(0.f, 0.f, 0.f, 0.f);
      return;
    }
    if (a.x_bf16) {
      const uint4 r = *(const uint4 *)((const uint16_t *)a.x + xrow + k0 + xc);
      p.x0 = make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u), __uint_as_float(r.y << 16),
                         __uint_as_float(r.y & 0xFFFF0000u));
      p.x1 = make_float4(__uint_as_float(r.z << 16), __uint_as_float(r.z & 0xFFFF0000u), __uint_as_float(r.w << 16),
                         __uint_as_float(r.w & 0xFFFF0000u));
    } else {
      p.x0 = *(const float4 *)((const float *)a.x + xrow + k0 + xc);
      p.x1 = *(const float4 *)((const float *)a.x + xrow + k0 + xc + 4);
    }
    p.w0 = *(const float4 *)(wrow + k0 + wc);
    p.w1 = *(const float4 *)(wrow + k0 + wc + 4);
  };
  auto stage = [&](int b, const Ld &p) {
    *(float4 *)&xs[b][xr][xc] = p.x0;
    *(float4 *)&xs[b][xr][xc + 4] = p.x1;
    *(float4 *)&wsm[b][wr][wc] = p.w0;
    *(float4 *)&wsm[b][wr][wc + 4] = p.w1;
  };
  constexpr int kPf = 2;
  const int nk = (a.H + kLK - 1) / kLK;
  Ld pl[kPf];
#pragma unroll
  for (int d = 0; d < kPf; ++d) load(min(d, nk - 1) * kLK, pl[d]);
  stage(0, pl[0]);
  __syncthreads();
  f64x4 acc = {0.0, 0.0, 0.0, 0.0}, acc2 = {0.0, 0.0, 0.0, 0.0};
  const int tb = (wave & 1) * 16, eb = (wave >> 1) * 16, kq = lane >> 4;
  for (int kc0 = 0; kc0 < nk; kc0 += kPf) {
#pragma unroll
    for (int d = 0; d < kPf; ++d) {
      const int kc = kc0 + d;
      if (kc < nk) {  // uniform
        load(min(kc + kPf, nk - 1) * kLK, pl[d]);
        const int b = kc & 1;
#pragma unroll
        for (int kk = 0; kk < kLK; kk += 8) {
          const double av = (double)xs[b][tb + (lane & 15)][kk + kq];
          const double bv = (double)wsm[b][eb + (lane & 15)][kk + kq];
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
          const double av2 = (double)xs[b][tb + (lane & 15)][kk + 4 + kq];
          const double bv2 = (double)wsm[b][eb + (lane & 15)][kk + 4 + kq];
          acc2 = __builtin_amdgcn_mfma_f64_16x16x4f64(av2, bv2, acc2, 0, 0, 0);
        }
        stage(b ^ 1, pl[(d + 1) % kPf]);
        __syncthreads();
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + tb + (lane >> 4) + 4 * i, e = e0 + eb + (lane & 15);
    if (t < a.S && e < a.E) a.logits[(size_t)t * a.E + e] = acc[i] + acc2[i];
  }
}

// Few tokens, logits and selection inputs only (the selection runs in the
// consumer's first kernel): one workgroup per expert stores the tokens' scores
// and keys.  No completion count, so no workspace header is involved.
__global__ __launch_bounds__(256) void k_route_scores(RouteArgs a) {
  __shared__ double part[4][kFewTokens];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x;
  float4 wv[kFewChunks];
  few_logits_load(a, e, wave, lane, wv);
  few_logits_finish(a, e, wave, lane, wv, part);
}

// Few tokens, selection: one workgroup per token from the scores and keys that
// k_route_scores stored (the kernel boundary is the hand-off).  A workspace
// without the header's magic words gets idx = -1 and w = NaN.
template <int EPT>
__global__ __launch_bounds__(256) void k_route_select_few(RouteArgs a) {
  __shared__ SelLds sel;
  const int t = blockIdx.x;
  if (a.sync[0] != kWsMagic0 || a.sync[1] != kWsMagic1) {
    if ((int)threadIdx.x < a.k) {
      a.idx[(size_t)t * a.k + threadIdx.x] = -1;
      a.w[(size_t)t * a.k + threadIdx.x] = __builtin_nanf("");
    }
    return;
  }
  const SelCfg c = sel_cfg(a);
  SelIn<EPT> in;
  sel_load<EPT, false>(c, a.keys + (size_t)t * a.E, a.scores + (size_t)t * a.E, nullptr, in);
  select_block<EPT, false>(c, t, in, sel, a.idx, a.w);
}

__global__ void k_ws_init(uint32_t *sync) {
  const int i = threadIdx.x;
  if (i < kWsSyncBytes / 4) sync[i] = i == 0 ? kWsMagic0 : i == 1 ? kWsMagic1 : 0u;
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t st) {
  if (a.S == 0) return hipSuccess;
  const size_t sel_lds = (size_t)4 * a.E * (sizeof(double) + sizeof(float)) + (size_t)a.E * sizeof(float);
  if (a.S <= kFewTokens) {
    {
      ProfScope ps("route_scores", st);
      MOE_LAUNCH(k_route_scores, dim3(a.E), dim3(256), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ProfScope ps("route_select", st);
    if (a.E <= 256) {
      MOE_LAUNCH(k_route_select_few<1>, dim3(a.S), dim3(256), 0, st, a);
    } else {
      MOE_LAUNCH(k_route_select_few<4>, dim3(a.S), dim3(256), 0, st, a);
    }
    return hipGetLastError();
  }
  {
    ProfScope ps("route_logits", st);
    MOE_LAUNCH(k_route_logits_tiled, dim3((unsigned)((a.S + kLT - 1) / kLT), (unsigned)((a.E + kLE - 1) / kLE)),
               dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("route_select", st);
    MOE_LAUNCH(k_route_select, dim3((a.S + 3) / 4), dim3(256), sel_lds, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_route_scores(const RouteArgs &a, hipStream_t st) {
  if (a.S == 0) return hipSuccess;
  if (a.S > kFewTokens) return hipErrorInvalidValue;
  ProfScope ps("route_scores", st);
  MOE_LAUNCH(k_route_scores, dim3(a.E), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_ws_init(uint32_t *sync, hipStream_t st) {
  MOE_LAUNCH(k_ws_init, dim3(1), dim3(kWsSyncBytes / 4), 0, st, sync);
  return hipGetLastError();
}

}  // namespace moe
