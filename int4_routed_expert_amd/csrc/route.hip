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

// Raw buffer resource over `bytes` bytes at p: loads at byte offsets past the
// end return zeros (range-checked in hardware; 0x00020000 is the gfx9-family
// data-format word that raw dword loads need).
__device__ inline __amdgpu_buffer_rsrc_t share_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}
__device__ inline float4 buf_f4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
__device__ inline uint2 buf_u2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  return make_uint2(v.x, v.y);
}

// ---- selection ------------------------------------------------------------------
// Monotone map of fp32 keys to uint32 (0 is below every key), so that the
// wave-wide arg-max is an integer max; ties are then broken towards the lower
// expert index.
__device__ inline uint32_t ordered_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ inline uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Maximum over the wave, returned to every lane.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<0xB1>(v));        // quad_perm [1,0,3,2]
  v = max(v, dpp_u<0x4E>(v));        // quad_perm [2,3,0,1]
  v = max(v, dpp_u<0x141>(v));       // row_half_mirror
  v = max(v, dpp_u<0x140>(v));       // row_mirror
  v = max(v, dpp_u<0x142, 0xA>(v));  // row_bcast:15
  v = max(v, dpp_u<0x143, 0xC>(v));  // row_bcast:31: lane 63 holds the maximum
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// s = sigmoid(l) and key = fp32(s + bias) of one (token, expert), fp64.
__device__ inline void score(double l, float bias, double &s, float &key) {
  s = 1.0 / (1.0 + exp(-l));
  key = __double2float_rn(s + (double)bias);
}

// One wave selects for token t from its keys and scores already in LDS (skey,
// ssg: E entries each): group scores, the Gk kept groups, then k rounds of
// wave arg-max over the kept experts' keys.  Lane l holds experts l, l+64, ...
// (NPL experts per lane, E <= 64*NPL).
template <int NPL>
__device__ void select_wave(const RouteArgs &a, int t, const float *skey, const double *ssg, int lane) {
  const int E = a.E, G = a.G, per = a.E / a.G;
  // group score: fp32 sum of the group's two largest keys (one lane per group)
  float gs = -INFINITY;
  if (lane < G) {
    // top two with multiplicity, branch-free: k1 >= k2 always
    float k1 = -INFINITY, k2 = -INFINITY;
    const float *p = skey + lane * per;
    if ((per & 3) == 0) {
      const float4 *p4 = (const float4 *)p;
#pragma unroll 8
      for (int i = 0; i < per / 4; ++i) {
        const float4 v = p4[i];
        k2 = fmaxf(k2, fminf(k1, v.x)); k1 = fmaxf(k1, v.x);
        k2 = fmaxf(k2, fminf(k1, v.y)); k1 = fmaxf(k1, v.y);
        k2 = fmaxf(k2, fminf(k1, v.z)); k1 = fmaxf(k1, v.z);
        k2 = fmaxf(k2, fminf(k1, v.w)); k1 = fmaxf(k1, v.w);
      }
    } else {
      for (int i = 0; i < per; ++i) {
        const float v = p[i];
        k2 = fmaxf(k2, fminf(k1, v));
        k1 = fmaxf(k1, v);
      }
    }
    gs = per == 1 ? k1 : __double2float_rn((double)k1 + (double)k2);
  }
  // keep the Gk best groups (ties: lower group index)
  int rk = 0;
  for (int i = 0; i < G; ++i) {
    const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gs), i));
    rk += (v > gs || (v == gs && i < lane)) ? 1 : 0;
  }
  const uint64_t kept = __ballot(lane < G && rk < a.Gk);
  uint32_t cand[NPL];
#pragma unroll
  for (int m = 0; m < NPL; ++m) {
    const int e = lane + 64 * m;
    cand[m] = (e < E && ((kept >> (e / per)) & 1)) ? ordered_key(skey[e]) : 0u;
  }
  int my_idx = -1;  // lane r < k: expert of rank r
  for (int r = 0; r < a.k; ++r) {
    uint32_t loc = 0;
#pragma unroll
    for (int m = 0; m < NPL; ++m) loc = max(loc, cand[m]);
    const uint32_t K = wave_max_u32(loc);
    if (K == 0u) break;  // no candidate left (cannot happen for a valid cfg)
    int lowest = 0x7fffffff;  // this lane's lowest expert holding K
#pragma unroll
    for (int m = NPL - 1; m >= 0; --m)
      if (cand[m] == K) lowest = lane + 64 * m;
    uint64_t holders = __ballot(lowest != 0x7fffffff);
    int e = __builtin_amdgcn_readlane(lowest, (int)__builtin_ctzll(holders));
    holders &= holders - 1;
    while (holders) {  // more than one lane only on exactly equal keys
      e = min(e, __builtin_amdgcn_readlane(lowest, (int)__builtin_ctzll(holders)));
      holders &= holders - 1;
    }
#pragma unroll
    for (int m = 0; m < NPL; ++m)
      if (lane + 64 * m == e) cand[m] = 0u;
    if (lane == r) my_idx = e;
  }
  const double my_s = my_idx >= 0 ? ssg[my_idx] : 0.0;
  double denom = 0.0;  // scores summed in rank order
  for (int r = 0; r < a.k; ++r) {
    const int lo = __builtin_amdgcn_readlane((int)__double2loint(my_s), r);
    const int hi = __builtin_amdgcn_readlane((int)__double2hiint(my_s), r);
    denom += __hiloint2double(hi, lo);
  }
  if (lane < a.k) {
    const double wv = a.norm ? my_s / denom * (double)a.rsf : my_s * (double)a.rsf;
    a.idx[(size_t)t * a.k + lane] = my_idx;
    a.w[(size_t)t * a.k + lane] = my_idx >= 0 ? (float)wv : __builtin_nanf("");
  }
}

__device__ void select_wave_dispatch(const RouteArgs &a, int t, const float *skey, const double *ssg, int lane) {
  const int npl = (a.E + 63) / 64;
  if (npl <= 1) select_wave<1>(a, t, skey, ssg, lane);
  else if (npl <= 2) select_wave<2>(a, t, skey, ssg, lane);
  else if (npl <= 4) select_wave<4>(a, t, skey, ssg, lane);
  else if (npl <= 8) select_wave<8>(a, t, skey, ssg, lane);
  else select_wave<16>(a, t, skey, ssg, lane);
}

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
  select_wave_dispatch(a, t, skey, ssg, lane);
}

// fp64 sum over the wave into lane 63 (DPP on the two halves; fixed order).
template <int CTRL, int ROW_MASK = 0xF>
__device__ inline double dpp_d(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROW_MASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROW_MASK, 0xF, false);
  return __hiloint2double(hi, lo);
}
__device__ inline double wave_sum_f64_to63(double v) {
  v += dpp_d<0xB1>(v);
  v += dpp_d<0x4E>(v);
  v += dpp_d<0x141>(v);
  v += dpp_d<0x140>(v);
  v += dpp_d<0x142, 0xA>(v);
  v += dpp_d<0x143, 0xC>(v);
  return v;
}

// Many tokens: the logits GEMM in fp64, one workgroup per 64 tokens x 32
// experts.  K advances in chunks of 32 staged in LDS (double-buffered, as fp32:
// bf16 and fp32 inputs both widen to fp32 exactly); each
// thread accumulates 4 tokens (strided by 16, so that its LDS reads are free of
// bank conflicts) x 2 experts with fp64 FMA in h order.
constexpr int kLT = 64, kLE = 32, kLK = 32, kLPad = 36;  // row stride 144 B
__global__ __launch_bounds__(256) void k_route_logits_tiled(RouteArgs a) {
  __shared__ __align__(16) float xs[2][kLT][kLPad];
  __shared__ __align__(16) float wsm[2][kLE][kLPad];
  const int t0 = blockIdx.x * kLT, e0 = blockIdx.y * kLE;
  const int tid = threadIdx.x;
  const int xr = tid >> 2, xc = (tid & 3) * 8;  // loader: x row, 8 columns
  const int wr = tid >> 3, wc = (tid & 7) * 4;  // loader: W row, 4 columns
  const size_t xrow = (size_t)min(t0 + xr, a.S - 1) * a.H;  // rows past S / E are clamped, not stored
  const float *wrow = a.W + (size_t)min(e0 + wr, a.E - 1) * a.H;
  const int ct = tid & 15, ce = (tid >> 4) * 2;
  auto load_x = [&](int k0, float4 &p, float4 &q) {
    if (a.x_bf16) {
      const uint4 r = *(const uint4 *)((const uint16_t *)a.x + xrow + k0 + xc);
      p = make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u), __uint_as_float(r.y << 16),
                      __uint_as_float(r.y & 0xFFFF0000u));
      q = make_float4(__uint_as_float(r.z << 16), __uint_as_float(r.z & 0xFFFF0000u), __uint_as_float(r.w << 16),
                      __uint_as_float(r.w & 0xFFFF0000u));
    } else {
      p = *(const float4 *)((const float *)a.x + xrow + k0 + xc);
      q = *(const float4 *)((const float *)a.x + xrow + k0 + xc + 4);
    }
  };
  float4 px, qx, pw;
  load_x(0, px, qx);
  pw = *(const float4 *)(wrow + wc);
  *(float4 *)&xs[0][xr][xc] = px;
  *(float4 *)&xs[0][xr][xc + 4] = qx;
  *(float4 *)&wsm[0][wr][wc] = pw;
  __syncthreads();
  double acc[4][2];
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r][0] = acc[r][1] = 0.0;
  const int nk = a.H / kLK;
  for (int kc = 0; kc < nk; ++kc) {
    const int kn = min(kc + 1, nk - 1) * kLK;  // unconditional prefetch (the last one repeats)
    load_x(kn, px, qx);
    pw = *(const float4 *)(wrow + kn + wc);
    const int b = kc & 1;
#pragma unroll
    for (int kk = 0; kk < kLK; kk += 4) {
      float4 xv[4], wv[2];
#pragma unroll
      for (int r = 0; r < 4; ++r) xv[r] = *(const float4 *)&xs[b][ct + 16 * r][kk];
      wv[0] = *(const float4 *)&wsm[b][ce][kk];
      wv[1] = *(const float4 *)&wsm[b][ce + 1][kk];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          double t = acc[r][c];
          t = fma((double)xv[r].x, (double)wv[c].x, t);
          t = fma((double)xv[r].y, (double)wv[c].y, t);
          t = fma((double)xv[r].z, (double)wv[c].z, t);
          t = fma((double)xv[r].w, (double)wv[c].w, t);
          acc[r][c] = t;
        }
    }
    *(float4 *)&xs[b ^ 1][xr][xc] = px;
    *(float4 *)&xs[b ^ 1][xr][xc + 4] = qx;
    *(float4 *)&wsm[b ^ 1][wr][wc] = pw;
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int t = t0 + ct + 16 * r, e = e0 + ce + c;
      if (t < a.S && e < a.E) a.logits[(size_t)t * a.E + e] = acc[r][c];
    }
}

// Few tokens (S <= kFewTokens), one launch for the whole router: one workgroup
// per expert computes that expert's logits (its 4 waves split H; every load of
// a lane is issued before the FMAs; partial sums meet in LDS in a fixed order),
// publishes them and counts itself done on a device-scope counter in the
// workspace header; the workgroup that completes the count selects for all
// tokens (scores by all its threads, then one wave per token) and puts the
// counter back to zero.  A workspace without the header's magic words gets
// idx = -1 and w = NaN.
constexpr int kFewTokens = 8;
constexpr int kBiasRegs = kMaxE / 256;
__global__ __launch_bounds__(256) void k_route_fused(RouteArgs a) {
  extern __shared__ double sel_lds[];
  __shared__ double part[4][kFewTokens];
  __shared__ int s_last;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x;
  const int q = a.H / 4;  // each wave's share of H (a multiple of 8)
  const size_t seg = (size_t)wave * q;
  // buffer loads bounded to the wave's share: lanes past it read zeros, so every
  // load is unconditional and all of them are in flight together
  const __amdgpu_buffer_rsrc_t rw = share_rsrc(a.W + (size_t)e * a.H + seg, (uint32_t)q * 4u);
  constexpr int kMaxChunks = 8;  // ceil(q / 256) <= 8 for H <= 8192
  float4 wv[kMaxChunks];
#pragma unroll
  for (int m = 0; m < kMaxChunks; ++m) wv[m] = buf_f4(rw, (uint32_t)(m * 256 + lane * 4) * 4u);
  const uint32_t m0 = a.sync[0], m1 = a.sync[1];
  if (m0 != kWsMagic0 || m1 != kWsMagic1) {
    if (e == 0)
      for (int i = threadIdx.x; i < a.S * a.k; i += blockDim.x) {
        a.idx[i] = -1;
        a.w[i] = __builtin_nanf("");
      }
    return;
  }
  double acc[kFewTokens];
#pragma unroll
  for (int s = 0; s < kFewTokens; ++s) {
    acc[s] = 0.0;
    if (s < a.S) {
      float4 xv[kMaxChunks];
      if (a.x_bf16) {
        const __amdgpu_buffer_rsrc_t rx =
            share_rsrc((const uint16_t *)a.x + (size_t)s * a.H + seg, (uint32_t)q * 2u);
        uint2 raw[kMaxChunks];
#pragma unroll
        for (int m = 0; m < kMaxChunks; ++m) raw[m] = buf_u2(rx, (uint32_t)(m * 256 + lane * 4) * 2u);
#pragma unroll
        for (int m = 0; m < kMaxChunks; ++m)
          xv[m] = make_float4(__uint_as_float(raw[m].x << 16), __uint_as_float(raw[m].x & 0xFFFF0000u),
                              __uint_as_float(raw[m].y << 16), __uint_as_float(raw[m].y & 0xFFFF0000u));
      } else {
        const __amdgpu_buffer_rsrc_t rx = share_rsrc((const float *)a.x + (size_t)s * a.H + seg, (uint32_t)q * 4u);
#pragma unroll
        for (int m = 0; m < kMaxChunks; ++m) xv[m] = buf_f4(rx, (uint32_t)(m * 256 + lane * 4) * 4u);
      }
      double t = 0.0;
#pragma unroll
      for (int m = 0; m < kMaxChunks; ++m) {
        t = fma((double)wv[m].x, (double)xv[m].x, t);
        t = fma((double)wv[m].y, (double)xv[m].y, t);
        t = fma((double)wv[m].z, (double)xv[m].z, t);
        t = fma((double)wv[m].w, (double)xv[m].w, t);
      }
      acc[s] = t;
    }
  }
#pragma unroll
  for (int s = 0; s < kFewTokens; ++s)
    if (s < a.S) {
      const double v = wave_sum_f64_to63(acc[s]);
      if (lane == 63) part[wave][s] = v;
    }
  // bias for the selection, loaded while the count completes
  float bias[kBiasRegs];
#pragma unroll
  for (int j = 0; j < kBiasRegs; ++j) bias[j] = a.bias[min((int)threadIdx.x + 256 * j, a.E - 1)];
  __syncthreads();
  if (threadIdx.x < a.S) {
    const int s = threadIdx.x;
    a.logits[(size_t)s * a.E + e] = ((part[0][s] + part[1][s]) + part[2][s]) + part[3][s];
  }
  // wave 0 wrote this expert's logits; its release-ordered increment publishes them
  if (threadIdx.x == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(a.sync + kSyncRouteCtr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == (uint32_t)(a.E - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // tokens in rounds of four: all threads score the round's (token, expert)
  // pairs into per-wave LDS, then wave w selects for token r + w
  for (int r = 0; r < a.S; r += 4) {
    const int nt = min(4, a.S - r);
#pragma unroll
    for (int j = 0; j < kBiasRegs; ++j) {
      const int ee = (int)threadIdx.x + 256 * j;
      if (ee < a.E)
        for (int w2 = 0; w2 < nt; ++w2) {
          double sv;
          float kv;
          score(a.logits[(size_t)(r + w2) * a.E + ee], bias[j], sv, kv);
          sel_lds[(size_t)w2 * a.E + ee] = sv;
          ((float *)(sel_lds + (size_t)4 * a.E))[(size_t)w2 * a.E + ee] = kv;
        }
    }
    __syncthreads();
    if (wave < nt) {
      const double *ssg = sel_lds + (size_t)wave * a.E;
      const float *skey = (const float *)(sel_lds + (size_t)4 * a.E) + (size_t)wave * a.E;
      select_wave_dispatch(a, r + wave, skey, ssg, lane);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) __hip_atomic_store(a.sync + kSyncRouteCtr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void k_ws_init(uint32_t *sync) {
  const int i = threadIdx.x;
  if (i < kWsSyncBytes / 4) sync[i] = i == 0 ? kWsMagic0 : i == 1 ? kWsMagic1 : 0u;
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t st) {
  if (a.S == 0) return hipSuccess;
  const size_t sel_lds = (size_t)4 * a.E * (sizeof(double) + sizeof(float));
  if (a.S <= kFewTokens) {
    ProfScope ps("route_fused", st);
    MOE_LAUNCH(k_route_fused, dim3(a.E), dim3(256), sel_lds, st, a);
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

hipError_t launch_ws_init(uint32_t *sync, hipStream_t st) {
  MOE_LAUNCH(k_ws_init, dim3(1), dim3(kWsSyncBytes / 4), 0, st, sync);
  return hipGetLastError();
}

}  // namespace moe
