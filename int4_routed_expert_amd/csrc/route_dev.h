// Device helpers of the router, shared by the router kernels and the one-token
// layer kernel: bounded buffer loads, the per-token selection (one wave per
// token), and the few-token logits (one workgroup per expert) with its
// completion hand-off.  See route.hip for the method and its citations.
#pragma once

#include "dot.h"

namespace moe {

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

struct SelCfg {
  int E, G, Gk, k, norm;
  float rsf;
};

// One wave selects for one token from its keys and scores already in LDS
// (skey, ssg: E entries each): group scores, the Gk kept groups, then k rounds
// of wave arg-max over the kept experts' keys; lanes r < k store rank r's
// expert and weight into idx_row[r] and w_row[r] (global or LDS).  Lane l holds
// experts l, l+64, ... (NPL experts per lane, E <= 64*NPL).
template <int NPL>
__device__ void select_wave(const SelCfg &a, const float *skey, const double *ssg, int lane, int32_t *idx_row,
                            float *w_row) {
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
    idx_row[lane] = my_idx;
    w_row[lane] = my_idx >= 0 ? (float)wv : __builtin_nanf("");
  }
}

__device__ inline void select_wave_dispatch(const SelCfg &a, const float *skey, const double *ssg, int lane,
                                            int32_t *idx_row, float *w_row) {
  const int npl = (a.E + 63) / 64;
  if (npl <= 1) select_wave<1>(a, skey, ssg, lane, idx_row, w_row);
  else if (npl <= 2) select_wave<2>(a, skey, ssg, lane, idx_row, w_row);
  else if (npl <= 4) select_wave<4>(a, skey, ssg, lane, idx_row, w_row);
  else if (npl <= 8) select_wave<8>(a, skey, ssg, lane, idx_row, w_row);
  else select_wave<16>(a, skey, ssg, lane, idx_row, w_row);
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

constexpr int kFewTokens = 8;  // the one-launch router handles up to this many tokens

// Few-token logits of expert e, part 1: waves 0..3 issue the loads of their
// quarter of W's row (bounded buffer loads: lanes past the share read zeros,
// so every load is unconditional and all are in flight together).
constexpr int kFewChunks = 8;  // ceil((H/4) / 256) <= 8 for H <= 8192
__device__ inline void few_logits_load(const RouteArgs &a, int e, int wave, int lane, float4 (&wv)[kFewChunks]) {
  const int q = a.H / 4;  // each wave's share of H (a multiple of 8)
  const __amdgpu_buffer_rsrc_t rw = share_rsrc(a.W + (size_t)e * a.H + (size_t)(wave & 3) * q, (uint32_t)q * 4u);
#pragma unroll
  for (int m = 0; m < kFewChunks; ++m) wv[m] = buf_f4(rw, (uint32_t)(m * 256 + lane * 4) * 4u);
}

// Part 2: waves 0..3 form the fp64 dots with the tokens' activations (same
// bounded loads), reduce each to lane 63, and the four shares are added in a
// fixed order by thread s < S, which scores logit (s, e) and stores the score
// and the selection key.  Every thread of the workgroup must call it (one
// barrier); waves past the fourth only wait.
__device__ inline void few_logits_finish(const RouteArgs &a, int e, int wave, int lane, const float4 (&wv)[kFewChunks],
                                         double (*part)[kFewTokens]) {
  const int q = a.H / 4;
  const size_t seg = (size_t)wave * q;
  if (wave < 4) {
    double acc[kFewTokens];
    // the activations of up to four tokens are requested together, then used
    // (one load latency per four tokens instead of one per token)
#pragma unroll
    for (int sb = 0; sb < kFewTokens; sb += 4) {
      if (sb < a.S) {
        float4 xv[4][kFewChunks];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int s = sb + j;
          if (s < a.S) {
            if (a.x_bf16) {
              const __amdgpu_buffer_rsrc_t rx =
                  share_rsrc((const uint16_t *)a.x + (size_t)s * a.H + seg, (uint32_t)q * 2u);
              uint2 raw[kFewChunks];
#pragma unroll
              for (int m = 0; m < kFewChunks; ++m) raw[m] = buf_u2(rx, (uint32_t)(m * 256 + lane * 4) * 2u);
#pragma unroll
              for (int m = 0; m < kFewChunks; ++m)
                xv[j][m] = make_float4(__uint_as_float(raw[m].x << 16), __uint_as_float(raw[m].x & 0xFFFF0000u),
                                       __uint_as_float(raw[m].y << 16), __uint_as_float(raw[m].y & 0xFFFF0000u));
            } else {
              const __amdgpu_buffer_rsrc_t rx =
                  share_rsrc((const float *)a.x + (size_t)s * a.H + seg, (uint32_t)q * 4u);
#pragma unroll
              for (int m = 0; m < kFewChunks; ++m) xv[j][m] = buf_f4(rx, (uint32_t)(m * 256 + lane * 4) * 4u);
            }
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int s = sb + j;
          if (s < a.S) {
            double t = 0.0;
#pragma unroll
            for (int m = 0; m < kFewChunks; ++m) {
              t = fma((double)wv[m].x, (double)xv[j][m].x, t);
              t = fma((double)wv[m].y, (double)xv[j][m].y, t);
              t = fma((double)wv[m].z, (double)xv[j][m].z, t);
              t = fma((double)wv[m].w, (double)xv[j][m].w, t);
            }
            acc[s] = t;
          }
        }
      }
    }
#pragma unroll
    for (int s = 0; s < kFewTokens; ++s)
      if (s < a.S) {
        const double v = wave_sum_f64_to63(acc[s]);
        if (lane == 63) part[wave][s] = v;
      }
  }
  const float b = a.bias[e];
  __syncthreads();
  if ((int)threadIdx.x < a.S) {
    const int s = threadIdx.x;
    double sv;
    float kv;
    score(((part[0][s] + part[1][s]) + part[2][s]) + part[3][s], b, sv, kv);
    a.scores[(size_t)s * a.E + e] = sv;
    a.keys[(size_t)s * a.E + e] = kv;
  }
}

// ---- selection of one token by a whole workgroup ---------------------------------
// Each expert's key becomes a unique 64-bit value (ordered key above, inverted
// index below), so "larger value" is exactly "higher key, lower index on ties".
// Then, with one expert per thread (or a few):
//   1. rank of the expert within its group (compares with the group's values);
//      the group's best min(k, per) values and its two best keys go to LDS;
//   2. every wave: group score = fp32 sum of the two best keys, the Gk best
//      groups kept (ties: lower group index);
//   3. an expert of a kept group with in-group rank r < min(k, per) has global
//      rank r + (number of better values among the other kept groups' best
//      lists); ranks below k name the selection;
//   4. lanes r < k of wave 0: weight of rank r from the unbiased scores summed in
//      rank order.
// The result is the sequential definition's (k rounds of arg-max over the kept
// experts) because the packed values are distinct and totally ordered.
__device__ inline uint64_t packed_rank_value(float key, int e) {
  return ((uint64_t)ordered_key(key) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

struct SelLds {
  alignas(16) uint64_t v[kMaxE];            // packed values of the token's experts
  alignas(16) uint64_t top[kMaxG * kMaxK];  // [group][rank < kMaxK] best values (0 past min(k, per))
  float gtop[kMaxG][2];           // two best keys of each group
  int out_e[kMaxK];               // selected expert of each rank
  int out_slot[kMaxK];            // and its slot-table entry (when loaded)
  double out_s[kMaxK];            // and its unbiased score
};

// One token's inputs, experts threadIdx.x + j * blockDim.x (clamped).
template <int EPT>
struct SelIn {
  float key[EPT];
  double s[EPT];
  int slot[EPT];
};

// Loads of the token's keys and scores (and slot-table entries when SLOT).
template <int EPT, bool SLOT>
__device__ inline void sel_load(const SelCfg &c, const float *keys, const double *scores, const int32_t *table,
                                SelIn<EPT> &in) {
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = min((int)threadIdx.x + j * (int)blockDim.x, c.E - 1);
    in.key[j] = ldg<float>(keys + e);
    in.s[j] = ldg<double>(scores + e);
    in.slot[j] = SLOT ? ldg<int>(table + e) : 0;
  }
}

// Every thread of the workgroup calls it (three barriers).  Leaves the ranks'
// experts, scores and slots in L.out_* (readable by every thread on return);
// lanes r < k of wave 0 store idx/w row t when idx_out is not null.
template <int EPT, bool SLOT>
__device__ void select_block(const SelCfg &c, int t, const SelIn<EPT> &in, SelLds &L, int32_t *idx_out,
                             float *w_out) {
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63;
  const int E = c.E, G = c.G, per = E / G, k = c.k, kk = min(k, per);
  uint64_t v[EPT];
  int rin[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + j * nt;
    v[j] = packed_rank_value(in.key[j], e);
    if (e < E) L.v[e] = v[j];
  }
  for (int i = tid; i < G * kMaxK; i += nt)
    if ((i & (kMaxK - 1)) >= kk) L.top[i] = 0ull;  // below every packed value
  __syncthreads();
  // 1. rank within the group
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + j * nt;
    rin[j] = per;
    if (e < E) {
      const int g = e / per;
      const uint64_t *gv = L.v + (size_t)g * per;
      int r = 0;
      if ((per & 7) == 0) {
        for (int cc = 0; cc < per; cc += 8) {
          ulonglong2 p[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) p[q] = *(const ulonglong2 *)(gv + cc + 2 * q);
#pragma unroll
          for (int q = 0; q < 4; ++q) r += (p[q].x > v[j] ? 1 : 0) + (p[q].y > v[j] ? 1 : 0);
        }
      } else {
        for (int cc = 0; cc < per; ++cc) r += (gv[cc] > v[j]) ? 1 : 0;
      }
      rin[j] = r;
      if (r < kk) L.top[(size_t)g * kMaxK + r] = v[j];
      if (r < 2) L.gtop[g][r] = in.key[j];
    }
  }
  __syncthreads();
  // 2. kept groups (G <= 64, so lane g of every wave holds group g)
  float gsc = -INFINITY;
  if (lane < G) gsc = per == 1 ? L.gtop[lane][0] : __double2float_rn((double)L.gtop[lane][0] + (double)L.gtop[lane][1]);
  int grk = 0;
  for (int i = 0; i < G; ++i) {
    const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gsc), i));
    grk += (o > gsc || (o == gsc && i < lane)) ? 1 : 0;
  }
  const uint64_t kept = __ballot(lane < G && grk < c.Gk);
  // 3. global rank of the kept groups' leading experts
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + j * nt;
    if (e < E && rin[j] < kk) {
      const int g = e / per;
      if ((kept >> g) & 1) {
        int r = rin[j];
        for (uint64_t m = kept & ~(1ull << g); m; m &= m - 1) {
          const ulonglong2 *tv = (const ulonglong2 *)(L.top + (size_t)__builtin_ctzll(m) * kMaxK);
          ulonglong2 p[kMaxK / 2];
#pragma unroll
          for (int q = 0; q < kMaxK / 2; ++q) p[q] = tv[q];
#pragma unroll
          for (int q = 0; q < kMaxK / 2; ++q) r += (p[q].x > v[j] ? 1 : 0) + (p[q].y > v[j] ? 1 : 0);
        }
        if (r < k) {
          L.out_e[r] = e;
          L.out_s[r] = in.s[j];
          L.out_slot[r] = in.slot[j];
        }
      }
    }
  }
  __syncthreads();
  // 4. weights (wave 0)
  if (idx_out && tid < 64) {
    const int my_e = lane < k ? L.out_e[lane] : -1;
    const double my_s = lane < k ? L.out_s[lane] : 0.0;
    double denom = 0.0;
    for (int r = 0; r < k; ++r) {
      const int lo = __builtin_amdgcn_readlane((int)__double2loint(my_s), r);
      const int hi = __builtin_amdgcn_readlane((int)__double2hiint(my_s), r);
      denom += __hiloint2double(hi, lo);
    }
    if (lane < k) {
      const double wv = c.norm ? my_s / denom * (double)c.rsf : my_s * (double)c.rsf;
      idx_out[(size_t)t * k + lane] = my_e;
      w_out[(size_t)t * k + lane] = (float)wv;
    }
  }
}

__device__ inline SelCfg sel_cfg(const RouteArgs &a) { return SelCfg{a.E, a.G, a.Gk, a.k, a.norm, a.rsf}; }

}  // namespace moe
