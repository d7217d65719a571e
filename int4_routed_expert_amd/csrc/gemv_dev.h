// Device helpers of the GEMV kernels: activation staging in limb form, the
// gate/up feature ring (load one feature's two rows, compute its h), and the
// down tiles (load 8 rows, 8 row dots), for each weight format (template
// parameter WF, a moe_weight_format).  The tile math is the exact integer group
// dot of dot.h.
#pragma once

#include "dot.h"

namespace moe {

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// 32 activations (fp32, or bf16 bits) starting at element `off`.
__device__ inline void load32(const void *x, int bf16, size_t off, float *v) {
  if (bf16) {
    const uint16_t *p = (const uint16_t *)x + off;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 r = ldg<uint4>(p + 8 * m);
      const uint32_t d[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * m + 2 * j] = __uint_as_float(d[j] << 16);
        v[8 * m + 2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
      }
    }
  } else {
    const float *p = (const float *)x + off;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float4 r = ldg<float4>(p + 4 * m);
      v[4 * m] = r.x; v[4 * m + 1] = r.y; v[4 * m + 2] = r.z; v[4 * m + 3] = r.w;
    }
  }
}

// 32 int8 values (an int8-activation row's quantised integers) as floats, exact.
__device__ inline void load32_i8(const int8_t *p, float *v) {
  const uint4 r0 = ldg<uint4>(p), r1 = ldg<uint4>(p + 16);
  const uint32_t d[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = (float)(int8_t)(d[i >> 2] >> (8 * (i & 3)));
}

// The activations of one group as the contraction sees them: the exact values,
// or with int8 activations the row's quantised integers (the limbs' factor then
// takes the row scale d: T * 2^-sh * d is the group's dot with q * d).
__device__ inline void load_act32(const FfnArgs &a, bool x, size_t off, float *v) {
  if (!a.act_q) load32(x ? a.x : (const void *)a.h, x ? a.x_bf16 : 0, off, v);
  else load32_i8((x ? a.xq : a.hq) + off, v);
}
__device__ inline float act_scale(const FfnArgs &a, bool x, int row) {
  return a.act_q ? ldg<float>((x ? a.dx : a.dh) + row) : 1.0f;
}

__device__ inline void store_limbs(uint32_t *dst, float *fdst, const Limbs &L) {
  uint4 *d = (uint4 *)dst;
#pragma unroll
  for (int l = 0; l < 6; ++l) d[l] = make_uint4(L.L[l][0], L.L[l][1], L.L[l][2], L.L[l][3]);
  *fdst = L.f;
}
__device__ inline void load_limbs_lds(const uint32_t *src, const float *fsrc, Limbs &L) {
  const uint4 *s = (const uint4 *)src;
#pragma unroll
  for (int l = 0; l < 6; ++l) {
    const uint4 r = s[l];
    L.L[l][0] = r.x; L.L[l][1] = r.y; L.L[l][2] = r.z; L.L[l][3] = r.w;
  }
  L.f = *fsrc;
}
__device__ inline void load_limbs_global(const uint32_t *src, const float *fsrc, Limbs &L) {
#pragma unroll
  for (int l = 0; l < 6; ++l) {
    const uint4 r = ldg<uint4>(src + 4 * l);
    L.L[l][0] = r.x; L.L[l][1] = r.y; L.L[l][2] = r.z; L.L[l][3] = r.w;
  }
  L.f = ldg<float>(fsrc);
}

// ---- one token: gate/up ---------------------------------------------------------
// Scales: MOE_WF_Q4_G32 the fp16 (gate r, up r) pair of each of the lane's
// groups; the row-scaled formats the fp32 bits of the two row scales.
template <int NG, int WF>
struct GuFeat {
  QGroup<WF> g[NG], u[NG];
  uint32_t s[WF == kWfQ4G32 ? NG : 2];
  int valid;
};

// Loads of gate/up row pair r (feature r) of expert ex (null: an unresident
// expert, read from a stand-in and marked invalid).  Lanes past the last group
// read the last group and contribute zero because their activation limbs are
// zero.
template <int NG, int WF>
__device__ inline void gu_row_load(GuFeat<NG, WF> &b, const FfnArgs &a, const uint8_t *ex, int r, int lane) {
  const int H = a.H, ng = H / kGroup;
  const int64_t rb = row_bytes(H, WF);
  b.valid = ex != nullptr;
  if (!ex) ex = a.base;  // readable stand-in; the result is replaced by NaN
  const int pos = r & 3;
  const uint8_t *tile = ex + (size_t)(r >> 2) * gu_tile_bytes(H, WF);
  const uint8_t *rg = tile + (size_t)(2 * pos) * rb;
  const uint8_t *sc = tile + (size_t)kGuRows * rb;
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int g = min(lane + 64 * j, ng - 1);
    load_group(b.g[j], rg, g);
    load_group(b.u[j], rg + rb, g);
    if constexpr (WF == kWfQ4G32) b.s[j] = ldg<uint32_t>(sc + 4 * pos + g * 16);
  }
  if constexpr (WF != kWfQ4G32) {
    const uint2 s2 = ldg<uint2>(sc + 8 * pos);
    b.s[0] = s2.x;
    b.s[1] = s2.y;
  }
}

// Loads of feature i of this wave's list (clamped into range so that loads are
// unconditional): items [0, ns) are shared features s0 + i, the rest routed
// features r0 + i - ns of the list (expert j = feature / I, its pointer in lane j
// of my_ptr).
template <int NG, int WF>
__device__ inline void gu_feat_load(GuFeat<NG, WF> &b, const FfnArgs &a, int i, int n, int ns, int s0, int r0,
                                    uint64_t my_ptr, int lane) {
  i = min(i, n - 1);
  if (i < ns) {
    gu_row_load(b, a, a.shared, s0 + i, lane);
  } else {
    const int f = r0 + i - ns, j = f / a.I;
    gu_row_load(b, a, lane_ptr(my_ptr, j), f - j * a.I, lane);
  }
}

// h of one feature: the sums land in lane 63; the value is parked in lane
// `slot` of hout so that the loop issues no stores (stores would perturb the
// in-order load counter the prefetch ring relies on).
template <int NG, int WF>
__device__ inline float gu_feat_compute(const GuFeat<NG, WF> &b, const Limbs (&xv)[NG], int slot, float hout) {
  float g = 0.f, u = 0.f;
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    if constexpr (WF == kWfQ4G32) {
      g = group_fma(qdot(b.g[j], xv[j]), half_bits_to_float(b.s[j]), xv[j].f, g);
      u = group_fma(qdot(b.u[j], xv[j]), half_bits_to_float(b.s[j] >> 16), xv[j].f, u);
    } else {
      g = fmaf(qdot(b.g[j], xv[j]), xv[j].f, g);
      u = fmaf(qdot(b.u[j], xv[j]), xv[j].f, u);
    }
  }
  g = wave_sum_to63(g);
  u = wave_sum_to63(u);
  if constexpr (WF != kWfQ4G32) {
    g *= __uint_as_float(b.s[0]);
    u *= __uint_as_float(b.s[1]);
  }
  const float hv = b.valid ? silu_mul(g, u) : __builtin_nanf("");
  const float h63 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hv), 63));
  return (int)(threadIdx.x & 63) == slot ? h63 : hout;
}

constexpr int kGuMaxPerWave = 64;  // features per wave (one parked h per lane)

// ---- one token: down + route-order combine -----------------------------------------
// Scales: MOE_WF_Q4_G32 the 8 rows' fp16 scales of each of the lane's groups;
// the row-scaled formats the tile's 8 fp32 row scales.
template <int NGD, int WF>
struct DnTile {
  QGroup<WF> q[kDnRows][NGD];
  uint4 sc[WF == kWfQ4G32 ? NGD : 2];
};

// Tile t (clamped to the block's last tile: loads stay unconditional).
template <int NGD, int WF>
__device__ inline void dn_tile_load(DnTile<NGD, WF> &b, const uint8_t *dn, int inter, int t, int t1, int lane) {
  const int ng = inter / kGroup;
  const int64_t rb = row_bytes(inter, WF);
  const uint8_t *tile = dn + (size_t)min(t, t1 - 1) * dn_tile_bytes(inter, WF);
#pragma unroll
  for (int j = 0; j < NGD; ++j) {
    const int g = min(lane + 64 * j, ng - 1);
#pragma unroll
    for (int i = 0; i < kDnRows; ++i) load_group(b.q[i][j], tile + (size_t)i * rb, g);
    if constexpr (WF == kWfQ4G32) b.sc[j] = ldg<uint4>(tile + (size_t)kDnRows * rb + g * 16);
  }
  if constexpr (WF != kWfQ4G32) {
    b.sc[0] = ldg<uint4>(tile + (size_t)kDnRows * rb);
    b.sc[1] = ldg<uint4>(tile + (size_t)kDnRows * rb + 16);
  }
}

__device__ inline float scale_of(const uint4 sc, int i) {
  const uint32_t d[4] = {sc.x, sc.y, sc.z, sc.w};
  return half_bits_to_float(d[i >> 1] >> (16 * (i & 1)));
}
__device__ inline float row_scale_of(const uint4 (&sc)[2], int i) {
  const uint4 v = sc[i >> 2];
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
  return __uint_as_float(d[i & 3]);
}

// 8 row dots of one tile against one activation set; lane 63 holds the sums.
template <int NGD, int WF>
__device__ inline void dn_tile_dots(const DnTile<NGD, WF> &b, const Limbs (&hv)[NGD], float (&acc)[kDnRows]) {
#pragma unroll
  for (int i = 0; i < kDnRows; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < NGD; ++j)
#pragma unroll
    for (int i = 0; i < kDnRows; ++i) {
      if constexpr (WF == kWfQ4G32) acc[i] = group_fma(qdot(b.q[i][j], hv[j]), scale_of(b.sc[j], i), hv[j].f, acc[i]);
      else acc[i] = fmaf(qdot(b.q[i][j], hv[j]), hv[j].f, acc[i]);
    }
#pragma unroll
  for (int i = 0; i < kDnRows; ++i) {
    acc[i] = wave_sum_to63(acc[i]);
    if constexpr (WF != kWfQ4G32) acc[i] *= row_scale_of(b.sc, i);
  }
}

constexpr int kDnMaxTb = 8;    // down tiles per row block, at most
constexpr int kDnS1Waves = 9;  // waves per one-token down workgroup
// int8 tiles are twice as large: 8 waves (two per SIMD) leave each the
// registers for two tiles in flight
__host__ __device__ constexpr int dn_s1_waves(int wf) { return wf == kWfQ8Row ? 8 : kDnS1Waves; }

}  // namespace moe
