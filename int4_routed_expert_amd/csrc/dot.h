// Device helpers of the int4 GEMV kernels: global loads/stores, wave reductions,
// and the exact integer group dot product.
//
// Group dot product.  A 32-element weight group holds int4 values q (stored as
// 4-bit two's complement, element i of a dword in nibble i) with one fp16 scale
// s.  The matching 32 activations v are written in block fixed point,
//     v_c ~= X_c * 2^-sh,   X_c = rint(v_c * 2^sh),   |X_c| <= 2^22,
// with sh chosen from the group's largest |v| (so every element is kept to
// 2^-22 of the group maximum), and each X_c is split into six balanced base-16
// digits d_l in [-8, 7] (X_c = sum_l 16^l d_l).  Digit l of the 32 elements is
// packed like the weights (4 dwords, element i in nibble i), so
//     sum_c q_c X_c = sum_l 16^l * sum_c q_c d_{l,c}
// is six sums of 4 v_dot8_i32_i4 each: exact integers (|per-limb sum| <= 2048,
// |total| <= 2^30), combined exactly in int32 and rounded once to fp32.  The
// group's contribution is then (float)T * (s * 2^-sh).  Per weight this is about
// one instruction, against two (byte-to-float and FMA) for dequantise-and-FMA,
// with error at the level of fp32 rounding of the group's largest activation.
#pragma once

#include "common.h"

namespace moe {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Loads and stores through global (address space 1) pointers.  Pointers that
// come from lane reads or integer arithmetic would otherwise be generic, and
// generic (flat) loads make every wait also wait for LDS traffic.
template <class T>
__device__ inline T ldg(const void *p) {
  return *(const __attribute__((address_space(1))) T *)p;
}
template <>
__device__ inline uint4 ldg<uint4>(const void *p) {
  const u32x4_t v = *(const __attribute__((address_space(1))) u32x4_t *)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <>
__device__ inline uint2 ldg<uint2>(const void *p) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = *(const __attribute__((address_space(1))) u32x2_t *)p;
  return make_uint2(v.x, v.y);
}
template <>
__device__ inline float4 ldg<float4>(const void *p) {
  const f32x4_t v = *(const __attribute__((address_space(1))) f32x4_t *)p;
  return make_float4(v.x, v.y, v.z, v.w);
}
template <class T>
__device__ inline void stg(void *p, const T &v) {
  *(__attribute__((address_space(1))) T *)p = v;
}
template <>
__device__ inline void stg<uint4>(void *p, const uint4 &v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  *(__attribute__((address_space(1))) u32x4_t *)p = w;
}
template <>
__device__ inline void stg<float2>(void *p, const float2 &v) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t w = {v.x, v.y};
  *(__attribute__((address_space(1))) f32x2_t *)p = w;
}
template <>
__device__ inline void stg<float4>(void *p, const float4 &v) {
  const f32x4_t w = {v.x, v.y, v.z, v.w};
  *(__attribute__((address_space(1))) f32x4_t *)p = w;
}

// Wave-uniform 64-bit pointer (first active lane's value) in scalar registers.
__device__ inline const uint8_t *uniform_ptr(const uint8_t *p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (const uint8_t *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Lane j's 64-bit value, read by the whole wave (the lane-read builtin is 32 bits).
__device__ inline const uint8_t *lane_ptr(uint64_t p, int j) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)p, j);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(p >> 32), j);
  return (const uint8_t *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ inline void opaque(uint4 &v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }

// Sum over the wave's 64 lanes with DPP row operations; the total lands in
// lane 63 (other lanes hold partial sums).  Every kernel reduces with this one
// fixed order, so a token's result does not depend on the batch it is in.
template <int CTRL, int ROW_MASK = 0xF>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
__device__ inline float wave_sum_to63(float v) {
  v += dpp_f<0xB1>(v);        // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);        // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);       // row_half_mirror
  v += dpp_f<0x140>(v);       // row_mirror: every lane holds its row's sum
  v += dpp_f<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Activations of one group in limb form: L[l][m] holds digit l of elements
// 8m..8m+7; f = 2^-sh.
struct Limbs {
  uint32_t L[6][4];
  float f;
};

// v[32] (fp32) -> limbs.  Balanced digits: with Z = X + 0x888888 (0 <= Z < 2^24),
// digit l = z_l - 8, whose 4-bit two's complement is z_l ^ 8; so Y = Z ^ 0x888888
// holds all six digits of one element, and the limb words are a nibble
// transpose of the eight Y of each dword (two rounds of byte permutes).
__device__ inline void to_limbs(const float *v, Limbs &out) {
  float m = 0.f;
#pragma unroll
  for (int c = 0; c < 32; ++c) m = fmaxf(m, fabsf(v[c]));
  int E = 0;
  (void)frexpf(m, &E);  // m < 2^E (E = 0 for m = 0)
  // at most 149: 2^-149 is the smallest fp32 power of two, and a group whose
  // largest value is below 2^-127 (subnormal) is then still held exactly
  const int sh = min(22 - E, 149);
  out.f = ldexpf(1.0f, -sh);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t Y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int X = (int)rintf(ldexpf(v[8 * d + i], sh));
      Y[i] = ((uint32_t)(X + 0x888888)) ^ 0x888888u;
    }
    // pairs: A_p bytes b = (nibble 2b of Y_2p) | (nibble 2b of Y_2p+1) << 4  -> limbs 0, 2, 4
    //        B_p bytes b = (nibble 2b+1 of Y_2p) | (nibble 2b+1 of Y_2p+1) << 4 -> limbs 1, 3, 5
    uint32_t A[4], B[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      A[p] = (Y[2 * p] & 0x0F0F0Fu) | ((Y[2 * p + 1] & 0x0F0F0Fu) << 4);
      B[p] = ((Y[2 * p] >> 4) & 0x0F0F0Fu) | (Y[2 * p + 1] & 0xF0F0F0u);
    }
    // limb 2b   = bytes b of A_0..A_3;  limb 2b+1 = bytes b of B_0..B_3
    // perm(s0, s1, sel): byte selector k < 4 picks s1's byte k, 4..7 picks s0's byte k-4
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      const uint32_t lo_sel = (uint32_t)(b | ((b + 4) << 8));  // bytes: s1.b, s0.b
      const uint32_t pa01 = __builtin_amdgcn_perm(A[1], A[0], lo_sel);  // A0.b, A1.b in bytes 0,1
      const uint32_t pa23 = __builtin_amdgcn_perm(A[3], A[2], lo_sel);  // A2.b, A3.b
      out.L[2 * b][d] = __builtin_amdgcn_perm(pa23, pa01, 0x05040100u);
      const uint32_t pb01 = __builtin_amdgcn_perm(B[1], B[0], lo_sel);
      const uint32_t pb23 = __builtin_amdgcn_perm(B[3], B[2], lo_sel);
      out.L[2 * b + 1][d] = __builtin_amdgcn_perm(pb23, pb01, 0x05040100u);
    }
  }
}

// sum_c q_c X_c of one group (exact), returned as fp32: Horner over the limbs,
// T = 16 T + (limb l's four dot8), from the top limb down (|T| <= 2^30).
__device__ inline float group_dot(const uint4 q, const Limbs &x) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  int T = 0;
#pragma unroll
  for (int l = 5; l >= 0; --l) {
    T <<= 4;
#pragma unroll
    for (int d = 0; d < 4; ++d) T = __builtin_amdgcn_sdot8((int)w[d], (int)x.L[l][d], T, false);
  }
  return (float)T;
}

// int8 weights (v_dot4_i32_i8) take the same block fixed point X_c with three
// balanced base-256 digits d_l in [-128, 127] (X_c = sum_l 256^l d_l): with
// Z = X + 0x808080 (0 <= Z < 2^24), digit l is z_l - 128, whose 8-bit two's
// complement is z_l ^ 0x80, so Y = Z ^ 0x808080 holds the three digits of one
// element and the limb words are a byte transpose of four Y.  Limb l of
// elements 4m..4m+3 (element 4m+i in byte i, as the int8 weights) is stored at
// L[2l + m/4][m%4]: the same 24 words as the int4 limbs.
__device__ inline void to_limbs8(const float *v, Limbs &out) {
  float m = 0.f;
#pragma unroll
  for (int c = 0; c < 32; ++c) m = fmaxf(m, fabsf(v[c]));
  int E = 0;
  (void)frexpf(m, &E);
  const int sh = min(22 - E, 149);  // as in to_limbs
  out.f = ldexpf(1.0f, -sh);
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint32_t Y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) Y[i] = ((uint32_t)((int)rintf(ldexpf(v[4 * d + i], sh)) + 0x808080)) ^ 0x808080u;
#pragma unroll
    for (int l = 0; l < 3; ++l) {
      const uint32_t sel = (uint32_t)(l | ((l + 4) << 8));  // bytes: s1.l, s0.l
      const uint32_t p01 = __builtin_amdgcn_perm(Y[1], Y[0], sel);
      const uint32_t p23 = __builtin_amdgcn_perm(Y[3], Y[2], sel);
      out.L[2 * l + d / 4][d % 4] = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
    }
  }
}

// One group's contribution T * s * f (f = 2^-sh) to an fp32 sum.  The power of
// two is applied last: s * f alone underflows for very small activations (f
// down to 2^-149), while T * s keeps its precision and the final scaling is
// exact wherever the contribution itself is a normal number.
__device__ inline float group_fma(float T, float s, float f, float acc) { return fmaf(T * s, f, acc); }

template <int WF>
__device__ inline void to_limbs_wf(const float *v, Limbs &out) {
  if constexpr (WF == kWfQ8Row) to_limbs8(v, out);
  else to_limbs(v, out);
}

// sum_c q_c X_c of one group of int8 weights (w0: elements 0..15, w1: 16..31):
// three exact digit sums (|each| <= 32 * 128 * 128 = 2^19) combined exactly in
// fp64 (|total| < 2^35) and rounded once to fp32.
__device__ inline float group_dot8(const uint4 w0, const uint4 w1, const Limbs &x) {
  const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  int T[3];
#pragma unroll
  for (int l = 0; l < 3; ++l) {
    T[l] = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) T[l] = __builtin_amdgcn_sdot4((int)w[m], (int)x.L[2 * l + m / 4][m % 4], T[l], false);
  }
  return (float)fma((double)T[2], 65536.0, (double)(T[1] * 256 + T[0]));
}

// Weights of one 32-element group of one row: one uint4 (int4) or two (int8).
template <int WF>
struct QGroup {
  uint4 q[WF == kWfQ8Row ? 2 : 1];
};
template <int WF>
__device__ inline void load_group(QGroup<WF> &g, const uint8_t *row, int grp) {
  g.q[0] = ldg<uint4>(row + (size_t)grp * group_bytes(WF));
  if constexpr (WF == kWfQ8Row) g.q[1] = ldg<uint4>(row + (size_t)grp * group_bytes(WF) + 16);
}
template <int WF>
__device__ inline float qdot(const QGroup<WF> &g, const Limbs &x) {
  if constexpr (WF == kWfQ8Row) return group_dot8(g.q[0], g.q[1], x);
  else return group_dot(g.q[0], x);
}

// Slot s (the table entry of expert e) is usable when it is in [0, n_slots)
// and, for a generation-tagged view, still holds the generation the table was
// published with (a slot refilled since then holds another expert).
__device__ inline bool slot_ok(const FfnArgs &a, int e, int s) {
  if (s < 0 || s >= a.n_slots) return false;
  return !a.gen || ldg<uint32_t>(a.slot_gen + s) == ldg<uint32_t>(a.gen + e);
}

// Packed weights of routed expert e through the slot table, or null when its
// slot is not usable.
__device__ inline const uint8_t *expert_ptr(const FfnArgs &a, int e) {
  const int s = ldg<int>(a.table + e);
  if (!slot_ok(a, e, s)) return nullptr;
  return a.base + (size_t)s * (size_t)a.slot_bytes;
}

__device__ inline float half_bits_to_float(uint32_t bits16) {
  return __half2float(__ushort_as_half((uint16_t)(bits16 & 0xFFFFu)));
}

}  // namespace moe
