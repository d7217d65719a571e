// Expert FFN on the fp32 dequantise-and-multiply-accumulate path.
//
// Method: "GLM-5.2 on a 32 GB Mac - native MLX port of the Colibri hierarchy",
// N1 and "G2 implementation status": routed experts are SwiGLU FFNs over Q4
// weights whose nibbles are offset-binary (value = nibble - 8) with a scale per
// group; numerics are dequantise then f32 multiply-accumulate; the weighted
// expert outputs are composed in route order and the shared expert is added
// unweighted.  colibri README "What's implemented" (batch-union MoE): every
// unique expert of the batch is read once and applied to all tokens that chose it.
//
// Per 32-element group g of a weight row, with nibbles u and scale s:
//   sum_c (u_c - 8) s x_c = s * (sum_c u_c x_c - 8 * sum_c x_c)
// so the inner loop is one byte-to-float conversion and one FMA per weight, and
// the group sum of x is shared by the 8 rows of a tile.
//
// Decode path (S <= 4): two kernels.  Each workgroup derives the batch union
// from idx itself (at most 64 entries), so no planning launch is needed.
//  * k_gateup_small: one wave per gate/up tile (4 features: gate and up rows),
//    lanes own 32-element groups of K = H; h = silu(g) * u -> workspace.
//  * k_down_small: one workgroup per 8-row tile of y; its waves take the union's
//    experts, write per-(token, rank) dot products to LDS, and the workgroup
//    sums them in route order plus the shared expert: deterministic, no atomics,
//    and each token's result does not depend on the other tokens of the batch.
// Large-batch path: per-expert token lists (k_bucket), work items of up to 4
// tokens (k_schedule), the same tile math over items, and a combine kernel.
#include <algorithm>

#include "common.h"

namespace moe {
namespace {

constexpr int kTB = 4;  // tokens per work item

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// sum_c u_c x_c over one group: q holds 32 nibbles (element 2j low, 2j+1 high).
__device__ inline float dot_group(const uint4 q, const float *x) {
  const uint32_t d[4] = {q.x, q.y, q.z, q.w};
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = d[i] & 0x0F0F0F0Fu;
    const uint32_t hi = (d[i] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      acc = fmaf((float)((lo >> (8 * b)) & 0xFFu), x[8 * i + 2 * b], acc);
      acc = fmaf((float)((hi >> (8 * b)) & 0xFFu), x[8 * i + 2 * b + 1], acc);
    }
  }
  return acc;
}

__device__ inline float scale_of(const uint4 sc, int i) {
  const uint32_t d[4] = {sc.x, sc.y, sc.z, sc.w};
  const uint16_t bits = (uint16_t)(d[i >> 1] >> (16 * (i & 1)));
  return __half2float(__ushort_as_half(bits));
}

// Load a 32-element activation group (fp32 or bf16) and its sum.
__device__ inline float load_group(const void *x, int bf16, size_t off, float *xv) {
  if (bf16) {
    const uint4 *p = (const uint4 *)((const uint16_t *)x + off);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 r = p[v];
      const uint32_t d[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xv[8 * v + 2 * j] = __uint_as_float(d[j] << 16);
        xv[8 * v + 2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
      }
    }
  } else {
    const float4 *p = (const float4 *)((const float *)x + off);
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const float4 r = p[v];
      xv[4 * v] = r.x; xv[4 * v + 1] = r.y; xv[4 * v + 2] = r.z; xv[4 * v + 3] = r.w;
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 32; ++c) s += xv[c];
  return s;
}

// Keeps the compiler from hoisting the nibble unpacking of a whole tile out of
// the per-token loop (that would need 8 * 32 * NG registers per lane).
__device__ inline void opaque(uint4 &v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Batch union for S <= 4, in LDS.  uniq[0..U) ascending expert ids; for unique
// slot u: ntok[u] tokens tok[u][a] (ascending) with pair index pair[u][a] =
// token * (k+1) + rank.  Slot U is the shared expert with every token.
struct SmallPlan {
  int U;
  int tokbad[kSmallS];          // token's idx row names an expert outside [0, E) or twice
  int sidx[kSmallS * kMaxK];    // idx with invalid and repeated entries as -1
  int sfirst[kSmallS * kMaxK];  // entry is the first occurrence of its expert
  int uniq[kSmallS * kMaxK];
  int ntok[kSmallS * kMaxK + 1];
  int tok[kSmallS * kMaxK + 1][kSmallS];
  int pair[kSmallS * kMaxK + 1][kSmallS];
};

// Needs blockDim.x > S * k.
__device__ void build_small_plan(const FfnArgs &a, SmallPlan &p) {
  const int n = a.S * a.k, tid = threadIdx.x;
  if (tid == 0) p.U = 0;
  if (tid < a.S) p.tokbad[tid] = 0;
  __syncthreads();
  if (tid < n) {
    const int e = a.idx[tid];
    const int t = tid / a.k;
    bool ok = e >= 0 && e < a.E;
    for (int j = t * a.k; j < tid && ok; ++j) ok = a.idx[j] != e;
    p.sidx[tid] = ok ? e : -1;
    if (!ok) atomicOr(&p.tokbad[t], 1);
  }
  __syncthreads();
  if (tid < n) {
    const int e = p.sidx[tid];
    int first = e >= 0;
    for (int j = 0; j < tid; ++j) first &= (p.sidx[j] != e);
    p.sfirst[tid] = first;
  }
  __syncthreads();
  if (tid < n && p.sfirst[tid]) {
    const int e = p.sidx[tid];
    int pos = 0;
    for (int j = 0; j < n; ++j) pos += (p.sfirst[j] && p.sidx[j] < e) ? 1 : 0;
    p.uniq[pos] = e;
    atomicAdd(&p.U, 1);
  }
  __syncthreads();
  const int U = p.U;
  if (tid <= U) {
    int c = 0;
    for (int t = 0; t < a.S; ++t) {
      if (tid == U) {  // shared expert: every token, rank k
        p.tok[tid][c] = t; p.pair[tid][c] = t * (a.k + 1) + a.k; ++c;
      } else {
        for (int j = 0; j < a.k; ++j)
          if (p.sidx[t * a.k + j] == p.uniq[tid]) { p.tok[tid][c] = t; p.pair[tid][c] = t * (a.k + 1) + j; ++c; }
      }
    }
    p.ntok[tid] = c;
  }
  __syncthreads();
}

__device__ inline const uint8_t *expert_ptr(const FfnArgs &a, int e) {
  const int s = a.table[e];
  if (s < 0 || s >= a.n_slots) return nullptr;
  return a.base + (size_t)s * (size_t)a.slot_bytes;
}

// ---- one gate/up tile for a set of tokens -----------------------------------
// Lane owns groups lane + 64 j (j < NG) of K = H.  Activations come from LDS
// (xl: fp32 [S, H] and group sums xsum [S, H/32], staged by the workgroup) when
// XLDS is set, else from global memory (fp32 or bf16).
template <int NG, bool XLDS>
__device__ inline void gateup_tile(const FfnArgs &a, const uint8_t *tile, int ntok, const int *toks, const int *pairs,
                                   int feat0, int inter_stride, const float *xl, const float *xsum) {
  const int lane = threadIdx.x & 63, H = a.H, ng = H / kGroup;
  uint4 q[kGuRows][NG], sc[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int g = lane + 64 * j;
    if (g < ng) {
#pragma unroll
      for (int i = 0; i < kGuRows; ++i) q[i][j] = *(const uint4 *)(tile + (size_t)i * (H / 2) + g * 16);
      sc[j] = *(const uint4 *)(tile + (size_t)kGuRows * (H / 2) + g * 16);
    }
  }
  for (int tt = 0; tt < ntok; ++tt) {
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
      for (int i = 0; i < kGuRows; ++i) opaque(q[i][j]);
    float acc[kGuRows];
#pragma unroll
    for (int i = 0; i < kGuRows; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int g = lane + 64 * j;
      if (g < ng) {
        float xv[32], xs;
        if (XLDS) {
          const float4 *p = (const float4 *)(xl + (size_t)toks[tt] * H + g * kGroup);
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            const float4 r = p[v];
            xv[4 * v] = r.x; xv[4 * v + 1] = r.y; xv[4 * v + 2] = r.z; xv[4 * v + 3] = r.w;
          }
          xs = xsum[toks[tt] * ng + g];
        } else {
          xs = load_group(a.x, a.x_bf16, (size_t)toks[tt] * H + g * kGroup, xv);
        }
#pragma unroll
        for (int i = 0; i < kGuRows; ++i) {
          const float d = dot_group(q[i][j], xv);
          acc[i] = fmaf(scale_of(sc[j], i), fmaf(-8.f, xs, d), acc[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kGuRows; ++i) acc[i] = wave_sum(acc[i]);
    if (lane < kGuPairs) {
      float gv = acc[0], uv = acc[1];
#pragma unroll
      for (int r = 1; r < kGuPairs; ++r)
        if (lane == r) { gv = acc[2 * r]; uv = acc[2 * r + 1]; }
      a.h[(size_t)pairs[tt] * inter_stride + feat0 + lane] = silu_mul(gv, uv);
    }
  }
}

__device__ inline void poison_h(const FfnArgs &a, int ntok, const int *pairs, int feat0, int inter_stride) {
  const int lane = threadIdx.x & 63;
  if (lane < kGuPairs)
    for (int tt = 0; tt < ntok; ++tt) a.h[(size_t)pairs[tt] * inter_stride + feat0 + lane] = __builtin_nanf("");
}

constexpr int kGuWaves = 8;  // waves per gate/up workgroup, one tile each

// ---- decode path: gate/up ------------------------------------------------------
template <int NG, bool XLDS>
__global__ __launch_bounds__(kGuWaves * 64) void k_gateup_small(FfnArgs a) {
  extern __shared__ float xl[];  // XLDS: [S, H] fp32 then [S, H/32] group sums
  __shared__ SmallPlan plan;
  build_small_plan(a, plan);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ng = a.H / kGroup;
  float *xsum = xl + (size_t)a.S * a.H;
  if (XLDS) {
    const int n = a.S * ng;  // one thread per (token, group): copy 32 values and sum them in order
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      float xv[32];
      const float s = load_group(a.x, a.x_bf16, (size_t)i * kGroup, xv);
      float4 *d = (float4 *)(xl + (size_t)i * kGroup);
#pragma unroll
      for (int v = 0; v < 8; ++v) d[v] = make_float4(xv[4 * v], xv[4 * v + 1], xv[4 * v + 2], xv[4 * v + 3]);
      xsum[i] = s;
    }
    __syncthreads();
  }
  const int Imax = max(a.I, a.Is);
  const int tr = a.I / kGuPairs, ts = a.Is / kGuPairs;
  const int total = plan.U * tr + ts;
  const int tile = blockIdx.x * kGuWaves + wave;
  if (tile >= total) return;
  int u, t;
  const uint8_t *ex;
  if (tile < plan.U * tr) {
    u = tile / tr; t = tile - u * tr;
    ex = expert_ptr(a, plan.uniq[u]);
  } else {
    u = plan.U; t = tile - plan.U * tr;
    ex = a.shared;
  }
  (void)lane;
  if (!ex) { poison_h(a, plan.ntok[u], plan.pair[u], t * kGuPairs, Imax); return; }
  gateup_tile<NG, XLDS>(a, ex + (size_t)t * gu_tile_bytes(a.H), plan.ntok[u], plan.tok[u], plan.pair[u],
                        t * kGuPairs, Imax, xl, xsum);
}

// ---- one down tile: dots of 8 rows with h of each token ------------------------
// Lane i < 8 stores row i of token tt's dot at dst[pairs[tt] * dst_stride + i].
template <int NGD>
__device__ inline void down_tile(const FfnArgs &a, const uint8_t *tile, int inter, int ntok, const int *pairs,
                                 int inter_stride, float *dst, int dst_stride) {
  const int lane = threadIdx.x & 63, ng = inter / kGroup;
  uint4 q[kDnRows][NGD], sc[NGD];
#pragma unroll
  for (int j = 0; j < NGD; ++j) {
    const int g = lane + 64 * j;
    if (g < ng) {
#pragma unroll
      for (int i = 0; i < kDnRows; ++i) q[i][j] = *(const uint4 *)(tile + (size_t)i * (inter / 2) + g * 16);
      sc[j] = *(const uint4 *)(tile + (size_t)kDnRows * (inter / 2) + g * 16);
    }
  }
  for (int tt = 0; tt < ntok; ++tt) {
#pragma unroll
    for (int j = 0; j < NGD; ++j)
#pragma unroll
      for (int i = 0; i < kDnRows; ++i) opaque(q[i][j]);
    float acc[kDnRows];
#pragma unroll
    for (int i = 0; i < kDnRows; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < NGD; ++j) {
      const int g = lane + 64 * j;
      if (g < ng) {
        float hv[32];
        const float hs = load_group(a.h, 0, (size_t)pairs[tt] * inter_stride + g * kGroup, hv);
#pragma unroll
        for (int i = 0; i < kDnRows; ++i) {
          const float d = dot_group(q[i][j], hv);
          acc[i] = fmaf(scale_of(sc[j], i), fmaf(-8.f, hs, d), acc[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kDnRows; ++i) acc[i] = wave_sum(acc[i]);
    if (lane < kDnRows) {
      float v = acc[0];
#pragma unroll
      for (int i = 1; i < kDnRows; ++i)
        if (lane == i) v = acc[i];
      dst[(size_t)pairs[tt] * dst_stride + lane] = v;
    }
  }
}

// ---- decode path: down + route-order combine ------------------------------------
template <int NGD>
__global__ __launch_bounds__(1024) void k_down_small(FfnArgs a) {
  __shared__ SmallPlan plan;
  __shared__ float part[kSmallS * (kMaxK + 1)][kDnRows];
  build_small_plan(a, plan);
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  const int Imax = max(a.I, a.Is);
  const int rt = blockIdx.x;  // row tile of y
  const int nu = plan.U + (a.Is > 0 ? 1 : 0);
  for (int u = wave; u < nu; u += nw) {
    const bool sh = u == plan.U;
    const uint8_t *ex = sh ? a.shared : expert_ptr(a, plan.uniq[u]);
    const int inter = sh ? a.Is : a.I;
    if (!ex) {
      if (lane < kDnRows)
        for (int tt = 0; tt < plan.ntok[u]; ++tt) part[plan.pair[u][tt]][lane] = __builtin_nanf("");
      continue;
    }
    down_tile<NGD>(a, ex + down_offset(a.H, inter) + (size_t)rt * dn_tile_bytes(inter), inter, plan.ntok[u],
                   plan.pair[u], Imax, &part[0][0], kDnRows);
  }
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < a.S * kDnRows) {
    const int t = tid / kDnRows, i = tid % kDnRows;
    float acc = 0.f;
    const bool bad = plan.tokbad[t] != 0;
    if (!bad)
      for (int j = 0; j < a.k; ++j) acc = fmaf(a.w[t * a.k + j], part[t * (a.k + 1) + j][i], acc);
    if (a.Is > 0) acc += part[t * (a.k + 1) + a.k][i];
    a.y[(size_t)t * a.H + rt * kDnRows + i] = bad ? __builtin_nanf("") : acc;
  }
}

// ---- large-batch path ----------------------------------------------------------
// Per-expert token list in token order: block e scans idx in order and compacts
// the entries equal to e (each token names an expert at most once).
__global__ __launch_bounds__(256) void k_bucket(FfnArgs a) {
  __shared__ int wtot[4];
  __shared__ int base_s;
  const int e = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = a.S * a.k;
  if (tid == 0) base_s = 0;
  __syncthreads();
  for (int c0 = 0; c0 < n; c0 += 256) {
    const int i = c0 + tid;
    bool m = i < n && a.idx[i] == e;
    if (m) {  // a token that names e twice contributes once; the combine poisons it
      const int t0 = i / a.k * a.k;
      for (int j = t0; j < i; ++j) m = m && a.idx[j] != e;
    }
    const unsigned long long bal = __ballot(m);
    const int pre = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wtot[wave] = __popcll(bal);
    __syncthreads();
    int off = base_s;
    for (int w2 = 0; w2 < wave; ++w2) off += wtot[w2];
    if (m) {
      const int t = i / a.k, j = i - t * a.k;
      a.lists[(size_t)e * a.S + off + pre] = t * (a.k + 1) + j;
    }
    __syncthreads();
    if (tid == 0) base_s += wtot[0] + wtot[1] + wtot[2] + wtot[3];
    __syncthreads();
  }
  if (tid == 0) a.counts[e] = base_s;
}

// Work items {expert, first list position, n tokens}: routed experts in id order,
// then the shared expert (id E) over all tokens.
__global__ __launch_bounds__(1024) void k_schedule(FfnArgs a) {
  __shared__ int pre[kMaxE + 1];
  const int tid = threadIdx.x, E = a.E;
  for (int e = tid; e < E; e += blockDim.x) pre[e] = (a.counts[e] + kTB - 1) / kTB;
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int e = 0; e < E; ++e) { const int c = pre[e]; pre[e] = s; s += c; }
    pre[E] = s;
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    const int c = a.counts[e];
    for (int s = 0; s * kTB < c; ++s) {
      int *it = a.items + 3 * (size_t)(pre[e] + s);
      it[0] = e; it[1] = s * kTB; it[2] = min(kTB, c - s * kTB);
    }
  }
  const int nr = pre[E];
  const int nsh = a.Is > 0 ? (a.S + kTB - 1) / kTB : 0;
  for (int s = tid; s < nsh; s += blockDim.x) {
    int *it = a.items + 3 * (size_t)(nr + s);
    it[0] = E; it[1] = s * kTB; it[2] = min(kTB, a.S - s * kTB);
  }
  if (tid == 0) { a.n_items[0] = nr; a.n_items[1] = nsh; }
}

__device__ inline int item_tokens(const FfnArgs &a, const int *it, int *toks, int *pairs) {
  const int e = it[0], s0 = it[1], n = it[2];
  for (int tt = 0; tt < n; ++tt) {
    if (e == a.E) { toks[tt] = s0 + tt; pairs[tt] = (s0 + tt) * (a.k + 1) + a.k; }
    else { const int p = a.lists[(size_t)e * a.S + s0 + tt]; pairs[tt] = p; toks[tt] = p / (a.k + 1); }
  }
  return n;
}

template <int NG>
__global__ __launch_bounds__(256) void k_gateup_items(FfnArgs a) {
  const int wave = threadIdx.x >> 6;
  const int nr = a.n_items[0], nsh = a.n_items[1];
  const int Imax = max(a.I, a.Is);
  const int tr = a.I / kGuPairs, ts = a.Is / kGuPairs;
  const long total = (long)nr * tr + (long)nsh * ts;
  for (long w = (long)blockIdx.x * 4 + wave; w < total; w += (long)gridDim.x * 4) {
    int item, t;
    if (w < (long)nr * tr) { item = (int)(w / tr); t = (int)(w - (long)item * tr); }
    else { const long r = w - (long)nr * tr; item = nr + (int)(r / ts); t = (int)(r - (long)(item - nr) * ts); }
    const int *it = a.items + 3 * (size_t)item;
    int toks[kTB], pairs[kTB];
    const int n = item_tokens(a, it, toks, pairs);
    const uint8_t *ex = it[0] == a.E ? a.shared : expert_ptr(a, it[0]);
    if (!ex) { poison_h(a, n, pairs, t * kGuPairs, Imax); continue; }
    gateup_tile<NG, false>(a, ex + (size_t)t * gu_tile_bytes(a.H), n, toks, pairs, t * kGuPairs, Imax, nullptr, nullptr);
  }
}

template <int NGD>
__global__ __launch_bounds__(256) void k_down_items(FfnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nr = a.n_items[0], nsh = a.n_items[1];
  const int Imax = max(a.I, a.Is);
  const int nt = a.H / kDnRows;
  const long total = (long)(nr + nsh) * nt;
  for (long w = (long)blockIdx.x * 4 + wave; w < total; w += (long)gridDim.x * 4) {
    const int item = (int)(w / nt), rt = (int)(w - (long)item * nt);
    const int *it = a.items + 3 * (size_t)item;
    int toks[kTB], pairs[kTB];
    const int n = item_tokens(a, it, toks, pairs);
    const bool sh = it[0] == a.E;
    const uint8_t *ex = sh ? a.shared : expert_ptr(a, it[0]);
    const int inter = sh ? a.Is : a.I;
    if (!ex) {
      if (lane < kDnRows)
        for (int tt = 0; tt < n; ++tt) a.part[(size_t)pairs[tt] * a.H + rt * kDnRows + lane] = __builtin_nanf("");
      continue;
    }
    down_tile<NGD>(a, ex + down_offset(a.H, inter) + (size_t)rt * dn_tile_bytes(inter), inter, n, pairs, Imax,
                   a.part + (size_t)rt * kDnRows, a.H);
  }
}

// y[t, c] = sum_j w[t, j] * part[t, j, c] (route order) + part[t, k, c]; a token
// whose idx row is out of range or repeats an expert gets NaN.
__global__ __launch_bounds__(256) void k_combine(FfnArgs a) {
  __shared__ int bad;
  const int t = blockIdx.y;
  if (threadIdx.x == 0) {
    int b = 0;
    for (int j = 0; j < a.k; ++j) {
      const int e = a.idx[t * a.k + j];
      b |= (e < 0 || e >= a.E);
      for (int i = 0; i < j; ++i) b |= a.idx[t * a.k + i] == e;
    }
    bad = b;
  }
  __syncthreads();
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= a.H) return;
  float acc = 0.f;
  for (int j = 0; j < a.k; ++j) acc = fmaf(a.w[t * a.k + j], a.part[((size_t)t * (a.k + 1) + j) * a.H + c], acc);
  if (a.Is > 0) acc += a.part[((size_t)t * (a.k + 1) + a.k) * a.H + c];
  a.y[(size_t)t * a.H + c] = bad ? __builtin_nanf("") : acc;
}

template <int NG>
hipError_t gateup_small_ng(const FfnArgs &a, hipStream_t st, int grid) {
  const size_t lds = (size_t)a.S * a.H * sizeof(float) + (size_t)a.S * (a.H / kGroup) * sizeof(float);
  ProfScope ps("gateup_small", st);
  if (lds <= 48 * 1024)
    hipLaunchKernelGGL((k_gateup_small<NG, true>), dim3(grid), dim3(kGuWaves * 64), lds, st, a);
  else
    hipLaunchKernelGGL((k_gateup_small<NG, false>), dim3(grid), dim3(kGuWaves * 64), 0, st, a);
  return hipGetLastError();
}

int ceil_groups(int K) { return (K / kGroup + 63) / 64; }

}  // namespace

hipError_t launch_ffn_small(const FfnArgs &a, hipStream_t st) {
  const int Umax = std::min(a.S * a.k, a.E);
  const long tiles = (long)Umax * (a.I / kGuPairs) + a.Is / kGuPairs;
  const int grid = (int)((tiles + kGuWaves - 1) / kGuWaves);
  hipError_t e;
  switch (ceil_groups(a.H)) {
    case 1: e = gateup_small_ng<1>(a, st, grid); break;
    case 2: e = gateup_small_ng<2>(a, st, grid); break;
    case 3: e = gateup_small_ng<3>(a, st, grid); break;
    default: e = gateup_small_ng<4>(a, st, grid); break;
  }
  if (e != hipSuccess) return e;
  const int nw = std::min(Umax + 1, 16);
  dim3 g2(a.H / kDnRows), b2(64 * nw);
  ProfScope ps("down_small", st);
  switch (ceil_groups(std::max(a.I, a.Is))) {
    case 1: hipLaunchKernelGGL(k_down_small<1>, g2, b2, 0, st, a); break;
    case 2: hipLaunchKernelGGL(k_down_small<2>, g2, b2, 0, st, a); break;
    case 3: hipLaunchKernelGGL(k_down_small<3>, g2, b2, 0, st, a); break;
    default: hipLaunchKernelGGL(k_down_small<4>, g2, b2, 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_ffn_large(const FfnArgs &a, hipStream_t st) {
  {
    ProfScope ps("bucket", st);
    hipLaunchKernelGGL(k_bucket, dim3(a.E), dim3(256), 0, st, a);
  }
  {
    ProfScope ps("schedule", st);
    hipLaunchKernelGGL(k_schedule, dim3(1), dim3(1024), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long tiles_max = (long)a.max_items * (std::max(a.I, a.Is) / kGuPairs);
  const int grid = (int)std::min<long>((tiles_max + 3) / 4, 8192);
  ProfScope ps1("gateup_items", st);
  switch (ceil_groups(a.H)) {
    case 1: hipLaunchKernelGGL(k_gateup_items<1>, dim3(grid), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL(k_gateup_items<2>, dim3(grid), dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL(k_gateup_items<3>, dim3(grid), dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL(k_gateup_items<4>, dim3(grid), dim3(256), 0, st, a); break;
  }
  const long dtiles = (long)a.max_items * (a.H / kDnRows);
  const int g2 = (int)std::min<long>((dtiles + 3) / 4, 8192);
  ProfScope ps2("down_items", st);
  switch (ceil_groups(std::max(a.I, a.Is))) {
    case 1: hipLaunchKernelGGL(k_down_items<1>, dim3(g2), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL(k_down_items<2>, dim3(g2), dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL(k_down_items<3>, dim3(g2), dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL(k_down_items<4>, dim3(g2), dim3(256), 0, st, a); break;
  }
  {
    ProfScope ps3("combine", st);
    hipLaunchKernelGGL(k_combine, dim3((a.H + 255) / 256, a.S), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace moe
