// Many-token experts: grouped int4 x bf16 GEMM on the matrix cores (gfx950
// v_mfma_f32_16x16x32_bf16), used for experts that received at least
// mfma_min_tokens tokens of a batch (and for the shared expert when the batch
// is that large).
//
// Method: "GLM-5.2 on a 32 GB Mac - native MLX port of the Colibri hierarchy",
// "Prefill" (int4 experts dequantised to bf16 and contracted on the matrix
// units for a batch of tokens; the threshold on tokens per expert separates
// this from the per-token GEMV path).  Weights are the slot layout of the
// packer: gate/up row tiles (rows g0 u0 g1 u1 ... of four features, fp16
// scale per row and group of 32) and down row tiles of eight output rows.
//
// Tiles: a workgroup (4 waves) owns up to 128 token rows of one expert's list
// (kMT; wave w takes rows 32w .. 32w+31) and 64 output columns (kNT).  One
// MFMA contracts exactly one quantisation group (K = 32), so each lane's B
// fragment carries a single scale.  Per group the 64 x 32 B tile is
// dequantised once by the whole workgroup (8 values per thread: exact n*s - 8s
// in fp32, then round-to-nearest-even to bf16) into LDS and read by all four
// waves; A fragments (token rows, 8 consecutive K per lane) come straight from
// global memory.  The next group's weights and activations are loaded while
// the current group's MFMAs run; one barrier per group (double-buffered B).
//
// Gate/up: column c of an N tile is tile row c % 8 of gate/up tile c / 8, so
// gate and up of a feature sit in adjacent lanes of the accumulator layout;
// the epilogue forms h = silu(g) * u there and stores it (fp32) for the down
// GEMM, which rounds it to bf16 as its A operand.  Down: columns are output
// rows of Wd; results go to the per-(token, rank) partials that the combine
// sums in route order.
#include "dot.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMT = kMfmaTileTokens;  // token rows per workgroup tile
constexpr int kNT = 64;               // output columns per workgroup tile
constexpr int kBStride = 80;          // bytes per column of an LDS B stage (64 + 16 padding: no bank conflicts)
constexpr int kBStage = kNT * kBStride;

__device__ inline uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// Eight int4 weights (slot layout: two's-complement nibbles, element 2j in the
// low nibble of byte j) times their scale, as eight bf16 (RNE).  With the
// offset-binary nibble n = q + 8, n * s - 8 s = q * s is exact in fp32 (a 4-bit
// times an 11-bit significand), so the only rounding is the final one to bf16.
__device__ inline uint4 dequant8(uint32_t w, float s) {
  const uint32_t u = w ^ 0x88888888u;
  const uint32_t lo = u & 0x0F0F0F0Fu, hi = (u >> 4) & 0x0F0F0F0Fu;
  const float m8 = -8.0f * s;
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = fmaf((float)((lo >> (8 * j)) & 0xFFu), s, m8);
    v[2 * j + 1] = fmaf((float)((hi >> (8 * j)) & 0xFFu), s, m8);
  }
  return make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7]));
}

// Eight consecutive activations, raw: bf16 bits, or fp32 values that become
// bf16 (RNE) only where they are used, so that a prefetch does not wait.
template <bool ABF>
struct ARaw;
template <>
struct ARaw<true> {
  uint4 v;
  __device__ inline void load(const void *base, size_t off) { v = ldg<uint4>((const uint16_t *)base + off); }
  __device__ inline bf16x8 get() const { return __builtin_bit_cast(bf16x8, v); }
};
template <>
struct ARaw<false> {
  float4 p, q;
  __device__ inline void load(const void *base, size_t off) {
    p = ldg<float4>((const float *)base + off);
    q = ldg<float4>((const float *)base + off + 4);
  }
  __device__ inline bf16x8 get() const {
    return __builtin_bit_cast(
        bf16x8, make_uint4(pack_bf16(p.x, p.y), pack_bf16(p.z, p.w), pack_bf16(q.x, q.y), pack_bf16(q.z, q.w)));
  }
};

struct MTile {
  int e, s0, n;  // expert (E = shared), first position in its list, rows
};

__device__ inline MTile mtile_of(const FfnArgs &a, int m) {
  const int *t = a.mtiles + 3 * (size_t)m;
  return MTile{t[0], t[1], t[2]};
}

// Token and (token, rank) pair of row j of a tile.
__device__ inline void tile_rows(const FfnArgs &a, const MTile &mt, int *s_tok, int *s_pair) {
  for (int j = threadIdx.x; j < kMT; j += blockDim.x) {
    const int jj = min(j, mt.n - 1);
    int p, t;
    if (mt.e == a.E) {
      t = mt.s0 + jj;
      p = t * (a.k + 1) + a.k;
    } else {
      p = ldg<int>(a.lists + (size_t)mt.e * a.S + mt.s0 + jj);
      t = p / (a.k + 1);
    }
    s_tok[j] = t;
    s_pair[j] = p;
  }
}

// The grouped GEMM main loop shared by gate/up and down.  For group g the B
// column c (0..63) reads 32 nibbles at colp[c] + 16 g and its scale at
// sclp[c] + 16 g (pointers precomputed per column in LDS); A row r of this
// wave's M block mb is arow(mb) + 32 g + octet*8 elements.
struct GemmAcc {
  f32x4 acc[2][4];  // [M block of 16 rows][N block of 16 columns]
};

template <bool ABF>
__device__ inline void gemm_loop(GemmAcc &C, int ng, const uint8_t *const *s_colp, const uint8_t *const *s_sclp,
                                 uint8_t *s_b, const void *abase, const size_t *arow, int lane) {
  const int tid = threadIdx.x;
  const int bc = tid >> 2, bo = tid & 3;  // this thread's B column and K octet for dequantisation
  const uint8_t *colp = s_colp[bc];
  const uint8_t *sclp = s_sclp[bc];
  const int oct = lane >> 4;  // this lane's K octet in A and B fragments
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) C.acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // prologue: group 0
  {
    const uint32_t w = ldg<uint32_t>(colp + bo * 4);
    const float s = half_bits_to_float(ldg<uint16_t>(sclp));
    *(uint4 *)(s_b + bc * kBStride + bo * 16) = dequant8(w, s);
  }
  ARaw<ABF> A[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) A[mb].load(abase, arow[mb] + oct * 8);
  __syncthreads();
  for (int g = 0; g < ng; ++g) {
    const int gn = min(g + 1, ng - 1);  // unconditional prefetch (the last one repeats)
    const uint32_t wn = ldg<uint32_t>(colp + (size_t)gn * 16 + bo * 4);
    const uint16_t sn = ldg<uint16_t>(sclp + (size_t)gn * 16);
    ARaw<ABF> An[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) An[mb].load(abase, arow[mb] + (size_t)gn * 32 + oct * 8);
    const uint8_t *sb = s_b + (g & 1) * kBStage;
    bf16x8 B[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      B[nb] = __builtin_bit_cast(bf16x8, *(const uint4 *)(sb + (nb * 16 + (lane & 15)) * kBStride + oct * 16));
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const bf16x8 a8 = A[mb].get();
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        C.acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, B[nb], C.acc[mb][nb], 0, 0, 0);
    }
    *(uint4 *)(s_b + ((g + 1) & 1) * kBStage + bc * kBStride + bo * 16) = dequant8(wn, half_bits_to_float(sn));
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) A[mb] = An[mb];
    __syncthreads();
  }
}

// Gate/up for one (M tile, N tile of 32 features): h[pair][feature] = silu(g) * u.
__global__ __launch_bounds__(256) void k_gu_mfma(FfnArgs a) {
  __shared__ __align__(16) uint8_t s_b[2 * kBStage];
  __shared__ const uint8_t *s_colp[kNT];
  __shared__ const uint8_t *s_sclp[kNT];
  __shared__ int s_tok[kMT], s_pair[kMT];
  const int m = blockIdx.x;
  const int n_mt = a.n_items[2] + a.n_items[3];
  if (m >= n_mt) return;
  const MTile mt = mtile_of(a, m);
  const bool sh = mt.e == a.E;
  const int inter = sh ? a.Is : a.I;
  const int nt = blockIdx.y;
  if (nt * (kNT / 2) >= inter) return;
  const uint8_t *ex = sh ? a.shared : expert_ptr(a, mt.e);
  if (!ex) return;  // the down GEMM poisons this tile's rows
  const int Imax = max(a.I, a.Is);
  const size_t gtb = gu_tile_bytes(a.H);
  if (threadIdx.x < kNT) {
    const int c = threadIdx.x;
    const uint8_t *tile = ex + (size_t)(nt * 8 + c / 8) * gtb;
    s_colp[c] = tile + (size_t)(c % 8) * (a.H / 2);
    s_sclp[c] = tile + (size_t)kGuRows * (a.H / 2) + 2 * (c % 8);
  }
  tile_rows(a, mt, s_tok, s_pair);
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  size_t arow[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) arow[mb] = (size_t)s_tok[wave * 32 + mb * 16 + (lane & 15)] * a.H;
  GemmAcc C;
  if (a.x_bf16)
    gemm_loop<true>(C, a.H / kGroup, s_colp, s_sclp, s_b, a.x, arow, lane);
  else
    gemm_loop<false>(C, a.H / kGroup, s_colp, s_sclp, s_b, a.x, arow, lane);
  // epilogue: even columns are gate, the next lane holds the matching up
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gv = C.acc[mb][nb][i];
        const float uv = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(gv), 0xB1, 0xF, 0xF, false));
        const int j = wave * 32 + mb * 16 + (lane >> 4) * 4 + i;
        const int c = nb * 16 + (lane & 15);
        if ((c & 1) == 0 && j < mt.n) {
          const int f = nt * (kNT / 2) + (c / 8) * kGuPairs + (c % 8) / 2;
          a.h[(size_t)s_pair[j] * Imax + f] = gv / (1.0f + expf(-gv)) * uv;
        }
      }
}

// Down for one (M tile, N tile of 64 output rows): part[pair][row] = Wd h.
__global__ __launch_bounds__(256) void k_dn_mfma(FfnArgs a) {
  __shared__ __align__(16) uint8_t s_b[2 * kBStage];
  __shared__ const uint8_t *s_colp[kNT];
  __shared__ const uint8_t *s_sclp[kNT];
  __shared__ int s_tok[kMT], s_pair[kMT];
  const int m = blockIdx.x;
  const int n_mt = a.n_items[2] + a.n_items[3];
  if (m >= n_mt) return;
  const MTile mt = mtile_of(a, m);
  const bool sh = mt.e == a.E;
  const int inter = sh ? a.Is : a.I;
  const int n0 = blockIdx.y * kNT;
  const uint8_t *ex = sh ? a.shared : expert_ptr(a, mt.e);
  tile_rows(a, mt, s_tok, s_pair);
  if (!ex) {
    __syncthreads();
    for (int i = threadIdx.x; i < mt.n * kNT; i += blockDim.x) {
      const int j = i / kNT, n = n0 + i % kNT;
      if (n < a.H) a.part[(size_t)s_pair[j] * a.H + n] = __builtin_nanf("");
    }
    return;
  }
  const int Imax = max(a.I, a.Is);
  if (threadIdx.x < kNT) {
    const int n = min(n0 + (int)threadIdx.x, a.H - 1);  // columns past H read row H-1 and are not stored
    const uint8_t *tile = ex + down_offset(a.H, inter) + (size_t)(n / kDnRows) * dn_tile_bytes(inter);
    s_colp[threadIdx.x] = tile + (size_t)(n % kDnRows) * (inter / 2);
    s_sclp[threadIdx.x] = tile + (size_t)kDnRows * (inter / 2) + 2 * (n % kDnRows);
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  size_t arow[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) arow[mb] = (size_t)s_pair[wave * 32 + mb * 16 + (lane & 15)] * Imax;
  GemmAcc C;
  gemm_loop<false>(C, inter / kGroup, s_colp, s_sclp, s_b, a.h, arow, lane);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = wave * 32 + mb * 16 + (lane >> 4) * 4 + i;
        const int n = n0 + nb * 16 + (lane & 15);
        if (j < mt.n && n < a.H) a.part[(size_t)s_pair[j] * a.H + n] = C.acc[mb][nb][i];
      }
}

}  // namespace

hipError_t launch_gu_mfma(const FfnArgs &a, hipStream_t st) {
  if (a.mfma_thr <= 0 || a.max_mtiles <= 0) return hipSuccess;
  ProfScope ps("gateup_mfma", st);
  const int Imax = std::max(a.I, a.Is);
  MOE_LAUNCH(k_gu_mfma, dim3((unsigned)a.max_mtiles, (unsigned)(Imax / (kNT / 2))), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dn_mfma(const FfnArgs &a, hipStream_t st) {
  if (a.mfma_thr <= 0 || a.max_mtiles <= 0) return hipSuccess;
  ProfScope ps("down_mfma", st);
  MOE_LAUNCH(k_dn_mfma, dim3((unsigned)a.max_mtiles, (unsigned)((a.H + kNT - 1) / kNT)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
