// Many-token experts: grouped int4 x bf16 GEMM on the matrix cores (gfx950
// v_mfma_f32_16x16x32_bf16), used for experts that received at least
// mfma_min_tokens tokens of a batch (and for the shared expert when the batch
// is that large).
//
// Method: colibri README, "Experimental Metal backend (Apple Silicon)": the
// large GEMMs of prefill run on the GPU, and a tunable count of rows (here:
// tokens per expert) decides which experts take that path instead of the
// per-token one; "GLM-5.2 on a 32 GB Mac - native MLX port of the Colibri
// hierarchy", "What Colibri is actually doing" item 11 (large prefill GEMMs on
// the GPU).  Dequantising the int4 weights to bf16 for the matrix cores is this
// library's choice, not the pages' (their GPU paths dequantise to f32 and
// multiply-accumulate in f32); it carries its own, wider error bar.  Weights
// are the slot layout of the packer: gate/up row tiles (rows g0 u0 g1 u1 ... of
// four features, fp16 scale per row and group of 32) and down row tiles of
// eight output rows.
//
// Tiles: a workgroup (8 waves) owns up to 256 token rows of one expert's list
// (kMT) and 256 output columns (kNT); wave w computes two 16-row blocks (blocks
// w and w + 8, so that a partial tile's rows spread over all SIMDs) x all 256
// columns.  Every wave reads the whole dequantised B stage from LDS (at this
// wave tile the CU's LDS read bandwidth and its matrix-core time per stage are
// about equal; a 64 x 128 wave tile halves the LDS reads but doubles the
// activation loads and measured slower).  One MFMA contracts exactly one
// quantisation group (K = 32), so each lane's B fragment carries a single
// scale.  A pipeline stage is two groups: the two threads of a B column read its
// contiguous weight bytes of the stage and each dequantises one group (32
// values: n*s - 8s in fp32, exact for fp16 scales, then round-to-nearest-even to
// bf16) into LDS, read by all eight waves; A fragments (token rows, 8
// consecutive K per lane) come straight from global memory.  Weights come from a
// register ring three stages deep for gate/up (two for down), activations one
// stage ahead; one barrier per stage (double-buffered B, 80 KB of LDS).  The
// weight format is a template parameter (row scales: one fp32 scale per column,
// loaded once; int8 weights: 32 bytes per group).
//
// Gate/up: column c of an N tile is tile row c % 8 of gate/up tile c / 8, so
// gate and up of a feature sit in adjacent lanes of the accumulator layout;
// the epilogue forms h = silu(g) * u there and stores it rounded to bf16 (in
// the first half of the row's fp32 storage) as the down GEMM's A operand.  Down: columns are output
// rows of Wd; results go to the per-(token, rank) partials that the combine
// sums in route order.
//
// int8 activations (moe_cfg.act_int8): with fp16 group scales the same tiles
// run over integers on both sides (quantised activation bytes, weight nibbles
// dequantised with scale 1), each group's MFMA starts from zero and its exact
// integer dot is scaled into the accumulators (group_mfma_gs); with row scales
// the integer kernels at the end of this file run v_mfma_i32_16x16x64_i8.
#include "dot.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;             // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMT = kMfmaTileTokens;  // token rows per workgroup tile
constexpr int kNT = 256;              // output columns per workgroup tile
constexpr int kWM = 8;                // row bands of a tile (wave w: band w % kWM)
constexpr int kWN = kWaves / kWM;     // column parts of a tile (wave w: part w / kWM)
constexpr int kMB = kMT / 16 / kWM;   // MFMA row blocks (16 rows) per wave
constexpr int kNB = kNT / 16 / kWN;   // MFMA column blocks (16 columns) per wave
constexpr int kKG = 2;                // quantisation groups (K = 32 each) per pipeline stage
constexpr int kBStride = 80;          // bytes per column of an LDS B group (64 + 16 padding, see below)
// The 16 bytes of padding put the 16-byte fragment reads of eight consecutive
// columns on distinct banks, and the second group of a stage starts 64 bytes
// past the first group's end: the two threads of a column store their groups in
// the same instruction, and without the skew their stores met in the same LDS
// banks (measured: the gate/up GEMM's bank-conflict cycles fell by a quarter).
// The hardware still counts conflict cycles for these 128-bit accesses (about
// four per fragment read, as many in a kernel that only reads fragments): they
// come from how it groups the lanes of wide accesses, not from this layout.
constexpr int kBGroup = kNT * kBStride + 64;
constexpr int kBStage = kKG * kBGroup;
constexpr int kBParts = kThreads / kNT;  // threads that dequantise one column of a group (8 bytes each)
static_assert(kMT == kWM * 16 * kMB && kNT == kWN * 16 * kNB && kKG == 2 && kBParts == kKG, "tile shape");

// Two fp32 values as bf16 (RNE), lo in the low half: one v_cvt_pk_bf16_f32 (two
// scalar conversions would cost a shift and an or on top).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Eight int4 weights (slot layout: two's-complement nibbles, element 2j in the
// low nibble of byte j) times their scale, as eight bf16 (RNE).  With the
// offset-binary nibble n = q + 8, n * s - 8 s = q * s is exact in fp32 (a 4-bit
// times an 11-bit significand), so the only rounding is the final one to bf16.
__device__ inline uint4 dequant8(uint32_t w, float s) {
  const uint32_t u = w ^ 0x88888888u;
  uint32_t lo = u & 0x0F0F0F0Fu, hi = (u >> 4) & 0x0F0F0F0Fu;
  // kept opaque so that each element converts straight from its byte
  // (v_cvt_f32_ubyte1..3) instead of a bit-field extract per element
  asm volatile("" : "+v"(lo), "+v"(hi));
  const float m8 = -8.0f * s;
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = fmaf((float)((lo >> (8 * j)) & 0xFFu), s, m8);
    v[2 * j + 1] = fmaf((float)((hi >> (8 * j)) & 0xFFu), s, m8);
  }
  return make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7]));
}

// Eight int8 weights (two dwords, element 4m+i in byte i of dword m) times the
// row scale, as eight bf16: q * s rounded to fp32, then to bf16 (RNE).
__device__ inline uint4 dequant8_i8(uint32_t w0, uint32_t w1, float s) {
  const uint32_t d[2] = {w0, w1};
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (float)(int8_t)(d[j >> 2] >> (8 * (j & 3))) * s;
  return make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7]));
}

// Eight consecutive activations, raw: bf16 bits (kActBf16), fp32 values that
// become bf16 (RNE) only where they are used, so that a prefetch does not wait
// (kActF32), or the int8 integers of a quantised row (kActI8: exact in bf16,
// the row's scale is applied to the accumulators).
constexpr int kActF32 = 0, kActBf16 = 1, kActI8 = 2;
template <int AK>
struct ARaw;
template <>
struct ARaw<kActBf16> {
  uint4 v;
  __device__ inline void load(const void *base, size_t off) { v = ldg<uint4>((const uint16_t *)base + off); }
  __device__ inline bf16x8 get() const { return __builtin_bit_cast(bf16x8, v); }
};
template <>
struct ARaw<kActF32> {
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
template <>
struct ARaw<kActI8> {
  uint2 v;
  __device__ inline void load(const void *base, size_t off) { v = ldg<uint2>((const int8_t *)base + off); }
  __device__ inline bf16x8 get() const {
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (float)(int8_t)((j < 4 ? v.x : v.y) >> (8 * (j & 3)));
    return __builtin_bit_cast(
        bf16x8, make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7])));
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
// column c (0..kNT-1) reads 32 nibbles at colp[c] + 16 g and its scale at
// sclp[c] + 16 g (pointers precomputed per column in LDS); A row r of this
// wave's M block mb is arow(mb) + 32 g + octet*8 elements.
struct GemmAcc {
  f32x4 acc[kMB][kNB];  // [M block of 16 rows][N block of 16 columns] of this wave
};

// One quantisation group's MFMAs for the first MBV row blocks of this wave:
// A[mb] holds the group's activations of row block mb, sb the group's
// dequantised B columns of this wave.  Each B fragment is read from LDS
// kFragAhead column blocks before its MFMAs; the scheduling groups pin that
// order (left to itself the compiler reads each fragment right before its MFMAs,
// two at a time, and the wave waits out the LDS latency at every column block).
constexpr int kFragAhead = 4;
template <int MBV>
__device__ inline void group_mfma(GemmAcc &C, const bf16x8 (&A)[kMB], const uint8_t *sb, int lane, int oct) {
  auto frag = [&](int n) {
    return __builtin_bit_cast(bf16x8, *(const uint4 *)(sb + (n * 16 + (lane & 15)) * kBStride + oct * 16));
  };
  constexpr int P = kFragAhead;
  bf16x8 B[kNB];
#pragma unroll
  for (int n = 0; n < P; ++n) B[n] = frag(n);
  __builtin_amdgcn_sched_group_barrier(0x100, P, 0);  // DS reads
#pragma unroll
  for (int n = 0; n < kNB; ++n) {
    if (n + P < kNB) B[n + P] = frag(n + P);
#pragma unroll
    for (int mb = 0; mb < MBV; ++mb)
      C.acc[mb][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb], B[n], C.acc[mb][n], 0, 0, 0);
    if (n + P < kNB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, MBV, 0);  // MFMAs
  }
}

// Int8 activations with grouped weight scales: A and B both hold integers
// (|x| <= 127, |q| <= 8, exact in bf16), so one MFMA gives a group's integer dot
// exactly in fp32 (|sum| <= 32 * 127 * 8 < 2^24); it starts from zero, and its
// result times the group's scale is added to the accumulator, column by column
// (one scale per lane and column block).  The scales of the wave's columns come
// from LDS, column n*16 + c of the group at c * kScStride + n.  A block's scaling
// runs kGsLag column blocks behind its MFMAs, so that it does not wait for them.
constexpr int kScStride = 20;  // floats per column residue (16 blocks + 4 padding)
constexpr int kGsLag = 2;
constexpr bool group_scaled(int AK, int WF) { return AK == kActI8 && WF == kWfQ4G32; }
static_assert(kNT / 16 <= kScStride && kScStride % 4 == 0, "scale layout");
template <int MBV>
__device__ inline void group_mfma_gs(GemmAcc &C, const bf16x8 (&A)[kMB], const uint8_t *sb, const float *ssc,
                                     int lane, int oct) {
  auto frag = [&](int n) {
    return __builtin_bit_cast(bf16x8, *(const uint4 *)(sb + (n * 16 + (lane & 15)) * kBStride + oct * 16));
  };
  constexpr int P = kFragAhead, D = kGsLag;
  float sc[kNB];
#pragma unroll
  for (int n4 = 0; n4 < kNB; n4 += 4) {
    const float4 v = *(const float4 *)(ssc + n4);
    sc[n4] = v.x, sc[n4 + 1] = v.y, sc[n4 + 2] = v.z, sc[n4 + 3] = v.w;
  }
  bf16x8 B[kNB];
  f32x4 T[kMB][kNB];
#pragma unroll
  for (int n = 0; n < P; ++n) B[n] = frag(n);
  __builtin_amdgcn_sched_group_barrier(0x100, P + kNB / 4, 0);  // DS reads
#pragma unroll
  for (int n = 0; n < kNB + D; ++n) {
    if (n < kNB) {
      if (n + P < kNB) B[n + P] = frag(n + P);
#pragma unroll
      for (int mb = 0; mb < MBV; ++mb)
        T[mb][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb], B[n], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    }
    if (n >= D) {
#pragma unroll
      for (int mb = 0; mb < MBV; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) C.acc[mb][n - D][i] = fmaf(T[mb][n - D][i], sc[n - D], C.acc[mb][n - D][i]);
    }
    if (n + P < kNB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (n < kNB) __builtin_amdgcn_sched_group_barrier(0x008, MBV, 0);  // MFMAs
    if (n >= D) __builtin_amdgcn_sched_group_barrier(0x002, 4 * MBV, 0);  // scaling
  }
}

template <int AK, int kDepth, int MBV, int WF>
__device__ inline void gemm_loop(GemmAcc &C, int ng, const uint8_t *const *s_colp, const uint8_t *const *s_sclp,
                                 uint8_t *s_b, float *s_gsc, const void *abase, const size_t *arow, int wn,
                                 int lane) {
  constexpr bool kGS = group_scaled(AK, WF);
  const int tid = threadIdx.x;
  // this thread dequantises group kKG s + bp of B column bc: the two lanes of a
  // column read its 32 contiguous nibble bytes of the stage together
  const int bc = tid >> 1, bp = tid & 1;
  const uint8_t *colp = s_colp[bc];
  const uint8_t *sclp = s_sclp[bc];
  const int oct = lane >> 4;  // this lane's K octet in A and B fragments
  const int ns = (ng + kKG - 1) / kKG;  // stages
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) C.acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // a column's scale: per group (fp16, loaded with the group) or per row (fp32, once)
  const float row_sc = WF == kWfQ4G32 ? 0.f : ldg<float>(sclp);
  struct BRaw {
    QGroup<WF> w;
    uint16_t sc;
  };
  auto load_b = [&](int st) {
    const int g = min(st * kKG + bp, ng - 1);
    BRaw r;
    load_group(r.w, colp, g);
    r.sc = WF == kWfQ4G32 ? ldg<uint16_t>(sclp + (size_t)g * 16) : (uint16_t)0;
    return r;
  };
  auto store_b = [&](int buf, const BRaw &r) {
    uint8_t *d = s_b + buf * kBStage + bp * kBGroup + bc * kBStride;
    if constexpr (WF == kWfQ8Row) {
      *(uint4 *)(d) = dequant8_i8(r.w.q[0].x, r.w.q[0].y, row_sc);
      *(uint4 *)(d + 16) = dequant8_i8(r.w.q[0].z, r.w.q[0].w, row_sc);
      *(uint4 *)(d + 32) = dequant8_i8(r.w.q[1].x, r.w.q[1].y, row_sc);
      *(uint4 *)(d + 48) = dequant8_i8(r.w.q[1].z, r.w.q[1].w, row_sc);
    } else {
      float sc = WF == kWfQ4G32 ? half_bits_to_float(r.sc) : row_sc;
      if constexpr (kGS) {  // integers in LDS, the scale beside them (column bc = 16 (bc / 16) + bc % 16)
        s_gsc[((buf * kKG + bp) * 16 + (bc & 15)) * kScStride + (bc >> 4)] = sc;
        sc = 1.0f;
      }
      *(uint4 *)(d) = dequant8(r.w.q[0].x, sc);
      *(uint4 *)(d + 16) = dequant8(r.w.q[0].y, sc);
      *(uint4 *)(d + 32) = dequant8(r.w.q[0].z, sc);
      *(uint4 *)(d + 48) = dequant8(r.w.q[0].w, sc);
    }
  };
  // activations of group gi of stage st (clamped to the last group)
  auto load_a = [&](int st, int gi, ARaw<AK> (&r)[kMB]) {
    const int g = min(st * kKG + gi, ng - 1);
#pragma unroll
    for (int mb = 0; mb < MBV; ++mb) r[mb].load(abase, arow[mb] + (size_t)g * 32 + oct * 8);
  };
  // Rings: the activations of group gi of stage s + 1 are requested right after
  // the MFMAs of group gi of stage s (they come mostly from L2); B of stage s is
  // requested kDepth stages before it is dequantised into LDS (one stage before
  // its MFMAs).  Loads are clamped to the last group, so every one is
  // unconditional; the MFMAs of groups past the last one (an odd group count,
  // padding to a multiple of kDepth stages) are skipped.
  ARaw<AK> aq[kKG][kMB];
  BRaw bq[kDepth];
#pragma unroll
  for (int gi = 0; gi < kKG; ++gi) load_a(0, gi, aq[gi]);
#pragma unroll
  for (int d = 0; d < kDepth; ++d) bq[d] = load_b(d);
  store_b(0, bq[0]);
  bq[0] = load_b(kDepth);
  __syncthreads();
  const int nsp = (ns + kDepth - 1) / kDepth * kDepth;
  for (int st = 0; st < nsp; st += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int s = st + d;
      const uint8_t *sb = s_b + (s & 1) * kBStage + (wn * 16 * kNB) * kBStride;
#pragma unroll
      for (int gi = 0; gi < kKG; ++gi) {
        bf16x8 A[kMB];
#pragma unroll
        for (int mb = 0; mb < MBV; ++mb) A[mb] = aq[gi][mb].get();
        // rows past the tile's end repeat its last row (not stored); groups past
        // the last one (a wave-uniform condition) are skipped
        if (MBV > 0 && s * kKG + gi < ng) {
          if constexpr (kGS)
            group_mfma_gs<MBV>(C, A, sb + gi * kBGroup,
                               s_gsc + (((s & 1) * kKG + gi) * 16 + (lane & 15)) * kScStride + wn * kNB, lane, oct);
          else
            group_mfma<MBV>(C, A, sb + gi * kBGroup, lane, oct);
        }
        load_a(s + 1, gi, aq[gi]);  // after the MFMAs: the slot's registers are free again
      }
      store_b((s + 1) & 1, bq[(d + 1) % kDepth]);
      bq[(d + 1) % kDepth] = load_b(s + 1 + kDepth);
      __syncthreads();
    }
  }
}

// Row block rb (16 rows) of a tile belongs to row band rb % kWM (slot rb /
// kWM), so that a partial tile's valid blocks spread over all bands; a wave
// multiplies only its valid blocks (MBV), every wave dequantises its share of B.
__device__ inline int row_of(int wave, int mb, int r16) { return (wave % kWM + kWM * mb) * 16 + r16; }

template <int AK, int kDepth, int WF>
__device__ inline void gemm_rows(GemmAcc &C, int rows, int ng, const uint8_t *const *s_colp,
                                 const uint8_t *const *s_sclp, uint8_t *s_b, float *s_gsc, const void *abase,
                                 const size_t *arow, int wave, int lane) {
  const int nblk = (rows + 15) / 16, band = wave % kWM, wn = wave / kWM;
  const int mbv = min(kMB, max(0, (nblk - band + kWM - 1) / kWM));  // valid blocks band, band + kWM, ...
  switch (mbv) {
    case 4: if constexpr (kMB >= 4) gemm_loop<AK, kDepth, 4, WF>(C, ng, s_colp, s_sclp, s_b, s_gsc, abase, arow, wn, lane); break;
    case 3: if constexpr (kMB >= 3) gemm_loop<AK, kDepth, 3, WF>(C, ng, s_colp, s_sclp, s_b, s_gsc, abase, arow, wn, lane); break;
    case 2: gemm_loop<AK, kDepth, 2, WF>(C, ng, s_colp, s_sclp, s_b, s_gsc, abase, arow, wn, lane); break;
    case 1: gemm_loop<AK, kDepth, 1, WF>(C, ng, s_colp, s_sclp, s_b, s_gsc, abase, arow, wn, lane); break;
    default: gemm_loop<AK, kDepth, 0, WF>(C, ng, s_colp, s_sclp, s_b, s_gsc, abase, arow, wn, lane); break;
  }
}

// Workgroups go to the 8 XCDs (each with its own L2) round-robin in launch
// order, so block b runs on XCD b % 8.  M tile m is given to XCD m % 8 with all
// its N tiles back to back: the N tiles of an M tile share its activation rows
// and run together in one L2 instead of fetching the rows once per N tile.
constexpr int kXcds = 8;
__device__ inline void tile_of_block(int n_tiles, int &m, int &nt) {
  const int b = blockIdx.x, x = b % kXcds, local = b / kXcds;
  m = (local / n_tiles) * kXcds + x;
  nt = local % n_tiles;
}
inline unsigned tile_blocks(int max_mtiles, int n_tiles) {
  return (unsigned)((max_mtiles + kXcds - 1) / kXcds * kXcds * n_tiles);
}

// Gate/up for one (M tile, N tile of kNT/2 features): h[pair][feature] = silu(g) * u.
// AK = kActI8 (int8 activations with grouped weight scales): A is the tokens'
// quantised integers, g and u are scaled by the token's d, and h is stored in
// fp32 for the per-row quantisation of the down projection's input.
template <int WF, int AK = kActBf16>
__global__ __launch_bounds__(kThreads) void k_gu_mfma(FfnArgs a) {
  __shared__ __align__(16) uint8_t s_b[2 * kBStage];
  __shared__ __align__(16) float s_gsc[group_scaled(AK, WF) ? 2 * kKG * 16 * kScStride : 4];
  __shared__ const uint8_t *s_colp[kNT];
  __shared__ const uint8_t *s_sclp[kNT];
  __shared__ int s_tok[kMT], s_pair[kMT];
  int m, nt;  // features nt*kNT/2 ..
  tile_of_block((2 * max(a.I, a.Is) + kNT - 1) / kNT, m, nt);
  const int n_mt = a.n_items[2] + a.n_items[3];
  if (m >= n_mt) return;
  const MTile mt = mtile_of(a, m);
  const bool sh = mt.e == a.E;
  const int inter = sh ? a.Is : a.I;
  if (nt * (kNT / 2) >= inter) return;
  const uint8_t *ex = sh ? a.shared : expert_ptr(a, mt.e);
  if (!ex) return;  // the down GEMM poisons this tile's rows
  const int Imax = max(a.I, a.Is);
  const size_t gtb = gu_tile_bytes(a.H, WF), rb = row_bytes(a.H, WF);
  if (threadIdx.x < kNT) {
    const int c = threadIdx.x;
    // columns past 2 * inter (a partial last tile) read the last gate/up tile and are not stored
    const int tt = min(nt * (kNT / 8) + c / 8, inter / kGuPairs - 1);
    const uint8_t *tile = ex + (size_t)tt * gtb;
    s_colp[c] = tile + (size_t)(c % 8) * rb;
    s_sclp[c] = tile + (size_t)kGuRows * rb + (WF == kWfQ4G32 ? 2 : 4) * (c % 8);
  }
  tile_rows(a, mt, s_tok, s_pair);
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave / kWM;  // column part
  size_t arow[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) arow[mb] = (size_t)s_tok[row_of(wave, mb, lane & 15)] * a.H;
  GemmAcc C;
  gemm_rows<AK, 3, WF>(C, mt.n, a.H / kGroup, s_colp, s_sclp, s_b, s_gsc,
                       AK == kActI8 ? (const void *)a.xq : a.x_bf16 ? a.x : (const void *)a.xb, arow, wave, lane);
  // epilogue: even columns are gate, the next lane holds the matching up
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = row_of(wave, mb, (lane >> 4) * 4 + i);
        const float gv = AK == kActI8 ? C.acc[mb][nb][i] * ldg<float>(a.dx + s_tok[min(j, mt.n - 1)]) : C.acc[mb][nb][i];
        const float uv = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(gv), 0xB1, 0xF, 0xF, false));
        const int c = wn * 16 * kNB + nb * 16 + (lane & 15);
        const int f = nt * (kNT / 2) + (c / 8) * kGuPairs + (c % 8) / 2;
        if ((c & 1) == 0 && j < mt.n && f < inter) {
          const float hv = gv / (1.0f + expf(-gv)) * uv;
          if constexpr (AK == kActI8) {
            a.h[(size_t)s_pair[j] * Imax + f] = hv;
          } else {
            // bf16 in the first half of the row's fp32 storage: the down GEMM's A operand
            ((__bf16 *)a.h)[(size_t)s_pair[j] * 2 * Imax + f] = (__bf16)hv;
          }
        }
      }
}

// Down for one (M tile, N tile of kNT output rows): part[pair][row] = Wd h.
// AK = kActI8: A is the quantised h rows, the results are scaled by each row's d.
template <int WF, int AK = kActBf16>
__global__ __launch_bounds__(kThreads) void k_dn_mfma(FfnArgs a) {
  __shared__ __align__(16) uint8_t s_b[2 * kBStage];
  __shared__ __align__(16) float s_gsc[group_scaled(AK, WF) ? 2 * kKG * 16 * kScStride : 4];
  __shared__ const uint8_t *s_colp[kNT];
  __shared__ const uint8_t *s_sclp[kNT];
  __shared__ int s_tok[kMT], s_pair[kMT];
  int m, nt;
  tile_of_block((a.H + kNT - 1) / kNT, m, nt);
  const int n_mt = a.n_items[2] + a.n_items[3];
  if (m >= n_mt) return;
  const MTile mt = mtile_of(a, m);
  const bool sh = mt.e == a.E;
  const int inter = sh ? a.Is : a.I;
  const int n0 = nt * kNT;
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
    const size_t rb = row_bytes(inter, WF);
    const uint8_t *tile = ex + down_offset(a.H, inter, WF) + (size_t)(n / kDnRows) * dn_tile_bytes(inter, WF);
    s_colp[threadIdx.x] = tile + (size_t)(n % kDnRows) * rb;
    s_sclp[threadIdx.x] = tile + (size_t)kDnRows * rb + (WF == kWfQ4G32 ? 2 : 4) * (n % kDnRows);
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave / kWM;  // column part
  size_t arow[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
    arow[mb] = (size_t)s_pair[row_of(wave, mb, lane & 15)] * (AK == kActI8 ? Imax : 2 * Imax);
  GemmAcc C;
  gemm_rows<AK, 2, WF>(C, mt.n, inter / kGroup, s_colp, s_sclp, s_b, s_gsc, AK == kActI8 ? (const void *)a.hq : a.h, arow,
                       wave, lane);
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = row_of(wave, mb, (lane >> 4) * 4 + i);
        const int n = n0 + wn * 16 * kNB + nb * 16 + (lane & 15);
        if (j < mt.n && n < a.H)
          a.part[(size_t)s_pair[j] * a.H + n] =
              AK == kActI8 ? C.acc[mb][nb][i] * ldg<float>(a.dh + s_pair[j]) : C.acc[mb][nb][i];
      }
}

// ---- int8 activations with row-scaled weights: integer matrix cores ---------------
// With one scale per weight row and one per activation row, a whole row of K
// products accumulates exactly in int32 (|sum| <= K * 127 * 128 < 2^31 for K <=
// 8192), so the tile runs v_mfma_i32_16x16x64_i8 over int8 activations (the
// quantised rows) and int8 weights (int4 nibbles sign-extended to bytes, or the
// int8 weights themselves) and scales once in the epilogue:
// y = fp32(acc) * d_row * s_col.  Lane layout (checked on the GPU against a host
// matmul): A lane l = (row l % 16, k 16 (l / 16) .. + 15), B lane l = (column
// l % 16, the same k), D as for the bf16 MFMA.  A pipeline stage is K = 64 (two
// quantisation groups, one MFMA per 16 x 16 block); the two threads of a B column
// each write one group's 32 bytes into LDS.
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kBStageI8 = kNT * kBStride;  // one 64-byte column (+ 16 padding) per output column

// Eight int4 weights (two's-complement nibbles, element 2j in the low nibble of
// byte j) as eight int8 in element order: each nibble n becomes the byte
// ((n ^ 8) + 0x78) ^ 0x80 = n - 16 (n >= 8) or n (no carry leaves a byte), then
// the low- and high-nibble bytes are interleaved.
__device__ inline uint2 nib_to_i8(uint32_t w) {
  uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  lo = ((lo ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
  hi = ((hi ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
  return make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u));
}

struct GemmAccI {
  i32x4 acc[kMB][kNB];
};

template <int kDepth, int MBV, int WF>
__device__ inline void gemm_loop_i8(GemmAccI &C, int ng, const uint8_t *const *s_colp, uint8_t *s_b,
                                    const int8_t *abase, const size_t *arow, int wn, int lane) {
  const int tid = threadIdx.x;
  const int bc = tid >> 1, bp = tid & 1;  // this thread writes group 2 st + bp of B column bc
  const uint8_t *colp = s_colp[bc];
  const int kq = lane >> 4;               // this lane's 16-byte quarter of the stage's K = 64
  const int ns = (ng + 1) / 2;            // stages
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) C.acc[mb][nb] = i32x4{0, 0, 0, 0};
  auto load_b = [&](int st) {
    QGroup<WF> r;
    load_group(r, colp, min(st * 2 + bp, ng - 1));
    return r;
  };
  auto store_b = [&](int buf, const QGroup<WF> &r) {
    uint8_t *d = s_b + buf * kBStageI8 + bc * kBStride + bp * 32;
    if constexpr (WF == kWfQ8Row) {
      *(uint4 *)(d) = r.q[0];
      *(uint4 *)(d + 16) = r.q[1];
    } else {
      const uint2 a0 = nib_to_i8(r.q[0].x), a1 = nib_to_i8(r.q[0].y), a2 = nib_to_i8(r.q[0].z),
                  a3 = nib_to_i8(r.q[0].w);
      *(uint4 *)(d) = make_uint4(a0.x, a0.y, a1.x, a1.y);
      *(uint4 *)(d + 16) = make_uint4(a2.x, a2.y, a3.x, a3.y);
    }
  };
  // activations of stage st: this lane's 16 bytes of K (clamped to the last group)
  auto load_a = [&](int st, uint4 (&r)[kMB]) {
    const int g = min(st * 2 + (kq >> 1), ng - 1);
#pragma unroll
    for (int mb = 0; mb < MBV; ++mb) r[mb] = ldg<uint4>(abase + arow[mb] + (size_t)g * 32 + (kq & 1) * 16);
  };
  uint4 aq[kMB];
  QGroup<WF> bq[kDepth];
  load_a(0, aq);
#pragma unroll
  for (int d = 0; d < kDepth; ++d) bq[d] = load_b(d);
  store_b(0, bq[0]);
  bq[0] = load_b(kDepth);
  __syncthreads();
  const int nsp = (ns + kDepth - 1) / kDepth * kDepth;
  for (int st = 0; st < nsp; st += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int s = st + d;
      const uint8_t *sb = s_b + (s & 1) * kBStageI8 + (wn * 16 * kNB) * kBStride;
      // a lane whose group is past the last one (odd group count, padded stages)
      // contributes zero; the masking is needed only in such a stage (uniform)
      if (s * 2 + 1 >= ng) {
        const uint32_t live = s * 2 + (kq >> 1) < ng ? ~0u : 0u;
#pragma unroll
        for (int mb = 0; mb < MBV; ++mb)
          aq[mb] = make_uint4(aq[mb].x & live, aq[mb].y & live, aq[mb].z & live, aq[mb].w & live);
      }
      i32x4 A[kMB];
#pragma unroll
      for (int mb = 0; mb < MBV; ++mb) A[mb] = __builtin_bit_cast(i32x4, aq[mb]);
      load_a(s + 1, aq);
      if (MBV > 0) {
#pragma unroll
        for (int n4 = 0; n4 < kNB; n4 += 4) {
          i32x4 B[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            B[q] = __builtin_bit_cast(i32x4, *(const uint4 *)(sb + ((n4 + q) * 16 + (lane & 15)) * kBStride + kq * 16));
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int mb = 0; mb < MBV; ++mb)
              C.acc[mb][n4 + q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[mb], B[q], C.acc[mb][n4 + q], 0, 0, 0);
          asm volatile("" ::: "memory");
        }
      }
      store_b((s + 1) & 1, bq[(d + 1) % kDepth]);
      bq[(d + 1) % kDepth] = load_b(s + 1 + kDepth);
      __syncthreads();
    }
  }
}

template <int kDepth, int WF>
__device__ inline void gemm_rows_i8(GemmAccI &C, int rows, int ng, const uint8_t *const *s_colp, uint8_t *s_b,
                                    const int8_t *abase, const size_t *arow, int wave, int lane) {
  const int nblk = (rows + 15) / 16, band = wave % kWM, wn = wave / kWM;
  const int mbv = min(kMB, max(0, (nblk - band + kWM - 1) / kWM));
  switch (mbv) {
    case 4: if constexpr (kMB >= 4) gemm_loop_i8<kDepth, 4, WF>(C, ng, s_colp, s_b, abase, arow, wn, lane); break;
    case 3: if constexpr (kMB >= 3) gemm_loop_i8<kDepth, 3, WF>(C, ng, s_colp, s_b, abase, arow, wn, lane); break;
    case 2: gemm_loop_i8<kDepth, 2, WF>(C, ng, s_colp, s_b, abase, arow, wn, lane); break;
    case 1: gemm_loop_i8<kDepth, 1, WF>(C, ng, s_colp, s_b, abase, arow, wn, lane); break;
    default: gemm_loop_i8<kDepth, 0, WF>(C, ng, s_colp, s_b, abase, arow, wn, lane); break;
  }
}

// Gate/up with int8 activations: h[pair][feature] = silu(g) * u in fp32 (the
// down projection quantises h per row).
template <int WF>
__global__ __launch_bounds__(kThreads) void k_gu_mfma_i8(FfnArgs a) {
  __shared__ __align__(16) uint8_t s_b[2 * kBStageI8];
  __shared__ const uint8_t *s_colp[kNT];
  __shared__ float s_cs[kNT];
  __shared__ int s_tok[kMT], s_pair[kMT];
  int m, nt;
  tile_of_block((2 * max(a.I, a.Is) + kNT - 1) / kNT, m, nt);
  const int n_mt = a.n_items[2] + a.n_items[3];
  if (m >= n_mt) return;
  const MTile mt = mtile_of(a, m);
  const bool sh = mt.e == a.E;
  const int inter = sh ? a.Is : a.I;
  if (nt * (kNT / 2) >= inter) return;
  const uint8_t *ex = sh ? a.shared : expert_ptr(a, mt.e);
  if (!ex) return;  // the down GEMM poisons this tile's rows
  const int Imax = max(a.I, a.Is);
  const size_t gtb = gu_tile_bytes(a.H, WF), rb = row_bytes(a.H, WF);
  if (threadIdx.x < kNT) {
    const int c = threadIdx.x;
    const int tt = min(nt * (kNT / 8) + c / 8, inter / kGuPairs - 1);
    const uint8_t *tile = ex + (size_t)tt * gtb;
    s_colp[c] = tile + (size_t)(c % 8) * rb;
    s_cs[c] = ldg<float>(tile + (size_t)kGuRows * rb + 4 * (c % 8));
  }
  tile_rows(a, mt, s_tok, s_pair);
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave / kWM;
  size_t arow[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) arow[mb] = (size_t)s_tok[row_of(wave, mb, lane & 15)] * a.H;
  GemmAccI C;
  gemm_rows_i8<3, WF>(C, mt.n, a.H / kGroup, s_colp, s_b, a.xq, arow, wave, lane);
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = row_of(wave, mb, (lane >> 4) * 4 + i);
      const float dxr = ldg<float>(a.dx + s_tok[min(j, mt.n - 1)]);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const int c = wn * 16 * kNB + nb * 16 + (lane & 15);
        const float gv = (float)C.acc[mb][nb][i] * dxr * s_cs[c];
        const float uv = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(gv), 0xB1, 0xF, 0xF, false));
        const int f = nt * (kNT / 2) + (c / 8) * kGuPairs + (c % 8) / 2;
        if ((c & 1) == 0 && j < mt.n && f < inter) a.h[(size_t)s_pair[j] * Imax + f] = gv / (1.0f + expf(-gv)) * uv;
      }
    }
}

// Down with int8 activations (the quantised h rows): part[pair][row] = acc * dh * s.
template <int WF>
__global__ __launch_bounds__(kThreads) void k_dn_mfma_i8(FfnArgs a) {
  __shared__ __align__(16) uint8_t s_b[2 * kBStageI8];
  __shared__ const uint8_t *s_colp[kNT];
  __shared__ float s_cs[kNT];
  __shared__ int s_tok[kMT], s_pair[kMT];
  int m, nt;
  tile_of_block((a.H + kNT - 1) / kNT, m, nt);
  const int n_mt = a.n_items[2] + a.n_items[3];
  if (m >= n_mt) return;
  const MTile mt = mtile_of(a, m);
  const bool sh = mt.e == a.E;
  const int inter = sh ? a.Is : a.I;
  const int n0 = nt * kNT;
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
    const int n = min(n0 + (int)threadIdx.x, a.H - 1);
    const size_t rb = row_bytes(inter, WF);
    const uint8_t *tile = ex + down_offset(a.H, inter, WF) + (size_t)(n / kDnRows) * dn_tile_bytes(inter, WF);
    s_colp[threadIdx.x] = tile + (size_t)(n % kDnRows) * rb;
    s_cs[threadIdx.x] = ldg<float>(tile + (size_t)kDnRows * rb + 4 * (n % kDnRows));
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave / kWM;
  size_t arow[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) arow[mb] = (size_t)s_pair[row_of(wave, mb, lane & 15)] * Imax;
  GemmAccI C;
  gemm_rows_i8<2, WF>(C, mt.n, inter / kGroup, s_colp, s_b, a.hq, arow, wave, lane);
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = row_of(wave, mb, (lane >> 4) * 4 + i);
      const float dhr = ldg<float>(a.dh + s_pair[min(j, mt.n - 1)]);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const int c = wn * 16 * kNB + nb * 16 + (lane & 15);
        const int n = n0 + c;
        if (j < mt.n && n < a.H) a.part[(size_t)s_pair[j] * a.H + n] = (float)C.acc[mb][nb][i] * dhr * s_cs[c];
      }
    }
}

// fp32 activations -> bf16 (RNE), eight per thread.
__global__ __launch_bounds__(256) void k_x_to_bf16(const float *x, uint16_t *xb, long n8) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const float4 p = ldg<float4>(x + 8 * i), q = ldg<float4>(x + 8 * i + 4);
  stg<uint4>(xb + 8 * i, make_uint4(pack_bf16(p.x, p.y), pack_bf16(p.z, p.w), pack_bf16(q.x, q.y), pack_bf16(q.z, q.w)));
}

}  // namespace

hipError_t launch_gu_mfma(const FfnArgs &a, hipStream_t st) {
  if (a.mfma_thr <= 0 || a.max_mtiles <= 0) return hipSuccess;
  if (a.act_q) {  // int8 activations: integer tiles for row scales, bf16 tiles over the integers for group scales
    ProfScope ps("gateup_mfma", st);
    const dim3 g(tile_blocks(a.max_mtiles, (2 * std::max(a.I, a.Is) + kNT - 1) / kNT));
    if (a.wf == kWfQ8Row) MOE_LAUNCH(k_gu_mfma_i8<kWfQ8Row>, g, dim3(kThreads), 0, st, a);
    else if (a.wf == kWfQ4Row) MOE_LAUNCH(k_gu_mfma_i8<kWfQ4Row>, g, dim3(kThreads), 0, st, a);
    else MOE_LAUNCH((k_gu_mfma<kWfQ4G32, kActI8>), g, dim3(kThreads), 0, st, a);
    return hipGetLastError();
  }
  if (!a.x_bf16) {
    ProfScope ps("x_bf16", st);
    const long n8 = (long)a.S * a.H / 8;
    MOE_LAUNCH(k_x_to_bf16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, (const float *)a.x, a.xb, n8);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ProfScope ps("gateup_mfma", st);
  const int Imax = std::max(a.I, a.Is);
  const dim3 g(tile_blocks(a.max_mtiles, (2 * Imax + kNT - 1) / kNT));
  switch (a.wf) {
    case kWfQ4Row: MOE_LAUNCH(k_gu_mfma<kWfQ4Row>, g, dim3(kThreads), 0, st, a); break;
    case kWfQ8Row: MOE_LAUNCH(k_gu_mfma<kWfQ8Row>, g, dim3(kThreads), 0, st, a); break;
    default: MOE_LAUNCH(k_gu_mfma<kWfQ4G32>, g, dim3(kThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_dn_mfma(const FfnArgs &a, hipStream_t st) {
  if (a.mfma_thr <= 0 || a.max_mtiles <= 0) return hipSuccess;
  ProfScope ps("down_mfma", st);
  if (a.act_q) {
    const dim3 g(tile_blocks(a.max_mtiles, (a.H + kNT - 1) / kNT));
    if (a.wf == kWfQ8Row) MOE_LAUNCH(k_dn_mfma_i8<kWfQ8Row>, g, dim3(kThreads), 0, st, a);
    else if (a.wf == kWfQ4Row) MOE_LAUNCH(k_dn_mfma_i8<kWfQ4Row>, g, dim3(kThreads), 0, st, a);
    else MOE_LAUNCH((k_dn_mfma<kWfQ4G32, kActI8>), g, dim3(kThreads), 0, st, a);
    return hipGetLastError();
  }
  const dim3 g(tile_blocks(a.max_mtiles, (a.H + kNT - 1) / kNT));
  switch (a.wf) {
    case kWfQ4Row: MOE_LAUNCH(k_dn_mfma<kWfQ4Row>, g, dim3(kThreads), 0, st, a); break;
    case kWfQ8Row: MOE_LAUNCH(k_dn_mfma<kWfQ8Row>, g, dim3(kThreads), 0, st, a); break;
    default: MOE_LAUNCH(k_dn_mfma<kWfQ4G32>, g, dim3(kThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace moe
