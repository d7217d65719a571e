// Internal definitions shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kGroup = 32;       // int4 elements per fp16 scale (along the contraction)
constexpr int kGuRows = 8;       // rows per gate/up tile: gate r, up r for 4 consecutive r
constexpr int kGuPairs = 4;      // feature rows per gate/up tile
constexpr int kDnRows = 8;       // rows per down tile
constexpr int kSmallS = 4;       // batches up to this size take the decode path
constexpr int kMfmaTileTokens = 256;  // token rows per matrix-core tile (many-token experts)
constexpr int kMaxK = 16;        // top_k limit
constexpr int kMaxE = 1024;      // n_experts limit
constexpr int kMaxG = 64;        // n_group limit

// Workspace header (first kWsSyncBytes bytes): two magic words written by
// moe_workspace_init (the router refuses a workspace without them), then zeros.
constexpr int kWsSyncBytes = 256;
constexpr int kWsPlanBytes = 4096;  // the eptr region: k pointers, or a small batch's union and pointers
constexpr uint32_t kWsMagic0 = 0x6D6F6534u, kWsMagic1 = 0x77733031u;

// ---- slot layout of one packed expert (inter = I, hidden = H) -------------
// gate/up: I/4 tiles.  Tile t holds 8 rows, in order (g 4t, u 4t, g 4t+1, u 4t+1,
// ..., g 4t+3, u 4t+3), then the tile's scales.
// down: H/8 tiles.  Tile t holds rows 8t..8t+7, then the tile's scales.
// A row of K elements takes K/2 bytes (int4) or K bytes (int8).  Scales of a
// tile: MOE_WF_Q4_G32 [K/32 groups][8 rows] fp16; the row-scaled formats 8 fp32
// in the tile's row order.
// int4 element order within a row is the interchange order (element 2j in the
// low nibble of byte j), but each nibble holds the value in two's complement
// (interchange nibble XOR 8), the operand format of v_dot8_i32_i4; int8
// elements are the interchange bytes (two's complement, v_dot4_i32_i8's).
constexpr int kWfQ4G32 = MOE_WF_Q4_G32, kWfQ4Row = MOE_WF_Q4_ROW, kWfQ8Row = MOE_WF_Q8_ROW;
__host__ __device__ constexpr int64_t row_bytes(int K, int wf) { return wf == kWfQ8Row ? K : K / 2; }
// bytes of one 32-element group of a row: 16 (int4) or 32 (int8)
__host__ __device__ constexpr int group_bytes(int wf) { return wf == kWfQ8Row ? 32 : 16; }
__host__ __device__ constexpr int64_t tile_scale_bytes(int K, int wf) {
  return wf == kWfQ4G32 ? (int64_t)(K / kGroup) * 8 * 2 : 8 * 4;
}
__host__ __device__ inline int64_t gu_tile_bytes(int H, int wf) { return (int64_t)kGuRows * row_bytes(H, wf) + tile_scale_bytes(H, wf); }
__host__ __device__ inline int64_t dn_tile_bytes(int I, int wf) { return (int64_t)kDnRows * row_bytes(I, wf) + tile_scale_bytes(I, wf); }
__host__ __device__ inline int64_t down_offset(int H, int I, int wf) { return (int64_t)(I / kGuPairs) * gu_tile_bytes(H, wf); }
__host__ __device__ inline int64_t packed_bytes(int H, int I, int wf) {
  return down_offset(H, I, wf) + (int64_t)(H / kDnRows) * dn_tile_bytes(I, wf);
}
inline int64_t slot_stride(int H, int I, int wf) { return (packed_bytes(H, I, wf) + 4095) / 4096 * 4096; }

// ---- kernel arguments -------------------------------------------------------
struct RouteArgs {
  int H, E, G, Gk, k, S, x_bf16, norm;
  float rsf;
  const void *x;
  const float *W;
  const float *bias;
  double *logits;  // [S, E] (many tokens)
  double *scores;  // [S, E] sigmoid of the logit (few tokens)
  float *keys;     // [S, E] fp32 selection key, sigmoid + bias (few tokens)
  int32_t *idx;
  float *w;
  uint32_t *sync;  // workspace header
};

struct FfnArgs {
  int H, E, k, I, Is, S, x_bf16;
  int wf;  // moe_weight_format
  int act_q;  // int8 activations: x and h rows quantised (xq/dx, hq/dh) before their matmuls
  const void *x;
  const int32_t *idx;
  const float *w;
  const uint8_t *base;
  int64_t slot_bytes;
  const int32_t *table;
  int32_t n_slots;
  const uint32_t *gen;       // [E] generation each expert's slot held when the table was published (null: no check)
  const uint32_t *slot_gen;  // [n_slots] the slots' current generations
  const uint8_t *shared;
  float *y;
  // workspace views
  float *h;        // [S * (k+1), max(I, Is)] fp32 hidden activations
  float *part;     // [S, k+1, H] fp32 per-(token, rank) expert outputs (large-batch path)
  int32_t *lists;  // [E+1, S] token lists per expert (large-batch path), entry = token*(k+1)+rank
  int32_t *counts; // [E+1]
  int32_t *items;  // GEMV work items {expert, list position, tokens} (large-batch path)
  int32_t *n_items;  // [0] routed items, [1] shared items, [2] routed MFMA tiles, [3] shared MFMA tiles
  int32_t max_items;
  int32_t *mtiles;   // MFMA tiles {expert, list position, rows <= kMfmaTileTokens}
  uint16_t *xb;      // [S, H] bf16 copy of fp32 x (matrix-core path)
  int32_t max_mtiles;
  int32_t mfma_thr;  // experts with at least this many tokens use the matrix cores (0: never)
  // activations in limb form (see dot.h): [rows][groups][24] words and [rows][groups] factors
  uint32_t *xl;    // x: S rows of H/32 groups
  float *xf;
  uint32_t *hl;    // h: S*(k+1) rows of Imax/32 groups
  float *hf;
  // int8 activations: quantised rows and their scales
  int8_t *xq;      // [S, H]
  float *dx;       // [S]
  int8_t *hq;      // [S * (k+1), Imax]
  float *dh;       // [S * (k+1)]
  // one-token decode path
  // one-token calls: [k] routed experts' packed weights (0: not resident), resolved by the gate/up
  // kernel; two to four tokens: the batch union and its experts' weights, as the gate/up kernel
  // derived them (kWsPlanBytes)
  uint64_t *eptr;
  int32_t n_blk;   // row blocks of the down kernel
  int32_t tb;      // down tiles (8 rows) per row block
  int32_t dn_slots;  // two to four tokens: (token, expert) h rows the down kernel may hold in LDS per workgroup
  int32_t n_cu;    // compute units of the device
  // one-token layer: the gate/up kernel selects the experts itself from the
  // router's scores and keys (then idx and w above are written, not read)
  int32_t sel;
  int32_t G, Gk, norm;
  float rsf;
  const float *keys;     // [E] selection keys of the token
  const double *scores;  // [E] unbiased sigmoid scores
  int32_t *idx_out;
  float *w_out;
};

// ---- timing instrumentation (host) --------------------------------------------
// When enabled (moe_profile_enable), a launcher names the kernel it is about to
// launch (ProfScope); the next MOE_LAUNCH on this thread then goes through
// hipExtLaunchKernel with a start and a stop event that the command processor
// stamps at the kernel's own begin and end, so the per-kernel averages that
// moe_profile_report sums cover the same span as a kernel trace.
bool prof_on();
void prof_arm(const char *name);
bool prof_take(hipEvent_t *start, hipEvent_t *stop);
struct ProfScope {
  ProfScope(const char *name, hipStream_t) { if (prof_on()) prof_arm(name); }
};

// Every kernel of the library is launched through this macro: a plain launch, or,
// when a ProfScope has armed a record, one stamped with kernel start/stop events.
#define MOE_LAUNCH(KERNEL, GRID, BLOCK, LDS, ST, ...)                                        \
  do {                                                                                      \
    hipEvent_t moe_e0_ = nullptr, moe_e1_ = nullptr;                                        \
    if (::moe::prof_take(&moe_e0_, &moe_e1_))                                               \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, (uint32_t)(LDS), ST, moe_e0_, moe_e1_, 0,  \
                            __VA_ARGS__);                                                   \
    else                                                                                    \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, ST, __VA_ARGS__);                        \
  } while (0)

// Keeps a failed HIP call's message for moe_last_hip_error().
void set_hip_error(hipError_t e);

// ---- launchers (host) --------------------------------------------------------
hipError_t launch_route(const RouteArgs &a, hipStream_t st);
hipError_t launch_ws_init(uint32_t *sync, hipStream_t st);
hipError_t launch_route_scores(const RouteArgs &a, hipStream_t st);  // S <= 8: scores and keys only
hipError_t launch_ffn_decode(const FfnArgs &a, hipStream_t st);  // S <= kSmallS
hipError_t launch_gateup_s1(const FfnArgs &a, hipStream_t st);   // S = 1: gate/up (+ selection)
hipError_t launch_down_s1(const FfnArgs &a, hipStream_t st);     // S = 1: down + combine
hipError_t launch_ffn_batch(const FfnArgs &a, hipStream_t st);   // S > kSmallS
hipError_t launch_gu_mfma(const FfnArgs &a, hipStream_t st);
hipError_t launch_dn_mfma(const FfnArgs &a, hipStream_t st);
hipError_t launch_to_limbs(const void *src, int src_bf16, int rows, int K, int src_stride, uint32_t *limbs,
                           float *factors, int wf, const int8_t *q, const float *dq, hipStream_t st);
hipError_t launch_quant_x(const FfnArgs &a, hipStream_t st);  // x -> xq, dx (int8 activations)
hipError_t launch_quant_h(const FfnArgs &a, hipStream_t st);  // h -> hq, dh (int8 activations)
hipError_t launch_pack(int H, int I, const uint8_t *qg, const uint16_t *sg, const uint8_t *qu, const uint16_t *su,
                       const uint8_t *qd, const uint16_t *sd, uint8_t *dst, hipStream_t st);
hipError_t launch_pack_rows(int H, int I, int wf, const uint8_t *qg, const float *sg, const uint8_t *qu,
                            const float *su, const uint8_t *qd, const float *sd, uint8_t *dst, hipStream_t st);

// workspace layout (bytes, each region 256-aligned)
struct WsLayout {
  size_t sync, logits, scores, keys, h, xl, xf, hl, hf, eptr, part, lists, counts, items, n_items, mtiles, xb, xq,
      dx, hq, dh, total;
  int32_t max_items, max_mtiles;
};
WsLayout ws_layout(const moe_cfg &c, int32_t S);

}  // namespace moe
