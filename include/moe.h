/* int4 routed-expert MoE layer for AMD Instinct MI355X (gfx950): C ABI.
 *
 * One GLM-5.2-style (glm_moe_dsa) MoE layer forward, split in two calls:
 *   moe_route : router logits, sigmoid scores, group-limited top-k selection and
 *               renormalised weights  ->  idx[S,k], w[S,k]
 *   moe_ffn   : the selected experts' int4 SwiGLU FFN, the weighted sum of their
 *               outputs and the always-on shared expert  ->  y[S,H]
 * plus host helpers (configuration checks, buffer sizes, the packer that turns
 * interchange-format weights into the library's slot layout) and an HBM expert
 * slot pool whose misses are filled from pinned host memory on a side stream.
 *
 * Sources (web pages, cited by title and section):
 *  [PORT]   "GLM-5.2 on a 32 GB Mac - native MLX port of the Colibri hierarchy":
 *           N1 "GLM-5.2 graph" (router and shared expert), "G2 implementation
 *           status" (the int4 nibble encoding, the tie rule between equal keys,
 *           the weights taken from the sigmoid without its bias, the scaling of
 *           the routed sum, the shared expert's weight of one, the dequantise-
 *           and-accumulate contract), "G3 implementation status" (the slot
 *           catalog and its per-layer LRU, the batch union, resident work first).
 *  [README] colibri README, "What's implemented" (the sigmoid noaux_tc router
 *           of the DeepSeek-V3 kind with its scaling factor, the batch union).
 *  [MODELS] "Model support" doc, 4.3 UniversalMoE (grouped routing) and 6.4.
 *  [SCOUT]  "opus colibri scout" (the Colibri-vs-strata Metal audit): sections 1
 *           and 5 (a whole decode window submitted as one command buffer).
 *
 * Conventions for every call below:
 *  - Tensor pointers are DEVICE pointers owned by the caller unless stated.
 *    Nothing here allocates device memory except moe_pool_create.
 *  - `stream` is a hipStream_t (NULL: the default stream).  GPU work is enqueued
 *    on it and the call returns without synchronising.
 *  - Return value: MOE_OK (0) or a negative moe_status.  Arguments are checked
 *    before anything is enqueued; a failed call enqueues nothing and leaves the
 *    outputs untouched.  MOE_EHIP reports a failed launch or copy; the HIP error
 *    string is kept for moe_last_hip_error().
 *  - Values that only the GPU sees (an idx entry outside [0, E), a slot-table
 *    entry outside [0, n_slots)) cannot be checked on the host without a
 *    synchronisation; the kernels never read out of bounds for them and write
 *    NaN into the affected output rows instead.
 */
#ifndef INT4_ROUTED_EXPERT_MOE_H
#define INT4_ROUTED_EXPERT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = -1,     /* configuration or shape not supported */
  MOE_ENULL = -2,      /* a required pointer is NULL */
  MOE_EDTYPE = -3,     /* unknown activation dtype */
  MOE_EWORKSPACE = -4, /* workspace smaller than moe_workspace_bytes() */
  MOE_ENOSLOT = -5,    /* slot pool: the union of experts exceeds the layer's slots */
  MOE_ESTALE = -6,     /* slot pool: a view whose slots have been refilled since it was published */
  MOE_EHIP = -7,       /* a HIP call failed */
  MOE_ELEASE = -8,     /* slot pool: acquire of a leased layer, or release without acquire */
};

enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };

/* Expert weight formats (moe_cfg.weight_format).  In each, W[r,c] = q[r,c] * scale:
 *  MOE_WF_Q4_G32: int4, fp16 scale per 32 consecutive elements of a row (the
 *                 grouped-int4 container);
 *  MOE_WF_Q4_ROW: int4, one fp32 scale per row ([PORT] "G2 implementation
 *                 status": Colibri's production Q4 format, whose group is the
 *                 whole row; "G3 implementation status": 18,939,904 B per GLM-5.2
 *                 expert there, nibbles and fp32 row scales in page-aligned parts);
 *  MOE_WF_Q8_ROW: signed int8, one fp32 scale per row ([PORT] "G4": the MTP
 *                 layer's signed-Q8 routed experts; [README] "What's implemented":
 *                 int8 and packed int4 with per-row scales). */
enum moe_weight_format { MOE_WF_Q4_G32 = 0, MOE_WF_Q4_ROW = 1, MOE_WF_Q8_ROW = 2 };

/* Layer constants.  Limits checked by moe_validate_cfg:
 *  hidden H, moe_inter I, shared_inter Is: multiples of 32, H and I in [32, 8192],
 *  Is = 0 (no shared expert) or in [32, 8192]; group_size = 32;
 *  1 <= n_experts E <= 1024, n_group G divides E, 1 <= topk_group Gk <= G <= 64,
 *  1 <= top_k k <= min(16, Gk * E / G); norm_topk_prob 0 or 1;
 *  routed_scaling_factor finite; weight_format a moe_weight_format; act_int8 0 or 1. */
typedef struct moe_cfg {
  int32_t hidden;
  int32_t n_experts;
  int32_t n_group;
  int32_t topk_group;
  int32_t top_k;
  int32_t moe_inter;
  int32_t shared_inter;
  int32_t group_size;
  float routed_scaling_factor;
  int32_t norm_topk_prob;
  /* Batches of more than 4 tokens: an expert (routed or shared) that receives at
   * least this many tokens is contracted on the matrix cores in bf16 (x and h
   * rounded to bf16, weights dequantised to bf16, fp32 accumulation; with
   * act_int8 the matrix cores take the quantised integers exactly, see act_int8);
   * the others keep the exact fp32 path.  0 disables the matrix-core path.  >= 0.
   * The binding's default is 3. */
  int32_t mfma_min_tokens;
  /* moe_weight_format of every expert of the layer (routed and shared). */
  int32_t weight_format;
  /* 1: int8 activations, an approximate mode ([PORT] "G2 implementation status":
   * the IDOT=1 setting of Colibri, where every activation row becomes int8 ahead
   * of its dot products with the packed int4 weights; [README] "Integer-dot
   * kernels").  Each token's x and each
   * (token, expert) hidden row h (in fp32) is replaced by q * d with
   * d = fp32(max|v| / 127) and q = rint(fp32(v / d)) in [-127, 127] (a row with a
   * NaN gets d = NaN); the dot products of q with the weights are exact integers
   * on every path: per group (then scaled in fp32) with fp16 group scales, per
   * row with row scales, on the GEMV items and on the matrix cores alike.
   * 0: the exact contract (no activation quantisation). */
  int32_t act_int8;
} moe_cfg;

/* Where the routed experts live.  Expert e's packed weights start at
 * base + table[e] * slot_bytes.  `table` is a DEVICE array of E int32 slot
 * numbers (entries outside [0, n_slots) poison the rows that use them).
 * With every expert resident in one array, table[e] = e and gen = NULL.
 *
 * Generation tags ([PORT] N3 "Explicit ExpertResidencyManager": slots carry a
 * generation so that a stale user cannot consume storage that has been reused
 * for another expert).  When gen is not NULL, slot_gen is a DEVICE array of
 * n_slots generation numbers that the owner of the slots changes before it
 * refills a slot, and gen is a DEVICE array of E numbers: the generation that
 * table[e]'s slot held when the table was published.  A kernel uses expert e
 * only if slot_gen[table[e]] == gen[e]; otherwise it writes NaN into the rows
 * of the tokens that chose e, never another expert's values.  The slot pool's
 * views are tagged; a caller's own resident arrays pass gen = NULL.  `lease`
 * identifies the pool acquire that published the view (0 otherwise); the host
 * can ask moe_pool_check_view whether the view has gone stale. */
typedef struct moe_slot_view {
  const void *base;
  int64_t slot_bytes; /* >= moe_expert_bytes(cfg, moe_inter), multiple of 256 */
  const int32_t *table;
  int32_t n_slots;
  const uint32_t *gen;      /* [E] expected generations, or NULL (no check) */
  const uint32_t *slot_gen; /* [n_slots] current generations; required when gen is set */
  uint64_t lease;
} moe_slot_view;

int moe_validate_cfg(const moe_cfg *cfg);
const char *moe_status_string(int status);
const char *moe_last_hip_error(void);

/* Bytes of one packed expert with intermediate size `inter` in the slot layout
 * (gate/up row tiles, then down row tiles; see the packer), rounded up to 4096.
 * Returns a negative moe_status on a bad configuration. */
int64_t moe_expert_bytes(const moe_cfg *cfg, int32_t inter);

/* Device workspace needed by moe_route and moe_ffn for up to max_S tokens.
 * 0 on a bad configuration. */
size_t moe_workspace_bytes(const moe_cfg *cfg, int32_t max_S);

/* Initialise a workspace once, before its first use by moe_route or moe_ffn:
 * writes the 256-byte header at its start (two magic words, then zeros) with a
 * small kernel on `stream` (no memset node, so it may be captured in a graph).
 * No call changes the header, so it stays valid across calls and graph
 * replays.  A workspace is used by one call at a time (calls that share one
 * must be stream-ordered).  moe_route with S <= 8 checks the magic words and,
 * on a workspace that was not initialised, writes idx = -1 and w = NaN for
 * every token (moe_ffn then yields NaN rows).  ws_bytes must be at least 256.
 * Errors: MOE_ENULL, MOE_EWORKSPACE, MOE_EHIP. */
int moe_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Pack one expert from the interchange format into the slot layout.
 * Interchange format of an R x K matrix (K = contraction, groups of 32 along K):
 *   q: uint8 [R, K/2], element (r, 2j) in the low nibble of byte (r, j), (r, 2j+1)
 *      in the high nibble; offset binary, value = nibble - 8 ([PORT] G2 status);
 *   s: uint16 [R, K/32] fp16 bits, scale of elements (r, 32g .. 32g+31).
 * Gate and up are [inter, H], down is [H, inter].  dst receives
 * moe_expert_bytes(cfg, inter) bytes.  where = 0: all pointers are host memory and
 * the packing runs on the CPU (stream ignored); where = 1: all pointers are device
 * memory and a kernel packs on `stream`.  The device packer writes the packed
 * bytes only (the slot's padding up to moe_expert_bytes is left as it was).
 * cfg->weight_format must be MOE_WF_Q4_G32 (MOE_EINVAL otherwise; the row-scaled
 * formats use moe_pack_expert_rows).  Errors: MOE_EINVAL (configuration, inter,
 * where), MOE_ENULL, MOE_EHIP. */
int moe_pack_expert(const moe_cfg *cfg, int32_t inter, const uint8_t *q_gate, const uint16_t *s_gate,
                    const uint8_t *q_up, const uint16_t *s_up, const uint8_t *q_down, const uint16_t *s_down,
                    void *dst, int32_t where, void *stream);

/* Inverse of moe_pack_expert for host memory (round-trip checks). */
int moe_unpack_expert(const moe_cfg *cfg, int32_t inter, const void *src, uint8_t *q_gate, uint16_t *s_gate,
                      uint8_t *q_up, uint16_t *s_up, uint8_t *q_down, uint16_t *s_down);

/* moe_pack_expert for the row-scaled formats (cfg->weight_format MOE_WF_Q4_ROW or
 * MOE_WF_Q8_ROW; MOE_EINVAL otherwise, and moe_pack_expert returns MOE_EINVAL
 * for them).  Interchange format of an R x K matrix:
 *   MOE_WF_Q4_ROW: q uint8 [R, K/2], offset-binary nibbles as for moe_pack_expert;
 *   MOE_WF_Q8_ROW: q int8 [R, K], two's complement, element (r, c) at byte (r, c);
 *   s: fp32 [R], the scale of row r.
 * Gate and up are [inter, H], down is [H, inter]; dst receives
 * moe_expert_bytes(cfg, inter) bytes; `where` and `stream` as for moe_pack_expert. */
int moe_pack_expert_rows(const moe_cfg *cfg, int32_t inter, const void *q_gate, const float *s_gate,
                         const void *q_up, const float *s_up, const void *q_down, const float *s_down, void *dst,
                         int32_t where, void *stream);

/* Inverse of moe_pack_expert_rows for host memory. */
int moe_unpack_expert_rows(const moe_cfg *cfg, int32_t inter, const void *src, void *q_gate, float *s_gate,
                           void *q_up, float *s_up, void *q_down, float *s_down);

/* Router ([PORT] N1 and G2 status; [README] "What's implemented"; [MODELS] 4.3):
 *   l[t,e] = sum_h x[t,h] W_gate[e,h]         (fp64 accumulation)
 *   s = sigmoid(l) (fp64); key = fp32(s + bias)
 *   group score = fp32(sum of the group's two largest keys), groups are G
 *   contiguous blocks of E/G experts; keep the Gk best groups (ties: lower group);
 *   top-k keys over the kept experts (ties: lower expert ID), rank order;
 *   w = s[idx] / sum(s[idx]) * rsf (or s[idx] * rsf without renormalisation).
 * x: [S, H] fp32 or bf16 (x_dtype); W_gate: [E, H] fp32 row-major; bias: [E] fp32.
 * Out: idx [S, k] int32, w [S, k] fp32, both rank-ordered.  S = 0 is a no-op.
 * ws: device workspace of at least moe_workspace_bytes(cfg, S) bytes, initialised
 * by moe_workspace_init.  S <= 8: one workgroup per expert computes its logits
 * and stores the tokens' scores and keys, then one workgroup per token selects
 * (two kernels); larger S: an fp64 matrix-core logits GEMM, then one wave per
 * token selects. */
int moe_route(const moe_cfg *cfg, const void *x, int32_t x_dtype, int32_t S, const float *W_gate,
              const float *bias, int32_t *idx, float *w, void *ws, size_t ws_bytes, void *stream);

/* Expert FFN ([PORT] N1 and G2 status; [README] batch-union MoE):
 *   y[t] = sum_j w[t,j] * FFN_{idx[t,j]}(x_t) + FFN_shared(x_t),
 *   FFN(x) = Wd (silu(Wg x) * (Wu x)),  W = dequant(q, s) = (nibble - 8) * scale.
 * Every expert named by idx is streamed once per call and applied to all the
 * tokens that chose it.  x: [S, H] fp32 or bf16; idx/w: [S, k] as from moe_route;
 * experts: routed slots (host struct holding device pointers); shared: the packed
 * shared expert (moe_expert_bytes(cfg, shared_inter) bytes), ignored when
 * shared_inter = 0.  Out: y [S, H] fp32.  Arithmetic: each 32-element group's
 * dot product of int4 (or int8) weights with the activations in block fixed
 * point (2^-22 of the group's largest |value|) is an exact integer, rounded once
 * to fp32, scaled by the group's scale (MOE_WF_Q4_G32) and summed in fp32; the
 * row-scaled formats multiply the row's sum by its scale instead.  Larger
 * batches use the same for experts with fewer than mfma_min_tokens tokens and
 * bf16 MFMA (fp32 accumulation) for the others.  With act_int8 the quantised
 * integers take the activations' place in the same exact dot products (the row
 * scale folds into each group's factor); larger batches with row-scaled weights
 * send the many-token experts to int8 MFMA (exact int32 row sums, scaled once),
 * and with MOE_WF_Q4_G32 weights every expert stays on the exact path. */
int moe_ffn(const moe_cfg *cfg, const void *x, int32_t x_dtype, int32_t S, const int32_t *idx, const float *w,
            const moe_slot_view *experts, const void *shared, float *y, void *ws, size_t ws_bytes, void *stream);

/* One MoE layer forward: moe_route followed by moe_ffn on the same stream, with
 * the same arguments and bit-identical results (idx, w and y); [PORT] N1 (the
 * layer is the router, then the routed experts, then their route-order
 * combine with the shared expert).  For S = 1 the router kernel only stores
 * each expert's score and key and the gate/up kernel selects the experts itself
 * in every workgroup from those values (workgroup 0 also writes idx and w), so
 * the selection needs no kernel of its own (and the workspace header is not
 * read).  Other S: moe_route then moe_ffn.  Errors: those of moe_route and
 * moe_ffn. */
int moe_layer(const moe_cfg *cfg, const void *x, int32_t x_dtype, int32_t S, const float *W_gate, const float *bias,
              int32_t *idx, float *w, const moe_slot_view *experts, const void *shared, float *y, void *ws,
              size_t ws_bytes, void *stream);

/* moe_layer for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It takes
 * no workspace: the library's own fixed per-device array of MOE_SCRATCH_BYTES
 * (8 MiB; each GPU the library runs on holds one until the process ends) serves
 * as the workspace, and the call allocates nothing.  Same arguments as
 * moe_layer without ws/ws_bytes, same kernels, bit-identical idx, w and y; for
 * S > 1 it first rewrites the workspace header with a kernel on `stream`.
 * Errors: those of moe_layer, and MOE_EWORKSPACE when moe_workspace_bytes(cfg,
 * S) exceeds MOE_SCRATCH_BYTES (the GLM-5.2 shape fits up to S = 16; the
 * largest supported shape up to S = 4), with nothing enqueued.  Every call on
 * one GPU uses that GPU's array, which keeps the last call's contents: calls
 * that overlap on one GPU (on different streams, or in graphs replayed
 * concurrently) race and must not be made. */
#define MOE_SCRATCH_BYTES ((size_t)8 << 20)
int moe_layer_noalloc(const moe_cfg *cfg, const void *x, int32_t x_dtype, int32_t S, const float *W_gate,
                      const float *bias, int32_t *idx, float *w, const moe_slot_view *experts, const void *shared,
                      float *y, void *stream);

/* ---- recorded chains of layer calls: one library-owned HIP graph ----------------
 * [SCOUT] section 1 "architecture side by side" and section 5 "where strata is
 * ahead", item 1: the faster Metal design submits a whole decode window (every
 * layer's router and MoE) as one command buffer, instead of one submission per
 * layer or op.  Here that is a HIP graph: moe_chain_create records n moe_layer
 * calls, in order, each with its own arguments, and instantiates them as one
 * graph; moe_chain_launch enqueues the whole chain on a stream as a single graph
 * launch.  [MODELS] "History" records a single-dispatch megakernel that was
 * shelved at about 0.94x of the split kernels, and a one-launch kernel built for
 * this layer measured slower too, so the chain keeps the split kernels and only
 * removes the host's per-kernel submissions.
 *
 * moe_layer_call holds the arguments of one moe_layer call.  Everything in it is
 * read at record time and kept by value: the configuration, S, the dtypes, every
 * pointer, and the fields of the slot view.  The device memory behind those
 * pointers is read at every launch.  So the caller writes new inputs into the
 * same buffers between launches, and a slot pool's table updates (its device
 * table and generation arrays) are seen by the next launch.  The output of one
 * call may be the input of a later one (y of call i as x of call i + 1): calls
 * run in recorded order.  The caller keeps every buffer alive, and at the same
 * address, until moe_chain_destroy.
 *
 * moe_chain_create: every call is checked as moe_layer checks it before anything
 * is recorded; the first failing call's status is returned (MOE_EINVAL also for
 * n < 1, or while moe_profile_enable is on: kernel-stamped profiling events are
 * not recorded in graphs).  HIP errors while recording or instantiating return
 * MOE_EHIP; MOE_EINVAL if the host cannot allocate the chain's record.  On any
 * error *out is NULL and nothing is enqueued.  The chain
 * belongs to the device that is current at creation; the calls are recorded on
 * a private stream (default priority) that is destroyed before return.
 * moe_chain_launch: MOE_ENULL for a NULL chain, MOE_EINVAL if the current device
 * is not the chain's; otherwise one graph launch on `stream`.  Results are
 * bit-identical to the same moe_layer calls made one by one.  Launches of chains
 * that share a workspace or output buffers must not overlap (different streams
 * without ordering race, as the same moe_layer calls would).
 * moe_chain_destroy: frees the graph (NULL is a no-op).  Launches already
 * enqueued finish normally. */
typedef struct moe_layer_call {
  const moe_cfg *cfg;
  const void *x;
  int32_t x_dtype;
  int32_t S;
  const float *W_gate;
  const float *bias;
  int32_t *idx;
  float *w;
  const moe_slot_view *experts;
  const void *shared;
  float *y;
  void *ws;
  size_t ws_bytes;
} moe_layer_call;
typedef struct moe_chain moe_chain;
int moe_chain_create(const moe_layer_call *calls, int32_t n, moe_chain **out);
int moe_chain_launch(const moe_chain *chain, void *stream);
void moe_chain_destroy(moe_chain *chain);

/* ---- HBM expert-slot pool ([PORT] N3 and G3 status; [README] per-layer LRU) ----
 * One device slab of n_layers * slots_per_layer slots of moe_expert_bytes(cfg,
 * moe_inter) bytes, a device table per layer (table[e] = slot, or -1), and a
 * host-side LRU per layer.  The packed experts live in caller-owned host memory
 * (pinned: hipHostMalloc) registered with moe_pool_register_host.
 *
 * moe_pool_acquire(layer, idx[n]) takes the union of the experts named by idx
 * (host memory, n entries, e.g. S*k routing results copied back), leases the
 * resident ones, and for each miss takes a free slot or evicts the least recently
 * used unleased slot of the layer (ties: lowest slot).  Miss copies are enqueued
 * on `side` after the victim slot's previous consumer has finished; the layer's
 * table is updated on `compute` after the copies completed, so a kernel on
 * `compute` never sees a partially filled slot.  view_out then addresses the
 * layer (pass it to moe_ffn on `compute`).  Each acquire must be followed by
 * moe_pool_release(layer, compute) after the consuming work is enqueued; it
 * records the consumer-done event of every leased slot.
 * Generations: every fill takes a new pool-wide generation number, written into
 * the slot's slot_gen entry on `side` before the copy; the table upload carries
 * each resident expert's generation (view gen).  A slot whose prefetch copy is
 * still running is published as absent (-1) until an acquire that leases it
 * has waited for the copy.  A view used after its release, once its slots have
 * been refilled, gives NaN rows for the refilled experts (see moe_slot_view);
 * such a use must still be stream-ordered after the refill's start (a kernel
 * that runs concurrently with a refill of its slot is a race).
 * Errors: MOE_ENOSLOT (union larger than slots_per_layer), MOE_ELEASE (acquire
 * of a layer with an unreleased lease, or release without acquire), MOE_ENULL
 * (a missing expert has no registered host source), MOE_EINVAL (bad layer or
 * expert id).  All calls on one pool must come from one host thread. */
typedef struct moe_pool moe_pool;
enum { MOE_POOL_NO_DEVICE = 1, /* policy only: no device memory, no copies (host tests) */
       MOE_POOL_POISON = 2 /* overwrite a slot with 0xFF bytes before refilling it (ordering tests) */ };
int moe_pool_create(const moe_cfg *cfg, int32_t n_layers, int32_t slots_per_layer, int32_t flags, moe_pool **out);
void moe_pool_destroy(moe_pool *pool);
int moe_pool_register_host(moe_pool *pool, int32_t layer, int32_t expert, const void *packed_host_src);
int moe_pool_acquire(moe_pool *pool, int32_t layer, const int32_t *idx_host, int32_t n, moe_slot_view *view_out,
                     int32_t *n_miss_out, void *compute_stream, void *side_stream);
int moe_pool_release(moe_pool *pool, int32_t layer, void *compute_stream);
/* Predictive prefetch ([PORT] "What Colibri is actually doing", item 10: the
 * next layer's router applied ahead of time, real loads only for a future
 * layer, residency rechecked, no partially filled slot ever published; [README]
 * "What's implemented", router-lookahead prefetch).  idx_host (host memory, n
 * entries) is a predicted routing of `layer`.  Its resident experts become
 * recently used; each missing one takes a free slot or the least recently used
 * unleased slot of the layer (ties: lowest; never a leased slot) and its copy
 * is enqueued on side_stream after the victim's last consumer, with nothing
 * leased and nothing published.  The next moe_pool_acquire of the layer finds
 * those experts resident, makes its compute stream wait for their copies and
 * uploads the table, so results are the same as without the prefetch; a
 * prediction that is never acquired only takes slots (and may evict experts
 * that would have hit: [PORT] "What not to copy blindly").  When every slot is
 * leased the rest of the prediction is dropped.  n_fill_out (optional): copies
 * enqueued.  Errors: MOE_ENOSLOT (union larger than slots_per_layer), MOE_ENULL
 * (a missing expert has no registered host source), MOE_EINVAL, MOE_EHIP. */
int moe_pool_prefetch(moe_pool *pool, int32_t layer, const int32_t *idx_host, int32_t n, int32_t *n_fill_out,
                      void *side_stream);
/* The last acquire's decisions as (expert, slot, hit) triples in out[3 * i ..];
 * returns the number of triples, or a negative status (cap too small). */
int moe_pool_trace(const moe_pool *pool, int32_t *out, int32_t cap);
/* {"acquires", "hits", "misses", "evictions", "fill_bytes", "prefetches",
 * "prefetch_fills", "prefetch_hits", ...} as JSON (prefetch_hits: acquire hits
 * on prefetched slots). */
int moe_pool_stats(const moe_pool *pool, char *out_json, size_t cap);
/* Host-side staleness check of a view of `layer` made by moe_pool_acquire:
 * MOE_OK while its lease is open, or when no slot of the layer has been given
 * to another expert since the view was published; MOE_ESTALE when its lease
 * has ended and a slot of the layer has been refilled since (its kernels would
 * then write NaN for the refilled experts); MOE_EINVAL when the view does not
 * address this pool's layer. */
int moe_pool_check_view(const moe_pool *pool, int32_t layer, const moe_slot_view *view);

/* Timing instrumentation (not part of the layer's computation).  While enabled,
 * the library brackets each kernel it launches with two hipEvents recorded on the
 * launch stream.  moe_profile_report waits for the recorded events, writes
 * {"kernel": [total_ms, launches], ...} as a NUL-terminated JSON string into out
 * (cap bytes; MOE_EINVAL if too small) and forgets the records.  Host state is
 * process-wide and not thread-safe. */
int moe_profile_enable(int on);
int moe_profile_report(char *out, size_t cap);

#ifdef __cplusplus
}
#endif
#endif
