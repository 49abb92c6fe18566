/*
 * fm.h — C ABI of the MI355X (gfx950) block drafter forward.
 *
 * One drafter handle drives three calls, in the order a speculative-decoding loop makes them:
 *
 *   fm_context_append   tapped target hidden states -> fused context -> per-layer K/V rows in the cache
 *   fm_draft_block      one single-pass block forward (16 flow-map slots, gamma KV-injection slots or M MTP rows)
 *   fm_lm_argmax        lm_head GEMM fused with a per-row argmax
 *
 * Sources (page title, unit on the page):
 *   flow-map   "diskformer 0.5.4 -> 0.6.6", engines/flashmap_drafter.js: FlashMapDrafter.extendContext,
 *              FlashMapDrafter.draft, the file header
 *   KV-inject  "mlx-bun 0.4.0 -> 1.0.0", src/spec/dspark/module-dflash.ts: projectContextRows, forwardRows,
 *              #backbone / #layer (DSpark Eq 2 and Eq 3)
 *   MTP        "diskformer 0.5.3 -> 0.6.4", engines/ternary_bonsai_2_mtp.js: MTPHead.forward, the file header
 *
 * Conventions
 *   - Every data pointer is DEVICE memory owned by the caller (weights, caches, workspace, inputs, outputs). The
 *     library never allocates or frees device memory and never synchronises a stream.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Every call only enqueues work on it;
 *     results are valid once the caller synchronises that stream.
 *   - Every argument is validated on the host BEFORE anything is enqueued; on error nothing is launched and the
 *     call returns a non-zero fm_status with a message in fm_last_error().
 *   - A handle is not thread-safe; one handle is used from one host thread and one stream at a time.
 *   - Weights: bf16 matrices row-major [out][in]; Q8_0 matrices as an int8 code array [out][in] plus an f16 scale
 *     array [out][in/32] (one scale per 32 consecutive codes of a row). Norm weights bf16 (flow-map, KV-inject) or
 *     f32 (MTP).
 */
#ifndef FM_H
#define FM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fm_status {
    FM_OK = 0,
    FM_E_INVALID = 1,        /* bad argument: null pointer, out-of-range size/position, inconsistent config */
    FM_E_CONTEXT_FULL = 2,   /* the append (or draft) would run past max_ctx */
    FM_E_HIP = 3,            /* a HIP runtime call failed (message holds hipGetErrorString) */
    FM_E_UNSUPPORTED = 4,    /* a config combination the library does not implement */
    FM_E_MISSING_WEIGHT = 5, /* a weight the variant needs is not in the name table */
    FM_E_DEVICE = 6          /* reported by fm_device_status: a persistent draft launch gave up waiting */
} fm_status;

enum fm_variant { FM_VARIANT_FLOWMAP = 0, FM_VARIANT_KVINJECT = 1, FM_VARIANT_MTP = 2 };
enum fm_rope { FM_ROPE_NONE = 0, FM_ROPE_INTERLEAVED = 1, FM_ROPE_NEOX = 2 };
enum fm_mlp { FM_MLP_GELU_ERF = 0, FM_MLP_GEGLU_TANH = 1, FM_MLP_SWIGLU = 2 };
enum fm_kv_dtype { FM_KV_F16 = 0, FM_KV_F32 = 1 };
enum fm_wtype { FM_W_BF16 = 0, FM_W_Q8_0 = 1 };

/* Shape and constants of one drafter.
 *   dim        D, the drafter width (flow-map CFG.dim, DflashConfig.dDraft, MCFG.H)
 *   heads      query heads; head_dim hd; kv_heads K/V heads (== heads except grouped-query MTP)
 *   layers     drafter layers (MTP: 1)
 *   ffn        MLP width (F)
 *   block      rows per draft: flow-map slots (16), KV-inject gamma, MTP maximum M (8); at most 16
 *   target_dim Ht, width of a tapped target layer, of the head output and of the lm_head rows
 *   n_taps     tapped target layers concatenated on the feature axis (flow-map / KV-inject context input)
 *   vocab      lm_head rows
 *   max_ctx    cache rows (positions) held per layer
 *   rope       FM_ROPE_*; rope_dims rotated dims per head (NEOX partial); rope_theta the base
 *   ln_eps / rms_eps / qk_eps   LayerNorm, RMSNorm and q/k head-norm epsilons
 *   mlp        FM_MLP_*; kv_dtype FM_KV_* (cache element type); wtype FM_W_* (matrix storage)
 * Supported shapes (FM_E_UNSUPPORTED otherwise): target_dim a multiple of 512; head_dim 64 or 128 (flow-map), 128
 * (KV-inject), 256 (MTP); kv_heads == heads except for the MTP head; n_taps * target_dim at most 16384; dim at most
 * 4096 for the flow-map and KV-inject drafters (their norms are folded into the products, whose statistics cover at
 * most 256 tiles of 16 columns), 6144 for the MTP head.
 * dim, target_dim and ffn must be multiples of 256, and for the MTP head heads * head_dim too (FM_E_INVALID). */
typedef struct fm_config {
    int32_t variant;
    int32_t dim;
    int32_t heads;
    int32_t head_dim;
    int32_t kv_heads;
    int32_t layers;
    int32_t ffn;
    int32_t block;
    int32_t target_dim;
    int32_t n_taps;
    int32_t vocab;
    int32_t max_ctx;
    int32_t rope;
    int32_t rope_dims;
    double rope_theta;
    float ln_eps;
    float rms_eps;
    float qk_eps;
    int32_t mlp;
    int32_t kv_dtype;
    int32_t wtype;
} fm_config;

typedef struct fm_drafter fm_drafter;

/* Bytes of the K/V cache the caller allocates for `cfg` (0 if cfg is invalid).
 * Flow-map / KV-inject layout: for layer l, K at byte offset 2*l*max_ctx*dim*es and V right after (es = 2 for F16,
 * 4 for F32), each max_ctx*dim elements. K is [max_ctx][dim] (position-major). V is [max_ctx][dim] in an F32 cache
 * and tiled [max_ctx/32][dim][32] in an F16 cache: each block of 32 positions is stored dimension-major, so that
 * attention reads one dimension's 32 consecutive positions as the matrix-core operand, and a head's block of
 * 32 positions as contiguous memory; an F16 cache needs max_ctx % 32 == 0.
 * MTP layout: K [max_ctx][kv_heads*head_dim] f32, then V likewise. */
size_t fm_kv_bytes(const fm_config* cfg);

/* Bytes of the device workspace the caller allocates for `cfg` (0 if cfg is invalid): activations, split-K
 * partials, the RoPE table (and its prefill copy), the zero-noise slot row, argmax scratch, prefill buffers (an f16
 * copy of one append's taps; f16 copies of the context-projection and K/V weights, made at create); for Q8_0
 * weights (the MTP head) a copy of every Q8_0 matrix, the lm_head included, in the order its matrix-core kernels
 * read it (made at create: 1.79 GB at the MTP head shape).
 * Owned by the caller; reserved for one handle. */
size_t fm_workspace_bytes(const fm_config* cfg);

/* Create a drafter. `names` / `ptrs` is a table of n_weights (name, device pointer) pairs naming every tensor the
 * variant needs (the parameter names of the pages; Q8_0 matrices as "<name>.q" codes and "<name>.d" scales).
 * Borrowed: the library keeps the pointers, never frees them; they must outlive the handle. kv_cache and
 * workspace must be at least fm_kv_bytes / fm_workspace_bytes and 256-byte aligned.
 * Enqueues the create-time work on `stream`: clearing the workspace's counters, the RoPE table (angles in f64,
 * stored f32, and its permuted prefill copy), f16 copies of the context-projection and per-layer K/V weights
 * (flow-map and KV-inject), copies of the Q8_0 matrices in the matrix-core operand order (MTP: every "<name>.q"
 * must be 8-byte aligned and every "<name>.d" 2-byte aligned, else FM_E_INVALID before any work is enqueued) and,
 * for the flow-map, a private copy of the modulation table "mod", the zero-noise slot
 * input x_embed(state_norm(mean row of lm_head)) + bias (flashmap_drafter.js, init), and layer 0 of a draft from
 * that row up to the cross-attention's q projection (the same for every draft: each slot starts from that row, and
 * the self-attention of identical v rows returns v, so this holds at zero noise, the only slot input built here).
 * The weights must keep their values while the handle lives.
 * Context length starts at 0.
 * Errors: FM_E_INVALID (null pointer, dim % heads, sizes not multiples of 32/256, block > 16 ...),
 * FM_E_MISSING_WEIGHT, FM_E_UNSUPPORTED, FM_E_HIP. */
fm_status fm_create(const fm_config* cfg, int32_t n_weights, const char* const* names, const void* const* ptrs,
                    void* kv_cache, void* workspace, void* stream, fm_drafter** out);

/* Append n rows of tapped features taps[n][n_taps*target_dim] (f32, device) as context positions
 * start .. start+n-1 (flashmap_drafter.js extendContext; module-dflash.ts projectContextRows):
 *   flow-map   c = RMSNorm(fc(taps); hidden_norm), per layer K = RoPE(headRMSNorm(k_proj c; k_norm)), V = v_proj c
 *   KV-inject  c = RMSNorm(W_c taps; ctx_norm), per layer K = W_k RMSNorm(c; attn_norm), V likewise
 * written to the cache (f16 or f32). Any start <= current length may be rewritten (a rewind); the length becomes
 * start + n. taps must be 16-byte aligned (it is read in 16-byte pieces). Appends of more than 16 rows round the
 * taps to f16 for the matrix cores after scaling each row by a power of two into f16's range (undone in f32), so
 * any finite magnitude is accepted; smaller appends keep f32 range (hi + lo bf16 operands).
 * Errors: FM_E_INVALID (n < 1, start < 0, start > length, null or misaligned taps, MTP handle),
 * FM_E_CONTEXT_FULL when start + n + block + 1 > max_ctx (extendContext's own check). */
fm_status fm_context_append(fm_drafter* d, const float* taps, int32_t n, int32_t start, void* stream);

/* Per-call arguments of a draft. */
typedef struct fm_block_args {
    const int32_t* anchor;    /* device: the anchor token id (flow-map, KV-inject); unused by MTP */
    int32_t pos;              /* flow-map: the anchor's context position (slots sit at pos+1 ..); MTP: pos0 */
    int32_t rows;             /* MTP: M in [1, block]; ignored by the other variants (block rows) */
    int32_t kv_lo;            /* MTP: first cache row attended to; ignored otherwise */
    const float* embed_rows;  /* MTP: device [M][dim] f32 embedding rows e */
    const float* prev_hidden; /* MTP: device [M][dim] f32 normed trunk rows h */
    float* debug_layers;      /* nullable device [layers][rows][dim] f32: the residual stream after each layer */
} fm_block_args;

/* One block forward; writes hidden_out[rows][target_dim] (f32, device), the rows that go to the lm_head.
 *   flow-map  (flashmap_drafter.js draft): writes the anchor's context slot at `pos` into the cache (side effect),
 *             then the T zero-noise slots through every DiT layer (adaLN self-attention over the slots,
 *             cross-attention over cache rows [0, pos], GELU MLP), final modulation and head. Needs pos <= length.
 *   KV-inject (module-dflash.ts forwardRows / #backbone): block = [tok_proj(E[anchor]) + block_pos[0];
 *             mask_emb + block_pos[1..]], every layer attends over [cache rows [0, length) ++ block], out_proj.
 *             A one-row block (block = 1) is the anchor row alone and needs no mask_emb in the weight table.
 *   MTP       (ternary_bonsai_2_mtp.js MTPHead.forward): rows M at positions pos .. pos+M-1, writes their K/V to
 *             the cache there, causal grouped-query attention over rows [kv_lo, pos+m]; output shared_head_norm(x).
 * Anchor ids outside [0, vocab) are clamped into the table (a device-side id cannot be checked by the host).
 * Errors: FM_E_INVALID (null pointers, pos > length, rows out of range, kv_lo > pos), FM_E_CONTEXT_FULL
 * (pos + rows (+1) > max_ctx). */
fm_status fm_draft_block(fm_drafter* d, const fm_block_args* a, float* hidden_out, void* stream);

/* tokens[r] = argmax_v (hidden[r] . lm_head[v]) for r < rows (ties to the lowest index), int32 on the device: the
 * target's lm_head applied to the draft's head output and a greedy argmax per row (flashmap_drafter.js draft: the
 * verify-block matvec over the target's head (mvT_ / mm_) and argmaxRows; module-dflash.ts #baseLogits and
 * argmaxAxis; ternary_bonsai_2_mtp.js MTPRunner's lm micro-graph), fused so the [rows][vocab] logits are never
 * stored. hidden is device f32 [rows][target_dim]; the table is the "lm_head.weight" (bf16 [vocab][target_dim]) or
 * "lm_head" (Q8_0) tensor named at fm_create.
 * logits, if not NULL, receives the full [rows][vocab] f32 logits (a debug path; the fused path never writes them).
 * rows <= 16; a flow-map handle (bf16 table) takes up to 32, the rows of a two-request fm_draft_batch, and streams
 * the table once for all of them.
 * Errors: FM_E_INVALID (rows < 1 or above that limit, null hidden / tokens). */
fm_status fm_lm_argmax(fm_drafter* d, const float* hidden, int32_t rows, int32_t* tokens, float* logits,
                       void* stream);

/* fm_lm_argmax without the handle's workspace, for callers that cannot allocate device memory where they call it
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the same product and
 * argmax, the same tokens, with its scratch -- 16 argmax keys and the fragments of the rows -- in the library's own
 * static device array (256 B + 16 x 8192 x 4 B on each GPU, held until the process ends). No allocation, no host
 * synchronisation. Every call on one GPU shares that array: calls that overlap on one GPU (two streams, two host
 * threads) race and must be serialised by the caller; each call clears the keys it needs first.
 * Errors: FM_E_INVALID (rows < 1 or > 16, null hidden / tokens, target_dim > 8192), FM_E_HIP. */
fm_status fm_lm_argmax_static(fm_drafter* d, const float* hidden, int32_t rows, int32_t* tokens, void* stream);

/* Chained MTP depth (ternary_bonsai_2_mtp.js: the file header's "Depth N chains the head", MTPRunner's draft loop):
 * `steps` further single-row passes, pass i at position pos + i, each on the embedding row of the previous draft
 * token (tokens[i]: the row of the lm_head table, dequantised) and the previous pass's output h' (h for pass 0),
 * each followed by the lm_head argmax, all on the device with no host synchronisation.
 *   tokens      device int32 [steps + 1]: tokens[0] is given (the draft the chain starts from); pass i writes
 *               tokens[i + 1]
 *   h           device f32 [dim]: the output row h' of the pass that drafted tokens[0]
 *   hidden_out  device f32 [steps][dim]: pass i's output h'; each pass writes its K/V row into the cache at pos + i
 * Errors: FM_E_INVALID (null pointers, not an MTP drafter, steps < 1, kv_lo > pos), FM_E_CONTEXT_FULL
 * (pos + steps > max_ctx). Token ids outside [0, vocab) are clamped into the table. */
fm_status fm_mtp_chain(fm_drafter* d, int32_t* tokens, const float* h, int32_t steps, int32_t pos, int32_t kv_lo,
                       float* hidden_out, void* stream);

/* Greedy decode of a KV-injection block with the DSpark Markov correction and confidence head (module-dflash.ts:
 * forwardRows' loop with #markov and #confidence). For r < rows, in order: e1 = markov.w1[prev] (prev = *anchor for
 * r = 0, else tokens[r - 1]), tokens[r] = argmax_v (hidden[r] . lm_head[v] + (e1 . markov.w2)[v]) (ties to the
 * lowest index), conf[r] = sigmoid([block_r; e1] . conf.w + conf.b) with block_r = RMSNorm(H_d; out_norm) row r of
 * the last fm_draft_block on this handle (hidden = that call's output).
 *   weights (named at fm_create): markov.w1 bf16 [vocab][rank], markov.w2 bf16 [rank][vocab],
 *            conf.w bf16 [dim + rank], conf.b bf16 [1]
 *   anchor   device int32 [1]; tokens, conf device [rows]; scores nullable device f32 [rows][vocab] (debug)
 * Confidence pruning (forwardRows with thresholds / minConf): thresholds, if not NULL, is a host float [rows], the
 * minimum confidence to keep each position (a uniform minConf is every entry equal). Position 0 is always kept;
 * at the first r >= 1 with conf[r] < thresholds[r] the block ends: positions r .. rows - 1 are dropped (tokens -1,
 * conf 0) and their decode steps do no work (the correction table is not streamed for them; the decision is taken
 * on the device, no host synchronisation). length, if not NULL, receives on the device the positions kept (rows
 * without a cut). With thresholds NULL every position is decoded.
 * Errors: FM_E_INVALID (null pointers, not a KV-injection drafter, rows outside [1, block], rank outside [1, 1024],
 * missing weights), FM_E_UNSUPPORTED (vocab % 4 != 0). */
fm_status fm_markov_argmax(fm_drafter* d, const float* hidden, int32_t rows, const int32_t* anchor, int32_t rank,
                           int32_t* tokens, float* conf, float* scores, const float* thresholds, int32_t* length,
                           void* stream);

/* Time conditioning of the flow-map jump s -> t (flashmap_drafter.js timeConditioning, the model's
 * time_conditioning): sinusoidal embeddings of s and t (time_dim values, frequencies 10000^(-i / (time_dim / 2)),
 * angles of time * time_scale rounded to f32 as the page rounds them) through the time_embed / jump_embed MLPs
 * (linear_1 [cond_dim][time_dim], SiLU, linear_2 [cond_dim][cond_dim], bf16, with biases), cond = SiLU(sum), then
 * every norm's [scale | shift | gate] = its adaLN linear (layers.<l>.{self_attn,cross_attn,mlp}_adaln.linear and
 * final_adaln.linear, bf16 [3 dim][cond_dim] + bias) of cond. Create-time work: the page computes it once per jump
 * (zero noise to tokens: s = 0, t = 1).
 * The table goes into this handle's own copy of the modulation table (taken from the "mod" tensor at fm_create;
 * the caller's "mod" tensor is never written, so other handles created on the same weights keep their tables), and
 * the draft's cached layer-0 projections of the zero-noise slot row, which depend on it, are recomputed.
 * table_out, if not NULL, receives a copy of the new table (device f32 [3 layers + 1][3 dim]).
 * Errors: FM_E_INVALID (not a flow-map drafter, missing weights, time_dim odd or outside [2, 1024], cond_dim
 * outside [1, 1024]), FM_E_UNSUPPORTED (more than 49 norms). */
fm_status fm_time_condition(fm_drafter* d, float s, float t, int32_t time_dim, int32_t cond_dim, float time_scale,
                            float* table_out, void* stream);

/* Batched drafting (module-dflash.ts forwardRows over anchors[]; for the MTP head, several sequences' rows in one
 * pass): one block forward for B requests. Handle ds[b] holds request b's context (its KV cache); all handles share
 * the same weight tensors and block shape (max_ctx may differ). args[b] is request b's fm_draft_block argument
 * (flow-map and KV-injection: anchor, and for flow-map pos; MTP: rows, pos, kv_lo, embed_rows, prev_hidden;
 * debug_layers is ignored). Every projection streams its weights once for all rows; each request attends over its
 * own cache (flow-map: cross-attention over its cache rows [0, pos], self-attention among its own slots, its anchor
 * slot written into its own cache at pos; KV-injection: its context rows ++ its block rows; MTP: causal over
 * [kv_lo, pos + m], after writing its rows' K/V at pos). hidden_out gets the rows in request order (flow-map and
 * KV-injection: block rows per request; MTP: args[b].rows each); the lm_head over them is
 * fm_lm_argmax(ds[0], hidden_out, rows, ...). KV-injection and MTP take at most 16 rows in all; flow-map takes
 * B <= 2 requests (32 rows: each weight tile multiplied against two 16-row blocks), with 16-slot blocks, bf16
 * weights, dim and ffn multiples of 512, and handles whose modulation tables agree (the same fm_time_condition
 * jump, or none). KV-injection: each handle keeps its own request's normed backbone rows, so
 * fm_markov_argmax(ds[b], request b's rows of hidden_out, ...) decodes request b.
 * Errors: FM_E_INVALID (null pointers, B < 1, more than 16 rows, handles with other shapes, other weight tensors or
 * (flow-map) another modulation table, a handle twice, a request's own fm_draft_block errors), FM_E_CONTEXT_FULL (a
 * request past its cache), FM_E_UNSUPPORTED (a flow-map batch of more than 2 requests or of another shape). */
fm_status fm_draft_batch(fm_drafter* const* ds, int32_t B, const fm_block_args* args, float* hidden_out, void* stream);

/* How fm_draft_block runs a flow-map draft. The draft is one forward pass either way (the same arithmetic, results
 * within rounding); this only chooses how its phases are scheduled on the GPU:
 *   0  automatic (the default): one launch per phase, the faster of the two on MI355X at every shape the persistent
 *      kernel takes (its phases are latency-bound, and a launch spreads each over more work-groups)
 *   1  one launch per phase
 *   2  the persistent kernel: every phase of the draft in one launch, one work-group per CU, weights and context K/V
 *      streamed ahead of the arithmetic into LDS, activations passed between work-groups through device-coherent
 *      memory with grid barriers between phases; it applies to 128-wide heads, 16 slots and widths that are
 *      multiples of 256 up to 2048 with one work-group per CU resident (FM_E_UNSUPPORTED elsewhere)
 * The persistent kernel needs its whole grid resident: a caller that runs other work on the GPU at the same time may
 * delay it (each of its waits gives up after 0.2 s, leaving the draft's outputs invalid; fm_device_status reports
 * it). Errors: FM_E_INVALID (null handle, path outside [0, 2]), FM_E_UNSUPPORTED. */
fm_status fm_set_draft_path(fm_drafter* d, int32_t path);

/* The path fm_draft_block takes now: 1 (one launch per phase) or 2 (persistent); -1 for a null handle. */
int32_t fm_draft_path(const fm_drafter* d);

/* Diagnostics: the time of a flow-map draft's skinny weight-streaming GEMM launches (K1) and of the whole draft,
 * with HIP events on `stream`. Runs the draft (one launch per phase) once while recording its K1 launches; then
 * those launches alone, in order, `reps` times over between two events; then the draft once more between two events
 * (its outputs and cache writes are those of fm_draft_block; hidden_out holds them on return). A 2 ms one-wave hold
 * kernel goes ahead of each timed sequence so the host has queued it before the GPU reaches it. Synchronises
 * `stream` and returns, on the host: *skinny_us, the time of one pass over the K1 launches (microseconds);
 * *skinny_launches, their count; *draft_us, the timed draft. Errors: FM_E_INVALID (null pointer, pos outside the
 * cache, null anchor, reps outside [1, 64]), FM_E_UNSUPPORTED (not a flow-map drafter). */
fm_status fm_profile_draft(fm_drafter* d, const fm_block_args* a, float* hidden_out, int32_t reps, float* skinny_us,
                           int32_t* skinny_launches, float* draft_us, void* stream);

/* Synchronises `stream` and reports whether a persistent draft launch on this handle gave up
 * waiting since the last check (FM_E_DEVICE; the flag is then cleared). FM_OK for handles without the persistent
 * kernel. For tests and diagnostics. */
fm_status fm_device_status(fm_drafter* d, void* stream);

/* Current context length (rows appended and not rewound), or -1 for a null handle. */
int32_t fm_context_length(const fm_drafter* d);

/* Free the handle's host-side state; device memory stays with the caller. NULL is ignored. */
void fm_destroy(fm_drafter* d);

/* Message of the last failed call on this host thread ("" if none). */
const char* fm_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FM_H */
