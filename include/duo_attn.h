/*
 * duo_attn.h -- C ABI of the MI355X (gfx950) hybrid GQA attention library:
 * causal full-attention layers, causal sliding-window layers, and
 * DuoAttention per-KV-head routing (full-context heads vs. streaming heads
 * that keep sink + recent tokens in a compacted cache).
 *
 * Sources of the method (titles and sections of the pages):
 *  - Hugging Face model card "DuoAttention Laguna Adapter": "Summary" (KV heads
 *    split into full-context and streaming heads; sink size 64, recent size
 *    256; a learned full_attention_heads tensor), "Why It Works" (full-context
 *    heads hold every earlier position, a streaming head holds only the
 *    first positions and the newest ones), "Changes In This Submission" (head
 *    reordering so
 *    full and streaming heads are separated; static Duo KV cache).
 *  - Blog post on Laguna-M.1-8bit attention: sliding-window section (a token
 *    looks back over a fixed-width window, cost O(n*w) instead of O(n^2)),
 *    implementation section (per-layer layer_types / sliding_window, None for
 *    full layers), mask-generation section (causal and sliding-window causal
 *    masks chosen per layer type).
 *  - SGLang cookbook "Laguna-XS-2.1", section 1 "Model Introduction": 48 Q / 8
 *    KV heads, window 512, 30 sliding + 10 full layers; DFlash speculative
 *    decoding (the target verifies a drafted block in one pass).
 *  - Blog post on Laguna-XS-2.1 sliding-window attention, section on its
 *    optimisations: q/k RMSNorm before the rotary embedding, an optional
 *    learnable attention-sink bias on sliding layers, output gating through
 *    a g_proj projection. Blog post on Laguna-M.1-8bit, YaRN section: the
 *    rotary parameters of full-attention layers.
 *
 * Visibility of key position j for a query at position i (G = Hq / Hkv, query
 * head h uses KV head h / G):
 *   full-context head, FULL layer (or window <= 0):  0 <= j <= i
 *   full-context head, SLIDING layer, window W > 0:  i - W + 1 <= j <= i
 *   streaming head (any layer):                      j <= i and (j < sink or j > i - recent)
 *
 * Conventions for every entry point:
 *  - Tensors are bfloat16 (16-bit bit patterns), row-major, densely packed,
 *    head_dim = 128, and 16-byte aligned, except the float32 lse outputs,
 *    sink logits and RMSNorm weights (4-byte aligned). Device pointers are
 *    owned by the caller; the library never allocates, frees or retains them.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream). Calls only
 *    enqueue work and return; results are visible after the stream is
 *    synchronised.
 *  - Validation is synchronous and has no side effects: a non-zero return
 *    means nothing was launched. duo_last_error() then describes the problem
 *    (thread-local, valid until the next call on the same thread).
 *  - Calls on different streams that write the same cache or workspace race.
 *  - Positions (start_pos + num_tokens, max_seq_len, max_end_pos,
 *    max_past_len + num_tokens) must stay at or below 2^31 - 1025
 *    (INVALID_ARG otherwise): the kernels use 32-bit positions and form tile
 *    bounds a little past the last one.
 *  - Inputs are finite numbers. The prefill is built without NaN semantics,
 *    so a NaN in its inputs gives unspecified (but in-bounds) results.
 */
#ifndef DUO_ATTN_H
#define DUO_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DUO_ATTN_VERSION 2
#define DUO_HEAD_DIM 128
#define DUO_MAX_KV_HEADS 32
#define DUO_MAX_GROUP 16

typedef enum duo_status {
  DUO_OK = 0,
  DUO_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad size or range   */
  DUO_ERR_UNSUPPORTED = -2,  /* head_dim != 128, group > 16, kv heads > 32     */
  DUO_ERR_CAPACITY = -3,     /* positions beyond the caller's cache capacity  */
  DUO_ERR_WORKSPACE = -4,    /* workspace missing, too small or misaligned    */
  DUO_ERR_HIP = -5           /* a HIP launch failed                          */
} duo_status;

typedef enum duo_layer_kind {
  DUO_LAYER_FULL = 0,        /* causal attention over the whole prefix        */
  DUO_LAYER_SLIDING = 1      /* causal sliding window of `window` positions   */
} duo_layer_kind;

/* One attention layer (host memory, read only during the call).
 * `full_attention_heads` is this layer's row of the adapter's learned
 * full_attention_heads tensor (model card "DuoAttention Laguna Adapter",
 * "Summary"/"Training"), reduced to a binary mask: nonzero = full-context KV
 * head. NULL = no Duo routing, every KV head keeps full context.
 * `window` applies to SLIDING layers only; <= 0 means no window (Laguna-M.1-8bit
 * blog post, implementation section: sliding_window is None for non-sliding
 * layers). `scale` 0 means 1/sqrt(head_dim). */
typedef struct duo_layer {
  int32_t num_q_heads;       /* Hq (48 for Laguna-XS-2.1)                     */
  int32_t num_kv_heads;      /* Hkv (8); Hq % Hkv == 0, Hq / Hkv <= 16        */
  int32_t head_dim;          /* must be 128                                   */
  int32_t kind;              /* duo_layer_kind                                */
  int32_t window;            /* 512 on sliding layers                         */
  int32_t sink;              /* 64: first positions kept by streaming heads   */
  int32_t recent;            /* 256: newest positions kept by streaming heads */
  const uint8_t* full_attention_heads; /* host [num_kv_heads] or NULL        */
  float scale;
} duo_layer;

/* The static KV cache of one layer (device memory, caller owned).
 * Heads are split by class; within a class they are numbered by ascending KV
 * head index ("rank"), the cache-side image of the adapter's head reordering
 * (model card, "Changes In This Submission"). n_main = number of full-context
 * KV heads (all Hkv without a mask), n_stream = Hkv - n_main.
 *   k_main/v_main     [B, n_main, main_capacity, 128]
 *       FULL layer (or window <= 0): slot = position; main_capacity is the
 *       largest position count the cache can hold.
 *       SLIDING layer with window W > 0: a ring, slot = position mod W;
 *       main_capacity must equal W.
 *   k_stream/v_stream [B, n_stream, sink + recent, 128]
 *       slot = position if position < sink,
 *              else sink + (position - sink) mod recent.
 * Pointers of an empty class may be NULL. */
typedef struct duo_kv_cache {
  void* k_main;
  void* v_main;
  int64_t main_capacity;
  void* k_stream;
  void* v_stream;
} duo_kv_cache;

/* Optional input prologue: RMSNorm of each head's 128 channels, then the
 * rotary position embedding, applied to q (fused into the attention calls'
 * query loads), to k on its way into the cache (duo_kv_append), or to any
 * [batch, tokens, heads, 128] tensor (duo_qk_prologue).
 * Laguna-XS-2.1 blog post, sliding-window optimisations: q and k are
 * RMS-normalised before the rotary embedding is applied. Laguna-M.1-8bit blog
 * post, YaRN dynamic RoPE: full-attention layers use rope_theta 500000, YaRN
 * factor 64, original_max_position_embeddings 4096, beta_fast 64, beta_slow 1,
 * attention_factor 1, all 128 channels rotated.
 *
 * norm_weight : device float [128] or NULL (no RMSNorm): y = x / sqrt(mean(x^2)
 *               + norm_eps) * norm_weight over one head's channels (the pages
 *               give neither the axis nor eps; per head is the plainest
 *               reading, eps is the caller's). 4-byte aligned.
 * rope        : host duo_rope or NULL (no rotation); read during the call only.
 * Rotation: channel i pairs with channel i + 64 and the pair turns by
 * pos * f_i: (x_i cos - x_{i+64} sin, x_{i+64} cos + x_i sin), both times
 * attention_factor. f_i = theta^(-2i/128); with factor > 1, YaRN (Peng et
 * al. 2023, section 3.2, NTK-by-parts) blends f_i and f_i / factor with a
 * ramp over the pair index between floor(c(beta_fast)) and
 * ceil(c(beta_slow)), c(r) being the pair index that turns r times over
 * original_max_position positions. pos is the row's absolute position.
 * Errors: theta <= 1, a non-finite or non-positive factor or
 * attention_factor, original_max_position < 1, beta_fast <= beta_slow or
 * beta_slow <= 0 (with factor > 1), a negative or non-finite eps:
 * INVALID_ARG. */
typedef struct duo_rope {
  float theta;
  float factor;                   /* <= 1: plain RoPE */
  int32_t original_max_position;
  float beta_fast, beta_slow;
  float attention_factor;
} duo_rope;

typedef struct duo_prologue {
  const float* norm_weight;
  float norm_eps;
  const duo_rope* rope;
} duo_prologue;

/* Optional output epilogue of the attention calls (pass NULL for none).
 * sink_logits : device float [Hq] or NULL. Attention sink of a sliding layer
 *               (Laguna-M.1-8bit post, sliding-window optimisations: a
 *               learnable bias added for sliding-window layers): one logit per
 *               query head, in the units of the scaled logits, that joins the
 *               softmax normaliser as a key whose value row is zero
 *               (w_j = e^{s_j} / (sum_i e^{s_i} + e^{b_h})); lse includes it.
 * gate        : device bf16 or NULL. Output gate (same post, attention output
 *               gating through a g_proj projection): out = attention output x
 *               logistic(gate). DUO_GATE_PER_ELEMENT: gate laid out like `out`;
 *               DUO_GATE_PER_HEAD: like `out` without its last dimension (one
 *               value per row and query head, broadcast over the 128 channels).
 * The pages do not name the gate's nonlinearity; the logistic function is the
 * plainest reading. Both are applied where the kernel normalises each output
 * row, before the bf16 rounding. Alignment: sink_logits 4 bytes, gate 16
 * bytes (INVALID_ARG otherwise); gate given without a mode, a mode without a
 * gate or an unknown mode is INVALID_ARG. The library keeps no pointer after
 * the call is enqueued; the buffers must stay valid until it completes. */
enum duo_gate_mode { DUO_GATE_NONE = 0, DUO_GATE_PER_ELEMENT = 1, DUO_GATE_PER_HEAD = 2 };

typedef struct duo_epilogue {
  const float* sink_logits;
  const void* gate;
  int32_t gate_mode;
} duo_epilogue;

/* Write new K/V rows into the cache (the streaming-head cache manager).
 * Defined by the model card "DuoAttention Laguna Adapter": "Summary" (KV heads
 * are full-context or streaming; a streaming head keeps the 64 sink and the
 * 256 most recent positions) and "Changes In This Submission" (a static Duo
 * KV cache, heads reordered so that the two classes are stored apart). The
 * slot of each position is the library's reading of those passages (the
 * pages never describe slots): see duo_kv_cache.
 * k_new, v_new : device [batch, num_tokens, Hkv, 128] (token-major, as the
 *                projections emit them); token t of sequence b is position
 *                start_pos[b] + t.
 * start_pos    : device int32 [batch], >= 0.
 * max_end_pos  : host upper bound on max_b(start_pos[b]) + num_tokens; checked
 *                against main_capacity for contiguous caches (CAPACITY error).
 *                The kernel also drops any write whose slot would fall outside
 *                a contiguous cache, so a wrong bound cannot corrupt memory.
 * When one call brings more positions than a ring holds, only the newest
 * positions of each slot are written, so every slot has exactly one writer.
 * Bit copy, no rounding, unless k_prologue is given: then each written K row
 * is the bf16 (round to nearest even) of the prologue of k_new at its
 * position; V stays a bit copy. */
int duo_kv_append(const duo_layer* layer, const duo_kv_cache* cache, int32_t batch,
                  const void* k_new, const void* v_new, int32_t num_tokens,
                  const int32_t* start_pos, int64_t max_end_pos, const duo_prologue* k_prologue,
                  void* stream);

/* Prefill attention for a chunk of num_tokens query positions
 * [start_pos, start_pos + num_tokens) of every sequence in the batch.
 * Defined by the blog post on Laguna-M.1-8bit attention, sliding-window
 * section (each token attends a fixed-width window of earlier tokens) and
 * mask-generation section (a causal or a sliding-window causal mask per layer
 * type), and by the model card "DuoAttention Laguna Adapter", "Why It Works"
 * (full-context heads see every earlier position, streaming heads only the
 * sink and the most recent ones). The visibility rules at the top of this
 * file restate them; the result is the exact masked softmax.
 * q   : device [batch, num_tokens, Hq, 128]
 * k,v : device [batch, num_tokens, Hkv, 128] -- the chunk's own keys/values.
 * past: the cache holding positions [0, start_pos) as duo_kv_append left it;
 *       may be NULL when start_pos == 0. The chunk's K/V are read from k/v,
 *       not from the cache (attend, then append the chunk).
 * out : device [batch, num_tokens, Hq, 128] bf16 (round to nearest even).
 * lse : NULL or device float [batch, Hq, num_tokens], natural-log
 *       log-sum-exp of the scaled logits of each row.
 * q_prologue : NULL or the RMSNorm / rotary embedding of q (duo_prologue),
 *       applied as the query rows are loaded, at positions start_pos + t; k
 *       must already hold the prologue's output (duo_qk_prologue).
 * epilogue : NULL or the attention sink / output gate (duo_epilogue); a
 *       per-element gate is [batch, num_tokens, Hq, 128], a per-head gate
 *       [batch, num_tokens, Hq].
 * workspace : NULL, or device scratch of at least
 *       duo_attn_prefill_workspace_bytes() bytes (256-byte aligned, caller
 *       owned, zero-filled once before its first use with
 *       duo_attn_decode_workspace_init or any zero fill; every completed call
 *       leaves its counters at zero again). With a workspace, the full-context
 *       query tiles of a chunk over a long past are cut into key-range pieces
 *       that run as separate workgroups and are merged in the same launch
 *       (partial max, sum and output, as the decode's split-K), so the longest
 *       work items no longer set the launch's length; the size is 0 (and the
 *       workspace unused) when no piece would be cut. Without one, every query
 *       tile runs whole. The result is the same either way up to fp32
 *       summation order. A workspace smaller than needed, or misaligned, is
 *       DUO_ERR_WORKSPACE. Calls that share a workspace must be ordered. */
int duo_attn_prefill(const duo_layer* layer, const duo_kv_cache* past, int32_t batch,
                     const void* q, const void* k, const void* v, int32_t num_tokens,
                     int64_t start_pos, void* out, float* lse, void* workspace,
                     size_t workspace_bytes, const duo_prologue* q_prologue,
                     const duo_epilogue* epilogue, void* stream);

/* Workspace size for duo_attn_prefill at these sizes (0 when the call would
 * cut no query tile into pieces, and on invalid arguments). Host only. */
size_t duo_attn_prefill_workspace_bytes(const duo_layer* layer, int32_t batch, int32_t num_tokens,
                                        int64_t start_pos);

/* Decode attention: one query token per sequence at position seq_lens[b]-1,
 * whose K/V have already been appended (seq_lens counts them).
 * Defined by the same passages as duo_attn_prefill (Laguna-M.1-8bit post,
 * sliding-window and mask-generation sections; model card "DuoAttention
 * Laguna Adapter", "Why It Works"), applied to the newest token: the
 * decode-time KV reads that the model card's "Benefits" section says the
 * streaming heads shrink.
 * q         : device [batch, Hq, 128]
 * seq_lens  : device int32 [batch], each in [1, max_seq_len]; a 0 entry
 *             yields a zero output row (lse = -inf, or the sink logit when
 *             the epilogue has one).
 * q_prologue: NULL or duo_prologue, applied to q at position seq_lens[b] - 1.
 * epilogue  : NULL or duo_epilogue; gate [batch, Hq, 128] or [batch, Hq].
 * max_seq_len : host bound used to size the split-K grid.
 * out       : device [batch, Hq, 128] bf16.  lse: NULL or device float [batch, Hq].
 * workspace : device scratch of at least duo_attn_decode_workspace_bytes()
 *             bytes, 256-byte aligned, owned by the caller. It holds split-K
 *             partial results and per-(sequence, KV head) arrival counters.
 *             It must be zero-filled once before its first use
 *             (duo_attn_decode_workspace_init, or any zero fill); every
 *             completed call leaves the counters at zero again, so it can be
 *             reused without clearing. Calls that share a workspace must be
 *             ordered (same stream). */
int duo_attn_decode(const duo_layer* layer, const duo_kv_cache* cache, int32_t batch,
                    const void* q, const int32_t* seq_lens, int64_t max_seq_len,
                    void* out, float* lse, void* workspace, size_t workspace_bytes,
                    const duo_prologue* q_prologue, const duo_epilogue* epilogue, void* stream);

/* duo_attn_decode without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). The split-K partials and arrival counters live in
 * scratch the library holds: one 32 MiB device array per GPU, resolved on the
 * first call on each device and kept until the process ends. Arguments and
 * results are those of duo_attn_decode. A decode whose workspace
 * (duo_attn_decode_workspace_bytes) would exceed 32 MiB is refused with
 * DUO_ERR_WORKSPACE before anything is launched. Each call first clears the
 * counters it uses (a fill kernel on `stream`, so it may be captured). The
 * call allocates and frees nothing. Every call on one GPU shares that GPU's
 * scratch: calls that may overlap on one GPU (different streams without
 * ordering) race and give wrong results; order them on one stream. */
int duo_attn_decode_noalloc(const duo_layer* layer, const duo_kv_cache* cache, int32_t batch,
                            const void* q, const int32_t* seq_lens, int64_t max_seq_len, void* out,
                            float* lse, const duo_prologue* q_prologue, const duo_epilogue* epilogue,
                            void* stream);

/* Block decode: num_tokens consecutive query tokens per sequence, at
 * positions past_lens[b] .. past_lens[b] + num_tokens - 1 -- the block a
 * speculative-decoding target verifies in one pass (SGLang cookbook
 * "Laguna-XS-2.1", DFlash speculative decoding: the target checks a whole
 * drafted block at once). Each token sees the visible cached positions
 * (the same rules as duo_attn_prefill: full-context heads the causal prefix,
 * a sliding layer its window, streaming heads sink + recent) and the block's
 * tokens up to itself. Attend, then append: the cache holds positions
 * [0, past_lens[b]) as duo_kv_append left it, the block's own K/V come from
 * k_new/v_new; append them afterwards for the next step.
 * q, out      : device [batch, num_tokens, Hq, 128] bf16.
 * k_new,v_new : device [batch, num_tokens, Hkv, 128] bf16.
 * past_lens   : device int32 [batch], each in [0, max_past_len].
 * max_past_len: host bound; sizes the split-K grid and the workspace.
 * lse         : NULL or device float [batch, num_tokens, Hq].
 * num_tokens  : 1 .. 64.
 * workspace   : as for duo_attn_decode, of duo_attn_decode_block_workspace_bytes()
 *               bytes (zero-filled once before first use).
 * q_prologue  : NULL or duo_prologue, applied to q at positions past_lens[b] + t;
 *               k_new must already hold the prologue's output.
 * epilogue    : NULL or duo_epilogue; gate [batch, num_tokens, Hq, 128] or
 *               [batch, num_tokens, Hq]. */
int duo_attn_decode_block(const duo_layer* layer, const duo_kv_cache* cache, int32_t batch,
                          const void* q, const void* k_new, const void* v_new, int32_t num_tokens,
                          const int32_t* past_lens, int64_t max_past_len, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, const duo_prologue* q_prologue,
                          const duo_epilogue* epilogue, void* stream);

/* Workspace size for duo_attn_decode_block; 0 on invalid arguments. Host only. */
size_t duo_attn_decode_block_workspace_bytes(const duo_layer* layer, int32_t batch,
                                             int32_t num_tokens, int64_t max_past_len);

/* Zero-fill a decode or prefill workspace (enqueued on `stream`; a small fill
 * kernel, so it is also safe under graph capture). */
int duo_attn_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Host only: the angular frequency f_i (radians per position) of each of the
 * 64 rotary pairs that the prologue uses for `rope` (YaRN blend included).
 * freqs: host double [64]. */
int duo_rope_frequencies(const duo_rope* rope, double* freqs);

/* The prologue on its own: y[b, t, h, :] = bf16(prologue(x[b, t, h, :])) at
 * position start_pos[b] + t (round to nearest even). Used for the K of a
 * prefill chunk or a verify block, which the attention reads before it is
 * appended (attend, then append; append it afterwards without a prologue).
 * x, y      : device bf16 [batch, num_tokens, heads, 128], 16-byte aligned;
 *             y == x works in place, other overlaps are undefined.
 * start_pos : device int32 [batch]; start_pos[b] + num_tokens must respect
 *             the position limit above (device data: not checked).
 * heads     : 1 .. 4096. One HBM pass over x and y. */
int duo_qk_prologue(const duo_prologue* prologue, int32_t batch, int32_t num_tokens, int32_t heads,
                    const void* x, void* y, const int32_t* start_pos, void* stream);

/* Workspace size for duo_attn_decode; 0 on invalid arguments. Host only. */
size_t duo_attn_decode_workspace_bytes(const duo_layer* layer, int32_t batch,
                                       int64_t max_seq_len);

/* Bytes of the static cache for `capacity` positions per sequence (model
 * card, "Changes In This Submission": static Duo KV cache). Host only.
 * main_bytes/stream_bytes receive the size of ONE of k/v for each class. */
int duo_kv_cache_bytes(const duo_layer* layer, int32_t batch, int64_t capacity,
                       int64_t* main_bytes, int64_t* stream_bytes);

/* Static-cache footprint and occupancy for sequences of the given lengths
 * (HOST array seq_lens[batch]), per head class, beside the same layer without
 * Duo routing (every KV head keeps its whole context). Host only, no GPU.
 * Model card "DuoAttention Laguna Adapter": "Benefits" (smaller KV-cache
 * footprint), "Changes In This Submission" (a static Duo KV cache).
 * Bytes count K and V together (2 x 128 bf16 per slot and head). Slots are
 * (sequence, head, slot) triples; a slot is occupied when duo_kv_append has
 * written a position there: min(len, slots per head) per sequence and head. */
typedef struct duo_cache_report {
  int64_t main_slots, stream_slots;     /* allocated, per class */
  int64_t main_active, stream_active;   /* occupied, per class */
  int64_t main_bytes, stream_bytes;     /* allocated K+V bytes, per class */
  int64_t base_slots, base_active;      /* the same layer with every head full context */
  int64_t base_bytes;
} duo_cache_report;

int duo_kv_cache_report(const duo_layer* layer, int32_t batch, int64_t capacity,
                        const int32_t* seq_lens, duo_cache_report* out);

/* Head-class plan (host only, no GPU): for each KV head, its class
 * (1 = streaming, 0 = full context) and its rank within the class. */
int duo_head_plan(const duo_layer* layer, int32_t* head_class, int32_t* head_rank,
                  int32_t* n_main, int32_t* n_stream);

/* Prefill work plan (host only): the number of workgroups the prefill launch
 * uses, with a workspace (with_workspace != 0) or without one; when `items`
 * is not NULL it receives, per workgroup, seven int32 (batch, q_head, q_tile,
 * key_tiles, piece, pieces, heads), or (-1, -1, -1, 0, 0, 0, 0) for padding:
 * the workgroup computes query heads q_head .. q_head + heads - 1 on the
 * q_tile-th duo_prefill_tile_rows()-row tile of the chunk, visiting key_tiles
 * 64-key tiles after masked tiles are skipped; piece / pieces are its
 * key-range piece and the number of non-empty pieces of its query tile (1
 * when the tile runs whole; a workgroup with key_tiles 0 is an empty piece). */
int duo_prefill_plan(const duo_layer* layer, int32_t batch, int32_t num_tokens,
                     int64_t start_pos, int32_t with_workspace, int32_t* items, int64_t* n_items);

/* Query rows per prefill work item of this layer (the q_tile unit of
 * duo_prefill_plan): 64 when a workgroup computes two query heads (even
 * group sizes), else 128. A negative duo_status on an invalid layer. */
int duo_prefill_tile_rows(const duo_layer* layer);

/* Decode work plan (host only): keys per split and number of split-K work
 * items; when `items` is not NULL it receives per item four int32
 * (batch, kv_head, split, class). */
int duo_decode_plan(const duo_layer* layer, int32_t batch, int64_t max_seq_len,
                    int32_t* split_keys, int32_t* items, int64_t* n_items);

/* Out-of-contract device data that kernels had to clamp (host only; a
 * checked mode for debugging). Device-side arguments (start_pos, seq_lens,
 * past_lens) cannot be validated before launch; where they break the
 * contracts above, the kernels keep every access inside the caller's buffers
 * (as those entries state) and record here that they did. Not defined by the
 * pages: it checks the library's own contracts (duo_kv_cache slots, the
 * max_seq_len / max_past_len bounds). Bits, or'ed since the last clear on the
 * current device:
 *   DUO_DEVICE_APPEND_PAST_CAPACITY: duo_kv_append dropped a position at or
 *     past a contiguous main cache's capacity;
 *   DUO_DEVICE_LENGTH_PAST_CAPACITY: a decode took a length past a
 *     contiguous main cache's capacity as that capacity;
 *   DUO_DEVICE_LENGTH_PAST_PLAN: a decode cut a length beyond its
 *     max_seq_len / max_past_len bound to the planned splits.
 * bits  : host output.
 * clear : nonzero zeroes the bits after they are read.
 * Waits for all work on the current device first. Calls still being issued
 * by other threads may set bits after the read. */
#define DUO_DEVICE_APPEND_PAST_CAPACITY 1u
#define DUO_DEVICE_LENGTH_PAST_CAPACITY 2u
#define DUO_DEVICE_LENGTH_PAST_PLAN 4u
int duo_device_errors(uint32_t* bits, int32_t clear);

const char* duo_last_error(void);
int duo_attn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DUO_ATTN_H */
