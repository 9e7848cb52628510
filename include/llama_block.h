/*
 * llama_block.h -- C ABI of a gfx950 (MI355X) library that runs the forward
 * pass of one Llama pre-norm decoder block:
 *
 *     h = x + Attn(RMSNorm_1(x)),     y = h + FFN(RMSNorm_2(h))
 *
 * ("Full Llama 3 transformer block", How it works; "The Evolving Transformer
 *  04 LLaMA", 06 BLOCK).  Attn = bias-free q/k/v projections, RoPE on q and k
 * (interleaved pairs (2i, 2i+1) turned by (start_pos+s) * theta^(-2i/d_head),
 * "The Evolving Transformer 04 LLaMA", 02 RoPE), a KV-cache write at start_pos
 * ("Full Llama 3 transformer block", How it works), causal grouped-query
 * attention in which query head h reads KV head floor(h / (n_heads/n_kv_heads))
 * ("The Evolving Transformer 04 LLaMA", 05 GQA), and the output projection.
 * FFN = down(SiLU(gate n) * up n) ("The Evolving Transformer 04 LLaMA",
 * 04 SWIGLU).  RMSNorm: v / sqrt(mean(v^2) + eps) * g (same page, 03 RMSNORM).
 *
 * Conventions
 *  - Every tensor pointer passed to init/forward is a DEVICE pointer (HIP
 *    device memory of the current device), row-major and densely packed.
 *  - Weights use the nn.Linear convention, weight[out][in]:
 *      wq [n_heads*d_head][d_model]   wk, wv [n_kv_heads*d_head][d_model]
 *      wo [d_model][n_heads*d_head]   w_gate, w_up [d_ff][d_model]
 *      w_down [d_model][d_ff]         attn_norm, ffn_norm [d_model]
 *    Head h owns rows/columns [h*d_head, (h+1)*d_head).
 *  - Activations x and out: [batch][seq_len][d_model].
 *  - Element type of x, out, the weights and the cache: cfg.dtype (fp32 or
 *    bf16).  Internally bf16 blocks run their matrix products with fp16 (or,
 *    on request, bf16) MFMA operands and fp32 accumulation; the residual
 *    stream h is kept in fp32.
 *  - Errors: every function validates its arguments before touching device
 *    memory, and an argument error (LB_ERR_INVALID_ARG, LB_ERR_UNSUPPORTED)
 *    launches nothing and writes nothing.  A forward that fails with
 *    LB_ERR_HIP (a launch refused by the runtime) stops at the failing
 *    kernel: the kernels before it have run, so `out`, the workspace and the
 *    cache rows [start_pos, start_pos + seq_len) of that call may be partly
 *    written; no other cache row is touched.  The text of the last error of a
 *    handle is available from llama_block_last_error().
 */
#ifndef LLAMA_BLOCK_H
#define LLAMA_BLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LB_F32 = 0, LB_BF16 = 1 } lb_dtype;

/* Operand type of the matrix-core products for bf16 blocks (ignored for fp32
 * blocks, which run in fp32 throughout).
 *   F16: bf16 weights are widened to fp16 at init and the activations that
 *     feed matrix products (RMSNorm outputs, q, k, v, the attention output
 *     and SiLU(gate)*up) are rounded to fp16: three more mantissa bits than
 *     bf16 at the same MFMA rate.  The residual stream stays fp32.  fp16's
 *     range is narrower than bf16's, so init checks, from the weights and
 *     gains on the device, bounds that hold for ANY input x: |RMSNorm out|
 *     <= sqrt(d_model) max|gain|; |q|, |k| <= sqrt(2) sqrt(d_model)
 *     max_j ||gain * W_j|| (RoPE turns pairs within their norm), |v| and the
 *     attention output <= sqrt(d_model) max_j ||gain * Wv_j||; |SiLU(gate)*up|
 *     <= d_model max_j ||g2 * Wgate_j|| ||g2 * Wup_j||.  Every bound and every
 *     |weight| must stay below 65504 (with a 2^-8 margin), and no weight row
 *     may change by more than 2^-11 of its norm when widened (bf16 values
 *     below 2^-17 lose bits in fp16).  Otherwise init returns
 *     LB_ERR_UNSUPPORTED.
 *   AUTO: F16 when that check passes, else BF16 (llama_block_operand_type
 *     tells which was taken).
 *   BF16: every operand in bf16 (8 significant bits).  An experimental mode:
 *     at the 8B width its operand rounding, amplified by the FFN, reaches
 *     about 2e-2 of rms(y) against an fp64 reference, so it is not held to
 *     the 2e-2 bar that F16 meets; its tests hold it to 4e-2. */
typedef enum { LB_OPERANDS_AUTO = 0, LB_OPERANDS_F16 = 1, LB_OPERANDS_BF16 = 2 } lb_operands;

typedef enum {
    LB_OK = 0,
    LB_ERR_INVALID_ARG = 1,  /* a pointer, size or config value is invalid */
    LB_ERR_UNSUPPORTED = 2,  /* valid, but a shape this library does not run */
    LB_ERR_OOM = 3,          /* device allocation failed */
    LB_ERR_HIP = 4           /* a HIP runtime call failed */
} lb_status;

/* Pairing of the rotated dimensions of a head.  INTERLEAVED turns (2i, 2i+1)
 * ("The Evolving Transformer 04 LLaMA", 02 RoPE); HALF turns (i, i + d_head/2),
 * the rotate_half form of "From GPT-2 to Llama", Positions become a rotation
 * (the layout the SmolLM2 / Hugging Face weights expect).  Either way q, k and
 * the K cache hold head dimensions in their natural order. */
typedef enum { LB_ROPE_INTERLEAVED = 0, LB_ROPE_HALF = 1 } lb_rope_layout;

typedef struct {
    int32_t d_model;      /* model width; must equal n_heads * d_head */
    int32_t n_heads;      /* query heads H */
    int32_t n_kv_heads;   /* key/value heads; must divide n_heads */
    int32_t d_head;       /* head width; even */
    int32_t d_ff;         /* SwiGLU inner width */
    int32_t max_tokens;   /* largest batch*seq_len of one forward (sizes the workspace) */
    int32_t max_seq_len;  /* RoPE table rows: every start_pos+seq_len must be <= this */
    double rope_theta;    /* rotation base theta (> 0) */
    double norm_eps;      /* RMSNorm epsilon (> 0), added to mean(v^2) inside the root */
    lb_dtype dtype;
    lb_operands operands;
    /* RoPE variants (all zero: interleaved pairs, no frequency scaling). */
    lb_rope_layout rope_layout;
    /* Frequency scaling as in Llama 3.1 ("From GPT-2 to Llama", Positions become
     * a rotation: the slowest pairs are slowed by the factor, the fastest left
     * alone, those between blended).  rope_scale_factor <= 1: none.  Otherwise,
     * with wavelength L = 2 pi / speed of a pair: L < original / high_freq_factor
     * keeps its speed, L > original / low_freq_factor is divided by the factor,
     * and between them the speed is (1-t) speed / factor + t speed with
     * t = (original / L - low) / (high - low).  Needs 0 < low < high and
     * original > 0. */
    double rope_scale_factor;
    double rope_low_freq_factor;
    double rope_high_freq_factor;
    double rope_original_max_pos;
} lb_config;

/* Device pointers in cfg.dtype, layouts as above.  init copies (and repacks)
 * them into library-owned memory: the caller may free them once init returns. */
typedef struct {
    const void *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm, *w_gate, *w_up, *w_down;
} lb_weights;

/* KV cache, caller-owned device memory in cfg.dtype:
 *   k: [batch][n_kv_heads][max_seq_len][d_head]   one row per position
 *   v: [batch][n_kv_heads][max_seq_len][d_head]   one row per position
 * (each (sequence, KV head) is one contiguous run of positions, so decode
 * streams both tensors with contiguous reads and appends contiguous rows).
 * A forward with start_pos p and seq_len S reads positions [0, p) of
 * sequences 0..B-1 and writes positions [p, p+S); no other entry changes.
 * The "Llama 4 From Scratch" worked example counts 2*n_kv*d_head values per
 * token per layer: exactly what one token adds here. */
typedef struct {
    void* k;
    void* v;
    int32_t batch;        /* sequences the cache holds (>= forward batch) */
    int32_t max_seq_len;  /* positions per sequence */
} lb_kv_cache;

typedef struct lb_block lb_block;

/* Create a block on the current HIP device: the set-up half of the pages'
 * block module ("Full Llama 3 transformer block", How it works: the block
 * holds the q/k/v/o projections, the two RMSNorm gains and the gate/up/down
 * FFN; the RoPE table freqs_cis is computed once, "The Evolving Transformer
 * 04 LLaMA", 02 RoPE).  Validates cfg: d_model ==
 * n_heads*d_head, n_heads % n_kv_heads == 0, d_head even, d_ff, max_tokens,
 * max_seq_len, rope_theta, norm_eps > 0 (LB_ERR_INVALID_ARG).  Supported
 * shapes (else LB_ERR_UNSUPPORTED): d_model <= 16384; bf16 blocks need d_head
 * in {64, 128}, d_model % 64 == 0, d_ff % 64 == 0 and n_heads/n_kv_heads <= 16;
 * fp32 blocks need d_head % 8 == 0, d_head <= 256, d_model % 8 == 0 and
 * d_ff % 4 == 0.  Packs the weights, builds
 * the RoPE cos/sin table (angles in fp64, stored as fp32) and allocates the
 * workspace.  Synchronous.  *out receives the handle (NULL on error). */
lb_status llama_block_init(const lb_config* cfg, const lb_weights* weights, lb_block** out);

/* One forward pass, the pages' forward(x, start_pos, freqs_cis, mask) ("Full
 * Llama 3 transformer block", How it works): freqs_cis is the handle's table
 * and the mask is the causal rule (key t is visible to the query at position
 * start_pos + s iff t <= start_pos + s), so neither is passed.  Enqueued on
 * `stream` (a hipStream_t; NULL = the null stream), asynchronous to the host.
 *   x   [batch][seq_len][d_model], device, cfg.dtype
 *   out [batch][seq_len][d_model], device, cfg.dtype; must not overlap x
 * seq_len == 1 runs the decode kernels, seq_len > 1 the prefill kernels; one
 * start_pos applies to every sequence.  Checks: batch, seq_len >= 1,
 * batch*seq_len <= max_tokens, start_pos >= 0, start_pos+seq_len <=
 * min(cfg.max_seq_len, kv->max_seq_len), batch <= kv->batch, non-null
 * pointers (LB_ERR_INVALID_ARG).  One call per handle may be in flight: the
 * workspace is shared by every call on the handle. */
lb_status llama_block_forward(lb_block* blk, const void* x, int32_t batch, int32_t seq_len,
                              int32_t start_pos, const lb_kv_cache* kv, void* out,
                              void* stream);

/* llama_block_forward with a start position per sequence, for batches whose
 * sequences have different lengths (decode of sequences at different
 * positions, or prefill chunks at different offsets): sequence b has its
 * queries at positions start_pos[b] + s, reads its cache positions
 * [0, start_pos[b]) and writes [start_pos[b], start_pos[b] + seq_len); no
 * other cache entry changes.  start_pos is a HOST array of `batch` values,
 * read during the call (they travel in the kernel arguments), so the caller
 * may reuse it as soon as the call returns.  batch <= LB_MAX_RAGGED_BATCH.
 * Checks as llama_block_forward, per sequence; a NULL start_pos is
 * LB_ERR_INVALID_ARG.  With every start_pos[b] equal it computes exactly what
 * llama_block_forward computes for that start_pos.  ("Full Llama 3
 * transformer block", How it works: the cache offset and the causal rule are
 * per sequence.) */
#define LB_MAX_RAGGED_BATCH 64
lb_status llama_block_forward_ragged(lb_block* blk, const void* x, int32_t batch,
                                     int32_t seq_len, const int32_t* start_pos,
                                     const lb_kv_cache* kv, void* out, void* stream);

/* For callers that cannot allocate device memory while they run (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * llama_block_forward for one decode step (seq_len == 1) whose scratch
 * buffers (normalised rows, q, the attention output and its split partials,
 * the fp32 residual, SiLU(gate)*up, split-K partials) live in one static device
 * array of LB_STATIC_SCRATCH_BYTES bytes per GPU, held by the library until
 * the process ends, instead of the handle's workspace.  It calls no
 * allocator.  Arguments as llama_block_forward with seq_len = 1; bf16 dense
 * blocks only, batch <= 64, and a block whose decode buffers do not fit the
 * array is refused with LB_ERR_UNSUPPORTED (the 70B width fits at 64
 * sequences).  The result equals llama_block_forward's for the same call.
 * Every call on one GPU shares that array, whatever the handle, and the array
 * keeps the last call's contents: calls that overlap on one GPU (other
 * streams, other threads) race, and the caller must serialise them.  The
 * stage buffers that llama_block_copy_stage reads are not written. */
#define LB_STATIC_SCRATCH_BYTES (32u << 20)
lb_status llama_block_forward_decode_static(lb_block* blk, const void* x, int32_t batch,
                                            int32_t start_pos, const lb_kv_cache* kv, void* out,
                                            void* stream);

/* ---- Mixture-of-experts blocks ----------------------------------------------
 * The FFN becomes a mixture of experts with a shared expert ("Llama 4 From
 * Scratch", The idea: N expert FFNs, a router that sends each token to its
 * top k, one always-on shared expert):
 *     FFN(n) = shared(n) + sum_{j<k} w_j expert_{e_j}(n)
 * where logits = n router^T (a bias-free linear layer), e_0..e_{k-1} are the
 * k largest logits (larger first; the lower expert index among equal
 * logits), w = softmax of those k logits, and every expert is a SwiGLU FFN
 * like the dense one.  The shared expert IS the block's dense FFN: the
 * lb_weights w_gate / w_up / w_down, width cfg.d_ff.  The page leaves the
 * router, the choice among equal scores and the weighting open; the rules
 * above are this library's reading.  Logits are fp32 dot products of the
 * operand-type n and router weights, so near-equal logits may be ordered
 * differently from an exact computation. */
typedef struct {
    int32_t n_experts;    /* routed experts E, 1..256 */
    int32_t top_k;        /* experts per token, 1..min(E, 8) */
    int32_t d_ff_expert;  /* width of each routed expert; a multiple of 64 */
} lb_moe_config;

/* Device pointers in cfg.dtype, experts stacked along the first index:
 *   router [E][d_model]   w_gate, w_up [E][d_ff_expert][d_model]
 *   w_down [E][d_model][d_ff_expert]
 * Copied (and repacked) by init. */
typedef struct {
    const void *router, *w_gate, *w_up, *w_down;
} lb_moe_weights;

/* Create a MoE block: weights as for llama_block_init (its FFN is the shared
 * expert) plus the routed experts.  bf16 blocks only (LB_ERR_UNSUPPORTED
 * otherwise).  The handle is used with llama_block_forward /
 * llama_block_forward_ragged / llama_block_destroy like any block; the
 * profiler's gate/up stage then covers the shared gate/up, the router, the
 * grouping and the experts' gate/up, and its down stage the shared and the
 * experts' down projections and the combine. */
lb_status llama_moe_block_init(const lb_config* cfg, const lb_weights* weights, const lb_moe_config* moe,
                               const lb_moe_weights* experts, lb_block** out);

/* Routing of the last forward of a MoE block, for its batch*seq_len token
 * rows: sel [rows][top_k] expert indices, weights [rows][top_k], logits
 * [rows][n_experts] (fp32).  Any pointer may be NULL; others receive a copy
 * (device or host memory) ordered on `stream`.  LB_ERR_INVALID_ARG for a
 * dense block. */
lb_status llama_block_copy_routing(lb_block* blk, int32_t* sel, float* weights, float* logits,
                                   void* stream);

/* Free the handle and everything it owns (synchronises the device first). */
void llama_block_destroy(lb_block* blk);

/* ---- Stacks of blocks ------------------------------------------------------
 * n_layers blocks of one config, each with its own weights and its own KV
 * cache, followed by the final RMSNorm ("The Evolving Transformer 04 LLaMA",
 * 07 ASSEMBLE LLAMA: token embedding, N blocks, final norm, output projection;
 * "Full Llama 3 transformer block", Overview: the block is the unit stacked L
 * times).  Block 0 maps x, block l maps block l-1's output, and
 *     y = RMSNorm(output of the last block) * final_norm   (eps = cfg.norm_eps).
 * The embedding and the output projection are not part of the stack.  Block
 * outputs pass from block to block in cfg.dtype.  The blocks share one
 * workspace, so one call per stack may be in flight. */
#define LB_MAX_STACK_LAYERS 1024
typedef struct lb_stack lb_stack;
typedef struct lb_stack_graph lb_stack_graph;

/* Create a stack on the current device: layers[0..n_layers) are the blocks'
 * weights (device pointers as for llama_block_init), final_norm [d_model]
 * the final gain in cfg.dtype.  Everything is copied; the caller may free its
 * tensors when the call returns.  Checks as llama_block_init, plus 1 <=
 * n_layers <= LB_MAX_STACK_LAYERS (LB_ERR_INVALID_ARG).  Synchronous. */
lb_status llama_stack_init(const lb_config* cfg, int32_t n_layers, const lb_weights* layers,
                           const void* final_norm, lb_stack** out);

/* One forward of the whole stack, enqueued on `stream`.
 *   x, out   [batch][seq_len][d_model] device, cfg.dtype; out must not overlap x
 *   kv       HOST array of n_layers caches (block l reads and writes kv[l],
 *            laid out as for llama_block_forward)
 *   hidden   optional device buffer [n_layers][batch][seq_len][d_model] in
 *            cfg.dtype that receives every block's output (NULL: kept in the
 *            workspace); must not overlap x or out
 *   starts   NULL: every sequence at start_pos; else a HOST array of batch
 *            start positions (batch <= LB_MAX_RAGGED_BATCH), as in
 *            llama_block_forward_ragged.
 * Checks as llama_block_forward against every cache. */
lb_status llama_stack_forward(lb_stack* st, const void* x, int32_t batch, int32_t seq_len,
                              int32_t start_pos, const int32_t* starts, const lb_kv_cache* kv,
                              void* out, void* hidden, void* stream);

/* llama_stack_forward with the start positions in DEVICE memory: positions
 * [batch] int32, read by the kernels when they run, so a captured graph of
 * this call can be replayed while the positions move.  Each value is clamped
 * to [0, min(cfg.max_seq_len, smallest cache max_seq_len) - seq_len] when it
 * is read: a position past the end rewrites the last rows of the cache instead
 * of leaving it, so callers stop before the capacity.  With advance != 0 a
 * last kernel adds seq_len to every position, after every read of them.
 * Launches are shaped for the largest start the clamp allows, which costs
 * decode launches with few (sequence, KV head) pairs some idle blocks. */
lb_status llama_stack_forward_device_pos(lb_stack* st, const void* x, int32_t batch,
                                         int32_t seq_len, int32_t* positions, int32_t advance,
                                         const lb_kv_cache* kv, void* out, void* hidden,
                                         void* stream);

/* Capture llama_stack_forward_device_pos(st, x, batch, seq_len, positions,
 * advance = 1, kv, out, hidden = NULL) into a HIP graph: each launch runs one
 * step of the stack at the current device positions and moves them on by
 * seq_len, with no host work but the launch.  x, out, positions and the
 * caches are bound at capture; the caller rewrites x (and, if it wishes,
 * positions) between launches.  Arguments are checked as for the eager call
 * before anything is captured.  Synchronous; the stack must outlive the
 * graph, and graph launches count as calls on the stack. */
lb_status llama_stack_graph_create(lb_stack* st, const void* x, int32_t batch, int32_t seq_len,
                                   int32_t* positions, const lb_kv_cache* kv, void* out,
                                   lb_stack_graph** g);
/* Enqueue one replay of the graph on `stream`. */
lb_status llama_stack_graph_launch(lb_stack_graph* g, void* stream);
/* Free the graph (synchronises the device first). */
void llama_stack_graph_destroy(lb_stack_graph* g);

/* Free the stack and everything it owns (synchronises the device first). */
void llama_stack_destroy(lb_stack* st);
int32_t llama_stack_num_layers(const lb_stack* st);
/* Last error text of the stack ("" if none); NULL: that of the last failed
 * llama_stack_init or llama_block_init on this thread. */
const char* llama_stack_last_error(const lb_stack* st);

/* Static text for a status code. */
const char* llama_block_status_string(lb_status s);

/* Text of the last error recorded on this handle ("" if none); with a NULL
 * handle, the last error of a failed llama_block_init on this thread. */
const char* llama_block_last_error(const lb_block* blk);

/* Intermediates of the last forward, for stage-by-stage checks.  They live in
 * the workspace, are valid until the next forward on the handle, and are
 * [batch*seq_len][cols] row-major:
 *   N1 RMSNorm_1(x) [d_model]     Q q after RoPE [n_heads*d_head]
 *   O attention output [n_heads*d_head]   H residual h, always fp32 [d_model]
 *   N2 RMSNorm_2(h) [d_model]     Z SiLU(gate)*up [d_ff]
 * Element type: fp32 for fp32 blocks and for H; otherwise the operand type.
 * MoE blocks add ROUTED: each routed expert's output for its token before
 * the routing weight ("Llama 4 From Scratch", The idea: the chosen expert
 * FFNs of a token), fp32 [batch*seq_len*top_k][d_model], row t*top_k + j for
 * choice j of token row t; its buffer holds top_k rows per token row, and it
 * is copied only to device memory (LB_ERR_INVALID_ARG for host memory or a
 * dense block). */
typedef enum { LB_STAGE_N1 = 0, LB_STAGE_Q = 1, LB_STAGE_O = 2, LB_STAGE_H = 3,
               LB_STAGE_N2 = 4, LB_STAGE_Z = 5, LB_STAGE_ROUTED = 6 } lb_stage;
typedef enum { LB_ELEM_F32 = 0, LB_ELEM_BF16 = 1, LB_ELEM_F16 = 2 } lb_elem;

/* Operand type the handle's matrix products run in: LB_ELEM_F32 for fp32
 * blocks, else LB_ELEM_F16 or LB_ELEM_BF16 as chosen by cfg.operands and the
 * range check of init (see lb_operands).  LB_ELEM_F32 for a NULL handle. */
lb_elem llama_block_operand_type(const lb_block* blk);
lb_elem llama_stack_operand_type(const lb_stack* st);

/* Device memory of a dense block or stack, in bytes as requested from the
 * allocator (it may round each allocation up), computed from the config alone
 * on the host: no GPU call, so a deployment can be sized before any weight
 * exists ("The Evolving Transformer 04 LLaMA", 07 ASSEMBLE LLAMA: a model is
 * N such blocks).  A block holds one copy of its weights, in the operand type
 * (2 bytes an element for bf16 blocks, 4 for fp32), plus its gains in fp32.
 *   n_layers   0: one block handle (llama_block_init); 1..LB_MAX_STACK_LAYERS:
 *              a stack of that many blocks (llama_stack_init)
 *   weights    the packed weights and gains of every block
 *   workspace  the RoPE table, activations and scratch one handle shares
 *              across its blocks (for a stack also the final gain and two
 *              activation buffers)
 *   init_staging  device memory init also holds while it packs (0 for fp32)
 * KV caches are the caller's and not counted.  MoE blocks are not covered.
 * Errors: NULL cfg or out, n_layers out of range, or any config that init
 * rejects (the same status and message as init). */
typedef struct lb_footprint {
    uint64_t weights;
    uint64_t workspace;
    uint64_t init_staging;
} lb_footprint;
lb_status llama_block_footprint(const lb_config* cfg, int32_t n_layers, lb_footprint* out);
/* Bytes a live handle holds (weights + workspace as above); 0 for NULL. */
uint64_t llama_block_device_bytes(const lb_block* blk);
uint64_t llama_stack_device_bytes(const lb_stack* st);

/* Describe a stage buffer: element type and columns per token row. */
lb_status llama_block_stage_info(const lb_block* blk, lb_stage which, lb_elem* elem,
                                 int64_t* cols);

/* Copy `bytes` bytes from the start of a stage buffer to dst (device or host
 * memory), ordered on `stream`.  bytes must not exceed the buffer. */
lb_status llama_block_copy_stage(lb_block* blk, lb_stage which, void* dst, size_t bytes,
                                 void* stream);

/* Per-stage GPU timing.  While enabled, each forward records HIP events
 * (timing only, no system-scope fence) on its stream at the boundaries of the
 * selected stages:
 *   0 RMSNorm_1   1 q/k/v projection (+RoPE, cache append)   2 attention
 *   3 o projection (+x)   4 RMSNorm_2   5 gate/up (+SiLU*up)   6 down (+h)
 * llama_block_profile(blk, mask) resets the sums and times the stages whose
 * bit is set in mask (LB_PROFILE_ALL: every stage; 0 stops).  Fewer stages
 * mean fewer events between kernels.  llama_block_profile_read waits for the
 * recorded events and returns the summed milliseconds per stage in
 * stage_ms[0..n) (n <= LB_NUM_STAGES; 0 for stages not timed) and the number
 * of profiled forwards in *calls. */
#define LB_NUM_STAGES 7
#define LB_PROFILE_ALL ((1u << LB_NUM_STAGES) - 1u)
lb_status llama_block_profile(lb_block* blk, uint32_t stage_mask);
lb_status llama_block_profile_read(lb_block* blk, double* stage_ms, int n, int64_t* calls);

#ifdef __cplusplus
}
#endif
#endif /* LLAMA_BLOCK_H */
