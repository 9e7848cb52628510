/*
 * fp64 CPU oracle for the forward pass of one Llama pre-norm decoder block.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it.  The HIP library neither links
 * nor calls it, and the two share no source, header, table or helper.
 *
 * Every value is double precision; inputs are the exact (already quantised)
 * workload values widened to double.  All arrays are host memory, row-major.
 *
 * Layouts used by this oracle (its own choice, independent of the library):
 *   x, y            [B][S][d]
 *   wq              [H*d_head][d]      wk, wv [n_kv*d_head][d]
 *   wo              [d][H*d_head]
 *   w_gate, w_up    [d_ff][d]          w_down [d][d_ff]
 *   attn_norm, ffn_norm [d]
 *   k_cache, v_cache [B][n_kv][cap][d_head]  (one row per absolute position)
 */
#ifndef LLAMA_BLOCK_ORACLE_H
#define LLAMA_BLOCK_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int d, n_heads, n_kv_heads, d_head, d_ff;
    double rope_theta, norm_eps;
    /* RoPE variants ("From GPT-2 to Llama", Positions become a rotation):
     * rope_half = 0 turns the interleaved pairs (2i, 2i+1), 1 the pairs
     * (i, i + d_head/2) of the rotate_half form.  rope_scale > 1 stretches the
     * slow pairs as Llama 3.1 does (rope_low / rope_high: the low and high
     * frequency factors, rope_orig: the original context length); <= 1: none. */
    int rope_half;
    double rope_scale, rope_low, rope_high, rope_orig;
} orc_cfg;

typedef struct {
    const double *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm, *w_gate, *w_up, *w_down;
} orc_weights;

/* Optional per-row intermediates (any pointer may be NULL), all [B*S][...]:
 * n1 [d], q [H*d_head] (after RoPE), k, v [n_kv*d_head] (k after RoPE),
 * o [H*d_head] (concatenated heads), h [d], n2 [d], z [d_ff]. */
typedef struct {
    double *n1, *q, *k, *v, *o, *h, *n2, *z;
} orc_stages;

int orc_num_threads(void);

/* Single steps, exposed so tests can pin each one on its own. */
void orc_rms_norm(const double* v, const double* g, int d, double eps, double* out);
void orc_linear(const double* in, const double* w, int n_out, int n_in, double* out);
void orc_rope(double* v, int d_head, long pos, double theta);
double orc_rope_freq(const orc_cfg* c, int i);
void orc_rope_cfg(double* v, long pos, const orc_cfg* c);
double orc_silu(double a);
void orc_attend(const double* q, const double* k_rows, const double* v_rows, long n_keys,
                int d_head, double* scratch, double* out);

/* Whole block.  Reads cache rows [0, start_pos) of every sequence, writes rows
 * [start_pos, start_pos+S).  rows/n_rows (optional): compute y (and stages)
 * only for these flat row indices b*S+s; the cache is still written for every
 * position up to the last requested one of each sequence.  rows == NULL
 * computes every row.  Returns 0, or a negative code for an invalid argument. */
int orc_block_forward(const orc_cfg* cfg, int B, int S, long start_pos, long cap,
                      const double* x, const orc_weights* w, double* k_cache, double* v_cache,
                      double* y, const int* rows, int n_rows, orc_stages* stages);

/* Mixture-of-experts FFN ("Llama 4 From Scratch", The idea: N expert FFNs,
 * a router sending each token to the top k, one always-on shared expert).
 * Readings where the page is silent: the router is a bias-free linear layer
 * [E][d]; the top k are the k largest logits, larger first, the lower expert
 * index first among equal logits; the chosen experts are weighted by the
 * softmax of their logits; every expert, the shared one included, is a
 * SwiGLU FFN.  The shared expert is the block's own FFN (orc_weights
 * w_gate/w_up/w_down, width cfg.d_ff). */
typedef struct {
    int n_experts, top_k, d_ff_expert;
} orc_moe_cfg;

typedef struct {
    const double* router;  /* [E][d] */
    const double* w_gate;  /* [E][d_ff_expert][d] */
    const double* w_up;    /* [E][d_ff_expert][d] */
    const double* w_down;  /* [E][d][d_ff_expert] */
} orc_moe_weights;

/* Routing of one normalised row n [d]: logits [E] = n router^T; sel [k]
 * receives the top k (or, with force != 0, holds the experts to use, which
 * must be distinct and in range); wts [k] their softmax weights.  Returns 0
 * or a negative code. */
int orc_moe_route(const orc_moe_cfg* m, int d, const double* n, const double* router, int* sel,
                  int force, double* wts, double* logits);
/* out [d] = shared(n) + sum_j wts[j] * expert_{sel[j]}(n), routing as above. */
int orc_moe_ffn(const orc_cfg* c, const orc_moe_cfg* m, const double* n, const orc_weights* w,
                const orc_moe_weights* mw, int* sel, int force, double* wts, double* logits,
                double* out);
/* The block with the MoE FFN: y = h + MoE(RMSNorm_2(h)), everything else as
 * orc_block_forward.  sel [B*S][k] (in with force, else out), wts [B*S][k],
 * logits [B*S][E] per row. */
int orc_moe_block_forward(const orc_cfg* c, const orc_moe_cfg* m, int B, int S, long start_pos,
                          long cap, const double* x, const orc_weights* w, const orc_moe_weights* mw,
                          double* k_cache, double* v_cache, double* y, const int* rows, int n_rows,
                          int* sel, int force, double* wts, double* logits);

/* A stack of n_layers blocks and the final RMSNorm: block l takes the output
 * of block l-1 (block 0 takes x), and y = RMSNorm(output of the last block)
 * with gain final_norm and the config's epsilon ("The Evolving Transformer 04
 * LLaMA", 07 ASSEMBLE LLAMA; "Full Llama 3 transformer block", Overview: the
 * block is the unit stacked L times; embedding and output projection are not
 * part of this function).  layers, k_caches, v_caches: n_layers entries, block
 * l reading and writing its own cache pair as orc_block_forward does.
 * hidden (optional, may be NULL): [n_layers][B][S][d] receives each block's
 * output.  Returns 0, or a negative code for an invalid argument. */
int orc_stack_forward(const orc_cfg* cfg, int n_layers, int B, int S, long start_pos, long cap,
                      const double* x, const orc_weights* layers, const double* final_norm,
                      double* const* k_caches, double* const* v_caches, double* hidden,
                      double* y);

#ifdef __cplusplus
}
#endif
#endif
