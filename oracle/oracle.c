/*
 * fp64 CPU oracle for the forward pass of one Llama pre-norm decoder block.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline timing).  Plain,
 * slow, obviously correct: one token row at a time, one dot product at a time,
 * no blocking, no fusion.  OpenMP only distributes independent rows over host
 * threads; every sum runs in the same sequential order whatever the thread
 * count, so results do not depend on it.
 *
 * Sources (cited by page title and section):
 *  [LL]  "The Evolving Transformer 04 LLaMA": 02 RoPE, 03 RMSNORM, 04 SWIGLU,
 *        05 GQA, 06 BLOCK.
 *  [L3]  "Full Llama 3 transformer block": How it works (residual equations,
 *        start_pos / cache offset), Watch-outs.
 *  [L4]  "Llama 4 From Scratch": The idea, Worked example.
 *  [ML]  "Mini Llama 2 Implementation": RMS normalization, Rotary positional
 *        embeddings (real/imaginary = adjacent pairs).
 *  [G2L] "From GPT-2 to Llama": Keys and values get shared (query-head to
 *        key/value-head grouping).
 *
 * Readings taken where the pages leave a step open:
 *  - RoPE pairs are the interleaved (2i, 2i+1) dimensions [LL 02; ML], at the
 *    absolute position start_pos + s [L3 How it works, Watch-outs].
 *  - Query head h reads key/value head floor(h / (H / n_kv)) [LL 05 repeat_kv
 *    expands each KV head over n_rep consecutive query heads; G2L].
 *  - Key t is visible to the query at absolute position m iff t <= m (the
 *    lower-triangular mask of [LL 05], offset by the cache [L3]).
 *  - SiLU(a) = a / (1 + exp(-a)) (Swish with beta 1) [LL 04; L4 The idea].
 *  - softmax is evaluated as exp(e_t - max e) / sum exp(e_s - max e), equal
 *    to exp(e_t) / sum exp(e_s) exactly in real arithmetic.
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* Host threads the oracle's parallel loops use (reported with its timings). */
int orc_num_threads(void)
{
    return omp_get_max_threads();
}

/* [LL 03 RMSNORM; L3 How it works; ML RMS normalization]:
 * out_k = v_k / sqrt(mean_j v_j^2 + eps) * g_k  -- no centring, no bias,
 * eps inside the root. */
void orc_rms_norm(const double* v, const double* g, int d, double eps, double* out)
{
    double ss = 0.0;
    for (int k = 0; k < d; ++k) ss += v[k] * v[k];
    const double r = 1.0 / sqrt(ss / (double)d + eps);
    for (int k = 0; k < d; ++k) out[k] = v[k] * r * g[k];
}

/* Bias-free projection, nn.Linear convention (weight [out][in]) [LL 05 wq/wk/wv/wo;
 * LL 04 w1/w2/w3]: out_j = sum_k in_k * w[j][k]. */
void orc_linear(const double* in, const double* w, int n_out, int n_in, double* out)
{
    for (int j = 0; j < n_out; ++j) {
        const double* row = w + (size_t)j * (size_t)n_in;
        double acc = 0.0;
        for (int k = 0; k < n_in; ++k) acc += in[k] * row[k];
        out[j] = acc;
    }
}

/* RoPE on one head vector [LL 02 RoPE; ML Rotary positional embeddings;
 * L4 Worked example]: pair i = (v[2i], v[2i+1]) is turned by the angle
 * pos * theta^(-2i/d_head):
 *   (u, w) -> (u cos a - w sin a,  u sin a + w cos a). */
void orc_rope(double* v, int d_head, long pos, double theta)
{
    for (int i = 0; i < d_head / 2; ++i) {
        const double freq = pow(theta, -2.0 * (double)i / (double)d_head);
        const double a = (double)pos * freq;
        const double c = cos(a), s = sin(a);
        const double u = v[2 * i], w = v[2 * i + 1];
        v[2 * i] = u * c - w * s;
        v[2 * i + 1] = u * s + w * c;
    }
}

/* Rotation speed of pair i under a block's RoPE settings [LL 02 RoPE: the
 * base speed theta^(-2i/d_head); G2L Positions become a rotation: Llama 3.1
 * keeps its original 8192-position context and stretches the slowest pairs by
 * its scale factor, leaves the fastest alone and blends the ones between].
 * Reading of the blend (the page names it only): with wavelength
 * L = 2 pi / speed, pairs with L < orig / high keep their speed, pairs with
 * L > orig / low are slowed by `scale`, and in between the speed is
 * (1 - t) * speed / scale + t * speed with t = (orig / L - low) / (high - low),
 * which meets both neighbours at the class boundaries.  With the page's
 * 8B settings (theta 500 000, 64 pairs, scale 8, low 1, high 4, orig 8192)
 * this makes 29 slow, 29 fast and 6 blended pairs, the page's counts. */
double orc_rope_freq(const orc_cfg* c, int i)
{
    const double speed = pow(c->rope_theta, -2.0 * (double)i / (double)c->d_head);
    if (!(c->rope_scale > 1.0)) return speed;
    const double two_pi = 6.283185307179586476925286766559;
    const double wavelen = two_pi / speed;
    if (wavelen < c->rope_orig / c->rope_high) return speed;
    if (wavelen > c->rope_orig / c->rope_low) return speed / c->rope_scale;
    const double t = (c->rope_orig / wavelen - c->rope_low) / (c->rope_high - c->rope_low);
    return (1.0 - t) * speed / c->rope_scale + t * speed;
}

/* RoPE on one head vector with a block's settings: pair i is (v[2i], v[2i+1])
 * [LL 02 RoPE; ML] or, in the rotate_half form, (v[i], v[i + d_head/2])
 * [G2L Positions become a rotation: q*cos + rotate_half(q)*sin], turned by
 * pos * orc_rope_freq(i) exactly as in orc_rope. */
void orc_rope_cfg(double* v, long pos, const orc_cfg* c)
{
    const int dh = c->d_head, half = dh / 2;
    for (int i = 0; i < half; ++i) {
        const double a = (double)pos * orc_rope_freq(c, i);
        const double cs = cos(a), sn = sin(a);
        const int iu = c->rope_half ? i : 2 * i, iw = c->rope_half ? i + half : 2 * i + 1;
        const double u = v[iu], w = v[iw];
        v[iu] = u * cs - w * sn;
        v[iw] = u * sn + w * cs;
    }
}

/* SiLU [LL 04 SWIGLU (F.silu); L4 The idea (Swish)]: a * sigmoid(a). */
double orc_silu(double a)
{
    return a / (1.0 + exp(-a));
}

/* Scaled dot-product attention of one query over n_keys key/value rows
 * [LL 05 GQA, the equation softmax(Q K^T / sqrt(dk)) V]:
 *   e_t = q . k_t / sqrt(d_head);  p = softmax(e);  out = sum_t p_t v_t.
 * k_rows, v_rows: [n_keys][d_head].  scratch: n_keys doubles. */
void orc_attend(const double* q, const double* k_rows, const double* v_rows, long n_keys,
                int d_head, double* scratch, double* out)
{
    const double scale = 1.0 / sqrt((double)d_head);
    double mx = -INFINITY;
    for (long t = 0; t < n_keys; ++t) {
        const double* kr = k_rows + (size_t)t * (size_t)d_head;
        double e = 0.0;
        for (int j = 0; j < d_head; ++j) e += q[j] * kr[j];
        e *= scale;
        scratch[t] = e;
        if (e > mx) mx = e;
    }
    double sum = 0.0;
    for (long t = 0; t < n_keys; ++t) {
        scratch[t] = exp(scratch[t] - mx);
        sum += scratch[t];
    }
    for (int j = 0; j < d_head; ++j) out[j] = 0.0;
    for (long t = 0; t < n_keys; ++t) {
        const double p = scratch[t] / sum;
        const double* vr = v_rows + (size_t)t * (size_t)d_head;
        for (int j = 0; j < d_head; ++j) out[j] += p * vr[j];
    }
}

/* One SwiGLU feed-forward of width f on n [L4 The idea; LL 04 SWIGLU]:
 * out = down(SiLU(gate n) * up n), gate/up [f][d], down [d][f]. */
static void swiglu(const double* n, const double* gate, const double* up, const double* down, int d,
                   int f, double* out)
{
    double* a = (double*)malloc(sizeof(double) * (size_t)f * 2);
    double* u = a + f;
    orc_linear(n, gate, f, d, a);
    orc_linear(n, up, f, d, u);
    for (int j = 0; j < f; ++j) a[j] = orc_silu(a[j]) * u[j];
    orc_linear(a, down, d, f, out);
    free(a);
}

int orc_moe_route(const orc_moe_cfg* m, int d, const double* n, const double* router, int* sel,
                  int force, double* wts, double* logits)
{
    const int E = m->n_experts, K = m->top_k;
    if (E < 1 || K < 1 || K > E) return -10;
    /* the router: a bias-free linear layer scoring every expert [L4 The idea] */
    orc_linear(n, router, E, d, logits);
    if (force) {
        for (int j = 0; j < K; ++j) {
            if (sel[j] < 0 || sel[j] >= E) return -11;
            for (int i = 0; i < j; ++i)
                if (sel[i] == sel[j]) return -11;
        }
    } else {
        /* the top-k: repeatedly the largest logit not yet taken, the lower
         * index first among equal logits */
        for (int j = 0; j < K; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                int taken = 0;
                for (int i = 0; i < j; ++i) taken |= sel[i] == e;
                if (!taken && (best < 0 || logits[e] > logits[best])) best = e;
            }
            sel[j] = best;
        }
    }
    /* weights: softmax over the chosen experts' logits */
    double mx = logits[sel[0]];
    for (int j = 1; j < K; ++j) mx = logits[sel[j]] > mx ? logits[sel[j]] : mx;
    double sum = 0.0;
    for (int j = 0; j < K; ++j) {
        wts[j] = exp(logits[sel[j]] - mx);
        sum += wts[j];
    }
    for (int j = 0; j < K; ++j) wts[j] /= sum;
    return 0;
}

/* out += sum_j wts[j] * expert_{sel[j]}(n), in the order of sel. */
static void moe_add_routed(const orc_moe_cfg* m, int d, const double* n, const orc_moe_weights* mw,
                           const int* sel, const double* wts, double* out)
{
    const int f = m->d_ff_expert;
    double* t = (double*)malloc(sizeof(double) * (size_t)d);
    for (int j = 0; j < m->top_k; ++j) {
        const size_t e = (size_t)sel[j];
        swiglu(n, mw->w_gate + e * (size_t)f * d, mw->w_up + e * (size_t)f * d,
               mw->w_down + e * (size_t)d * f, d, f, t);
        for (int i = 0; i < d; ++i) out[i] += wts[j] * t[i];
    }
    free(t);
}

int orc_moe_ffn(const orc_cfg* c, const orc_moe_cfg* m, const double* n, const orc_weights* w,
                const orc_moe_weights* mw, int* sel, int force, double* wts, double* logits,
                double* out)
{
    const int d = c->d;
    int rc = orc_moe_route(m, d, n, mw->router, sel, force, wts, logits);
    if (rc) return rc;
    swiglu(n, w->w_gate, w->w_up, w->w_down, d, c->d_ff, out); /* the shared expert */
    moe_add_routed(m, d, n, mw, sel, wts, out);
    return 0;
}

static int check_cfg(const orc_cfg* c, int B, int S, long start_pos, long cap)
{
    if (!c || c->d <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->d_head <= 0 || c->d_ff <= 0)
        return -1;
    if (c->n_heads % c->n_kv_heads != 0) return -2;
    if (c->d_head % 2 != 0) return -3;
    if (B < 0 || S < 0 || start_pos < 0 || start_pos + S > cap) return -4;
    if (c->rope_half != 0 && c->rope_half != 1) return -7;
    if (c->rope_scale > 1.0 && !(c->rope_low > 0.0 && c->rope_high > c->rope_low && c->rope_orig > 0.0))
        return -8;
    return 0;
}

static double* cache_row(double* cache, const orc_cfg* c, long cap, int b, int g, long t)
{
    return cache + (((size_t)b * (size_t)c->n_kv_heads + (size_t)g) * (size_t)cap + (size_t)t) *
                       (size_t)c->d_head;
}

/* One block [LL 06 BLOCK; L3 How it works]:
 *   h = x + Attn(RMSNorm_1(x)),   y = h + FFN(RMSNorm_2(h)),
 * Attn: q, k, v projections, RoPE on q and k, cache write of k and v at
 * start_pos + s [L3], causal grouped-query attention, output projection;
 * FFN: down(SiLU(gate n) * up n) [LL 04]. */
/* The block, with a dense FFN (mc == NULL) or with the MoE FFN, whose
 * shared expert is w's gate/up/down. */
static int block_forward(const orc_cfg* c, int B, int S, long start_pos, long cap, const double* x,
                         const orc_weights* w, double* k_cache, double* v_cache, double* y,
                         const int* rows, int n_rows, orc_stages* st, const orc_moe_cfg* mc,
                         const orc_moe_weights* mw, int* sel, int force, double* wts,
                         double* logits)
{
    int rc = check_cfg(c, B, S, start_pos, cap);
    if (rc) return rc;
    if (mc && (mc->n_experts < 1 || mc->top_k < 1 || mc->top_k > mc->n_experts || mc->d_ff_expert < 1 ||
               !mw || !sel || !wts || !logits))
        return -10;
    int moe_rc = 0;
    const int d = c->d, H = c->n_heads, G = c->n_kv_heads, dh = c->d_head, dff = c->d_ff;
    const int n_rep = H / G;
    const int qd = H * dh, kvd = G * dh;
    const long M = (long)B * S;

    /* Which rows are asked for, and how far each sequence needs its cache. */
    char* want = (char*)calloc((size_t)(M > 0 ? M : 1), 1);
    int* need = (int*)calloc((size_t)(B > 0 ? B : 1), sizeof(int));
    if (!want || !need) { free(want); free(need); return -5; }
    if (rows == NULL) {
        for (long r = 0; r < M; ++r) want[r] = 1;
        for (int b = 0; b < B; ++b) need[b] = S;
    } else {
        for (int i = 0; i < n_rows; ++i) {
            if (rows[i] < 0 || rows[i] >= M) { free(want); free(need); return -6; }
            want[rows[i]] = 1;
            const int b = rows[i] / S, s = rows[i] % S;
            if (s + 1 > need[b]) need[b] = s + 1;
        }
    }

    /* Steps 1-4 for every position a requested row can see: RMSNorm_1, the k
     * and v projections, RoPE on k, and the cache write at start_pos + s. */
    double* n1_all = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1) * (size_t)d);
    if (!n1_all) { free(want); free(need); return -5; }
#pragma omp parallel for schedule(dynamic, 1)
    for (long r = 0; r < M; ++r) {
        const int b = (int)(r / S), s = (int)(r % S);
        if (s >= need[b]) continue;
        double* n1 = n1_all + (size_t)r * d;
        double* kv = (double*)malloc(sizeof(double) * (size_t)kvd * 2);
        double* k = kv;
        double* v = kv + kvd;
        const long pos = start_pos + s;
        orc_rms_norm(x + (size_t)r * d, w->attn_norm, d, c->norm_eps, n1);
        orc_linear(n1, w->wk, kvd, d, k);
        orc_linear(n1, w->wv, kvd, d, v);
        for (int g = 0; g < G; ++g) {
            orc_rope_cfg(k + (size_t)g * dh, pos, c);
            memcpy(cache_row(k_cache, c, cap, b, g, pos), k + (size_t)g * dh, sizeof(double) * dh);
            memcpy(cache_row(v_cache, c, cap, b, g, pos), v + (size_t)g * dh, sizeof(double) * dh);
        }
        if (st && st->n1) memcpy(st->n1 + (size_t)r * d, n1, sizeof(double) * d);
        if (st && st->k) memcpy(st->k + (size_t)r * kvd, k, sizeof(double) * kvd);
        if (st && st->v) memcpy(st->v + (size_t)r * kvd, v, sizeof(double) * kvd);
        free(kv);
    }

    /* Steps 5-7 for each requested row. */
#pragma omp parallel for schedule(dynamic, 1)
    for (long r = 0; r < M; ++r) {
        if (!want[r]) continue;
        const int b = (int)(r / S), s = (int)(r % S);
        const long pos = start_pos + s;
        const long n_keys = pos + 1; /* causal: keys 0 .. pos */
        const double* n1 = n1_all + (size_t)r * d;
        const double* xr = x + (size_t)r * d;
        double* q = (double*)malloc(sizeof(double) * (size_t)qd);
        double* o = (double*)malloc(sizeof(double) * (size_t)qd);
        double* h = (double*)malloc(sizeof(double) * (size_t)d);
        double* n2 = (double*)malloc(sizeof(double) * (size_t)d);
        double* a = (double*)malloc(sizeof(double) * (size_t)dff);
        double* u = (double*)malloc(sizeof(double) * (size_t)dff);
        double* z = (double*)malloc(sizeof(double) * (size_t)dff);
        double* f = (double*)malloc(sizeof(double) * (size_t)d);
        double* scr = (double*)malloc(sizeof(double) * (size_t)n_keys);

        orc_linear(n1, w->wq, qd, d, q);
        for (int hh = 0; hh < H; ++hh) orc_rope_cfg(q + (size_t)hh * dh, pos, c);
        for (int hh = 0; hh < H; ++hh) {
            const int g = hh / n_rep;
            orc_attend(q + (size_t)hh * dh, cache_row(k_cache, c, cap, b, g, 0),
                       cache_row(v_cache, c, cap, b, g, 0), n_keys, dh, scr, o + (size_t)hh * dh);
        }
        /* h = x + o Wo^T */
        orc_linear(o, w->wo, d, qd, h);
        for (int i = 0; i < d; ++i) h[i] = xr[i] + h[i];
        /* y = h + down(SiLU(gate n2) * up n2) */
        orc_rms_norm(h, w->ffn_norm, d, c->norm_eps, n2);
        orc_linear(n2, w->w_gate, dff, d, a);
        orc_linear(n2, w->w_up, dff, d, u);
        for (int j = 0; j < dff; ++j) z[j] = orc_silu(a[j]) * u[j];
        orc_linear(z, w->w_down, d, dff, f);
        if (mc) {
            /* MoE: the FFN above is the always-on shared expert; add the
             * chosen experts, weighted [L4 The idea] */
            const int K = mc->top_k;
            int* sr = sel + (size_t)r * K;
            double* wr = wts + (size_t)r * K;
            const int rr = orc_moe_route(mc, d, n2, mw->router, sr, force, wr,
                                         logits + (size_t)r * mc->n_experts);
            if (rr) {
#pragma omp atomic write
                moe_rc = rr;
            } else {
                moe_add_routed(mc, d, n2, mw, sr, wr, f);
            }
        }
        for (int i = 0; i < d; ++i) y[(size_t)r * d + i] = h[i] + f[i];

        if (st && st->q) memcpy(st->q + (size_t)r * qd, q, sizeof(double) * qd);
        if (st && st->o) memcpy(st->o + (size_t)r * qd, o, sizeof(double) * qd);
        if (st && st->h) memcpy(st->h + (size_t)r * d, h, sizeof(double) * d);
        if (st && st->n2) memcpy(st->n2 + (size_t)r * d, n2, sizeof(double) * d);
        if (st && st->z) memcpy(st->z + (size_t)r * dff, z, sizeof(double) * dff);
        free(q); free(o); free(h); free(n2); free(a); free(u); free(z); free(f); free(scr);
    }
    free(n1_all);
    free(want);
    free(need);
    return moe_rc;
}

int orc_block_forward(const orc_cfg* c, int B, int S, long start_pos, long cap, const double* x,
                      const orc_weights* w, double* k_cache, double* v_cache, double* y,
                      const int* rows, int n_rows, orc_stages* st)
{
    return block_forward(c, B, S, start_pos, cap, x, w, k_cache, v_cache, y, rows, n_rows, st, NULL,
                         NULL, NULL, 0, NULL, NULL);
}

int orc_moe_block_forward(const orc_cfg* c, const orc_moe_cfg* m, int B, int S, long start_pos,
                          long cap, const double* x, const orc_weights* w, const orc_moe_weights* mw,
                          double* k_cache, double* v_cache, double* y, const int* rows, int n_rows,
                          int* sel, int force, double* wts, double* logits)
{
    if (!m) return -10;
    return block_forward(c, B, S, start_pos, cap, x, w, k_cache, v_cache, y, rows, n_rows, NULL, m,
                         mw, sel, force, wts, logits);
}

int orc_stack_forward(const orc_cfg* c, int n_layers, int B, int S, long start_pos, long cap,
                      const double* x, const orc_weights* layers, const double* final_norm,
                      double* const* k_caches, double* const* v_caches, double* hidden,
                      double* y)
{
    if (n_layers < 1 || !layers || !final_norm || !k_caches || !v_caches) return -9;
    int rc = check_cfg(c, B, S, start_pos, cap);
    if (rc) return rc;
    const int d = c->d;
    const long M = (long)B * S;
    const size_t n = (size_t)(M > 0 ? M : 1) * (size_t)d;
    double* buf[2] = {NULL, NULL};
    if (!hidden) {
        buf[0] = (double*)malloc(sizeof(double) * n);
        buf[1] = (double*)malloc(sizeof(double) * n);
        if (!buf[0] || !buf[1]) { free(buf[0]); free(buf[1]); return -5; }
    }
    /* the residual stream: each block maps the previous block's output */
    const double* stream = x;
    for (int l = 0; l < n_layers && rc == 0; ++l) {
        double* out = hidden ? hidden + (size_t)l * n : buf[l & 1];
        rc = orc_block_forward(c, B, S, start_pos, cap, stream, &layers[l], k_caches[l], v_caches[l],
                               out, NULL, 0, NULL);
        stream = out;
    }
    if (rc == 0) {
        for (long r = 0; r < M; ++r)
            orc_rms_norm(stream + (size_t)r * d, final_norm, d, c->norm_eps, y + (size_t)r * d);
    }
    free(buf[0]);
    free(buf[1]);
    return rc;
}
