/*
 * CPU oracle for the routed-expert MoE feed-forward layer of the
 * HunyuanImage-3.0 decoder.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline use it. It shares no code, header, table or constant with the
 * HIP implementation.
 *
 * It is written to be checked by eye against the pages, not to be fast:
 * plain loops, fp64 arithmetic (except the router, which the pages keep in
 * fp32: its logits are rounded once to fp32 and its softmax, selection and
 * renormalisation run in fp32), and one rounding at each point where the
 * layer stores a value in its working precision. OpenMP parallelises over token
 * rows only, so results do not depend on the thread count.
 *
 * What it computes, per real (non-padding) token row x of length H:
 *
 *   1. Router logits l[e] = sum_h x[h] * Wr[e,h] for e < E.  The gate linear
 *      is kept in fp32 (HunyuanImage-3.0 model-coverage page, "Train":
 *      the router stays in fp32, gate_precision float32; model API page,
 *      HunyuanImage3ForCausalMM: 'mlp.gate' is in _keep_in_fp32_modules_strict),
 *      so the exact dot product (fp64; products of bf16/fp32 by fp32 are exact
 *      in fp64) is rounded once to fp32.
 *   2. p = softmax(l) over ALL E experts (model API page, build_moe_config:
 *      softmax over all experts, top-k, renormalized, one shared expert),
 *      in fp32 like the rest of the router: m = max l, s[e] = expf(l[e] - m)
 *      (host libm), Z = sum of s in ascending e, p[e] = s[e] / Z.
 *   3. Top-K: the K experts with the largest p. Softmax preserves the order
 *      of the logits strictly, so this is the K largest logits; the choice is
 *      made on the fp32 logits, because fp32 p can underflow and make
 *      distinct logits tie. On equal logits the lower expert index is taken
 *      first. Output order: descending logit (so non-increasing weight), ties
 *      by ascending index. A NaN logit counts as -infinity in steps 2-4.
 *   4. Renormalise: w[k] = p[idx[k]] / sum_k' p[idx[k']], sum in k order,
 *      in fp32.
 *   5. For each selected expert e: [u; g] = W13[e] x with W13[e] of shape
 *      [2I, H] holding the up rows first and the gate rows second
 *      (layers API page, HunyuanSharedMLP: gate_and_up_proj holds [up; gate],
 *      up first; model-coverage page: fused [up; gate] expert projections
 *      converted to grouped experts); h = SiLU(g) * u with
 *      SiLU(z) = z / (1 + exp(-z)); h is an activation, stored in the layer's
 *      dtype (rounded once: bf16 round-to-nearest-even, or fp32);
 *      y_e = W2[e] h with W2[e] of shape [H, I] (down_proj), kept unrounded.
 *   6. Shared expert (model API page, HunyuanImage3Block: routed experts plus
 *      the fused shared expert; report section 3.1.1: one shared MLP): the
 *      same SwiGLU with Ws13 [2Is, H], Ws2 [H, Is], applied to every real
 *      token and added without any weight.
 *   7. out = (((w[0] y_0 + w[1] y_1) + ...) + w[K-1] y_{K-1}) + y_shared,
 *      rounded once to the layer's dtype.
 *   8. Padding rows (padding_mask true at padding, model API page,
 *      HunyuanImage3Block.forward): x is not read, out is not written, and the
 *      route outputs are idx = -1, w = 0.
 *
 * orc_rmsnorm adds the block's normalisation in front of the layer (the
 * residual add after the layer is composed in the Python wrapper).
 *
 * dtype codes: 0 = fp32, 1 = bf16 (uint16 bit patterns).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

/* ------------------------------------------------------------ numbers */

static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double elem(const void *base, int dtype, int64_t i)
{
    if (dtype == ORC_BF16)
        return bf16_bits_to_double(((const uint16_t *)base)[i]);
    return (double)((const float *)base)[i];
}

/* Nearest bf16 value to v, ties to even, computed directly from the double
 * (no intermediate fp32 rounding). bf16 keeps 8 significant bits and fp32's
 * exponent range. */
static double round_bf16(double v)
{
    if (v == 0.0 || isnan(v) || isinf(v))
        return v;
    double a = fabs(v);
    int e;
    frexp(a, &e);                    /* a = m * 2^e, m in [0.5, 1) */
    int q = e - 8;                   /* spacing of 8-bit significands */
    if (q < -133)
        q = -133;                    /* bf16 subnormal spacing 2^-133 */
    double r = rint(ldexp(a, -q));   /* default rounding: nearest, ties even */
    double out = ldexp(r, q);
    if (out > 3.3895313892515355e38) /* beyond the largest finite bf16 */
        out = INFINITY;
    return v < 0 ? -out : out;
}

static double round_dtype(double v, int dtype)
{
    if (dtype == ORC_BF16)
        return round_bf16(v);
    return (double)(float)v;
}

static void store_dtype(void *base, int dtype, int64_t i, double rounded)
{
    float f = (float)rounded; /* exact: rounded is already representable */
    if (dtype == ORC_BF16) {
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        ((uint16_t *)base)[i] = (uint16_t)(u >> 16);
    } else {
        ((float *)base)[i] = f;
    }
}

/* ------------------------------------------------------------ router */

/* Step 1 for one token row: logits in fp32. */
static void router_logits_row(const void *x, int dtype, int64_t t, int64_t H,
                              const float *w_router, int E, float *logits)
{
    for (int e = 0; e < E; e++) {
        double acc = 0.0;
        for (int64_t h = 0; h < H; h++)
            acc += elem(x, dtype, t * H + h) * (double)w_router[(int64_t)e * H + h];
        logits[e] = (float)acc;
    }
}

/* Steps 2-4 for one row: softmax over all experts, top-K, renormalise
 * (fp32). */
static void softmax_topk_row(const float *logits_in, int E, int K,
                             float *probs, int32_t *idx, float *w)
{
    /* A NaN logit (from a NaN weight or input) counts as -infinity: ranked
     * after every number (equal values by index) and given probability 0,
     * so exactly K distinct experts are always selected. */
    float logits[1024];
    for (int e = 0; e < E; e++)
        logits[e] = isnan(logits_in[e]) ? -INFINITY : logits_in[e];
    float m = E > 0 ? logits[0] : -INFINITY;
    for (int e = 1; e < E; e++)
        if (logits[e] > m)
            m = logits[e];
    float z = 0.0f;
    for (int e = 0; e < E; e++) {
        probs[e] = expf(logits[e] - m);
        z += probs[e];
    }
    for (int e = 0; e < E; e++)
        probs[e] = probs[e] / z;

    char taken[1024];
    memset(taken, 0, sizeof taken);
    for (int k = 0; k < K; k++) {
        int best = -1;
        for (int e = 0; e < E; e++) {
            if (taken[e])
                continue;
            if (best < 0 || logits[e] > logits[best]) /* strict: lower index wins ties */
                best = e;
        }
        idx[k] = best;
        taken[best] = 1;
    }
    float s = 0.0f;
    for (int k = 0; k < K; k++)
        s += probs[idx[k]];
    for (int k = 0; k < K; k++)
        w[k] = probs[idx[k]] / s;
}

/* ------------------------------------------------------------ expert */

/* Step 5 (and 6): one SwiGLU expert on one token row xr (already in fp64).
 * w_up_gate: [2*I, H] with the up rows first; w_down: [H, I]. */
static void swiglu_row(const double *xr, const void *w_up_gate, const void *w_down,
                       int dtype, int64_t H, int64_t I, double *hbuf, double *y)
{
    for (int64_t i = 0; i < I; i++) {
        double u = 0.0, g = 0.0;
        for (int64_t h = 0; h < H; h++) {
            u += xr[h] * elem(w_up_gate, dtype, i * H + h);
            g += xr[h] * elem(w_up_gate, dtype, (I + i) * H + h);
        }
        double silu_g = g / (1.0 + exp(-g));
        hbuf[i] = round_dtype(silu_g * u, dtype);
    }
    for (int64_t j = 0; j < H; j++) {
        double acc = 0.0;
        for (int64_t i = 0; i < I; i++)
            acc += hbuf[i] * elem(w_down, dtype, j * I + i);
        y[j] = acc;
    }
}

static size_t expert_up_gate_elems(int64_t H, int64_t I) { return (size_t)(2 * I * H); }
static size_t expert_down_elems(int64_t H, int64_t I) { return (size_t)(H * I); }

static const void *offset_elems(const void *base, int dtype, size_t n)
{
    if (dtype == ORC_BF16)
        return (const uint16_t *)base + n;
    return (const float *)base + n;
}

/* ------------------------------------------------------------ public API */

/*
 * Router only, for the listed rows: fp32 logits [nrows, E], fp32 softmax
 * probabilities [nrows, E] (nullable), top-K ids [nrows, K] and fp32
 * renormalised weights [nrows, K]. Padding rows give idx = -1, w = 0 and do not read x.
 */
void orc_route(const void *x, int dtype, const float *w_router, const uint8_t *pad,
               int64_t H, int E, int K, const int64_t *rows, int64_t nrows,
               float *logits, float *probs, int32_t *idx, float *w)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; r++) {
        int64_t t = rows[r];
        float pbuf[1024];
        if (pad && pad[t]) {
            for (int e = 0; e < E; e++) {
                if (logits) logits[r * E + e] = 0.0f;
                if (probs) probs[r * E + e] = 0.0f;
            }
            for (int k = 0; k < K; k++) {
                idx[r * K + k] = -1;
                w[r * K + k] = 0.0f;
            }
            continue;
        }
        float lbuf[1024];
        router_logits_row(x, dtype, t, H, w_router, E, lbuf);
        softmax_topk_row(lbuf, E, K, pbuf, idx + r * K, w + r * K);
        for (int e = 0; e < E; e++) {
            if (logits) logits[r * E + e] = lbuf[e];
            if (probs) probs[r * E + e] = pbuf[e];
        }
    }
}

/*
 * The whole layer for the listed rows.
 *
 * If idx_in/w_in are given ([nrows, K]), they replace the router's choice
 * (used where two selections are both correct); otherwise steps 1-4 run.
 * idx_out/w_out ([nrows, K], nullable) receive the routes used.
 * out_exact ([nrows, H] fp64, nullable) receives the value before the final
 * rounding; out ([nrows, H] in dtype, nullable) the rounded output.
 * Padding rows: x not read, out/out_exact not written, idx -1, w 0.
 */
void orc_moe_rows(const void *x, int dtype, const float *w_router,
                  const void *w13, const void *w2, const void *ws13, const void *ws2,
                  const uint8_t *pad, int64_t H, int E, int K, int64_t I, int64_t Is,
                  const int64_t *rows, int64_t nrows,
                  const int32_t *idx_in, const double *w_in,
                  int32_t *idx_out, double *w_out, double *out_exact, void *out)
{
    int64_t Imax = I > Is ? I : Is;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; r++) {
        int64_t t = rows[r];
        if (pad && pad[t]) {
            for (int k = 0; k < K; k++) {
                if (idx_out) idx_out[r * K + k] = -1;
                if (w_out) w_out[r * K + k] = 0.0;
            }
            continue;
        }
        int32_t idx[1024];
        double w[1024];
        if (idx_in) {
            for (int k = 0; k < K; k++) {
                idx[k] = idx_in[r * K + k];
                w[k] = w_in[r * K + k];
            }
        } else {
            float lbuf[1024], pbuf[1024], wf[1024];
            router_logits_row(x, dtype, t, H, w_router, E, lbuf);
            softmax_topk_row(lbuf, E, K, pbuf, idx, wf);
            for (int k = 0; k < K; k++)
                w[k] = (double)wf[k];
        }
        double *xr = malloc(sizeof(double) * (size_t)H);
        double *hb = malloc(sizeof(double) * (size_t)Imax);
        double *y = malloc(sizeof(double) * (size_t)H);
        double *acc = malloc(sizeof(double) * (size_t)H);
        for (int64_t h = 0; h < H; h++)
            xr[h] = elem(x, dtype, t * H + h);
        for (int64_t j = 0; j < H; j++)
            acc[j] = 0.0;
        for (int k = 0; k < K; k++) {
            int e = idx[k];
            swiglu_row(xr, offset_elems(w13, dtype, (size_t)e * expert_up_gate_elems(H, I)),
                       offset_elems(w2, dtype, (size_t)e * expert_down_elems(H, I)),
                       dtype, H, I, hb, y);
            for (int64_t j = 0; j < H; j++)
                acc[j] += w[k] * y[j];
        }
        swiglu_row(xr, ws13, ws2, dtype, H, Is, hb, y);
        for (int64_t j = 0; j < H; j++) {
            double v = acc[j] + y[j];
            if (out_exact) out_exact[r * H + j] = v;
            if (out) store_dtype(out, dtype, r * H + j, round_dtype(v, dtype));
        }
        for (int k = 0; k < K; k++) {
            if (idx_out) idx_out[r * K + k] = idx[k];
            if (w_out) w_out[r * K + k] = w[k];
        }
        free(xr);
        free(hb);
        free(y);
        free(acc);
    }
}

/*
 * Dense brute force for the listed rows: every one of the E experts is
 * evaluated and weighted by its renormalised gate weight if it is among the
 * given routes (idx/w, [nrows, K]) and by zero otherwise; then the shared
 * expert is added. Summation runs in expert-index order. Output is the fp64
 * value before rounding, [nrows, H]. Padding rows are not written.
 */
void orc_moe_dense_rows(const void *x, int dtype, const void *w13, const void *w2,
                        const void *ws13, const void *ws2, const uint8_t *pad,
                        int64_t H, int E, int K, int64_t I, int64_t Is,
                        const int64_t *rows, int64_t nrows,
                        const int32_t *idx, const double *w, double *out_exact)
{
    int64_t Imax = I > Is ? I : Is;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; r++) {
        int64_t t = rows[r];
        if (pad && pad[t])
            continue;
        double *xr = malloc(sizeof(double) * (size_t)H);
        double *hb = malloc(sizeof(double) * (size_t)Imax);
        double *y = malloc(sizeof(double) * (size_t)H);
        double *acc = malloc(sizeof(double) * (size_t)H);
        for (int64_t h = 0; h < H; h++)
            xr[h] = elem(x, dtype, t * H + h);
        for (int64_t j = 0; j < H; j++)
            acc[j] = 0.0;
        for (int e = 0; e < E; e++) {
            double we = 0.0;
            for (int k = 0; k < K; k++)
                if (idx[r * K + k] == e)
                    we = w[r * K + k];
            swiglu_row(xr, offset_elems(w13, dtype, (size_t)e * expert_up_gate_elems(H, I)),
                       offset_elems(w2, dtype, (size_t)e * expert_down_elems(H, I)),
                       dtype, H, I, hb, y);
            for (int64_t j = 0; j < H; j++)
                acc[j] += we * y[j];
        }
        swiglu_row(xr, ws13, ws2, dtype, H, Is, hb, y);
        for (int64_t j = 0; j < H; j++)
            out_exact[r * H + j] = acc[j] + y[j];
        free(xr);
        free(hb);
        free(y);
        free(acc);
    }
}

/* Round an fp64 array to bf16 bit patterns (used by tests for the
 * tolerance-attainability check). */
/*
 * The block's normalisation before the experts (model API page,
 * HunyuanImage3Block: a pre-norm decoder layer, post_attention_layernorm
 * ahead of the routed and shared experts; layers API page, HunyuanRMSNorm:
 * normalizes in fp32 over the last axis and returns weight * x in the input
 * dtype, eps 1e-5 by default). For every real row t:
 *   m   = mean over h of x[t,h]^2: accumulated in fp64 (the squares are
 *         exact), divided by H and rounded to fp32
 *   d   = m + eps in fp32 (eps taken as an fp32 number)
 *   r   = 1 / sqrt(d), rounded once to fp32
 *   n_h = x[t,h] * r in fp32, then converted to the input dtype
 *   xn  = weight[h] * n_h in the input dtype (the product of two dtype
 *         values is exact in fp64 and rounded once)
 * Padding rows are neither read nor written.
 */
void orc_rmsnorm(const void *x, int dtype, const void *weight, double eps,
                 const uint8_t *pad, int64_t T, int64_t H, void *xn)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        if (pad && pad[t])
            continue;
        double ss = 0.0;
        for (int64_t h = 0; h < H; h++) {
            double v = elem(x, dtype, t * H + h);
            ss += v * v;
        }
        float m = (float)(ss / (double)H);
        float d = m + (float)eps;
        float r = (float)(1.0 / sqrt((double)d));
        for (int64_t h = 0; h < H; h++) {
            float p = (float)(elem(x, dtype, t * H + h) * (double)r);
            double n = round_dtype((double)p, dtype);
            store_dtype(xn, dtype, t * H + h, round_dtype(elem(weight, dtype, h) * n, dtype));
        }
    }
}

/*
 * Backward of the block's RMSNorm (fine-tuning the decoder block:
 * model-coverage page, "Train"; the forward is orc_rmsnorm). Given
 * g = dL/dxn (fp64 [T,H]) on the real rows: the derivative of
 * xn = weight * x * r(x), r = (mean over h of x^2 + eps)^(-1/2), taken at the
 * forward's fp32 r, with the roundings of n and xn passed straight through:
 *   dweight[h] += g[t,h] * n[t,h]  (n = the forward's dtype(x r); rows in
 *                                   ascending order)
 *   v_h = weight[h] g[t,h],  s = sum over h of x_h v_h
 *   dx[t,h] = r v_h - r^3 x_h s / H
 * (d r / d x_h = -r^3 x_h / H). With mg (the magnitudes of g, nullable), mdx
 * and mdw (nullable) receive the matching magnitudes:
 *   mdx = r |w_h| mg_h + r^3 |x_h| (sum over h of |x_h w_h| mg_h) / H,
 *   mdw += mg_h |n_h|.
 * Padding rows are neither read nor written. Single-threaded.
 */
void orc_rmsnorm_backward(const void *x, int dtype, const void *weight, double eps,
                          const uint8_t *pad, int64_t T, int64_t H, const double *g,
                          const double *mg, double *dx, double *dw, double *mdx, double *mdw)
{
    if (dw) memset(dw, 0, sizeof(double) * (size_t)H);
    if (mdw) memset(mdw, 0, sizeof(double) * (size_t)H);
    for (int64_t t = 0; t < T; t++) {
        if (pad && pad[t])
            continue;
        double ss = 0.0;
        for (int64_t h = 0; h < H; h++) {
            double v = elem(x, dtype, t * H + h);
            ss += v * v;
        }
        float m = (float)(ss / (double)H);
        float d = m + (float)eps;
        double r = (double)(float)(1.0 / sqrt((double)d));
        double s = 0.0, ms = 0.0;
        for (int64_t h = 0; h < H; h++) {
            double xv = elem(x, dtype, t * H + h);
            double wv = elem(weight, dtype, h);
            double n = round_dtype((double)(float)(xv * r), dtype);
            double gv = g[t * H + h];
            if (dw) dw[h] += gv * n;
            if (mdw && mg) mdw[h] += mg[t * H + h] * fabs(n);
            s += xv * (wv * gv);
            if (mg) ms += fabs(xv * wv) * mg[t * H + h];
        }
        for (int64_t h = 0; h < H; h++) {
            double xv = elem(x, dtype, t * H + h);
            double wv = elem(weight, dtype, h);
            if (dx) dx[t * H + h] = r * (wv * g[t * H + h]) - r * r * r * xv * s / (double)H;
            if (mdx && mg)
                mdx[t * H + h] = r * fabs(wv) * mg[t * H + h] + r * r * r * fabs(xv) * ms / (double)H;
        }
    }
}

/*
 * Backward pass of the layer (for the pages' fine-tuning: HunyuanImage-3.0
 * model-coverage page, "Train": LoRA and full fine-tuning of the MoE
 * decoder). Given dout = dL/dout for the real rows, the gradients of
 * L = sum_t dout[t] . out[t] with respect to x and every weight, with the
 * routes held fixed (top-k selection is piecewise constant; its gradient
 * flows only through the renormalised weights), evaluated at the forward's
 * stored values: the router's fp32 p and w, the SwiGLU activation h rounded
 * to the dtype as the forward stores it, the pre-activations u, g and every
 * product exact (fp64). Per real row t, for each routed k (expert e, weight
 * w_k) and then the shared expert (weight 1):
 *   y_k   = W2[e] h_k                      (h_k = dtype(SiLU(g) u))
 *   dw_k  = dout . y_k,  dy_k = w_k dout
 *   dW2[e]  += dy_k h_k^T,  dh = W2[e]^T dy_k
 *   du = dh SiLU(g),  dg = dh u SiLU'(g),  SiLU'(g) = s (1 + g (1 - s)),
 *        s = 1 / (1 + exp(-g))
 *   dW13[e] += [du; dg] x^T (up rows first),  dx += W13[e]^T [du; dg]
 * Router: w_k = p_k / S with S = sum of the selected p, so for a selected j
 *   dp_j = (dw_j - sum_k w_k dw_k) / S  (0 for the others);
 *   softmax: dl_e = p_e (dp_e - sum_j p_j dp_j);
 *   dWr += dl x^T,  dx += Wr^T dl.
 * idx_in / w_in ([T, K]) replace the router's choice when given (p is still
 * the router's). Weight gradients are summed over tokens in ascending t
 * (single-threaded, deterministic); padding rows contribute nothing and
 * their dx rows are not written. Any output pointer may be NULL.
 * The m* outputs (each may be NULL) hold, per element of the matching
 * gradient, the sum of the absolute values of the terms that the gradient
 * sums (|dy| |h| for dW2, |[du; dg]| |x| for dW13, |W13| |[du; dg]| +
 * |Wr| |dl| for dx, |dl| |x| for dWr): the scale that the rounding error of
 * a computation from rounded terms is bounded by.
 */
void orc_moe_backward(const void *x, int dtype, const float *w_router, const void *w13,
                      const void *w2, const void *ws13, const void *ws2, const uint8_t *pad,
                      const void *dout, int64_t T, int64_t H, int E, int K, int64_t I,
                      int64_t Is, const int32_t *idx_in, const double *w_in, double *dx,
                      double *dwr, double *dw13, double *dw2, double *dws13, double *dws2,
                      double *mdx, double *mdwr, double *mdw13, double *mdw2, double *mdws13,
                      double *mdws2)
{
    int64_t Imax = I > Is ? I : Is;
    double *xr = malloc(sizeof(double) * (size_t)H);
    double *dv = malloc(sizeof(double) * (size_t)H);
    double *dxr = malloc(sizeof(double) * (size_t)H);
    double *dy = malloc(sizeof(double) * (size_t)H);
    double *u = malloc(sizeof(double) * (size_t)Imax);
    double *g = malloc(sizeof(double) * (size_t)Imax);
    double *hb = malloc(sizeof(double) * (size_t)Imax);
    double *du = malloc(sizeof(double) * (size_t)Imax);
    double *dg = malloc(sizeof(double) * (size_t)Imax);
    double *mxr = malloc(sizeof(double) * (size_t)H);
    double *gs[12] = {dwr, dw13, dw2, dws13, dws2, NULL, mdwr, mdw13, mdw2, mdws13, mdws2, NULL};
    size_t gn[6] = {(size_t)E * (size_t)H, (size_t)E * 2 * (size_t)I * (size_t)H,
                    (size_t)E * (size_t)H * (size_t)I, 2 * (size_t)Is * (size_t)H,
                    (size_t)H * (size_t)Is, 0};
    for (int q = 0; q < 12; q++)
        if (gs[q]) memset(gs[q], 0, sizeof(double) * gn[q % 6]);
    for (int64_t t = 0; t < T; t++) {
        if (pad && pad[t])
            continue;
        float lbuf[1024], pbuf[1024], wf[1024];
        int32_t idx[1024];
        double w[1024], dw[1024];
        router_logits_row(x, dtype, t, H, w_router, E, lbuf);
        softmax_topk_row(lbuf, E, K, pbuf, idx, wf);
        for (int k = 0; k < K; k++)
            w[k] = (double)wf[k];
        if (idx_in) {
            for (int k = 0; k < K; k++) {
                idx[k] = idx_in[t * K + k];
                w[k] = w_in[t * K + k];
            }
        }
        for (int64_t h = 0; h < H; h++) {
            xr[h] = elem(x, dtype, t * H + h);
            dv[h] = elem(dout, dtype, t * H + h);
            dxr[h] = 0.0;
            mxr[h] = 0.0;
        }
        /* routed experts (k >= 0, weight w[k]) and the shared expert (k = K, weight 1) */
        for (int k = 0; k <= K; k++) {
            const int shared = k == K;
            const int e = shared ? 0 : idx[k];
            const int64_t II = shared ? Is : I;
            const void *W13 = shared ? ws13 : offset_elems(w13, dtype, (size_t)e * expert_up_gate_elems(H, I));
            const void *W2 = shared ? ws2 : offset_elems(w2, dtype, (size_t)e * expert_down_elems(H, I));
            double *gW13 = shared ? dws13 : (dw13 ? dw13 + (size_t)e * 2 * (size_t)I * (size_t)H : NULL);
            double *gW2 = shared ? dws2 : (dw2 ? dw2 + (size_t)e * (size_t)H * (size_t)I : NULL);
            double *mW13 = shared ? mdws13 : (mdw13 ? mdw13 + (size_t)e * 2 * (size_t)I * (size_t)H : NULL);
            double *mW2 = shared ? mdws2 : (mdw2 ? mdw2 + (size_t)e * (size_t)H * (size_t)I : NULL);
            const double wk = shared ? 1.0 : w[k];
            for (int64_t i = 0; i < II; i++) {
                double uu = 0.0, gg = 0.0;
                for (int64_t h = 0; h < H; h++) {
                    uu += xr[h] * elem(W13, dtype, i * H + h);
                    gg += xr[h] * elem(W13, dtype, (II + i) * H + h);
                }
                u[i] = uu;
                g[i] = gg;
                hb[i] = round_dtype(gg / (1.0 + exp(-gg)) * uu, dtype);
            }
            double dwk = 0.0;
            for (int64_t j = 0; j < H; j++) {
                double yj = 0.0;
                for (int64_t i = 0; i < II; i++)
                    yj += hb[i] * elem(W2, dtype, j * II + i);
                dwk += dv[j] * yj;
                dy[j] = wk * dv[j];
            }
            if (!shared)
                dw[k] = dwk;
            if (gW2)
                for (int64_t j = 0; j < H; j++)
                    for (int64_t i = 0; i < II; i++)
                        gW2[j * II + i] += dy[j] * hb[i];
            if (mW2)
                for (int64_t j = 0; j < H; j++)
                    for (int64_t i = 0; i < II; i++)
                        mW2[j * II + i] += fabs(dy[j]) * fabs(hb[i]);
            for (int64_t i = 0; i < II; i++) {
                double dh = 0.0;
                for (int64_t j = 0; j < H; j++)
                    dh += elem(W2, dtype, j * II + i) * dy[j];
                double sg = 1.0 / (1.0 + exp(-g[i]));
                du[i] = dh * g[i] * sg;
                dg[i] = dh * u[i] * sg * (1.0 + g[i] * (1.0 - sg));
            }
            for (int64_t i = 0; i < II; i++)
                for (int64_t h = 0; h < H; h++) {
                    if (gW13) {
                        gW13[i * H + h] += du[i] * xr[h];
                        gW13[(II + i) * H + h] += dg[i] * xr[h];
                    }
                    if (mW13) {
                        mW13[i * H + h] += fabs(du[i]) * fabs(xr[h]);
                        mW13[(II + i) * H + h] += fabs(dg[i]) * fabs(xr[h]);
                    }
                    dxr[h] += elem(W13, dtype, i * H + h) * du[i] +
                              elem(W13, dtype, (II + i) * H + h) * dg[i];
                    mxr[h] += fabs(elem(W13, dtype, i * H + h) * du[i]) +
                              fabs(elem(W13, dtype, (II + i) * H + h) * dg[i]);
                }
        }
        /* router */
        double S = 0.0, A = 0.0, B = 0.0;
        double dp[1024];
        for (int e = 0; e < E; e++)
            dp[e] = 0.0;
        for (int k = 0; k < K; k++) {
            S += (double)pbuf[idx[k]];
            A += w[k] * dw[k];
        }
        for (int k = 0; k < K; k++)
            dp[idx[k]] = (dw[k] - A) / S;
        for (int e = 0; e < E; e++)
            B += (double)pbuf[e] * dp[e];
        for (int e = 0; e < E; e++) {
            double dl = (double)pbuf[e] * (dp[e] - B);
            for (int64_t h = 0; h < H; h++) {
                if (dwr) dwr[(int64_t)e * H + h] += dl * xr[h];
                if (mdwr) mdwr[(int64_t)e * H + h] += fabs(dl * xr[h]);
                dxr[h] += (double)w_router[(int64_t)e * H + h] * dl;
                mxr[h] += fabs((double)w_router[(int64_t)e * H + h] * dl);
            }
        }
        for (int64_t h = 0; h < H; h++) {
            if (dx) dx[t * H + h] = dxr[h];
            if (mdx) mdx[t * H + h] = mxr[h];
        }
    }
    free(xr); free(dv); free(dxr); free(dy); free(u); free(g); free(hb); free(du); free(dg);
    free(mxr);
}

void orc_round_bf16_array(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        store_dtype(out, ORC_BF16, i, round_bf16(v[i]));
}

int orc_max_experts(void) { return 1024; }
