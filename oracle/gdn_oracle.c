/*
 * gdn_oracle.c -- plain CPU reference of the GatedDeltaNet speculative
 * verify / commit step.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline may load this file's library. The HIP library never calls it and
 * shares no code with it. It is slow on purpose: one request, one head, one
 * row at a time, every sum in fp64 over the stored (fp32 or bf16) inputs.
 *
 * What it computes, and where that comes from:
 *
 *  - A verify scores k+1 rows per request, the pending token plus k drafts
 *    (FreeToken PR #844 "MTP drafts for the Qwen3.5 family and Flash-Next",
 *    Design: the target scores [pending, d1..dk] and accepts n of them).
 *    The verify runs the rows as a uniform extend and only READS the
 *    committed GatedDeltaNet state; the commit then replays the accepted rows
 *    (FreeToken issue #828 "Speculative decoding: MTP and DFlash", Design).
 *    Here a verify copies the slot's state, runs the rows on the copy and
 *    returns the outputs; a commit runs the first n rows on the slot itself.
 *
 *  - The verify's conv applies the same width-W taps a decode step uses to
 *    each of its rows in turn, reading a window that joins the slot's stored
 *    history to the new rows' conv inputs; the commit then stores the
 *    history that results once only the accepted rows have been taken in
 *    (FreeToken PR #844, Design, "Flash-Next target verify", the paragraph
 *    on the PLE verify conv; the causal_conv1d_spec kernel named by LightLLM
 *    PR #1330, Summary, plays the same part for the GDN layer).
 *
 *  - The layer itself is the gated delta rule over L2-normalised q and k
 *    (LightLLM PR #1330, Summary, names the Gated Delta Net / qwen3next
 *    linear attention; the pages print no equations). Per value head, with
 *    S the d_v x d_k state:
 *
 *        S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *        o_t = scale * S_t q_t
 *
 *    Expanding the bracket gives the rank-1 form used below, with no
 *    d_k x d_k matrix:  S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T.
 *
 * Readings where the pages are silent (each is a parameter or a fixed choice):
 *  - conv input x holds the mixed channels [q (HK*d_k) | k (HK*d_k) | v (HV*d_v)];
 *    a depthwise causal conv of width W (cw[c][W-1] multiplies the newest
 *    input, no bias) is followed by SiLU (act = 0) or nothing (act = 1);
 *  - conv history = the last W-1 raw inputs, oldest first;
 *  - q and k are normalised per key head as x / sqrt(sum x^2 + eps);
 *  - value head h reads key head h / (HV / HK);
 *  - alpha and beta are given per (row, value head), already activated;
 *  - accept_len n in [0, rows]; n = 0 commits nothing; slot id -1 is padding.
 *
 * Storage layouts (the same buffers the HIP library takes):
 *  ssm   fp32 [num_slots][HV][d_k][d_v]: element (i = d_v index, j = d_k index)
 *        of head h's state S is ssm[((slot*HV + h)*d_k + j)*d_v + i], i.e. each
 *        head stores S transposed, d_v contiguous;
 *  conv  [num_slots][W-1][C], conv_w [C][W], x [B][rows][C],
 *  alpha/beta [B][rows][HV], all fp32 (dtype 0) or bf16 bits (dtype 1).
 *
 * Parity pins: the hand-derived d = 2 and conv-ring values, the identity-gate,
 * write-back and closed-form cases, and an independent transition-matrix
 * formulation (tests/test_oracle_pins.py); each planted mistake in this file
 * makes one of them fail (tests/test_oracle_mutants.py). Parity unpinned: the
 * readings listed above (scale, eps, SiLU, tap order, head map) are choices,
 * not values the pages fix.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t num_k_heads;
    int32_t num_v_heads;
    int32_t d_k;
    int32_t d_v;
    int32_t conv_width;
    int32_t dtype;   /* 0: fp32 storage, 1: bf16 storage */
    int32_t act;     /* 0: SiLU after the conv, 1: none */
    int32_t pad_;
    double scale;
    double l2_eps;
} oracle_desc;

enum { ERR_SLOT = 1, ERR_ACCEPT = 2, ERR_ARGS = 1 << 30 };

/* ---- storage decode / encode ------------------------------------------- */

static double bf16_to_double(uint16_t h)
{
    uint32_t bits = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static uint16_t float_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x40); /* keep NaN a NaN */
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static double ld(const void *p, size_t idx, int dtype)
{
    if (dtype == 0)
        return (double)((const float *)p)[idx];
    return bf16_to_double(((const uint16_t *)p)[idx]);
}

/* Conv history values are raw inputs, so they are exact in the storage type. */
static void st(void *p, size_t idx, int dtype, double v)
{
    if (dtype == 0)
        ((float *)p)[idx] = (float)v;
    else
        ((uint16_t *)p)[idx] = float_to_bf16_rne((float)v);
}

/* ---- one request's state in fp64 ---------------------------------------- */

typedef struct {
    int C, W, HK, HV, dk, dv;
    double *hist; /* [W-1][C]  conv history, oldest first */
    double *S;    /* [HV][dv][dk]  S[h][i][j], math orientation */
    double *cw;   /* [C][W] */
    /* work space for one row */
    double *y;    /* [C] conv output after the activation */
    double *qn;   /* [HK][dk] normalised q */
    double *kn;   /* [HK][dk] normalised k */
    double *Sk;   /* [dv] */
} req_state;

static int state_alloc(req_state *r, const oracle_desc *d)
{
    r->HK = d->num_k_heads;
    r->HV = d->num_v_heads;
    r->dk = d->d_k;
    r->dv = d->d_v;
    r->W = d->conv_width;
    r->C = 2 * r->HK * r->dk + r->HV * r->dv;
    r->hist = calloc((size_t)(r->W - 1) * r->C, sizeof(double));
    r->S = calloc((size_t)r->HV * r->dv * r->dk, sizeof(double));
    r->cw = calloc((size_t)r->C * r->W, sizeof(double));
    r->y = calloc((size_t)r->C, sizeof(double));
    r->qn = calloc((size_t)r->HK * r->dk, sizeof(double));
    r->kn = calloc((size_t)r->HK * r->dk, sizeof(double));
    r->Sk = calloc((size_t)r->dv, sizeof(double));
    return r->hist && r->S && r->cw && r->y && r->qn && r->kn && r->Sk;
}

static void state_free(req_state *r)
{
    free(r->hist); free(r->S); free(r->cw); free(r->y);
    free(r->qn); free(r->kn); free(r->Sk);
}

static void state_import(req_state *r, const oracle_desc *d, const float *ssm,
                         const void *conv, const void *conv_w, int slot)
{
    const int C = r->C, W = r->W, HV = r->HV, dk = r->dk, dv = r->dv;
    for (int c = 0; c < C; ++c)
        for (int w = 0; w < W; ++w)
            r->cw[(size_t)c * W + w] = ld(conv_w, (size_t)c * W + w, d->dtype);
    for (int w = 0; w < W - 1; ++w)
        for (int c = 0; c < C; ++c)
            r->hist[(size_t)w * C + c] = ld(conv, ((size_t)slot * (W - 1) + w) * C + c, d->dtype);
    for (int h = 0; h < HV; ++h)
        for (int i = 0; i < dv; ++i)
            for (int j = 0; j < dk; ++j)
                r->S[((size_t)h * dv + i) * dk + j] =
                    (double)ssm[(((size_t)slot * HV + h) * dk + j) * dv + i];
}

static void state_export(const req_state *r, const oracle_desc *d, float *ssm, void *conv, int slot)
{
    const int C = r->C, W = r->W, HV = r->HV, dk = r->dk, dv = r->dv;
    for (int w = 0; w < W - 1; ++w)
        for (int c = 0; c < C; ++c)
            st(conv, ((size_t)slot * (W - 1) + w) * C + c, d->dtype, r->hist[(size_t)w * C + c]);
    for (int h = 0; h < HV; ++h)
        for (int i = 0; i < dv; ++i)
            for (int j = 0; j < dk; ++j)
                ssm[(((size_t)slot * HV + h) * dk + j) * dv + i] =
                    (float)r->S[((size_t)h * dv + i) * dk + j];
}

/*
 * One decode step on one request: conv over [history | x_t], activation,
 * split into q, k, v, L2-normalise q and k per key head, gated delta update of
 * every value head, o_t = scale * S_t q_t, then shift x_t into the history.
 * x_t points at the row's C inputs, alpha_t / beta_t at its HV gates (storage
 * type); o_t receives HV*dv outputs (may be NULL).
 */
static void decode_step(req_state *r, const oracle_desc *d, const void *x, size_t x_off,
                        const void *alpha, const void *beta, size_t g_off, double *o_t)
{
    const int C = r->C, W = r->W, HK = r->HK, HV = r->HV, dk = r->dk, dv = r->dv;
    const int group = HV / HK;

    /* causal depthwise conv: window row w is history[w] for w < W-1, x_t for w = W-1 */
    for (int c = 0; c < C; ++c) {
        double acc = 0.0;
        for (int w = 0; w < W; ++w) {
            double in = (w < W - 1) ? r->hist[(size_t)w * C + c] : ld(x, x_off + c, d->dtype);
            acc += r->cw[(size_t)c * W + w] * in;
        }
        if (d->act == 0)
            acc = acc / (1.0 + exp(-acc)); /* SiLU */
        r->y[c] = acc;
    }

    /* split and normalise: q = y[0, HK*dk), k = y[HK*dk, 2*HK*dk), v = the rest */
    for (int kh = 0; kh < HK; ++kh) {
        const double *q = r->y + (size_t)kh * dk;
        const double *k = r->y + (size_t)HK * dk + (size_t)kh * dk;
        double qq = 0.0, kk = 0.0;
        for (int j = 0; j < dk; ++j) {
            qq += q[j] * q[j];
            kk += k[j] * k[j];
        }
        double qs = 1.0 / sqrt(qq + d->l2_eps);
        double ks = 1.0 / sqrt(kk + d->l2_eps);
        for (int j = 0; j < dk; ++j) {
            r->qn[(size_t)kh * dk + j] = q[j] * qs;
            r->kn[(size_t)kh * dk + j] = k[j] * ks;
        }
    }

    /* gated delta rule per value head */
    for (int h = 0; h < HV; ++h) {
        const int kh = h / group;
        const double *kn = r->kn + (size_t)kh * dk;
        const double *qn = r->qn + (size_t)kh * dk;
        const double *v = r->y + (size_t)2 * HK * dk + (size_t)h * dv;
        const double a = ld(alpha, g_off + h, d->dtype);
        const double b = ld(beta, g_off + h, d->dtype);
        double *S = r->S + (size_t)h * dv * dk;
        for (int i = 0; i < dv; ++i) {
            double s = 0.0;
            for (int j = 0; j < dk; ++j)
                s += S[(size_t)i * dk + j] * kn[j];
            r->Sk[i] = s;
        }
        for (int i = 0; i < dv; ++i) {
            const double u = b * (v[i] - a * r->Sk[i]);
            for (int j = 0; j < dk; ++j)
                S[(size_t)i * dk + j] = a * S[(size_t)i * dk + j] + u * kn[j];
        }
        if (o_t) {
            for (int i = 0; i < dv; ++i) {
                double s = 0.0;
                for (int j = 0; j < dk; ++j)
                    s += S[(size_t)i * dk + j] * qn[j];
                o_t[(size_t)h * dv + i] = d->scale * s;
            }
        }
    }

    /* the history keeps the newest W-1 inputs */
    for (int w = 0; w < W - 2; ++w)
        for (int c = 0; c < C; ++c)
            r->hist[(size_t)w * C + c] = r->hist[(size_t)(w + 1) * C + c];
    for (int c = 0; c < C; ++c)
        r->hist[(size_t)(W - 2) * C + c] = ld(x, x_off + c, d->dtype);
}

static int desc_ok(const oracle_desc *d)
{
    return d && d->num_k_heads > 0 && d->num_v_heads > 0 &&
           d->num_v_heads % d->num_k_heads == 0 && d->d_k > 0 && d->d_v > 0 &&
           d->conv_width >= 2 && (d->dtype == 0 || d->dtype == 1) &&
           (d->act == 0 || d->act == 1);
}

/*
 * Verify: for each request b with slot s = slot_ids[b], copy the slot's
 * committed state, run rows 0..rows-1 on the copy and write
 *   out[b][t][h][i]                  (fp64) o of row t,
 *   snap[b][t][h][j][i] (optional)   (fp64) S after row t, pool orientation.
 * The pool is only read. Padding (s = -1) and bad slots give zero outputs;
 * bad slots also set ERR_SLOT in the return value.
 */
int oracle_verify(const oracle_desc *d, const float *ssm, const void *conv, int32_t num_slots,
                  const void *conv_w, const void *x, const void *alpha, const void *beta,
                  const int32_t *slot_ids, int32_t batch, int32_t rows,
                  double *out, double *snap, int32_t nthreads)
{
    if (!desc_ok(d) || batch < 0 || rows < 1 || !out)
        return ERR_ARGS;
    const int HV = d->num_v_heads, dk = d->d_k, dv = d->d_v;
    const int C = 2 * d->num_k_heads * dk + HV * dv;
    const size_t out_row = (size_t)HV * dv;
    const size_t snap_row = (size_t)HV * dk * dv;
    int err = 0;
    memset(out, 0, sizeof(double) * (size_t)batch * rows * out_row);
    if (snap)
        memset(snap, 0, sizeof(double) * (size_t)batch * rows * snap_row);

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1) reduction(| : err)
    for (int b = 0; b < batch; ++b) {
        const int slot = slot_ids[b];
        if (slot == -1)
            continue;
        if (slot < -1 || slot >= num_slots) {
            err |= ERR_SLOT;
            continue;
        }
        req_state r;
        if (!state_alloc(&r, d)) {
            err |= ERR_ARGS;
            state_free(&r);
            continue;
        }
        state_import(&r, d, ssm, conv, conv_w, slot);
        for (int t = 0; t < rows; ++t) {
            const size_t row = (size_t)b * rows + t;
            decode_step(&r, d, x, row * C, alpha, beta, row * HV, out + row * out_row);
            if (snap)
                for (int h = 0; h < HV; ++h)
                    for (int i = 0; i < dv; ++i)
                        for (int j = 0; j < dk; ++j)
                            snap[row * snap_row + ((size_t)h * dk + j) * dv + i] =
                                r.S[((size_t)h * dv + i) * dk + j];
        }
        state_free(&r);
    }
    return err;
}

/*
 * Commit: for each request b, run its first n = accept_len[b] rows on the
 * slot's committed state (rounded back to fp32 once, at the end) and store the
 * conv history as it stands after those rows. n = 0 and padding slots leave
 * the pool alone; a bad slot or n outside [0, rows] skips the request and sets
 * ERR_SLOT / ERR_ACCEPT.
 */
int oracle_commit(const oracle_desc *d, float *ssm, void *conv, int32_t num_slots,
                  const void *conv_w, const void *x, const void *alpha, const void *beta,
                  const int32_t *slot_ids, const int32_t *accept_len, int32_t batch,
                  int32_t rows, int32_t nthreads)
{
    if (!desc_ok(d) || batch < 0 || rows < 1)
        return ERR_ARGS;
    const int HV = d->num_v_heads;
    const int C = 2 * d->num_k_heads * d->d_k + HV * d->d_v;
    int err = 0;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1) reduction(| : err)
    for (int b = 0; b < batch; ++b) {
        const int slot = slot_ids[b];
        const int n = accept_len[b];
        if (slot < -1 || slot >= num_slots) {
            err |= ERR_SLOT;
            continue;
        }
        if (n < 0 || n > rows) {
            err |= ERR_ACCEPT;
            continue;
        }
        if (slot == -1 || n == 0)
            continue;
        req_state r;
        if (!state_alloc(&r, d)) {
            err |= ERR_ARGS;
            state_free(&r);
            continue;
        }
        state_import(&r, d, ssm, conv, conv_w, slot);
        for (int t = 0; t < n; ++t) {
            const size_t row = (size_t)b * rows + t;
            decode_step(&r, d, x, row * C, alpha, beta, row * HV, NULL);
        }
        state_export(&r, d, ssm, conv, slot);
        state_free(&r);
    }
    return err;
}

/*
 * One plain decode step on the pool: x [B][C], alpha/beta [B][HV]; writes
 * out [B][HV][dv] and the slot's new state (S rounded to fp32).
 */
int oracle_decode_step(const oracle_desc *d, float *ssm, void *conv, int32_t num_slots,
                       const void *conv_w, const void *x, const void *alpha, const void *beta,
                       const int32_t *slot_ids, int32_t batch, double *out, int32_t nthreads)
{
    if (!desc_ok(d) || batch < 0 || !out)
        return ERR_ARGS;
    const int HV = d->num_v_heads, dv = d->d_v;
    const int C = 2 * d->num_k_heads * d->d_k + HV * dv;
    int err = 0;
    memset(out, 0, sizeof(double) * (size_t)batch * HV * dv);

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1) reduction(| : err)
    for (int b = 0; b < batch; ++b) {
        const int slot = slot_ids[b];
        if (slot == -1)
            continue;
        if (slot < -1 || slot >= num_slots) {
            err |= ERR_SLOT;
            continue;
        }
        req_state r;
        if (!state_alloc(&r, d)) {
            err |= ERR_ARGS;
            state_free(&r);
            continue;
        }
        state_import(&r, d, ssm, conv, conv_w, slot);
        decode_step(&r, d, x, (size_t)b * C, alpha, beta, (size_t)b * HV, out + (size_t)b * HV * dv);
        state_export(&r, d, ssm, conv, slot);
        state_free(&r);
    }
    return err;
}
