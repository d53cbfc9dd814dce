// spec_sample.hip -- speculative (rejection) sampling of draft tokens on the
// device for MI355X (gfx950): gdn_spec_accept_sample of include/gdn_spec.h.
//
// The target side accepts each draft token with probability min(1, p/q) and,
// at the first rejection, draws the replacement from max(0, p - q); if every
// draft is kept it draws a bonus token from the last row (FreeToken issue #828
// "Speculative decoding: MTP and DFlash", Plan: target-side verify with
// rejection sampling and per-row presence and frequency penalties; lmdeploy PR
// #5006, What's included, Verification path: speculative sampling op
// kernels). Row t's target distribution is the softmax of its logits after
// presence / frequency penalties counted over the earlier output and the
// tokens of rows 0..t, divided by the request's temperature.
//
// Draws are Gumbel-max: argmax_v (log w_v + G_v), G_v = -log(-log U_v), with
// U from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers:
// As Easy as 1, 2, 3", SC'11) keyed by the call's seed, so no cumulative sum
// over the vocabulary decides an index. Counters: (v >> 2, t, b, 0), word
// v & 3, for the noise of row t at entry v; (0, t, b, 1), word 0, for row t's
// acceptance uniform. U = (2 (word >> 9) + 1) / 2^24, exact in fp32.
//
// Two kernels, both over the logits in HBM order:
//   stats     grid (splits, requests): each workgroup takes its columns of
//             every row of its request, forms the penalised and tempered
//             logits in base 2 and leaves, per row, the running maximum and
//             sum of 2^x (online softmax). No random numbers.
//   draw      grid (splits, requests): every workgroup of a request combines
//             the partial sums in the same order, so all of them reach the
//             same acceptance of every draft and the same accept length n;
//             each then takes the best Gumbel key over its entries of row
//             n - 1: of the residual max(0, p - q) after a rejection, of p
//             when every draft was kept (the bonus token). The workgroups
//             fold their bests into one word per request with atomics; the
//             last of them to finish writes accept_len and next_token.

#include <hip/hip_runtime.h>

#include <algorithm>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn_spec.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSampleThreads = 256;
constexpr int kColumn = kSampleThreads * 8;   // entries of one step of a workgroup: a unit of 8 per thread
constexpr int kMaxSampleRows = 9;
constexpr int kMaxSplits = 256;               // workgroups per request in either pass
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---- Philox4x32-10 -----------------------------------------------------------

struct U4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ U4 philox(U4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;   // one 32x32 -> 64-bit multiply each
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
        c = U4{(uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0};
    }
    return c;
}

__device__ __forceinline__ float unit_uniform(uint32_t word)
{
    return (float)(2u * (word >> 9) + 1u) * (1.0f / 16777216.0f);   // exact
}

// Gumbel noise in base 2, up to a constant that no argmax sees:
// -log2(-ln U) = -log2(-log2 U) - log2(ln 2).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }   // 2^x, v_exp_f32
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }    // log2 x, v_log_f32

__device__ __forceinline__ float gumbel2(uint32_t word)
{
    return -fast_log2(-fast_log2(unit_uniform(word)));
}

// ---- inputs -----------------------------------------------------------------

struct SampleParams {
    const void *logits;
    const float *dprob;
    const int32_t *draft;
    const int32_t *pending;
    const int32_t *prior;
    const float *temp;
    const float *pres;
    const float *freq;
    const int32_t *slot_ids;
    int B, R, V;
    int S, U;     // stats pass: splits per request, units (columns) per thread in a split
    int Sd, Ud;   // draw pass: the same
    uint32_t k0, k1;
    float2 *stats;   // [B][R][S]: running maximum (base 2) and sum of 2^(x - max)
    unsigned long long *best;   // [B]: best (key, index) of the draw so far, as one ordered word
    int32_t *done;              // [B]: draw workgroups finished
    int32_t *accept;
    int32_t *next;
    int32_t *err;
};

__device__ __forceinline__ float load_logit(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_logit(const uint16_t *p, size_t i) { return __uint_as_float((uint32_t)p[i] << 16); }

// Per-request values that every lane of a workgroup reads: scalar loads
// through the constant address space (the sampling kernels never write
// these inputs), whose waits do not drain the vector loads in flight.
__device__ __forceinline__ int32_t ld_scalar(const int32_t *ptr, size_t i)
{
    return ((const __attribute__((address_space(4))) int32_t *)ptr)[i];
}
__device__ __forceinline__ float ld_scalar(const float *ptr, size_t i)
{
    return ((const __attribute__((address_space(4))) float *)ptr)[i];
}

// A request's tokens in row order: the pending token (or -1), then the drafts.
struct Tokens {
    int32_t tok[kMaxSampleRows];
};

__device__ __forceinline__ Tokens request_tokens(const SampleParams &p, int b)
{
    Tokens t;
    t.tok[0] = p.pending ? ld_scalar(p.pending, b) : -1;
#pragma unroll
    for (int s = 1; s < kMaxSampleRows; ++s)
        t.tok[s] = s < p.R ? ld_scalar(p.draft, (size_t)b * (p.R - 1) + s - 1) : -1;
    return t;
}

// Penalised logit of row t at entry v, in base 2 units scaled by 1/T:
// (l - f c - r [c > 0]) * log2(e) / T, c = prior + tokens of rows 0..t equal to v.
__device__ __forceinline__ float penalised2(float l, int prior_c, const Tokens &tk, int t, int v, float f, float r,
                                            float scale2)
{
    int c = prior_c;
#pragma unroll
    for (int s = 0; s < kMaxSampleRows; ++s)
        c += (s <= t && tk.tok[s] == v) ? 1 : 0;
    const float pen = l - f * (float)c - r * (c > 0 ? 1.0f : 0.0f);
    return pen * scale2;
}

// Best (key, index) with ties to the smaller index.
__device__ __forceinline__ bool better(float k, int i, float bk, int bi) { return k > bk || (k == bk && i < bi); }

// (key, index) as one word that orders like better(): the key's bits made
// monotonic in the high half, the complemented index in the low half. A NaN
// key counts as -inf, so the word is never all ones.
__device__ __forceinline__ unsigned long long order_key(float k, int i)
{
    const uint32_t u = __float_as_uint(k == k ? k : kNegInf);
    const uint32_t hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)hi << 32) | (uint32_t)~(uint32_t)i;
}

// ---- reductions ------------------------------------------------------------

__device__ __forceinline__ void combine_ms(float &m, float &s, float m2, float s2)
{
    const float mm = fmaxf(m, m2);
    if (mm == kNegInf)
        return;
    s = s * fast_exp2(m - mm) + s2 * fast_exp2(m2 - mm);
    m = mm;
}

__device__ __forceinline__ void wave_best(float &k, int &i)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float k2 = __shfl_xor(k, off, 64);
        const int i2 = __shfl_xor(i, off, 64);
        if (better(k2, i2, k, i)) {
            k = k2;
            i = i2;
        }
    }
}

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x += __shfl_xor(x, off, 64);
    return x;
}

// The wave's (max, sum of 2^(x - max)) from every lane's pair: the maximum
// first, then each lane's sum rescaled to it once, then the sum. Every lane
// gets the result.
__device__ __forceinline__ void wave_ms(float &m, float &s)
{
    const float mm = wave_max(m);
    const float ref = mm == kNegInf ? 0.0f : mm;
    s = wave_sum(s * fast_exp2(m - ref));
    m = mm;
}

// Workgroup best key; every thread gets the same result.
__device__ __forceinline__ void group_best(float &k, int &i, float2 *sh)
{
    wave_best(k, i);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        sh[wave] = float2{k, __int_as_float(i)};
    __syncthreads();
    k = sh[0].x;
    i = __float_as_int(sh[0].y);
#pragma unroll
    for (int w = 1; w < kSampleThreads / 64; ++w)
        if (better(sh[w].x, __float_as_int(sh[w].y), k, i)) {
            k = sh[w].x;
            i = __float_as_int(sh[w].y);
        }
    __syncthreads();
}

__device__ __forceinline__ bool padding(const SampleParams &p, int b) { return p.slot_ids && ld_scalar(p.slot_ids, b) == -1; }

__device__ __forceinline__ float temperature_scale(const SampleParams &p, int b)
{
    const float T = ld_scalar(p.temp, b);
    return (T > 0.0f && T <= 3.0e38f) ? kLog2e / T : 0.0f;   // invalid temperatures are flagged by the final kernel
}

// ---- unit loads ---------------------------------------------------------------
//
// A thread's unit is 8 consecutive vocabulary entries. With `vec` (the unit lies
// inside the vocabulary and its row is 16-byte aligned) a row's unit is one or
// two 16-byte loads; otherwise each entry is loaded on its own from a clamped
// (always valid) index and entries past the vocabulary read as -inf logits,
// zero counts and zero draft probabilities (the `fill` of a float row).

template <typename L> struct Unit;
template <> struct Unit<uint16_t> {   // bf16 pairs, low half first
    u32x4 w;
    __device__ __forceinline__ float at(int k) const
    {
        return __uint_as_float((k & 1) ? (w[k >> 1] & 0xffff0000u) : (w[k >> 1] << 16));
    }
    __device__ __forceinline__ void clear(int k)   // entry k := -inf
    {
        w[k >> 1] = (k & 1) ? ((w[k >> 1] & 0xffffu) | 0xff800000u) : ((w[k >> 1] & 0xffff0000u) | 0xff80u);
    }
};
template <> struct Unit<float> {
    f32x4 a, b;
    __device__ __forceinline__ float at(int k) const { return k < 4 ? a[k] : b[k - 4]; }
    __device__ __forceinline__ void clear(int k)
    {
        if (k < 4)
            a[k] = kNegInf;
        else
            b[k - 4] = kNegInf;
    }
};

__device__ __forceinline__ Unit<uint16_t> load_unit(const uint16_t *row, int v0, int V, bool vec)
{
    Unit<uint16_t> u;
    if (vec) {
        u.w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row + v0));
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = v0 + 2 * k;
            const uint32_t lo = row[min(i, V - 1)], hi = row[min(i + 1, V - 1)];   // clamped: always valid
            u.w[k] = (i < V ? lo : 0xff80u) | ((i + 1 < V ? hi : 0xff80u) << 16);   // bf16 -inf past the end
        }
    }
    return u;
}

__device__ __forceinline__ Unit<float> load_unit(const float *row, int v0, int V, bool vec, float fill = kNegInf)
{
    Unit<float> u;
    if (vec) {
        u.a = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + v0));
        u.b = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + v0) + 1);
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float x = row[min(v0 + k, V - 1)];
            const float y = v0 + k < V ? x : fill;
            if (k < 4)
                u.a[k] = y;
            else
                u.b[k - 4] = y;
        }
    }
    return u;
}

__device__ __forceinline__ void load_counts(const int32_t *row, int v0, int V, bool vec, int (&c)[8])
{
    if (vec) {
        const int4 a = *reinterpret_cast<const int4 *>(row + v0);
        const int4 d = *reinterpret_cast<const int4 *>(row + v0 + 4);
        c[0] = a.x; c[1] = a.y; c[2] = a.z; c[3] = a.w; c[4] = d.x; c[5] = d.y; c[6] = d.z; c[7] = d.w;
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int x = row[min(v0 + k, V - 1)];
            c[k] = v0 + k < V ? x : 0;
        }
    }
}

// Which rows may take 16-byte loads (whole units only): bit 0 the logits,
// bit 1 the prior counts, bit 2 the draft probabilities.
enum : int { kVecLogits = 1, kVecPrior = 2, kVecProbs = 4 };

// Penalty of an entry with count c, in tempered base-2 units.
__device__ __forceinline__ float penalty2(int c, float f, float r, float scale2)
{
    return __builtin_fmaf(f, (float)c, c > 0 ? r : 0.0f) * scale2;
}

// True when one of tokens 0..last lies in [v0, v0 + 8).
__device__ __forceinline__ bool unit_holds_token(const Tokens &tk, int last, int v0)
{
    bool hit = false;
#pragma unroll
    for (int j = 0; j < kMaxSampleRows; ++j)
        hit |= j <= last && (uint32_t)tk.tok[j] - (uint32_t)v0 < 8u;
    return hit;
}

// ---- stats kernel -----------------------------------------------------------
//
// Grid (splits, requests). A split is U columns of 2048 entries; each thread
// takes one unit of 8 entries per column, for every row of its request. The
// launch sizes U so that the whole grid is resident at once (about one round
// of workgroups), and a thread loads the next column while it works on the
// current one. Per row the penalised, tempered logits in base 2 are
// y = x log2(e)/T - pen and the thread keeps a running (m, sum of 2^(y - m)):
// the first unit sets m exactly (its maximum); later units are summed against
// that m without a maximum of their own, and only a unit whose sum leaves the
// safe range (a value far above m, or m still -inf) joins exactly instead.
// The penalty comes from the prior counts alone, except at the entries of the
// request's own tokens, whose counts grow from row to row: a unit that holds
// one (rare, and a thread's own branch) joins those entries to every row on
// their own first and then drops them from the unit.

// The running pair (m, s) of one row joined exactly by a unit's 8 values.
__device__ __forceinline__ void join_unit(float &m, float &s, const float (&y)[8])
{
    float mu = kNegInf;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        mu = fmaxf(mu, y[k]);
    const float mm = fmaxf(m, mu);
    const float ref = mm == kNegInf ? 0.0f : mm;   // all -inf so far: the sum stays zero
    float su = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        su += fast_exp2(y[k] - ref);
    s = __builtin_fmaf(s, fast_exp2(m - ref), su);
    m = mm;
}

// The running pair (m, s) of one row joined by one value.
__device__ __forceinline__ void join_one(float &m, float &s, float y)
{
    const float mm = fmaxf(m, y);
    const float ref = mm == kNegInf ? 0.0f : mm;
    s = __builtin_fmaf(s, fast_exp2(m - ref), fast_exp2(y - ref));
    m = mm;
}

// One unit's loads: every row's 8 logits and (PRIOR) the prior counts.
template <int R, typename L, bool PRIOR>
__device__ __forceinline__ void stats_fetch(const SampleParams &p, const L *lg, int b, int v0, Unit<L> (&x)[R],
                                            int (&c)[8])
{
    const int V = p.V;
#pragma unroll
    for (int t = 0; t < R; ++t)
        x[t] = load_unit(lg + (size_t)t * V, v0, V, true);
    if (PRIOR) {
        load_counts(p.prior + (size_t)b * V, v0, V, true, c);
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            c[k] = 0;
    }
}

// One unit's arithmetic: every row's running pair joined by the unit, exactly
// (EXACT) or against the running maximum. With RELOAD, each row's registers
// take the same row of the next unit (at vn) as soon as the row is consumed,
// and the counts take the next unit's once the penalties are formed: one unit
// of lookahead in the registers of one.
template <int R, typename L, bool PEN, bool PRIOR, bool EXACT, bool RELOAD>
__device__ __forceinline__ void stats_unit(const SampleParams &p, const L *lg, int b, int vn, const Tokens &tk, int v0,
                                           float f, float r, float scale2, Unit<L> (&x)[R], int (&c)[8],
                                           float (&m)[R], float (&s)[R])
{
    const int V = p.V;
    float ps[8];
    if (PEN) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            ps[k] = penalty2(c[k], f, r, scale2);
        if (unit_holds_token(tk, R - 1, v0)) {
            // entries holding one of the request's tokens: their counts grow
            // from row to row, so they join each row on their own, exactly,
            // and leave the unit as -inf
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                bool tok = false;
#pragma unroll
                for (int j = 0; j < R; ++j)
                    tok |= tk.tok[j] == v0 + k;
                if (tok) {
                    int ck = c[k];
#pragma unroll
                    for (int t = 0; t < R; ++t) {
                        ck += tk.tok[t] == v0 + k ? 1 : 0;
                        join_one(m[t], s[t], __builtin_fmaf(x[t].at(k), scale2, -penalty2(ck, f, r, scale2)));
                        x[t].clear(k);
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            ps[k] = 0.0f;
    }
    if (PRIOR && RELOAD)
        load_counts(p.prior + (size_t)b * V, vn, V, true, c);
#pragma unroll
    for (int t = 0; t < R; ++t) {
        if (EXACT) {
            float y[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                y[k] = __builtin_fmaf(x[t].at(k), scale2, -ps[k]);
            join_unit(m[t], s[t], y);
        } else {
            // 2^(y - m) = 2^(x log2(e)/T - (pen + m)); below 2^100 per unit the
            // sum is safe, otherwise the unit joins exactly
            float su = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k)
                su += fast_exp2(__builtin_fmaf(x[t].at(k), scale2, -(ps[k] + m[t])));
            if (su <= 0x1p100f) {
                s[t] += su;
            } else {
                float y[8];
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    y[k] = __builtin_fmaf(x[t].at(k), scale2, -ps[k]);
                join_unit(m[t], s[t], y);
            }
        }
        if (RELOAD)
            x[t] = load_unit(lg + (size_t)t * V, vn, V, true);
    }
}

// A unit that is not whole, or whose rows are not 16-byte aligned: every
// entry loaded on its own from a clamped index (entries past the vocabulary
// read as -inf logits and zero counts), all rows at once.
template <int R, typename L, bool PRIOR>
__device__ __forceinline__ void stats_fetch_general(const SampleParams &p, const L *lg, int b, int v0, Unit<L> (&x)[R],
                                                    int (&c)[8])
{
    const int V = p.V;
#pragma unroll
    for (int t = 0; t < R; ++t)
        x[t] = load_unit(lg + (size_t)t * V, v0, V, false);
    if (PRIOR) {
        load_counts(p.prior + (size_t)b * V, v0, V, false, c);
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            c[k] = 0;
    }
}

// Every row's (m, s) combined over the wave, the rows interleaved so that
// their shuffles overlap: maxima first, each lane's sum rescaled once, then
// the sums. Every lane gets the results.
template <int R> __device__ __forceinline__ void wave_ms_rows(float (&m)[R], float (&s)[R])
{
    float mx[R];
#pragma unroll
    for (int t = 0; t < R; ++t)
        mx[t] = m[t];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int t = 0; t < R; ++t)
            mx[t] = fmaxf(mx[t], __shfl_xor(mx[t], off, 64));
#pragma unroll
    for (int t = 0; t < R; ++t) {
        const float ref = mx[t] == kNegInf ? 0.0f : mx[t];
        s[t] *= fast_exp2(m[t] - ref);
        m[t] = mx[t];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int t = 0; t < R; ++t)
            s[t] += __shfl_xor(s[t], off, 64);
}

template <int R, typename L, bool PEN, bool PRIOR>
__global__ __launch_bounds__(kSampleThreads) void gdn_sample_stats_kernel(const SampleParams p, int vec_ok)
{
    __shared__ float2 sh_ms[R][kSampleThreads / 64];
    const int split = blockIdx.x, b = blockIdx.y;
    const int V = p.V, S = p.S, U = p.U;
    const int tid = threadIdx.x;
    const L *lg = static_cast<const L *>(p.logits) + (size_t)b * R * V;
    const int base = split * U * kColumn;
    const int cols = min(U, (V - base + kColumn - 1) / kColumn);   // columns inside the vocabulary
    const bool vec = (vec_ok & kVecLogits) && (!PRIOR || (vec_ok & kVecPrior));
    const int whole = vec ? min(cols, (V - base) / kColumn) : 0;   // columns of whole units only

    if (split == 0 && tid == 0) {   // the draw pass of this call gathers its result here
        p.best[b] = 0ull;
        p.done[b] = 0;
    }
    // the first column's loads go out before the per-request values are read
    // (rows of padding requests are still inside the logits)
    Unit<L> x[R];
    int c[8];
    if (whole > 0)
        stats_fetch<R, L, PRIOR>(p, lg, b, base + tid * 8, x, c);
    if (padding(p, b))
        return;
    const float scale2 = temperature_scale(p, b);
    Tokens tk;
    float f = 0.0f, r = 0.0f;
    if (PEN) {
        tk = request_tokens(p, b);
        f = p.freq ? ld_scalar(p.freq, b) : 0.0f;
        r = p.pres ? ld_scalar(p.pres, b) : 0.0f;
    }
    float m[R], s[R];
#pragma unroll
    for (int t = 0; t < R; ++t) {
        m[t] = kNegInf;
        s[t] = 0.0f;
    }
    const auto col = [&](int u) { return base + (u * kSampleThreads + tid) * 8; };
    if (whole > 1) {
        stats_unit<R, L, PEN, PRIOR, true, true>(p, lg, b, col(1), tk, col(0), f, r, scale2, x, c, m, s);
#pragma unroll 1
        for (int u = 1; u + 1 < whole; ++u)
            stats_unit<R, L, PEN, PRIOR, false, true>(p, lg, b, col(u + 1), tk, col(u), f, r, scale2, x, c, m, s);
        stats_unit<R, L, PEN, PRIOR, false, false>(p, lg, b, 0, tk, col(whole - 1), f, r, scale2, x, c, m, s);
    } else if (whole == 1) {
        stats_unit<R, L, PEN, PRIOR, true, false>(p, lg, b, 0, tk, col(0), f, r, scale2, x, c, m, s);
    }
    // the ragged last column (or every column of unaligned rows)
#pragma unroll 1
    for (int u = whole; u < cols; ++u) {
        stats_fetch_general<R, L, PRIOR>(p, lg, b, col(u), x, c);
        stats_unit<R, L, PEN, PRIOR, true, false>(p, lg, b, 0, tk, col(u), f, r, scale2, x, c, m, s);
    }
    wave_ms_rows<R>(m, s);
    const int wave = tid >> 6, lane = tid & 63;
    if (lane == 0) {
#pragma unroll
        for (int t = 0; t < R; ++t)
            sh_ms[t][wave] = float2{m[t], s[t]};
    }
    __syncthreads();
    if (tid < R) {
        float mm = kNegInf, ss = 0.0f;
#pragma unroll
        for (int w = 0; w < kSampleThreads / 64; ++w)
            combine_ms(mm, ss, sh_ms[tid][w].x, sh_ms[tid][w].y);
        p.stats[((size_t)b * R + tid) * S + split] = float2{mm, ss};
    }
}

// ---- draw kernel ------------------------------------------------------------
//
// Grid (splits, requests), a split being Ud columns as above. Every workgroup
// of a request combines the partial sums in the same order, so all of them
// reach the same acceptance of every draft and the same accept length n.
// Then each takes the best Gumbel key over its entries of row n - 1: of the
// residual max(0, p - q) after a rejection, or of p itself when every draft
// was kept (the bonus token). With a greedy drafter (q one on the draft, zero
// elsewhere) the residual is p without the rejected draft, so both of those
// draws rank y + G (y = log2 p up to a constant of the row); only a drafter
// with probabilities needs p - q itself.

struct DrawRow {   // what the draw needs of its row
    const void *lg;     // the row's logits
    const float *q;     // its draft probabilities (drafter with probabilities, after a rejection), or null
    int t, d;           // the row, the draft excluded (greedy drafter after a rejection) or -1
    float mm, inv;      // the row's softmax maximum and 1 / sum
};

template <typename L> struct DrawUnit {
    Unit<L> x;
    Unit<float> q;
    int c[8];
};

// One unit's loads: 16-byte loads (VEC: a whole unit of aligned rows) or
// entry by entry from clamped indices. Q: the row's draft probabilities are
// read (a drafter with probabilities after a rejection); PRIOR: the prior counts.
template <typename L, bool VEC, bool Q, bool PRIOR>
__device__ __forceinline__ void draw_fetch(const SampleParams &p, const DrawRow &w, int b, int v0, DrawUnit<L> &u)
{
    const int V = p.V;
    u.x = load_unit(static_cast<const L *>(w.lg), v0, V, VEC);
    if (Q)
        u.q = load_unit(w.q, v0, V, VEC, 0.0f);
    if (PRIOR) {
        load_counts(p.prior + (size_t)b * V, v0, V, VEC, u.c);
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            u.c[k] = 0;
    }
}

// One unit's keys. A thread visits its entries in increasing index order, so
// among equal keys the first one seen (the smaller index) is kept by a plain
// greater-than; entries past the vocabulary have -inf keys. PEN: the row has
// penalties (its counts are the prior counts, when given, plus its tokens).
template <typename L, bool Q, bool PEN>
__device__ __forceinline__ void draw_unit(const SampleParams &p, const DrawRow &w, const Tokens &tk, int b, int v0,
                                          float f2, float r2, float scale2, DrawUnit<L> &u, float &bk, int &bi)
{
    const int t = w.t;
    float ps[8];
    if (PEN) {
        if (unit_holds_token(tk, t, v0)) {
#pragma unroll
            for (int j = 0; j < kMaxSampleRows; ++j)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    u.c[k] += (j <= t && tk.tok[j] == v0 + k) ? 1 : 0;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
            ps[k] = __builtin_fmaf(f2, (float)u.c[k], u.c[k] > 0 ? r2 : 0.0f);
    }
    const U4 g0 = philox(U4{(uint32_t)(v0 >> 2), (uint32_t)t, (uint32_t)b, 0u}, p.k0, p.k1);
    const U4 g1 = philox(U4{(uint32_t)(v0 >> 2) + 1u, (uint32_t)t, (uint32_t)b, 0u}, p.k0, p.k1);
    const uint32_t gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float y = PEN ? __builtin_fmaf(u.x.at(k), scale2, -ps[k]) : u.x.at(k) * scale2;
        float key;
        if (Q) {
            const float res = fast_exp2(y - w.mm) * w.inv - u.q.at(k);
            key = res > 0.0f ? fast_log2(res) + gumbel2(gw[k]) : kNegInf;
        } else {
            key = v0 + k != w.d ? y + gumbel2(gw[k]) : kNegInf;
        }
        if (key > bk) {
            bk = key;
            bi = v0 + k;
        }
    }
}

// The workgroup's columns of the draw's row: whole columns in order, the
// next one's loads out before the current one's arithmetic; then the ragged
// last column entry by entry.
template <typename L, bool Q, bool PEN, bool PRIOR>
__device__ __forceinline__ void draw_columns(const SampleParams &p, const DrawRow &w, const Tokens &tk, int b, int base,
                                             int cols, int whole, float f2, float r2, float scale2, float &bk, int &bi)
{
    const int V = p.V, tid = threadIdx.x;
    DrawUnit<L> cur, nxt;
    if (whole > 0) {
        draw_fetch<L, true, Q, PRIOR>(p, w, b, base + tid * 8, cur);
#pragma unroll 1
        for (int u = 0; u + 1 < whole; ++u) {
            draw_fetch<L, true, Q, PRIOR>(p, w, b, base + ((u + 1) * kSampleThreads + tid) * 8, nxt);
            draw_unit<L, Q, PEN>(p, w, tk, b, base + (u * kSampleThreads + tid) * 8, f2, r2, scale2, cur, bk, bi);
            cur = nxt;
        }
        draw_unit<L, Q, PEN>(p, w, tk, b, base + ((whole - 1) * kSampleThreads + tid) * 8, f2, r2, scale2, cur, bk,
                             bi);
    }
#pragma unroll 1
    for (int u = whole; u < cols; ++u) {
        const int v0 = base + (u * kSampleThreads + tid) * 8;
        draw_fetch<L, false, Q, PRIOR>(p, w, b, min(v0, V - 1), cur);
        if (v0 < V)
            draw_unit<L, Q, PEN>(p, w, tk, b, v0, f2, r2, scale2, cur, bk, bi);
    }
}

template <int R, typename L>
__global__ __launch_bounds__(kSampleThreads) void gdn_sample_draw_kernel(const SampleParams p, int vec_ok)
{
    __shared__ float2 row_ms[kMaxSampleRows];
    __shared__ int acc[kMaxSampleRows];
    __shared__ float2 sh_best[kSampleThreads / 64];
    __shared__ int last;
    const int split = blockIdx.x, b = blockIdx.y;
    const int V = p.V, S = p.S, U = p.Ud;
    const int tid = threadIdx.x;
    if (padding(p, b)) {
        if (split == 0 && tid == 0) {
            p.accept[b] = 0;
            p.next[b] = -1;
        }
        return;
    }
    const Tokens tk = request_tokens(p, b);
    const float scale2 = temperature_scale(p, b);
    const float f = p.freq ? ld_scalar(p.freq, b) : 0.0f, r = p.pres ? ld_scalar(p.pres, b) : 0.0f;
    const float f2 = f * scale2, r2 = r * scale2;
    const bool pen = f != 0.0f || r != 0.0f;
    const L *lg = static_cast<const L *>(p.logits) + (size_t)b * R * V;
    const int base = split * U * kColumn;
    const int cols = min(U, (V - base + kColumn - 1) / kColumn);

    // thread t < R - 1 reads what the acceptance of draft t+1 needs at the
    // draft's entry, alongside the partial sums; every thread loads (from a
    // clamped, valid index) so that no load sits in a divergent branch
    const int ta = R > 1 ? min(tid, R - 2) : 0;
    int dt = tk.tok[1];
#pragma unroll
    for (int j = 2; j < R; ++j)
        dt = ta == j - 1 ? tk.tok[j] : dt;
    const int dd = min(max(dt, 0), V - 1);   // out of range: flagged by the final kernel
    const L xd_raw = static_cast<const L *>(p.logits)[((size_t)b * R + ta) * V + dd];
    const int pcd = p.prior ? p.prior[(size_t)b * V + dd] : 0;
    const float qd = p.dprob ? p.dprob[((size_t)b * (R - 1) + ta) * V + dd] : 1.0f;

    // row t's softmax statistics over the splits (wave t % 4, lanes taking
    // the splits in turn), then the acceptance of draft t+1; the same
    // arithmetic in the same order in every workgroup of the request
    const int wave = tid >> 6, lane = tid & 63;
    constexpr int RW = (R + kSampleThreads / 64 - 1) / (kSampleThreads / 64);   // rows per wave
    constexpr int PL = kMaxSplits / 64;                                          // partials per lane
    // one partial per lane when the splits fit a wave (the usual case), else
    // up to PL per lane; the branch is uniform and every load in it is
    // unconditional
    float mrow[RW], srow[RW];
    if (S <= 64) {
        float2 part[RW];
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const int t = wave + j * (kSampleThreads / 64);
            const float2 v = p.stats[((size_t)b * R + min(t, R - 1)) * S + min(lane, S - 1)];
            part[j] = (t < R && lane < S) ? v : float2{kNegInf, 0.0f};
        }
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            mrow[j] = part[j].x;
            srow[j] = part[j].y;
        }
    } else {
        float2 part[RW][PL];
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const int t = wave + j * (kSampleThreads / 64);
#pragma unroll
            for (int i = 0; i < PL; ++i) {
                const int sp = lane + 64 * i;
                const float2 v = p.stats[((size_t)b * R + min(t, R - 1)) * S + min(sp, S - 1)];
                part[j][i] = (t < R && sp < S) ? v : float2{kNegInf, 0.0f};
            }
        }
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            mrow[j] = kNegInf;
            srow[j] = 0.0f;
#pragma unroll
            for (int i = 0; i < PL; ++i)
                combine_ms(mrow[j], srow[j], part[j][i].x, part[j][i].y);
        }
    }
    wave_ms_rows<RW>(mrow, srow);
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const int t = wave + j * (kSampleThreads / 64);
            if (t < R)
                row_ms[t] = float2{mrow[j], srow[j]};
        }
    }
    __syncthreads();
    if (tid < R) {
        const int t = tid;
        const float mm = row_ms[t].x, ss = row_ms[t].y;
        int ok = 1;
        if (t < R - 1) {
            const float y = penalised2(load_logit(&xd_raw, 0), pcd, tk, t, dd, f, r, scale2);
            const float pd = fast_exp2(y - mm) / ss;
            const U4 w = philox(U4{0u, (uint32_t)t, (uint32_t)b, 1u}, p.k0, p.k1);
            ok = unit_uniform(w.x) * qd <= pd ? 1 : 0;
        }
        acc[t] = ok;
    }
    __syncthreads();
    int n = R;
    for (int t = 0; t < R - 1; ++t)
        if (!acc[t]) {
            n = t + 1;
            break;
        }

    DrawRow w;
    w.t = n - 1;
    const bool rejected = n < R;
    w.d = -1;
#pragma unroll
    for (int j = 1; j < R; ++j)
        w.d = rejected && w.t == j - 1 ? tk.tok[j] : w.d;
    w.lg = lg + (size_t)w.t * V;
    w.q = rejected && p.dprob ? p.dprob + ((size_t)b * (R - 1) + w.t) * V : nullptr;
    w.mm = row_ms[w.t].x;
    w.inv = 1.0f / row_ms[w.t].y;
    float bk = kNegInf;
    int bi = 0x7fffffff;
    const bool vec_all = (vec_ok & kVecLogits) && (!pen || !p.prior || (vec_ok & kVecPrior)) &&
                         (!w.q || (vec_ok & kVecProbs));
    const int whole = vec_all ? min(cols, (V - base) / kColumn) : 0;
    // one path per workgroup (uniform branches): drafter probabilities or
    // not, penalties or not
    const int pm = !pen ? 0 : p.prior ? 2 : 1;   // penalties: none, tokens only, prior counts and tokens
    if (w.q) {
        if (pm == 2)
            draw_columns<L, true, true, true>(p, w, tk, b, base, cols, whole, f2, r2, scale2, bk, bi);
        else if (pm == 1)
            draw_columns<L, true, true, false>(p, w, tk, b, base, cols, whole, f2, r2, scale2, bk, bi);
        else
            draw_columns<L, true, false, false>(p, w, tk, b, base, cols, whole, f2, r2, scale2, bk, bi);
    } else {
        if (pm == 2)
            draw_columns<L, false, true, true>(p, w, tk, b, base, cols, whole, f2, r2, scale2, bk, bi);
        else if (pm == 1)
            draw_columns<L, false, true, false>(p, w, tk, b, base, cols, whole, f2, r2, scale2, bk, bi);
        else
            draw_columns<L, false, false, false>(p, w, tk, b, base, cols, whole, f2, r2, scale2, bk, bi);
    }
    group_best(bk, bi, sh_best);

    // every workgroup folds its best into the request's word with an atomic
    // maximum, then counts itself done; the count waits for the maximum's
    // returned value, so it is performed after it. The last to count reads
    // the word back: the best over all splits. Only atomics cross workgroups.
    if (tid == 0) {
        const unsigned long long prev = atomicMax(&p.best[b], order_key(bk, bi));
        last = atomicAdd(&p.done[b], prev == ~0ull ? 2 : 1) == p.Sd - 1;   // never ~0: see order_key
    }
    __syncthreads();
    if (!last || tid != 0)
        return;
    const unsigned long long fin = atomicOr(&p.best[b], 0ull);
    const int ci = (int)~(uint32_t)fin;
    bool bad = !(scale2 > 0.0f);
    if (p.pending)
        bad |= tk.tok[0] < 0 || tk.tok[0] >= V;
#pragma unroll
    for (int j = 1; j < R; ++j)
        bad |= tk.tok[j] < 0 || tk.tok[j] >= V;
    if (bad) {
        if (p.err)
            atomicOr(p.err, 8);
        p.accept[b] = 0;
        p.next[b] = -1;
        return;
    }
    {
        p.accept[b] = n;
        // an empty residual (every p <= q after rounding) keeps the rejected draft
        p.next[b] = ci != 0x7fffffff ? ci : (n < R ? w.d : 0);
    }
}

// Workgroups of a kernel that one compute unit holds at once (its occupancy),
// asked of the runtime once per kernel.
template <typename K> int groups_per_cu(K kernel)
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kSampleThreads, 0) != hipSuccess || n < 1)
        n = 1;
    return n;
}

int compute_units(hipStream_t st)
{
    static int cached[64] = {};
    int dev = 0;
    if (hipStreamGetDevice(st, &dev) != hipSuccess && hipGetDevice(&dev) != hipSuccess)
        return 256;
    if (dev < 0 || dev >= 64)
        return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Columns per thread so that the batch's workgroups all fit on the device at
// once: each request gets at most resident / B splits, and at most kMaxSplits.
int columns_per_split(int B, int V, int resident)
{
    const int total = (V + kColumn - 1) / kColumn;
    const int per_request = std::max(1, std::min(kMaxSplits, resident / std::max(B, 1)));
    return std::max(1, (total + per_request - 1) / per_request);
}

template <int R, typename L> void launch_sample_kernels(SampleParams p, hipStream_t st)
{
    const auto row_aligned = [](const void *ptr, size_t row_bytes) {
        return ptr && (reinterpret_cast<uintptr_t>(ptr) & 15) == 0 && row_bytes % 16 == 0;
    };
    const int vec = (row_aligned(p.logits, (size_t)p.V * sizeof(L)) ? kVecLogits : 0) |
                    (row_aligned(p.prior, (size_t)p.V * sizeof(int32_t)) ? kVecPrior : 0) |
                    (row_aligned(p.dprob, (size_t)p.V * sizeof(float)) ? kVecProbs : 0);
    const int cus = compute_units(st);
    const bool pen = p.pres || p.freq;
    static const int occ_prior = groups_per_cu(gdn_sample_stats_kernel<R, L, true, true>);
    static const int occ_pen = groups_per_cu(gdn_sample_stats_kernel<R, L, true, false>);
    static const int occ_plain = groups_per_cu(gdn_sample_stats_kernel<R, L, false, false>);
    static const int occ_draw = groups_per_cu(gdn_sample_draw_kernel<R, L>);
    p.U = columns_per_split(p.B, p.V, cus * (!pen ? occ_plain : p.prior ? occ_prior : occ_pen));
    p.S = (p.V + p.U * kColumn - 1) / (p.U * kColumn);
    p.Ud = columns_per_split(p.B, p.V, cus * occ_draw);
    p.Sd = (p.V + p.Ud * kColumn - 1) / (p.Ud * kColumn);
    const dim3 block(kSampleThreads);
    const dim3 grid((unsigned)p.S, (unsigned)p.B);
    if (pen && p.prior)
        hipLaunchKernelGGL((gdn_sample_stats_kernel<R, L, true, true>), grid, block, 0, st, p, vec);
    else if (pen)
        hipLaunchKernelGGL((gdn_sample_stats_kernel<R, L, true, false>), grid, block, 0, st, p, vec);
    else
        hipLaunchKernelGGL((gdn_sample_stats_kernel<R, L, false, false>), grid, block, 0, st, p, vec);
    hipLaunchKernelGGL((gdn_sample_draw_kernel<R, L>), dim3((unsigned)p.Sd, (unsigned)p.B), block, 0, st, p, vec);
}

template <typename L> void launch_rows(int rows, const SampleParams &p, hipStream_t st)
{
    switch (rows) {
    case 1: launch_sample_kernels<1, L>(p, st); break;
    case 2: launch_sample_kernels<2, L>(p, st); break;
    case 3: launch_sample_kernels<3, L>(p, st); break;
    case 4: launch_sample_kernels<4, L>(p, st); break;
    case 5: launch_sample_kernels<5, L>(p, st); break;
    case 6: launch_sample_kernels<6, L>(p, st); break;
    case 7: launch_sample_kernels<7, L>(p, st); break;
    case 8: launch_sample_kernels<8, L>(p, st); break;
    default: launch_sample_kernels<9, L>(p, st); break;
    }
}

// Scratch: partial pairs [B][R][splits] (sized for the most splits any
// launch may use), the draw's best word [B] and finished-workgroup counts [B].
struct SampleLayout {
    size_t stats, best, done, total;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

gdn_status sample_layout(int batch, int rows, int vocab, SampleLayout *l)
{
    if (batch < 0 || rows < 1 || rows > kMaxSampleRows || vocab < 1)
        return GDN_ERR_INVALID_ARG;
    if (vocab > (1 << 20))
        return GDN_ERR_UNSUPPORTED;
    const size_t splits = std::min<size_t>(kMaxSplits, (vocab + kColumn - 1) / kColumn);
    size_t off = 0;
    l->stats = off;
    off = align256(off + (size_t)batch * rows * splits * sizeof(float2));
    l->best = off;
    off = align256(off + (size_t)batch * sizeof(unsigned long long));
    l->done = off;
    off = align256(off + (size_t)batch * sizeof(int32_t));
    l->total = off;
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_spec_sample_scratch_bytes(int32_t batch, int32_t rows, int32_t vocab, size_t *bytes)
{
    SampleLayout l;
    const gdn_status s = sample_layout(batch, rows, vocab, &l);
    if (s != GDN_OK)
        return s;
    if (!bytes)
        return GDN_ERR_INVALID_ARG;
    *bytes = l.total;
    return GDN_OK;
}

gdn_status gdn_spec_accept_sample(const gdn_sample_inputs *in, int32_t logits_dtype, int32_t batch, int32_t rows,
                                  int32_t vocab, uint64_t seed, void *scratch, size_t scratch_bytes,
                                  int32_t *accept_len, int32_t *next_token, int32_t *err_flag, void *stream)
{
    SampleLayout l;
    gdn_status s = sample_layout(batch, rows, vocab, &l);
    if (s != GDN_OK)
        return s;
    if (logits_dtype != GDN_F32 && logits_dtype != GDN_BF16)
        return GDN_ERR_INVALID_ARG;
    if (batch == 0)
        return GDN_OK;
    if (!in || !in->logits || !in->temperature || (rows > 1 && !in->draft) || !accept_len || !next_token ||
        !scratch || ((uintptr_t)scratch & 15u) != 0)
        return GDN_ERR_INVALID_ARG;
    if (scratch_bytes < l.total)
        return GDN_ERR_SCRATCH_TOO_SMALL;
    SampleParams p;
    char *base = static_cast<char *>(scratch);
    p.logits = in->logits;
    p.dprob = in->draft_probs;
    p.draft = in->draft;
    p.pending = in->pending;
    p.prior = in->prior_counts;
    p.temp = in->temperature;
    p.pres = in->presence;
    p.freq = in->frequency;
    p.slot_ids = in->slot_ids;
    p.B = batch;
    p.R = rows;
    p.V = vocab;
    p.k0 = (uint32_t)(seed & 0xffffffffu);
    p.k1 = (uint32_t)(seed >> 32);
    p.stats = reinterpret_cast<float2 *>(base + l.stats);
    p.best = reinterpret_cast<unsigned long long *>(base + l.best);
    p.done = reinterpret_cast<int32_t *>(base + l.done);
    p.accept = accept_len;
    p.next = next_token;
    p.err = err_flag;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (logits_dtype == GDN_F32)
        launch_rows<float>(rows, p, st);
    else
        launch_rows<uint16_t>(rows, p, st);
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"
