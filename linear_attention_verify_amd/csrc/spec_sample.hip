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
// Three kernels, all over the logits in HBM order:
//   stats     grid (splits, requests): each workgroup takes 4096 vocabulary
//             entries of every row of its request, forms the penalised and
//             tempered logits in base 2 and leaves, per row, the running
//             maximum and sum of 2^x (online softmax), plus the best Gumbel
//             key of the last row (the bonus draw).
//   residual  grid (splits, requests): every workgroup of a request combines
//             the partial sums in the same order, so all of them reach the
//             same acceptance of every draft and the same accept length n;
//             if a draft was rejected, each takes the best Gumbel key of the
//             residual max(0, p - q) over its entries of row n - 1.
//   final     one thread per request: the best key over the splits gives the
//             next token; accept_len and next_token are written.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn_spec.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSampleThreads = 256;
constexpr int kSampleChunk = 4096;                        // vocabulary entries per workgroup
constexpr int kPerThread = kSampleChunk / kSampleThreads;  // 16: two units of 8
constexpr int kMaxSampleRows = 9;
constexpr int kMaxSplits = 256;                            // vocabulary up to 2^20 entries
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
    int B, R, V, S;
    uint32_t k0, k1;
    float2 *stats;   // [B][R][S]: running maximum (base 2) and sum of 2^(x - max)
    float2 *bonus;   // [B][S]: best key of the last row and its index (bits)
    float2 *resid;   // [B][S]: best key of the residual and its index (bits)
    int32_t *nacc;   // [B]: accept length
    int32_t *accept;
    int32_t *next;
    int32_t *err;
};

__device__ __forceinline__ float load_logit(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_logit(const uint16_t *p, size_t i) { return __uint_as_float((uint32_t)p[i] << 16); }

template <typename L> __device__ __forceinline__ void load_unit(const L *row, int v0, int V, float (&x)[8]);

template <> __device__ __forceinline__ void load_unit<float>(const float *row, int v0, int V, float (&x)[8])
{
    if (v0 + 8 <= V && ((uintptr_t)(row + v0) & 15u) == 0) {
        const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + v0));
        const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + v0) + 1);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[k] = a[k];
            x[4 + k] = b[k];
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            x[k] = v0 + k < V ? row[v0 + k] : 0.0f;
    }
}

template <> __device__ __forceinline__ void load_unit<uint16_t>(const uint16_t *row, int v0, int V, float (&x)[8])
{
    if (v0 + 8 <= V && ((uintptr_t)(row + v0) & 15u) == 0) {
        const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row + v0));
        const uint32_t w[4] = {a[0], a[1], a[2], a[3]};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = __uint_as_float(w[k] << 16);
            x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            x[k] = v0 + k < V ? __uint_as_float((uint32_t)row[v0 + k] << 16) : 0.0f;
    }
}

// A request's tokens in row order: the pending token (or -1), then the drafts.
struct Tokens {
    int32_t tok[kMaxSampleRows];
};

__device__ __forceinline__ Tokens request_tokens(const SampleParams &p, int b)
{
    Tokens t;
    t.tok[0] = p.pending ? p.pending[b] : -1;
#pragma unroll
    for (int s = 1; s < kMaxSampleRows; ++s)
        t.tok[s] = s < p.R ? p.draft[(size_t)b * (p.R - 1) + s - 1] : -1;
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

__device__ __forceinline__ void wave_ms(float &m, float &s)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(m, off, 64);
        const float s2 = __shfl_xor(s, off, 64);
        combine_ms(m, s, m2, s2);
    }
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

__device__ __forceinline__ bool padding(const SampleParams &p, int b) { return p.slot_ids && p.slot_ids[b] == -1; }

__device__ __forceinline__ float temperature_scale(const SampleParams &p, int b)
{
    const float T = p.temp[b];
    return (T > 0.0f && T <= 3.0e38f) ? kLog2e / T : 0.0f;   // invalid temperatures are flagged by the final kernel
}

// Prior counts of a unit's 8 entries (zero without penalties or counts).
__device__ __forceinline__ void prior_unit(const SampleParams &p, int b, int v0, int V, bool pen, int (&c)[8])
{
    if (pen && p.prior && v0 + 8 <= V && (((size_t)b * V + v0) & 3) == 0) {
        const int4 a = *reinterpret_cast<const int4 *>(p.prior + (size_t)b * V + v0);
        const int4 d = *reinterpret_cast<const int4 *>(p.prior + (size_t)b * V + v0 + 4);
        c[0] = a.x; c[1] = a.y; c[2] = a.z; c[3] = a.w; c[4] = d.x; c[5] = d.y; c[6] = d.z; c[7] = d.w;
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            c[k] = (pen && p.prior && v0 + k < V) ? p.prior[(size_t)b * V + v0 + k] : 0;
    }
}

// ---- stats kernel -----------------------------------------------------------
//
// Per thread, two units of 8 consecutive entries. For each unit all R rows
// are loaded first (one 16-byte load per row), then row by row: with
// penalties, the counts grow by the row's own token (c_t = c_{t-1} + [token
// of row t == v], from the prior counts); the logits are scaled to base 2; and
// the unit's maximum and sum of 2^(y - max) (one exp2 per entry) join the
// thread's running pair for that row. R is a template parameter, so the row
// loops are straight-line code.

// FULL: all 8 entries inside the vocabulary and the rows 16-byte aligned, so
// the loads are plain 16-byte loads and no entry needs a range check.
template <bool FULL, typename L> __device__ __forceinline__ void load8(const L *row, int v0, int V, float (&x)[8])
{
    if constexpr (FULL) {
        if constexpr (sizeof(L) == 4) {
            const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + v0));
            const f32x4 c = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + v0) + 1);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[k] = a[k];
                x[4 + k] = c[k];
            }
        } else {
            const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row + v0));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[2 * k] = __uint_as_float(a[k] << 16);
                x[2 * k + 1] = __uint_as_float(a[k] & 0xffff0000u);
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            x[k] = v0 + k < V ? load_logit(row, v0 + k) : 0.0f;
    }
}

// The running pair (m, s) joined by a unit's (mu, su); mu is finite.
__device__ __forceinline__ void join_finite(float &m, float &s, float mu, float su)
{
    const float mm = fmaxf(m, mu);
    s = __builtin_fmaf(s, fast_exp2(m - mm), su * fast_exp2(mu - mm));
    m = mm;
}

template <int R, typename L, bool PEN, bool FULL>
__device__ __forceinline__ void stats_unit(const SampleParams &p, const L *lg, const Tokens &tk, int b, int v0,
                                           float f, float r, float scale2, float (&m)[R], float (&s)[R], float &bk,
                                           int &bi)
{
    const int V = p.V;
    float x[R][8];
#pragma unroll
    for (int t = 0; t < R; ++t)
        load8<FULL, L>(lg + (size_t)t * V, v0, V, x[t]);
    int c[8];
    if (PEN) {
        if constexpr (FULL) {
            if (p.prior) {
                const int4 a = *reinterpret_cast<const int4 *>(p.prior + (size_t)b * V + v0);
                const int4 d = *reinterpret_cast<const int4 *>(p.prior + (size_t)b * V + v0 + 4);
                c[0] = a.x; c[1] = a.y; c[2] = a.z; c[3] = a.w; c[4] = d.x; c[5] = d.y; c[6] = d.z; c[7] = d.w;
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    c[k] = 0;
            }
        } else {
            prior_unit(p, b, v0, V, true, c);
        }
    }
#pragma unroll
    for (int t = 0; t < R; ++t) {
        float y[8];
        float mu = kNegInf;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float l = x[t][k];
            if (PEN) {
                c[k] += tk.tok[t] == v0 + k ? 1 : 0;
                l = __builtin_fmaf(-f, (float)c[k], l) - (c[k] > 0 ? r : 0.0f);
            }
            y[k] = (FULL || v0 + k < V) ? l * scale2 : kNegInf;
            mu = fmaxf(mu, y[k]);
        }
        float su = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            su += fast_exp2(y[k] - mu);
        join_finite(m[t], s[t], mu, su);
        if (t == R - 1) {
            // noise of the last row: two Philox blocks cover the unit's 8 entries
            const U4 g0 = philox(U4{(uint32_t)(v0 >> 2), (uint32_t)t, (uint32_t)b, 0u}, p.k0, p.k1);
            const U4 g1 = philox(U4{(uint32_t)(v0 >> 2) + 1u, (uint32_t)t, (uint32_t)b, 0u}, p.k0, p.k1);
            const uint32_t gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float key = y[k] + gumbel2(gw[k]);
                if ((FULL || v0 + k < V) && better(key, v0 + k, bk, bi)) {
                    bk = key;
                    bi = v0 + k;
                }
            }
        }
    }
}

// Grid (splits, requests); the workgroups of one launch all take the same
// path: PEN when the call has penalty arrays (zero penalties through it are
// exact), FULL for the splits that lie wholly inside the vocabulary with
// 16-byte aligned rows (the ragged last split gets a launch of its own).
template <int R, typename L, bool PEN, bool FULL>
__global__ __launch_bounds__(kSampleThreads) void gdn_sample_stats_kernel(const SampleParams p, int split0)
{
    __shared__ float2 sh_ms[R][kSampleThreads / 64];
    __shared__ float2 sh_best[kSampleThreads / 64];
    const int split = split0 + blockIdx.x, b = blockIdx.y;
    const int V = p.V, S = p.S;
    const int tid = threadIdx.x;
    if (padding(p, b))
        return;
    const Tokens tk = request_tokens(p, b);
    const float scale2 = temperature_scale(p, b);
    const float f = p.freq ? p.freq[b] : 0.0f, r = p.pres ? p.pres[b] : 0.0f;
    const L *lg = static_cast<const L *>(p.logits) + (size_t)b * R * V;

    float m[R], s[R];
#pragma unroll
    for (int t = 0; t < R; ++t) {
        m[t] = kNegInf;
        s[t] = 0.0f;
    }
    float bk = kNegInf;
    int bi = 0x7fffffff;
    const int base = split * kSampleChunk;
#pragma unroll 1
    for (int u = 0; u < kPerThread / 8; ++u) {
        const int v0 = base + (u * kSampleThreads + tid) * 8;
        if (FULL || v0 < V)
            stats_unit<R, L, PEN, FULL>(p, lg, tk, b, v0, f, r, scale2, m, s, bk, bi);
    }
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int t = 0; t < R; ++t) {
        wave_ms(m[t], s[t]);
        if (lane == 0)
            sh_ms[t][wave] = float2{m[t], s[t]};
    }
    group_best(bk, bi, sh_best);   // includes a barrier after the sh_ms stores
    if (tid < R) {
        float mm = kNegInf, ss = 0.0f;
#pragma unroll
        for (int w = 0; w < kSampleThreads / 64; ++w)
            combine_ms(mm, ss, sh_ms[tid][w].x, sh_ms[tid][w].y);
        p.stats[((size_t)b * R + tid) * S + split] = float2{mm, ss};
    }
    if (tid == 0)
        p.bonus[(size_t)b * S + split] = float2{bk, __int_as_float(bi)};
}

// ---- residual kernel --------------------------------------------------------

template <int R, typename L>
__global__ __launch_bounds__(kSampleThreads) void gdn_sample_residual_kernel(const SampleParams p)
{
    __shared__ float2 row_ms[kMaxSampleRows];
    __shared__ int acc[kMaxSampleRows];
    __shared__ float2 sh_best[kSampleThreads / 64];
    __shared__ float2 parts[kMaxSampleRows * kMaxSplits];
    const int split = blockIdx.x, b = blockIdx.y;
    const int V = p.V, S = p.S;
    const int tid = threadIdx.x;
    if (padding(p, b))
        return;
    const Tokens tk = request_tokens(p, b);
    const float scale2 = temperature_scale(p, b);
    const float f = p.freq ? p.freq[b] : 0.0f, r = p.pres ? p.pres[b] : 0.0f;
    const L *lg = static_cast<const L *>(p.logits) + (size_t)b * R * V;

    // row t's softmax statistics, combined over the splits in index order, and
    // the acceptance of draft t+1 (the same arithmetic in every workgroup);
    // the partial pairs come in through LDS, every thread loading some
    for (int i = tid; i < R * S; i += kSampleThreads)
        parts[i] = p.stats[(size_t)b * R * S + i];
    __syncthreads();
    if (tid < R) {
        const int t = tid;
        float mm = kNegInf, ss = 0.0f;
        for (int i = 0; i < S; ++i) {
            const float2 ms = parts[t * S + i];
            combine_ms(mm, ss, ms.x, ms.y);
        }
        row_ms[t] = float2{mm, ss};
        int ok = 1;
        if (t < R - 1) {
            const int d = min(max(p.draft[(size_t)b * (R - 1) + t], 0), V - 1);   // out of range: flagged later
            const int pc = p.prior ? p.prior[(size_t)b * V + d] : 0;
            const float y = penalised2(load_logit(static_cast<const L *>(p.logits), ((size_t)b * R + t) * V + d), pc,
                                       tk, t, d, f, r, scale2);
            const float pd = fast_exp2(y - mm) / ss;
            const float qd = p.dprob ? p.dprob[((size_t)b * (R - 1) + t) * V + d] : 1.0f;
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
    if (split == 0 && tid == 0)
        p.nacc[b] = n;
    if (n == R)
        return;

    // residual max(0, p - q) of row n-1 over this workgroup's entries
    const int t = n - 1;
    const float mm = row_ms[t].x, inv = 1.0f / row_ms[t].y;
    const int d = p.draft[(size_t)b * (R - 1) + t];
    const float *q = p.dprob ? p.dprob + ((size_t)b * (R - 1) + t) * V : nullptr;
    float bk = kNegInf;
    int bi = 0x7fffffff;
    const int base = split * kSampleChunk;
#pragma unroll
    for (int u = 0; u < kPerThread / 8; ++u) {
        const int v0 = base + (u * kSampleThreads + tid) * 8;
        if (v0 >= V)
            break;
        float x[8], qv[8];
        load_unit<L>(lg + (size_t)t * V, v0, V, x);
        if (q)
            load_unit<float>(q, v0, V, qv);
        const U4 g0 = philox(U4{(uint32_t)(v0 >> 2), (uint32_t)t, (uint32_t)b, 0u}, p.k0, p.k1);
        const U4 g1 = philox(U4{(uint32_t)(v0 >> 2) + 1u, (uint32_t)t, (uint32_t)b, 0u}, p.k0, p.k1);
        const uint32_t gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        int c[8];
        const bool pen = f != 0.0f || r != 0.0f;
        prior_unit(p, b, v0, V, pen, c);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int v = v0 + k;
            if (v < V) {
            const float y = penalised2(x[k], c[k], tk, t, v, f, r, scale2);
            const float pv = fast_exp2(y - mm) * inv;
            const float qq = q ? qv[k] : (v == d ? 1.0f : 0.0f);
            const float res = pv - qq;
            if (res > 0.0f) {
                const float key = fast_log2(res) + gumbel2(gw[k]);
                if (better(key, v, bk, bi)) {
                    bk = key;
                    bi = v;
                }
            }
            }
        }
    }
    group_best(bk, bi, sh_best);
    if (tid == 0)
        p.resid[(size_t)b * S + split] = float2{bk, __int_as_float(bi)};
}

// ---- final kernel -----------------------------------------------------------

// One wave per request: the lanes take the splits' best keys in turn, then the
// wave's best (ties to the smaller index) is the next token.
__global__ __launch_bounds__(64) void gdn_sample_final_kernel(const SampleParams p)
{
    const int b = blockIdx.x, lane = threadIdx.x;
    if (padding(p, b)) {
        if (lane == 0) {
            p.accept[b] = 0;
            p.next[b] = -1;
        }
        return;
    }
    const int R = p.R, V = p.V, S = p.S;
    bool bad = !(p.temp[b] > 0.0f && p.temp[b] <= 3.0e38f);
    if (p.pending)
        bad |= p.pending[b] < 0 || p.pending[b] >= V;
    for (int s = 0; s < R - 1; ++s) {
        const int d = p.draft[(size_t)b * (R - 1) + s];
        bad |= d < 0 || d >= V;
    }
    if (bad) {
        if (lane == 0) {
            if (p.err)
                atomicOr(p.err, 8);
            p.accept[b] = 0;
            p.next[b] = -1;
        }
        return;
    }
    const int n = p.nacc[b];
    const float2 *src = (n == R ? p.bonus : p.resid) + (size_t)b * S;
    float bk = kNegInf;
    int bi = 0x7fffffff;
    for (int i = lane; i < S; i += 64)
        if (better(src[i].x, __float_as_int(src[i].y), bk, bi)) {
            bk = src[i].x;
            bi = __float_as_int(src[i].y);
        }
    wave_best(bk, bi);
    if (lane == 0) {
        p.accept[b] = n;
        // an empty residual (every p <= q after rounding) keeps the rejected draft
        p.next[b] = bi != 0x7fffffff ? bi : (n < R ? p.draft[(size_t)b * (R - 1) + n - 1] : 0);
    }
}

template <int R, typename L, bool PEN> void launch_stats(const SampleParams &p, hipStream_t st)
{
    const bool aligned = ((size_t)p.V * sizeof(L)) % 16 == 0 && (reinterpret_cast<uintptr_t>(p.logits) & 15) == 0 &&
                         (reinterpret_cast<uintptr_t>(p.prior) & 15) == 0;
    const int full = aligned ? p.V / kSampleChunk : 0;   // splits wholly inside the vocabulary
    if (full > 0)
        hipLaunchKernelGGL((gdn_sample_stats_kernel<R, L, PEN, true>), dim3((unsigned)full, (unsigned)p.B),
                           dim3(kSampleThreads), 0, st, p, 0);
    if (full < p.S)
        hipLaunchKernelGGL((gdn_sample_stats_kernel<R, L, PEN, false>), dim3((unsigned)(p.S - full), (unsigned)p.B),
                           dim3(kSampleThreads), 0, st, p, full);
}

template <int R, typename L> void launch_sample_kernels(dim3 grid, const SampleParams &p, hipStream_t st)
{
    if (p.pres || p.freq)
        launch_stats<R, L, true>(p, st);
    else
        launch_stats<R, L, false>(p, st);
    hipLaunchKernelGGL((gdn_sample_residual_kernel<R, L>), grid, dim3(kSampleThreads), 0, st, p);
}

template <typename L> void launch_rows(int rows, dim3 grid, const SampleParams &p, hipStream_t st)
{
    switch (rows) {
    case 1: launch_sample_kernels<1, L>(grid, p, st); break;
    case 2: launch_sample_kernels<2, L>(grid, p, st); break;
    case 3: launch_sample_kernels<3, L>(grid, p, st); break;
    case 4: launch_sample_kernels<4, L>(grid, p, st); break;
    case 5: launch_sample_kernels<5, L>(grid, p, st); break;
    case 6: launch_sample_kernels<6, L>(grid, p, st); break;
    case 7: launch_sample_kernels<7, L>(grid, p, st); break;
    case 8: launch_sample_kernels<8, L>(grid, p, st); break;
    default: launch_sample_kernels<9, L>(grid, p, st); break;
    }
}

struct SampleLayout {
    size_t stats, bonus, resid, nacc, total;
    int S;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

gdn_status sample_layout(int batch, int rows, int vocab, SampleLayout *l)
{
    if (batch < 0 || rows < 1 || rows > kMaxSampleRows || vocab < 1)
        return GDN_ERR_INVALID_ARG;
    if (vocab > kMaxSplits * kSampleChunk)
        return GDN_ERR_UNSUPPORTED;
    l->S = (vocab + kSampleChunk - 1) / kSampleChunk;
    size_t off = 0;
    l->stats = off;
    off = align256(off + (size_t)batch * rows * l->S * sizeof(float2));
    l->bonus = off;
    off = align256(off + (size_t)batch * l->S * sizeof(float2));
    l->resid = off;
    off = align256(off + (size_t)batch * l->S * sizeof(float2));
    l->nacc = off;
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
    p.S = l.S;
    p.k0 = (uint32_t)(seed & 0xffffffffu);
    p.k1 = (uint32_t)(seed >> 32);
    p.stats = reinterpret_cast<float2 *>(base + l.stats);
    p.bonus = reinterpret_cast<float2 *>(base + l.bonus);
    p.resid = reinterpret_cast<float2 *>(base + l.resid);
    p.nacc = reinterpret_cast<int32_t *>(base + l.nacc);
    p.accept = accept_len;
    p.next = next_token;
    p.err = err_flag;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)l.S, (unsigned)batch);
    if (logits_dtype == GDN_F32)
        launch_rows<float>(rows, grid, p, st);
    else
        launch_rows<uint16_t>(rows, grid, p, st);
    hipLaunchKernelGGL(gdn_sample_final_kernel, dim3((unsigned)batch), dim3(64), 0, st, p);
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"
