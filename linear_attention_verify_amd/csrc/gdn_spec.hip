// gdn_spec.hip -- GatedDeltaNet speculative verify / commit for MI355X (gfx950).
//
// Implements the C ABI of include/gdn_spec.h. One workgroup of 256 threads
// (four wave64s) owns one (request, value head) tile: its d x d fp32 state,
// its value channels and its key head's q/k channels.
//
// Verify (FreeToken issue #828, Design: the verify rows run as a uniform
// extend and only read the GatedDeltaNet state). Rather than stepping the
// state row by row (4 multiply-adds per state element per row), the kernel
// uses the exact unrolled form of the gated delta rule. With e_t the row's
// correction vector and g(t,u) = a_{u+1} ... a_t (g(t,t) = 1):
//
//     S_t     = g(t,-1) S_0 + sum_{u<=t} g(t,u) e_u k_u^T
//     e_t     = b_t (v_t - a_t S_{t-1} k_t)
//             = b_t (v_t - g(t,-1) S_0 k_t - sum_{u<t} g(t,u) (k_u . k_t) e_u)
//     o_t     = scale (g(t,-1) S_0 q_t + sum_{u<=t} g(t,u) (k_u . q_t) e_u)
//
// so one pass over S_0 computing the 2R products S_0 k_t and S_0 q_t (2
// multiply-adds per element per row) plus R x R scalar algebra per row of S
// gives every o_t. The state is streamed once from HBM and never written.
//
// Commit (same Design section: the commit replays the accepted rows). The
// verify leaves each row's e_t and normalised k_t in scratch, so replaying
// row t is the rank-1 update S <- a_t S + e_t k_t^T, applied for t < n to the
// committed state in one streaming pass. In snapshot mode (LightLLM PR #1330,
// Summary: snapshot/restore of committed state) the verify applies the same
// update to every row and stores each S_t; the commit copies S_{n-1}. Both
// modes run the identical update, so their results agree bit for bit.
//
// The conv history is a shift register of raw inputs; the commit stores the
// last W-1 entries of [history | rows 0..n-1] (FreeToken PR #844, Design,
// "Flash-Next target verify": the commit restores the conv state as it stands
// after the accepted rows).

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "gdn_spec.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWidth = 4;    // conv width this build supports
constexpr int kMaxRows = 9;  // k + 1 with k <= 8 drafts
constexpr size_t kAlign = 256;

// ---- storage types -------------------------------------------------------

struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float((uint32_t)v.bits << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v)
{
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return bf16_t{(uint16_t)((u >> 16) | 0x40u)};  // stay NaN
    u += 0x7fffu + ((u >> 16) & 1u);                     // nearest, ties to even
    return bf16_t{(uint16_t)(u >> 16)};
}

// Barrier that orders LDS only: global loads already in flight (the state
// prefetch) are not drained by it.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, 64);
    return v;
}

// One accepted row replayed on one state element: S <- a S + e k.
__device__ __forceinline__ float row_update(float s, float a, float e, float k)
{
    return __builtin_fmaf(e, k, a * s);
}

// ---- scratch layout (shared by host and device code) -----------------------

struct ScratchLayout {
    size_t xs, es, ks, as, snap, total;
};

__host__ __device__ inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Per request b (row b of every part):
//   xs   [B][R][C]       raw verify inputs (storage type), for the conv commit
//   es   [B][R][HV][D]   fp32 correction vector e_t of each row and value head
//   ks   [B][R][HK][D]   fp32 normalised key of each row and key head
//   as   [B][R][HV]      fp32 decay gate a_t
//   snap [B][R][HV][D][D] fp32 S_t after each row (snapshot mode only),
//                         same per-head layout as the pool
__host__ inline ScratchLayout scratch_layout(int HK, int HV, int D, int C, size_t esize, int B,
                                              int R, bool snapshot)
{
    ScratchLayout L;
    size_t off = 0;
    L.xs = off;
    off = align_up(off + (size_t)B * R * C * esize);
    L.es = off;
    off = align_up(off + (size_t)B * R * HV * D * sizeof(float));
    L.ks = off;
    off = align_up(off + (size_t)B * R * HK * D * sizeof(float));
    L.as = off;
    off = align_up(off + (size_t)B * R * HV * sizeof(float));
    L.snap = off;
    if (snapshot)
        off = align_up(off + (size_t)B * R * HV * D * D * sizeof(float));
    L.total = off;
    return L;
}

// ---- verify ----------------------------------------------------------------

template <typename T> struct VerifyParams {
    const float *ssm;
    const T *conv;
    const T *conv_w;
    const T *x;
    const T *alpha;
    const T *beta;
    const int32_t *slot_ids;
    T *out;
    int32_t *err;
    T *xs;
    float *es;
    float *ks;
    float *as;
    float *snap;
    int HK, HV, C, P;
    int act;
    float scale, eps;
};

// Inputs of one conv channel: taps, history (oldest first) and the verify rows.
template <int NR, typename T> struct ChanIn {
    T w[kWidth];
    T hist[kWidth - 1];
    T x[NR];
};

template <int NR, typename T>
__device__ __forceinline__ ChanIn<NR, T> load_channel(const VerifyParams<T> &p, int slot, int b, int c)
{
    ChanIn<NR, T> in;
#pragma unroll
    for (int k = 0; k < kWidth; ++k)
        in.w[k] = p.conv_w[(size_t)c * kWidth + k];
#pragma unroll
    for (int k = 0; k < kWidth - 1; ++k)
        in.hist[k] = p.conv[((size_t)slot * (kWidth - 1) + k) * p.C + c];
#pragma unroll
    for (int t = 0; t < NR; ++t)
        in.x[t] = p.x[((size_t)b * NR + t) * p.C + c];
    return in;
}

// Causal conv over [history | rows]: y_t = sum_k w_k window[t + k], w_{W-1} on
// the newest input, then the activation.
template <int NR, typename T>
__device__ __forceinline__ void conv_rows(const ChanIn<NR, T> &in, int act, float (&y)[NR])
{
    float win[kWidth - 1 + NR];
#pragma unroll
    for (int k = 0; k < kWidth - 1; ++k)
        win[k] = to_f32(in.hist[k]);
#pragma unroll
    for (int t = 0; t < NR; ++t)
        win[kWidth - 1 + t] = to_f32(in.x[t]);
#pragma unroll
    for (int t = 0; t < NR; ++t) {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < kWidth; ++k)
            acc = __builtin_fmaf(to_f32(in.w[k]), win[t + k], acc);
        y[t] = act == GDN_ACT_SILU ? acc / (1.0f + __expf(-acc)) : acc;
    }
}

template <int D, int NR, typename T, bool SNAP>
__global__ __launch_bounds__(kThreads) void gdn_verify_kernel(const VerifyParams<T> p)
{
    constexpr int NC = 2 * NR;              // columns: k_hat of rows 0..NR-1, then q_hat
    constexpr int MS = (NC + 3) / 4 * 4;    // row stride of the column table
    constexpr int LPJ = D / 4;              // lanes covering one key index (4 state rows each)
    constexpr int GJ = kThreads / LPJ;      // key-index groups
    constexpr int JPER = D / GJ;            // key indices per lane
    static_assert(JPER >= 1 && LPJ <= 64, "unsupported head dim");
    constexpr int NPAIR = NR * (NR + 1) / 2;

    __shared__ __align__(16) float Mt[D * MS];    // [j][c]: k_hat_t[j] (c < NR), q_hat_t[j]
    __shared__ float vb[NR * D];                  // v_t[i]
    __shared__ __align__(16) float red[4 * D * NC];  // per-wave partial products; later e_t
    __shared__ float inv[NC];
    __shared__ float gkk[NR * NR], gkq[NR * NR];
    __shared__ float cA[NR * NR], cB[NR * NR];
    __shared__ float gam[NR], bet[NR], alp[NR];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int HV = p.HV, HK = p.HK;
    const int G = HV / HK;
    const int b = blockIdx.x / HV;
    const int h = blockIdx.x % HV;
    const int kh = h / G;
    const int slot = p.slot_ids[b];

    if (slot < 0 || slot >= p.P) {
        if (slot != -1 && tid == 0 && p.err)
            atomicOr(p.err, 1);
        for (int idx = tid; idx < NR * D; idx += kThreads) {
            const int t = idx / D, i = idx % D;
            p.out[(((size_t)b * NR + t) * HV + h) * D + i] = from_f32<T>(0.0f);
        }
        return;
    }

    // Small loads first: vmcnt retires in issue order, so anything issued
    // after the state stream would wait for all of it. They are branch-free
    // (clamped indices) so that they share one basic block with the stream.
    const int tr = tid < NR ? tid : NR - 1;
    const size_t gi = ((size_t)b * NR + tr) * HV + h;
    const T ga = p.alpha[gi];
    const T gb = p.beta[gi];
    // channels: threads < D take the key head's q and k channel `tid`,
    // threads D..2D-1 the value channel tid - D of this head (loaded twice)
    const int tc = tid < 2 * D ? tid : 0;
    const int nch = tid < D ? 2 : (tid < 2 * D ? 1 : 0);
    const int chan0 = tid < D ? kh * D + tc : 2 * HK * D + h * D + (tc - D + (tid >= 2 * D ? D : 0));
    const int chan1 = tid < D ? HK * D + kh * D + tc : chan0;
    const int chan[2] = {chan0, chan1};
    ChanIn<NR, T> cin[2];
    cin[0] = load_channel<NR>(p, slot, b, chan0);
    cin[1] = load_channel<NR>(p, slot, b, chan1);

    // The whole state slice: lane (rq, g) holds rows 4rq..4rq+3 at key
    // indices j = jj*GJ + g. The prologue below runs while it lands.
    const int rq = tid % LPJ;
    const int g = tid / LPJ;
    const float *S0 = p.ssm + ((size_t)slot * HV + h) * D * D;
    float4 s[JPER];
#pragma unroll
    for (int jj = 0; jj < JPER; ++jj)
        s[jj] = *reinterpret_cast<const float4 *>(S0 + (size_t)(jj * GJ + g) * D + 4 * rq);
    __builtin_amdgcn_sched_barrier(0);

    if (tid < NR) {
        alp[tid] = to_f32(ga);
        bet[tid] = to_f32(gb);
    }
    if (nch == 2) {
        float y[NR];
        conv_rows(cin[0], p.act, y);
#pragma unroll
        for (int t = 0; t < NR; ++t)
            Mt[tid * MS + NR + t] = y[t];
        conv_rows(cin[1], p.act, y);
#pragma unroll
        for (int t = 0; t < NR; ++t)
            Mt[tid * MS + t] = y[t];
    } else if (nch == 1) {
        float y[NR];
        conv_rows(cin[0], p.act, y);
#pragma unroll
        for (int t = 0; t < NR; ++t)
            vb[t * D + (tid - D)] = y[t];
    }
    lds_barrier();

    // L2 norms of the 2*NR vectors (one wave per vector)
    for (int c = wave; c < NC; c += 4) {
        float ss = 0.0f;
        for (int j = lane; j < D; j += 64) {
            const float v = Mt[j * MS + c];
            ss = __builtin_fmaf(v, v, ss);
        }
        ss = wave_sum(ss);
        if (lane == 0)
            inv[c] = 1.0f / sqrtf(ss + p.eps);
    }
    lds_barrier();
    for (int idx = tid; idx < D * NC; idx += kThreads) {
        const int j = idx / NC, c = idx % NC;
        Mt[j * MS + c] *= inv[c];
    }
    lds_barrier();

    // Gram entries k_hat_u . k_hat_t and k_hat_u . q_hat_t for u <= t
    for (int idx = tid; idx < 2 * NPAIR; idx += kThreads) {
        const int which = idx / NPAIR;
        int pr = idx % NPAIR, t = 0;
        while (pr > t) {
            pr -= t + 1;
            ++t;
        }
        const int u = pr;
        const int ca = which ? NR + t : t;
        float acc = 0.0f;
        for (int j = 0; j < D; ++j)
            acc = __builtin_fmaf(Mt[j * MS + ca], Mt[j * MS + u], acc);
        (which ? gkq : gkk)[t * NR + u] = acc;
    }
    lds_barrier();

    // scalar coefficients: gam[t] = a_0...a_t; cA = g(t,u) k_u.k_t; cB = g(t,u) k_u.q_t
    if (tid < NR * NR) {
        const int t = tid / NR, u = tid % NR;
        float gtu = 1.0f;
        for (int m = u + 1; m <= t; ++m)
            gtu *= alp[m];
        cA[tid] = (u < t) ? gtu * gkk[tid] : 0.0f;
        cB[tid] = (u <= t) ? gtu * gkq[tid] : 0.0f;
    }
    if (tid < NR) {
        float gt = 1.0f;
        for (int m = 0; m <= tid; ++m)
            gt *= alp[m];
        gam[tid] = gt;
    }

    // S_0 times the 2*NR column vectors
    float acc[4][NC];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c)
            acc[r][c] = 0.0f;
#pragma unroll
    for (int jj = 0; jj < JPER; ++jj) {
        const int j = jj * GJ + g;
        float m[MS];
#pragma unroll
        for (int q = 0; q < MS / 4; ++q)
            *reinterpret_cast<float4 *>(&m[4 * q]) = *reinterpret_cast<const float4 *>(&Mt[j * MS + 4 * q]);
        const float sv[4] = {s[jj].x, s[jj].y, s[jj].z, s[jj].w};
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < NC; ++c)
                acc[r][c] = __builtin_fmaf(sv[r], m[c], acc[r][c]);
    }
#pragma unroll
    for (int off = LPJ; off < 64; off <<= 1)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < NC; ++c)
                acc[r][c] += __shfl_xor(acc[r][c], off, 64);
    if (lane < LPJ) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < NC; ++c)
                red[(wave * D + 4 * rq + r) * NC + c] = acc[r][c];
    }

    // Scratch for the commit; stores start only now that the state has landed.
    const bool owner = (h % G) == 0;  // one value head per key head stores q/k inputs
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (k < nch && (nch == 1 || owner)) {
#pragma unroll
            for (int t = 0; t < NR; ++t)
                p.xs[((size_t)b * NR + t) * p.C + chan[k]] = cin[k].x[t];
        }
    }
    if (tid < NR)
        p.as[((size_t)b * NR + tid) * HV + h] = alp[tid];
    if (owner) {
        for (int idx = tid; idx < NR * D; idx += kThreads) {
            const int t = idx / D, j = idx % D;
            p.ks[(((size_t)b * NR + t) * HK + kh) * D + j] = Mt[j * MS + t];
        }
    }
    lds_barrier();

    // per state row i: correction vectors and outputs
    float pk[NR], pq[NR];
    if (tid < D) {
#pragma unroll
        for (int c = 0; c < NR; ++c) {
            float a = 0.0f, q = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                a += red[(w * D + tid) * NC + c];
                q += red[(w * D + tid) * NC + NR + c];
            }
            pk[c] = a;
            pq[c] = q;
        }
    }
    if (SNAP)
        lds_barrier();  // red is reused for e_t below
    if (tid < D) {
        const int i = tid;
        float e[NR];
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            float sres = __builtin_fmaf(-gam[t], pk[t], vb[t * D + i]);
#pragma unroll
            for (int u = 0; u < t; ++u)
                sres = __builtin_fmaf(-cA[t * NR + u], e[u], sres);
            e[t] = bet[t] * sres;
            float o = gam[t] * pq[t];
#pragma unroll
            for (int u = 0; u <= t; ++u)
                o = __builtin_fmaf(cB[t * NR + u], e[u], o);
            const size_t oi = (((size_t)b * NR + t) * HV + h) * D + i;
            p.out[oi] = from_f32<T>(p.scale * o);
            p.es[oi] = e[t];
            if (SNAP)
                red[t * D + i] = e[t];
        }
    }

    if (SNAP) {
        lds_barrier();
        // S_t for every row, by the same update the replay commit applies
#pragma unroll 1
        for (int t = 0; t < NR; ++t) {
            const float a = alp[t];
            const float4 ev = *reinterpret_cast<const float4 *>(&red[t * D + 4 * rq]);
            float *dst = p.snap + (((size_t)b * NR + t) * HV + h) * D * D;
#pragma unroll
            for (int jj = 0; jj < JPER; ++jj) {
                const int j = jj * GJ + g;
                const float k = Mt[j * MS + t];
                s[jj].x = row_update(s[jj].x, a, ev.x, k);
                s[jj].y = row_update(s[jj].y, a, ev.y, k);
                s[jj].z = row_update(s[jj].z, a, ev.z, k);
                s[jj].w = row_update(s[jj].w, a, ev.w, k);
                *reinterpret_cast<float4 *>(dst + (size_t)j * D + 4 * rq) = s[jj];
            }
        }
    }
}

// ---- commit ----------------------------------------------------------------

template <typename T> struct CommitParams {
    float *ssm;
    T *conv;
    const int32_t *slot_ids;
    const int32_t *accept;
    int32_t *err;
    const T *xs;
    const float *es;
    const float *ks;
    const float *as;
    const float *snap;
    int HK, HV, C, P, R;
};

template <int D, typename T, bool SNAP>
__global__ __launch_bounds__(kThreads) void gdn_commit_kernel(const CommitParams<T> p)
{
    constexpr int LPJ = D / 4;
    constexpr int GJ = kThreads / LPJ;
    constexpr int JPER = D / GJ;

    __shared__ __align__(16) float eb[kMaxRows * D];
    __shared__ float kb[kMaxRows * D];
    __shared__ float al[kMaxRows];

    const int tid = threadIdx.x;
    const int HV = p.HV, HK = p.HK, R = p.R;
    const int G = HV / HK;
    const int b = blockIdx.x / HV;
    const int h = blockIdx.x % HV;
    const int kh = h / G;
    const int slot = p.slot_ids[b];
    const int n = p.accept[b];

    if (slot < -1 || slot >= p.P) {
        if (tid == 0 && p.err)
            atomicOr(p.err, 1);
        return;
    }
    if (n < 0 || n > R) {
        if (tid == 0 && p.err)
            atomicOr(p.err, 2);
        return;
    }
    if (slot == -1 || n == 0)
        return;

    const int rq = tid % LPJ;
    const int g = tid / LPJ;
    float *Sd = p.ssm + ((size_t)slot * HV + h) * D * D;

    if (SNAP) {
        const float4 *src = reinterpret_cast<const float4 *>(
            p.snap + (((size_t)b * R + (n - 1)) * HV + h) * D * D);
        float4 *dst = reinterpret_cast<float4 *>(Sd);
        float4 v[D * D / 4 / kThreads];
#pragma unroll
        for (int q = 0; q < D * D / 4 / kThreads; ++q)
            v[q] = src[q * kThreads + tid];
#pragma unroll
        for (int q = 0; q < D * D / 4 / kThreads; ++q)
            dst[q * kThreads + tid] = v[q];
    } else {
        // staging loads first (fixed count, clamped indices, no branches),
        // then the state stream
        constexpr int NSTAGE = (kMaxRows * D + kThreads - 1) / kThreads;
        float ev_in[NSTAGE], kv_in[NSTAGE];
#pragma unroll
        for (int q = 0; q < NSTAGE; ++q) {
            const int idx = min(q * kThreads + tid, n * D - 1);
            const int t = idx / D, i = idx % D;
            ev_in[q] = p.es[(((size_t)b * R + t) * HV + h) * D + i];
            kv_in[q] = p.ks[(((size_t)b * R + t) * HK + kh) * D + i];
        }
        const float a_in = p.as[((size_t)b * R + min(tid, n - 1)) * HV + h];
        float4 s[JPER];
#pragma unroll
        for (int jj = 0; jj < JPER; ++jj)
            s[jj] = *reinterpret_cast<const float4 *>(Sd + (size_t)(jj * GJ + g) * D + 4 * rq);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < NSTAGE; ++q) {
            const int idx = q * kThreads + tid;
            if (idx < n * D) {
                eb[idx] = ev_in[q];
                kb[idx] = kv_in[q];
            }
        }
        if (tid < n)
            al[tid] = a_in;
        lds_barrier();
        for (int t = 0; t < n; ++t) {
            const float a = al[t];
            const float4 ev = *reinterpret_cast<const float4 *>(&eb[t * D + 4 * rq]);
#pragma unroll
            for (int jj = 0; jj < JPER; ++jj) {
                const float k = kb[t * D + jj * GJ + g];
                s[jj].x = row_update(s[jj].x, a, ev.x, k);
                s[jj].y = row_update(s[jj].y, a, ev.y, k);
                s[jj].z = row_update(s[jj].z, a, ev.z, k);
                s[jj].w = row_update(s[jj].w, a, ev.w, k);
            }
        }
#pragma unroll
        for (int jj = 0; jj < JPER; ++jj)
            *reinterpret_cast<float4 *>(Sd + (size_t)(jj * GJ + g) * D + 4 * rq) = s[jj];
    }

    // conv history: the last W-1 entries of [history | rows 0..n-1]; the value
    // channels belong to this head, the key head's q/k channels to its first
    // value head
    const bool owner = (h % G) == 0;
    const int nch = owner ? 3 * D : D;
    for (int idx = tid; idx < nch; idx += kThreads) {
        int c;
        if (idx < D)
            c = 2 * HK * D + h * D + idx;
        else if (idx < 2 * D)
            c = kh * D + (idx - D);
        else
            c = HK * D + kh * D + (idx - 2 * D);
        T *hist = p.conv + (size_t)slot * (kWidth - 1) * p.C + c;
        T win[kWidth - 1];
#pragma unroll
        for (int w = 0; w < kWidth - 1; ++w) {
            const int src = n + w;  // index into [history (W-1) | rows]
            win[w] = src < kWidth - 1 ? hist[(size_t)src * p.C]
                                      : p.xs[((size_t)b * R + (src - (kWidth - 1))) * p.C + c];
        }
#pragma unroll
        for (int w = 0; w < kWidth - 1; ++w)
            hist[(size_t)w * p.C] = win[w];
    }
}

// ---- host side -------------------------------------------------------------

struct Checked {
    int HK, HV, D, C;
    size_t esize;
};

gdn_status check_desc(const gdn_layer_desc *d, Checked *c)
{
    if (!d)
        return GDN_ERR_INVALID_ARG;
    if (d->num_k_heads < 1 || d->num_v_heads < 1 || d->d_k < 1 || d->d_v < 1 ||
        d->num_v_heads % d->num_k_heads != 0)
        return GDN_ERR_INVALID_ARG;
    if (d->dtype != GDN_F32 && d->dtype != GDN_BF16)
        return GDN_ERR_INVALID_ARG;
    if (d->act != GDN_ACT_SILU && d->act != GDN_ACT_NONE)
        return GDN_ERR_INVALID_ARG;
    if (d->d_k != d->d_v || (d->d_k != 32 && d->d_k != 64 && d->d_k != 128))
        return GDN_ERR_UNSUPPORTED;
    if (d->conv_width != kWidth)
        return GDN_ERR_UNSUPPORTED;
    c->HK = d->num_k_heads;
    c->HV = d->num_v_heads;
    c->D = d->d_k;
    c->C = 2 * c->HK * c->D + c->HV * c->D;
    c->esize = d->dtype == GDN_F32 ? 4 : 2;
    return GDN_OK;
}

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

template <int D, int NR, typename T, bool SNAP>
hipError_t launch_verify(const VerifyParams<T> &vp, int blocks, hipStream_t st)
{
    hipLaunchKernelGGL((gdn_verify_kernel<D, NR, T, SNAP>), dim3(blocks), dim3(kThreads), 0, st, vp);
    return hipGetLastError();
}

template <int D, typename T, bool SNAP>
hipError_t verify_rows(int rows, const VerifyParams<T> &vp, int blocks, hipStream_t st)
{
    switch (rows) {
    case 1: return launch_verify<D, 1, T, SNAP>(vp, blocks, st);
    case 2: return launch_verify<D, 2, T, SNAP>(vp, blocks, st);
    case 3: return launch_verify<D, 3, T, SNAP>(vp, blocks, st);
    case 4: return launch_verify<D, 4, T, SNAP>(vp, blocks, st);
    case 5: return launch_verify<D, 5, T, SNAP>(vp, blocks, st);
    case 6: return launch_verify<D, 6, T, SNAP>(vp, blocks, st);
    case 7: return launch_verify<D, 7, T, SNAP>(vp, blocks, st);
    case 8: return launch_verify<D, 8, T, SNAP>(vp, blocks, st);
    case 9: return launch_verify<D, 9, T, SNAP>(vp, blocks, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, bool SNAP>
hipError_t verify_dim(int D, int rows, const VerifyParams<T> &vp, int blocks, hipStream_t st)
{
    switch (D) {
    case 32: return verify_rows<32, T, SNAP>(rows, vp, blocks, st);
    case 64: return verify_rows<64, T, SNAP>(rows, vp, blocks, st);
    case 128: return verify_rows<128, T, SNAP>(rows, vp, blocks, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t verify_typed(const Checked &c, const gdn_layer_desc *d, const gdn_pool *pool,
                        const void *conv_w, const void *x, const void *alpha, const void *beta,
                        const int32_t *slot_ids, int batch, int rows, bool snapshot, void *scratch,
                        const ScratchLayout &L, void *out, int32_t *err, hipStream_t st)
{
    VerifyParams<T> vp;
    char *base = static_cast<char *>(scratch);
    vp.ssm = pool->ssm;
    vp.conv = static_cast<const T *>(pool->conv);
    vp.conv_w = static_cast<const T *>(conv_w);
    vp.x = static_cast<const T *>(x);
    vp.alpha = static_cast<const T *>(alpha);
    vp.beta = static_cast<const T *>(beta);
    vp.slot_ids = slot_ids;
    vp.out = static_cast<T *>(out);
    vp.err = err;
    vp.xs = reinterpret_cast<T *>(base + L.xs);
    vp.es = reinterpret_cast<float *>(base + L.es);
    vp.ks = reinterpret_cast<float *>(base + L.ks);
    vp.as = reinterpret_cast<float *>(base + L.as);
    vp.snap = snapshot ? reinterpret_cast<float *>(base + L.snap) : nullptr;
    vp.HK = c.HK;
    vp.HV = c.HV;
    vp.C = c.C;
    vp.P = pool->num_slots;
    vp.act = d->act;
    vp.scale = d->scale;
    vp.eps = d->l2_eps;
    const int blocks = batch * c.HV;
    return snapshot ? verify_dim<T, true>(c.D, rows, vp, blocks, st)
                    : verify_dim<T, false>(c.D, rows, vp, blocks, st);
}

template <int D, typename T, bool SNAP>
hipError_t launch_commit(const CommitParams<T> &cp, int blocks, hipStream_t st)
{
    hipLaunchKernelGGL((gdn_commit_kernel<D, T, SNAP>), dim3(blocks), dim3(kThreads), 0, st, cp);
    return hipGetLastError();
}

template <typename T, bool SNAP>
hipError_t commit_dim(int D, const CommitParams<T> &cp, int blocks, hipStream_t st)
{
    switch (D) {
    case 32: return launch_commit<32, T, SNAP>(cp, blocks, st);
    case 64: return launch_commit<64, T, SNAP>(cp, blocks, st);
    case 128: return launch_commit<128, T, SNAP>(cp, blocks, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t commit_typed(const Checked &c, const gdn_pool *pool, const int32_t *slot_ids,
                        const int32_t *accept, int batch, int rows, bool snapshot,
                        const void *scratch, const ScratchLayout &L, int32_t *err, hipStream_t st)
{
    CommitParams<T> cp;
    const char *base = static_cast<const char *>(scratch);
    cp.ssm = pool->ssm;
    cp.conv = static_cast<T *>(pool->conv);
    cp.slot_ids = slot_ids;
    cp.accept = accept;
    cp.err = err;
    cp.xs = reinterpret_cast<const T *>(base + L.xs);
    cp.es = reinterpret_cast<const float *>(base + L.es);
    cp.ks = reinterpret_cast<const float *>(base + L.ks);
    cp.as = reinterpret_cast<const float *>(base + L.as);
    cp.snap = snapshot ? reinterpret_cast<const float *>(base + L.snap) : nullptr;
    cp.HK = c.HK;
    cp.HV = c.HV;
    cp.C = c.C;
    cp.P = pool->num_slots;
    cp.R = rows;
    const int blocks = batch * c.HV;
    return snapshot ? commit_dim<T, true>(c.D, cp, blocks, st)
                    : commit_dim<T, false>(c.D, cp, blocks, st);
}

gdn_status check_common(const gdn_layer_desc *desc, const gdn_pool *pool, int32_t batch,
                        int32_t rows, gdn_commit_mode mode, const void *scratch,
                        size_t scratch_bytes, Checked *c, ScratchLayout *L)
{
    gdn_status s = check_desc(desc, c);
    if (s != GDN_OK)
        return s;
    if (!pool || !pool->ssm || !pool->conv || pool->num_slots < 1 || !aligned16(pool->ssm))
        return GDN_ERR_INVALID_ARG;
    if (batch < 0 || rows < 1 || rows > kMaxRows)
        return GDN_ERR_INVALID_ARG;
    if (mode != GDN_COMMIT_REPLAY && mode != GDN_COMMIT_SNAPSHOT)
        return GDN_ERR_INVALID_ARG;
    if ((size_t)batch * c->HV > 0x7fffffffu)
        return GDN_ERR_UNSUPPORTED;
    *L = scratch_layout(c->HK, c->HV, c->D, c->C, c->esize, batch, rows, mode == GDN_COMMIT_SNAPSHOT);
    if (batch > 0 && (!scratch || !aligned16(scratch)))
        return GDN_ERR_INVALID_ARG;
    if (scratch_bytes < L->total)
        return GDN_ERR_SCRATCH_TOO_SMALL;
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_spec_scratch_bytes(const gdn_layer_desc *desc, int32_t batch, int32_t rows,
                                  gdn_commit_mode mode, size_t *bytes)
{
    Checked c;
    gdn_status s = check_desc(desc, &c);
    if (s != GDN_OK)
        return s;
    if (!bytes || batch < 0 || rows < 1 || rows > kMaxRows ||
        (mode != GDN_COMMIT_REPLAY && mode != GDN_COMMIT_SNAPSHOT))
        return GDN_ERR_INVALID_ARG;
    *bytes = scratch_layout(c.HK, c.HV, c.D, c.C, c.esize, batch, rows, mode == GDN_COMMIT_SNAPSHOT).total;
    return GDN_OK;
}

gdn_status gdn_spec_verify(const gdn_layer_desc *desc, const gdn_pool *pool, const void *conv_w,
                           const void *x, const void *alpha, const void *beta,
                           const int32_t *slot_ids, int32_t batch, int32_t rows,
                           gdn_commit_mode mode, void *scratch, size_t scratch_bytes, void *out,
                           int32_t *err_flag, void *stream)
{
    Checked c;
    ScratchLayout L;
    gdn_status s = check_common(desc, pool, batch, rows, mode, scratch, scratch_bytes, &c, &L);
    if (s != GDN_OK)
        return s;
    if (batch == 0)
        return GDN_OK;
    if (!conv_w || !x || !alpha || !beta || !slot_ids || !out)
        return GDN_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool snap = mode == GDN_COMMIT_SNAPSHOT;
    hipError_t e = desc->dtype == GDN_F32
        ? verify_typed<float>(c, desc, pool, conv_w, x, alpha, beta, slot_ids, batch, rows, snap,
                              scratch, L, out, err_flag, st)
        : verify_typed<bf16_t>(c, desc, pool, conv_w, x, alpha, beta, slot_ids, batch, rows, snap,
                               scratch, L, out, err_flag, st);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_spec_commit(const gdn_layer_desc *desc, const gdn_pool *pool,
                           const int32_t *slot_ids, const int32_t *accept_len, int32_t batch,
                           int32_t rows, gdn_commit_mode mode, const void *scratch,
                           size_t scratch_bytes, int32_t *err_flag, void *stream)
{
    Checked c;
    ScratchLayout L;
    gdn_status s = check_common(desc, pool, batch, rows, mode, scratch, scratch_bytes, &c, &L);
    if (s != GDN_OK)
        return s;
    if (batch == 0)
        return GDN_OK;
    if (!slot_ids || !accept_len)
        return GDN_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool snap = mode == GDN_COMMIT_SNAPSHOT;
    hipError_t e = desc->dtype == GDN_F32
        ? commit_typed<float>(c, pool, slot_ids, accept_len, batch, rows, snap, scratch, L, err_flag, st)
        : commit_typed<bf16_t>(c, pool, slot_ids, accept_len, batch, rows, snap, scratch, L, err_flag, st);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

const char *gdn_strerror(gdn_status status)
{
    switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported shape";
    case GDN_ERR_SCRATCH_TOO_SMALL: return "scratch buffer too small";
    case GDN_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

}  // extern "C"
