// gdn_spec.hip -- GatedDeltaNet speculative verify / commit for MI355X (gfx950).
//
// Implements the C ABI of include/gdn_spec.h.
//
// Verify (FreeToken issue #828, Design: the verify rows run as a uniform
// extend and only read the GatedDeltaNet state). Rather than stepping the
// state row by row (4 multiply-adds per state element per row), the kernels
// use the exact unrolled form of the gated delta rule. With e_t the row's
// correction vector and g(t,u) = a_{u+1} ... a_t (g(t,t) = 1):
//
//     S_t     = g(t,-1) S_0 + sum_{u<=t} g(t,u) e_u k_u^T
//     e_t     = b_t (v_t - a_t S_{t-1} k_t)
//             = b_t (v_t - g(t,-1) S_0 k_t - sum_{u<t} g(t,u) (k_u . k_t) e_u)
//     o_t     = scale (g(t,-1) S_0 q_t + sum_{u<=t} g(t,u) (k_u . q_t) e_u)
//
// One pass over S_0 computing the 2R products S_0 k_t and S_0 q_t, plus R x R
// scalar algebra per state row, gives every o_t. The state is streamed once
// from HBM and never written.
//
// For d = 128 (gdn_verify_d128_kernel) the 2R products, and the Gram entries
// k_u.k_t and k_u.q_t the scalar algebra needs, come out of one pass on the
// matrix cores; other head dims use a VALU kernel (gdn_verify_kernel).
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
constexpr int kWidth = 4;    // the one conv width the kernels support
constexpr int kMaxRows = 9;  // k + 1 with k <= 8 drafts
constexpr int kMaxGroup = 16; // value heads per key head
constexpr size_t kAlign = 256;
constexpr int kXcds = 8;       // accelerator complex dies, each with its own L2

typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// Buffer loads: an SGPR resource (base, size in bytes), a 32-bit per-lane
// byte offset and a uniform byte offset. Keeps address registers to one per
// lane, and the hardware returns zero for any byte outside the resource.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

template <typename T> __device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff);
template <> __device__ __forceinline__ float buf_load<float>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}
template <> __device__ __forceinline__ bf16_t buf_load<bf16_t>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return bf16_t{__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0)};
}

// State and snapshot traffic: every kernel streams it exactly once. The
// nontemporal hint (cache-policy bit nt) keeps it from displacing the small
// per-row inputs and the stash in the caches, and keeps dirty state lines from
// piling up in the memory-side cache for the next kernel to write back.
constexpr int kStreamPolicy = 2;

__device__ __forceinline__ f32x4 buf_stream_load_f4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kStreamPolicy));
}

__device__ __forceinline__ void buf_stream_store_f4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, f32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, v), r,
                                           (int)voff, (int)soff, kStreamPolicy);
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land
// at lds + 16 i (lds uniform across the wave). The host pass never sees the
// builtin: parsed there, it drops the host stub of every kernel that uses it.
__device__ __forceinline__ void lds_dma16(const float *src, float *lds)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
#endif
}

__device__ __forceinline__ float4 stream_load(const float *ptr)
{
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(ptr));
    return float4{v[0], v[1], v[2], v[3]};
}

__device__ __forceinline__ void stream_store(float *ptr, f32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(ptr));
}

__device__ __forceinline__ void stream_store(float *ptr, float4 v)
{
    stream_store(ptr, f32x4{v.x, v.y, v.z, v.w});
}

// The verify's outputs and the stash it leaves for the commit are written
// once and read by later kernels only. Written back (plain stores), they are
// still dirty in L2 when the last wave ends, and the release at the end of
// the kernel flushes them while the rest of the chip idles: about 4 us of
// the saturated batch's 28 MB. Nontemporal stores drain them as they go.
template <typename X> __device__ __forceinline__ void out_store(X *ptr, X v)
{
    __builtin_nontemporal_store(v, ptr);
}

__device__ __forceinline__ void out_store(bf16_t *ptr, bf16_t v)
{
    __builtin_nontemporal_store(v.bits, &ptr->bits);
}

__device__ __forceinline__ void out_store(uint4 *ptr, uint4 v)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4 *>(ptr));
}

// Barrier that orders LDS only: global loads already in flight (the state
// prefetch) are not drained by it.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int CTRL> __device__ __forceinline__ float dpp_mov(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float lane_value(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over the 64 lanes of a wave, returned to every lane. DPP butterflies
// within each 16-lane row (xor 1 and xor 2 by quad permutes, then the half-row
// and row mirrors), then the four row sums in a fixed order: every lane gets
// the same bits on every run.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);  // row_half_mirror
    v += dpp_mov<0x140>(v);  // row_mirror
    return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

__device__ __forceinline__ float silu(float y)
{
    return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y));
}

// One accepted row replayed on one state element: S <- a S + e k.
__device__ __forceinline__ float row_update(float s, float a, float e, float k)
{
    return __builtin_fmaf(e, k, a * s);
}

// Triangular index of a pair (t, u), u <= t, enumerated row by row.
__device__ __forceinline__ void tri_decode(int idx, int &t, int &u)
{
    t = 0;
    while (idx > t) {
        idx -= t + 1;
        ++t;
    }
    u = idx;
}

// ---- scratch layout (shared by host and device code) -----------------------

// Scalar coefficients of one value head, as the verify kernels keep them in
// LDS: a_t, g(t,-1), b_t, then the R x R blocks g(t,u) k_u.k_t (u < t) and
// g(t,u) k_u.q_t (u <= t).
__host__ __device__ constexpr int coef_count(int R) { return 3 * R + 2 * R * R; }

struct ScratchLayout {
    size_t xs, es, ks, as, xh, snap, total;
};

__host__ __device__ inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Per request b (row b of every part):
//   xs   [B][R][C]          raw verify inputs (storage type), for the conv commit
//   es   [B][R][HV][D]      fp32 correction vector e_t of each row and value head
//   ks   [B][HK][R][D]      fp32 normalised k_t of each row and key head
//   as   [B][HV][R]         fp32 decay gate a_t
//   xh   [B][W-1][C]        the conv history the verify read (storage type;
//                           written by the replay-mode bf16 d = 128 kernels,
//                           so that a commit-verify of the next step builds
//                           the committed history from scratch alone)
//   snap [B][HV][R][D][D]   fp32 S_t after each row (snapshot mode only), same
//                           per-head layout as the pool
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
    off = align_up(off + (size_t)B * HK * R * D * sizeof(float));
    L.as = off;
    off = align_up(off + (size_t)B * HV * R * sizeof(float));
    L.xh = off;
    off = align_up(off + (size_t)B * (kWidth - 1) * C * esize);
    L.snap = off;
    if (snapshot)
        off = align_up(off + (size_t)B * R * HV * D * D * sizeof(float));
    L.total = off;
    return L;
}

// ---- verify: shared pieces ---------------------------------------------------

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
    // commit of the previous step ahead of this verify (commit-verify only):
    // src_row[b] is the previous batch row whose accepted rows are still to
    // be applied to slot_ids[b] (-1: none), read from that step's stash
    float *ssm_out;
    T *hist_out;
    const int32_t *src_row;
    const int32_t *prev_slots;
    const int32_t *prev_accept;
    const T *pxs;
    const float *pes;
    const float *pks;
    const float *pas;
    const T *pxh;
    const float *psnap;   // snapshot mode: the previous step's S_1..S_R
    int Bp;
    T *xh;
};

// Inputs of one conv channel: taps, history (oldest first) and the verify rows.
template <int NR, typename T> struct ChanIn {
    T w[kWidth];
    T hist[kWidth - 1];
    T x[NR];
};

// Row bases are uniform across the workgroup and the channel is the only
// per-lane part, so every load is an SGPR base plus one 32-bit lane offset.
template <int NR, typename T>
__device__ __forceinline__ ChanIn<NR, T> load_channel(const VerifyParams<T> &p, int slot, int b, int c)
{
    ChanIn<NR, T> in;
    const uint32_t E = sizeof(T);
    const uint32_t row = (uint32_t)p.C * E;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.conv_w, row * kWidth);
    const __amdgpu_buffer_rsrc_t rh = make_rsrc(p.conv + (size_t)slot * (kWidth - 1) * p.C, row * (kWidth - 1));
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x + (size_t)b * NR * p.C, row * NR);
#pragma unroll
    for (int k = 0; k < kWidth; ++k)
        in.w[k] = buf_load<T>(rw, (uint32_t)c * kWidth * E, k * E);
#pragma unroll
    for (int k = 0; k < kWidth - 1; ++k)
        in.hist[k] = buf_load<T>(rh, (uint32_t)c * E, k * row);
#pragma unroll
    for (int t = 0; t < NR; ++t)
        in.x[t] = buf_load<T>(rx, (uint32_t)c * E, t * row);
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
        y[t] = act == GDN_ACT_SILU ? silu(acc) : acc;
    }
}

template <typename T>
__device__ __forceinline__ void zero_outputs(const VerifyParams<T> &p, int b, int h, int NR, int D)
{
    for (int idx = threadIdx.x; idx < NR * D; idx += kThreads) {
        const int t = idx / D, i = idx % D;
        out_store(&p.out[(((size_t)b * NR + t) * p.HV + h) * D + i], from_f32<T>(0.0f));
    }
}

// Per state row i (thread i): e_t and o_t from S_0 k_t (pk) and S_0 q_t (pq),
// the row's values v_t and the scalar coefficients cf (coef_count(NR) floats).
template <int NR, typename T>
__device__ __forceinline__ void solve_row(const VerifyParams<T> &p, const float *cf, const float (&pk)[NR],
                                          const float (&pq)[NR], const float (&v)[NR], float (&e)[NR],
                                          int b, int h, int i, int D)
{
    const float *gam = cf + NR, *bet = cf + 2 * NR, *cA = cf + 3 * NR, *cB = cf + 3 * NR + NR * NR;
#pragma unroll
    for (int t = 0; t < NR; ++t) {
        float sres = __builtin_fmaf(-gam[t], pk[t], v[t]);
#pragma unroll
        for (int u = 0; u < t; ++u)
            sres = __builtin_fmaf(-cA[t * NR + u], e[u], sres);
        e[t] = bet[t] * sres;
        float o = gam[t] * pq[t];
#pragma unroll
        for (int u = 0; u <= t; ++u)
            o = __builtin_fmaf(cB[t * NR + u], e[u], o);
        const size_t oi = (((size_t)b * NR + t) * p.HV + h) * D + i;
        out_store(&p.out[oi], from_f32<T>(p.scale * o));
        out_store(&p.es[oi], e[t]);
        __builtin_amdgcn_sched_barrier(0);  // one row at a time: bounds the hoisted coefficient reads
    }
}

// Coefficient idx (< NR*NR + NR) of one value head from the Gram entries
// gkk[t][u] = k_u.k_t and gkq[t][u] = k_u.q_t (u <= t) and the head's gates
// al[t], be[t] (LDS); written to cf.
template <int NR>
__device__ __forceinline__ void write_coefficients(const float *gkk, const float *gkq, const float *al,
                                                   const float *be, int idx, float *cf)
{
    if (idx < NR * NR) {
        const int t = idx / NR, u = idx % NR;
        float gtu = 1.0f;
        for (int q = u + 1; q <= t; ++q)
            gtu *= al[q];
        cf[3 * NR + idx] = (u < t) ? gtu * gkk[idx] : 0.0f;
        cf[3 * NR + NR * NR + idx] = (u <= t) ? gtu * gkq[idx] : 0.0f;
    } else if (idx < NR * NR + NR) {
        const int t = idx - NR * NR;
        float gt = 1.0f;
        for (int q = 0; q <= t; ++q)
            gt *= al[q];
        cf[t] = al[t];
        cf[NR + t] = gt;
        cf[2 * NR + t] = be[t];
    }
}

// ---- verify, d = 32 / 64: one fused kernel on the VALU ----------------------
//
// One workgroup per (request, value head). Lane (rq, g) holds state rows
// 4rq..4rq+3 at key indices jj*GJ + g and accumulates their products with the
// 2R columns from LDS; the partial sums of the key-index groups are added
// across lanes and waves.
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
    constexpr int NCF = coef_count(NR);

    __shared__ __align__(16) float Mt[D * MS];    // [j][c]: k_hat_t[j] (c < NR), q_hat_t[j]
    __shared__ __align__(16) float vb[NR * D];    // v_t[i]; e_t in snapshot mode
    __shared__ __align__(16) float red[4 * D * NC];  // per-wave partial products
    __shared__ float inv[NC];
    __shared__ float gkk[NR * NR], gkq[NR * NR];
    __shared__ float cf[NCF];
    __shared__ float al[NR], be[NR];

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
        zero_outputs(p, b, h, NR, D);
        return;
    }

    const size_t gi = ((size_t)b * NR + min(tid, NR - 1)) * HV + h;
    const T ga = p.alpha[gi], gb = p.beta[gi];

    // channels: threads < D take the key head's q and k channel `tid`,
    // threads D..2D-1 the value channel tid - D of this head
    const int tc = tid < 2 * D ? tid : 0;
    const int nch = tid < D ? 2 : (tid < 2 * D ? 1 : 0);
    const int chan0 = tid < D ? kh * D + tc : 2 * HK * D + h * D + (tc - D + (tid >= 2 * D ? D : 0));
    const int chan1 = tid < D ? HK * D + kh * D + tc : chan0;
    ChanIn<NR, T> cin0 = load_channel<NR>(p, slot, b, chan0);
    ChanIn<NR, T> cin1 = load_channel<NR>(p, slot, b, chan1);

    const int rq = tid % LPJ;
    const int g = tid / LPJ;
    const float *S0 = p.ssm + ((size_t)slot * HV + h) * D * D;
    float4 s[JPER];
#pragma unroll
    for (int jj = 0; jj < JPER; ++jj)
        s[jj] = stream_load(S0 + (size_t)(jj * GJ + g) * D + 4 * rq);
    __builtin_amdgcn_sched_barrier(0);

    if (tid < NR) {
        al[tid] = to_f32(ga);
        be[tid] = to_f32(gb);
    }
    if (nch == 2) {
        float y[NR];
        conv_rows(cin0, p.act, y);
#pragma unroll
        for (int t = 0; t < NR; ++t)
            Mt[tid * MS + NR + t] = y[t];
        conv_rows(cin1, p.act, y);
#pragma unroll
        for (int t = 0; t < NR; ++t)
            Mt[tid * MS + t] = y[t];
    } else if (nch == 1) {
        float y[NR];
        conv_rows(cin0, p.act, y);
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
        int t, u;
        tri_decode(idx % NPAIR, t, u);
        const int ca = which ? NR + t : t;
        float acc = 0.0f;
        for (int j = 0; j < D; ++j)
            acc = __builtin_fmaf(Mt[j * MS + ca], Mt[j * MS + u], acc);
        (which ? gkq : gkk)[t * NR + u] = acc;
    }
    lds_barrier();
    for (int idx = tid; idx < NR * NR + NR; idx += kThreads)
        write_coefficients<NR>(gkk, gkq, al, be, idx, cf);

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

    // scratch for the commit; stores start only now that the state has landed
    const bool owner = (h % G) == 0;  // one value head per key head stores q/k inputs and the table
#pragma unroll
    for (int t = 0; t < NR; ++t) {
        if (nch == 1 || (nch == 2 && owner)) {
            out_store(&p.xs[((size_t)b * NR + t) * p.C + chan0], cin0.x[t]);
            if (nch == 2)
                out_store(&p.xs[((size_t)b * NR + t) * p.C + chan1], cin1.x[t]);
        }
    }
    if (owner) {
        float *ks = p.ks + ((size_t)b * HK + kh) * NR * D;
        for (int idx = tid; idx < NR * D; idx += kThreads)
            out_store(&ks[idx], Mt[(idx % D) * MS + idx / D]);
    }
    if (tid < NR)
        out_store(&p.as[((size_t)b * HV + h) * NR + tid], al[tid]);
    lds_barrier();

    // per state row i: correction vectors and outputs
    if (tid < D) {
        float pk[NR], pq[NR], v[NR], e[NR];
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
            v[c] = vb[c * D + tid];
        }
        solve_row<NR>(p, cf, pk, pq, v, e, b, h, tid, D);
        if (SNAP) {
            // entries of column tid of vb are read and written by this thread only
#pragma unroll
            for (int t = 0; t < NR; ++t)
                vb[t * D + tid] = e[t];
        }
    }

    if (SNAP) {
        lds_barrier();
        // S_t for every row, by the same update the replay commit applies
#pragma unroll 1
        for (int t = 0; t < NR; ++t) {
            const float a = cf[t];
            const float4 ev = *reinterpret_cast<const float4 *>(&vb[t * D + 4 * rq]);
            float *dst = p.snap + (((size_t)b * HV + h) * NR + t) * D * D;
#pragma unroll
            for (int jj = 0; jj < JPER; ++jj) {
                const int j = jj * GJ + g;
                const float k = Mt[j * MS + t];
                s[jj].x = row_update(s[jj].x, a, ev.x, k);
                s[jj].y = row_update(s[jj].y, a, ev.y, k);
                s[jj].z = row_update(s[jj].z, a, ev.z, k);
                s[jj].w = row_update(s[jj].w, a, ev.w, k);
                stream_store(dst + (size_t)j * D + 4 * rq, s[jj]);
            }
        }
    }
}

// ---- verify, d = 128: one pass on the matrix cores --------------------------
//
// The 2R products S_0 k_t, S_0 q_t are a dense (128 x 128) x (128 x 2R)
// contraction, run with v_mfma_f32_16x16x4_f32 (fp32 in, fp32 accumulate).
//
// One workgroup per (request, pair of value heads on one key head): the conv
// of the key head's q/k channels is done once for both heads, and with 4
// workgroups per compute unit a 64-request batch is resident in one round.
// Thread t convolves q/k channel t and value channel t of the pair; after
// the column table M (the raw conv outputs [k_0..k_{R-1} | q_0..q_{R-1}]) is
// in LDS there is no further workgroup barrier: wave w owns state rows
// 64(w&1)..64(w&1)+63 of value head h0 + (w>>1), which are exactly the rows
// whose value channels its own lanes convolved, and it finishes them alone.
//
// Per wave: lane l (kg = l/16, m = l%16) loads rows 4m..4m+3 of the block at
// key index j = 4s + kg of K-step s as one 16-byte load, which is the A
// operand of four 16-row tiles (tile v holds rows 4m + v: A[m][k] =
// S[4m+v][4s+k]). The state streams in chunks of 4 K-steps, two chunks in
// flight. The first 16 columns of M go through one 16-wide B tile; with
// R = 9 the last two (q_7, q_8) are done on the VALU from the same registers.
// Between chunks, the wave forms M^T M with a tile whose A operand is the B
// value itself (A[m][k] = M[4s+k][m]), giving the column norms (diagonal) and
// every Gram entry k_u.k_t, k_u.q_t; the L2 normalisation is then a column
// scaling applied to the Gram entries and to S_0 M. Still between chunks it
// forms its head's scalar coefficients and L^{-1} diag(b) (below), so after
// the last chunk only the per-row solve remains.
//
// The per-row recurrence for e_t is a unit lower-triangular system shared by
// every state row, e = L^{-1} diag(b) (v - g S_0 k), L = I + diag(b) A with
// A[t][u] = g(t,u) k_u.k_t (u < t), so each row's e_t and o_t are two small
// matrix-vector products.

// Orders this wave's LDS writes before its later LDS reads (one wave: no
// workgroup barrier).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// This wave's share (K-steps 8w..8w+7) of M^T M: tile rows are columns 0..15
// of M; the VALU columns 16, 17 (NVL = 2) give gv (their products with the
// tile rows) and dv (their own squared norms), as per-lane partial sums over
// the lane's kg.
template <int NVL, int MS>
__device__ __forceinline__ void gram_share(int wave, int kg, int m, const float *Mt, f32x4 &accg,
                                           float (&gv)[2], float (&dv)[2])
{
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int j = 4 * (8 * wave + k) + kg;
        const float bm = Mt[j * MS + m];
        accg = __builtin_amdgcn_mfma_f32_16x16x4f32(bm, bm, accg, 0, 0, 0);
        if (NVL) {
            const float2 mv = *reinterpret_cast<const float2 *>(&Mt[j * MS + 16]);
            gv[0] = __builtin_fmaf(bm, mv.x, gv[0]);
            gv[1] = __builtin_fmaf(bm, mv.y, gv[1]);
            dv[0] = __builtin_fmaf(mv.x, mv.x, dv[0]);
            dv[1] = __builtin_fmaf(mv.y, mv.y, dv[1]);
        }
    }
}

// Issue the loads of chunk c exactly here: the empty asm statements keep the
// compiler from hoisting them (and the registers they fill) any earlier.
template <int CK>
__device__ __forceinline__ void load_chunk(f32x4 (&sc)[CK], __amdgpu_buffer_rsrc_t rs, uint32_t soff, int c)
{
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < CK; ++k)
        sc[k] = buf_stream_load_f4(rs, soff, (uint32_t)(c * CK + k) * 4 * 128 * 4);
    asm volatile("" ::: "memory");
}

// The same, with the chunk offset in the per-lane offset, which the
// resource's range check covers (the uniform offset is not checked): a chunk
// past the end of the state returns zeros and moves no bytes.
template <int CK>
__device__ __forceinline__ void load_chunk_checked(f32x4 (&sc)[CK], __amdgpu_buffer_rsrc_t rs, uint32_t soff, int c)
{
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < CK; ++k)
        sc[k] = buf_stream_load_f4(rs, soff + (uint32_t)(c * CK + k) * 4 * 128 * 4, 0);
    asm volatile("" ::: "memory");
}

// Chunk c of the state against the column table: four tiles on the matrix
// cores, and the two VALU columns (NVL = 2) as per-lane partial sums.
template <int CK, int NVL, int MS>
__device__ __forceinline__ void mfma_chunk(const f32x4 (&sc)[CK], int c, int kg, int m, const float *Mt,
                                           f32x4 (&acc)[4], float (&pv)[4][2])
{
#pragma unroll
    for (int k = 0; k < CK; ++k) {
        const int j = 4 * (c * CK + k) + kg;
        const float bm = Mt[j * MS + m];
#pragma unroll
        for (int v = 0; v < 4; ++v)
            acc[v] = __builtin_amdgcn_mfma_f32_16x16x4f32(sc[k][v], bm, acc[v], 0, 0, 0);
        if (NVL) {
            const float2 mv = *reinterpret_cast<const float2 *>(&Mt[j * MS + 16]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                pv[v][0] = __builtin_fmaf(sc[k][v], mv.x, pv[v][0]);
                pv[v][1] = __builtin_fmaf(sc[k][v], mv.y, pv[v][1]);
            }
        }
    }
}

template <int NR, typename T, bool SNAP, bool FUSED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void gdn_verify_d128_kernel(const VerifyParams<T> p)
{
    static_assert(!FUSED || (sizeof(T) == 2 && !SNAP), "commit-verify: bf16 storage, replay");
    constexpr int D = 128;
    constexpr int NC = 2 * NR;
    constexpr int NMF = NC < 16 ? NC : 16;   // columns on the matrix cores
    constexpr int NVL = NC - NMF;            // columns on the VALU (0, or 2 when NR = 9)
    static_assert(NVL == 0 || NVL == 2, "unsupported row count");
    constexpr int MS = NVL ? 20 : 16;        // column-table row stride
    constexpr int PS = NC + 1;               // product-table row stride (odd)
    constexpr int CK = 4;                    // K-steps per chunk
    constexpr int NCHUNK = D / 4 / CK;       // 8 chunks per wave
    constexpr int NT = NR * (NR + 1) / 2;      // pairs (t, u), u <= t
    static_assert(NT <= 64, "one coefficient pair per lane");
    // bf16 inputs are staged: rows [history (W-1) | verify rows] of the
    // workgroup's 512 channels (q 128 | k 128 | v 256), in 16-byte units
    constexpr bool STAGED = sizeof(T) == 2;
    constexpr int NROWS = kWidth - 1 + NR;
    constexpr int UPR = 64;                                 // units per row
    constexpr int NXU = (NR * UPR + kThreads - 1) / kThreads;   // verify-row units per thread
    constexpr int PFLOATS = 4 * 64 * PS > NROWS * 256 ? 4 * 64 * PS : NROWS * 256;

    __shared__ __align__(16) float Mt[D * MS];      // [j][c]: raw k_c[j] (c < NR), q_{c-NR}[j]; 0 beyond NC
    __shared__ __align__(16) float P[PFLOATS];       // staged inputs; then per wave [i][c]: (S_0 M^)[i][c], then e_t
    __shared__ float invs[4][NC];                   // per wave: 1 / |column c of M|
    __shared__ float4 cpark[4][64];                 // per wave: each lane's coefficients during the stream
    __shared__ float gp[4][NR * NC + NR];           // wave w's share: (M^T M)[u][c], u < NR; then |q_t|^2
    __shared__ float al[2][NR], be[2][NR];
    __shared__ float alo[2][FUSED ? NR : 1];         // commit-verify: the previous step's a_t

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: state resources stay in SGPRs
    const int HV = p.HV, HK = p.HK;
    const int G = HV / HK;
    const int npair = HV / 2;
    const int b = blockIdx.x / npair;
    const int h0 = 2 * (blockIdx.x % npair);
    const int kh = h0 / G;
    const int slot_in = p.slot_ids[b];   // its latency overlaps the slot-free loads below
    int src = -1;
    if constexpr (FUSED)
        src = p.src_row[b];

    // Small loads first, branch-free, so they retire ahead of the state
    // stream; those that need no slot (gates, verify rows, taps) go before the
    // slot id is waited for. Threads < 128 take q channel `tid`, threads 128..
    // k channel tid-128; thread tid takes value channel tid of the pair (head
    // h0 + tid/128).
    const int gidx = min(tid, 2 * NR - 1);
    const int ghh = gidx / NR, gtt = gidx % NR;
    const size_t gi = ((size_t)b * NR + gtt) * HV + h0 + ghh;
    const T ga = p.alpha[gi], gb = p.beta[gi];
    const int jc = tid & (D - 1);
    const bool isq = tid < D;
    const int chA = isq ? kh * D + jc : HK * D + kh * D + jc;
    const int chV = 2 * HK * D + h0 * D + tid;
    // staged units: unit u is row u / UPR; units 0..15 q, 16..31 k, 32..63 v
    // channels of that row; unit k of a row starts at local channel 8k
    auto unit_channel = [&](int k) {
        return k < 16 ? kh * D + 8 * k : (k < 32 ? HK * D + kh * D + 8 * (k - 16) : 2 * HK * D + h0 * D + 8 * (k - 32));
    };
    static_assert(NXU <= 3 && (kWidth - 1) * UPR <= kThreads, "staged units per thread");
    uint4 xu0 = {}, xu1 = {}, xu2 = {}, hu = {};   // separate registers: an array here ends up in scratch
    uint2 wA = {}, wV = {};
    ChanIn<NR, T> cinA, cinV;
    if constexpr (STAGED) {
        const T *xbase = p.x + (size_t)b * NR * p.C;
        auto load_xunit = [&](int q) {
            const int u = min(q * kThreads + tid, NR * UPR - 1);
            return *reinterpret_cast<const uint4 *>(xbase + (size_t)(u / UPR) * p.C + unit_channel(u % UPR));
        };
        xu0 = load_xunit(0);
        if constexpr (NXU > 1)
            xu1 = load_xunit(1);
        if constexpr (NXU > 2)
            xu2 = load_xunit(2);
        wA = *reinterpret_cast<const uint2 *>(p.conv_w + (size_t)chA * kWidth);
        wV = *reinterpret_cast<const uint2 *>(p.conv_w + (size_t)chV * kWidth);
    }
    // then the loads that need the slot: a bad slot id reads slot 0's history
    // (any address inside the pool) and the workgroup leaves before the state
    bool bad = slot_in < 0 || slot_in >= p.P;
    int errbits = bad && slot_in != -1 ? 1 : 0;
    // commit-verify: n accepted rows of the previous step's row src go into
    // the state before it is read (a padding request ignores src)
    int n = 0;
    if constexpr (FUSED) {
        if (!bad && src != -1) {
            if (src < 0 || src >= p.Bp || p.prev_slots[src] != slot_in) {
                bad = true;
                errbits |= 4;
            } else {
                n = p.prev_accept[src];
                if (n < 0 || n > NR) {
                    bad = true;
                    errbits |= 2;
                    n = 0;
                }
            }
        }
    }
    const int slot = bad ? 0 : slot_in;
    if constexpr (STAGED) {
        const int u = min(tid, (kWidth - 1) * UPR - 1);
        const int r = u / UPR;
        // (commit-verify with n > 0 pending rows: the committed history,
        // entry n + r of [the history the previous verify read | its rows],
        // all from the previous step's scratch, so no workgroup reads pool
        // history that another one is overwriting)
        const int e = r + n;
        const T *from = n == 0 ? p.conv + ((size_t)slot * (kWidth - 1) + r) * p.C + unit_channel(u % UPR)
            : e < kWidth - 1 ? p.pxh + ((size_t)src * (kWidth - 1) + e) * p.C + unit_channel(u % UPR)
                             : p.pxs + ((size_t)src * NR + e - (kWidth - 1)) * p.C + unit_channel(u % UPR);
        hu = *reinterpret_cast<const uint4 *>(from);
    } else {
        cinA = load_channel<NR>(p, slot, b, chA);
        cinV = load_channel<NR>(p, slot, b, chV);
    }
    if (bad) {
        if (errbits && tid == 0 && p.err)
            atomicOr(p.err, errbits);
        zero_outputs(p, b, h0, NR, D);
        zero_outputs(p, b, h0 + 1, NR, D);
        return;
    }

    const int kg = lane >> 4;
    const int m = lane & 15;
    const int hh = wave >> 1;                        // this wave's head: h0 + hh
    const int rb = 64 * (wave & 1);                  // and its 64-row block
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.ssm + ((size_t)slot * HV + h0 + hh) * D * D, D * D * 4);
    const uint32_t soff = (kg * D + rb + 4 * m) * 4;  // lane byte offset within each K-step block
    // chunks in flight: three; two in the commit-verify, whose stream is a
    // rolled loop over chunk pairs (unrolled, its replay loops keep too many
    // values live for four workgroups per compute unit)
    constexpr int DEPTH = FUSED ? 2 : 3;
    f32x4 c0[CK], c1[CK], c2[DEPTH == 3 ? CK : 1];
    load_chunk(c0, rs, soff, 0);
    load_chunk(c1, rs, soff, 1);
    __builtin_amdgcn_sched_barrier(0);

    if (tid < 2 * NR) {
        al[ghh][gtt] = to_f32(ga);
        be[ghh][gtt] = to_f32(gb);
        out_store(&p.as[((size_t)b * HV + h0 + ghh) * NR + gtt], to_f32(ga));
    }
    const bool owner = (h0 % G) == 0;
    if constexpr (STAGED) {
        // to LDS, and the verify rows' units straight to the raw-row stash
        // LDS rows: history 0..W-2, then the verify rows
        uint4 *Xs = reinterpret_cast<uint4 *>(P);
        if (tid < (kWidth - 1) * UPR)
            Xs[tid] = hu;
        auto stage_xunit = [&](int q, uint4 val) {
            const int u = q * kThreads + tid;
            if (u < NR * UPR) {
                const int r = u / UPR, k = u % UPR;
                Xs[(kWidth - 1) * UPR + u] = val;
                if (k >= 32 || owner)
                    out_store(reinterpret_cast<uint4 *>(p.xs + ((size_t)b * NR + r) * p.C + unit_channel(k)), val);
            }
        };
        stage_xunit(0, xu0);
        if constexpr (NXU > 1)
            stage_xunit(1, xu1);
        if constexpr (NXU > 2)
            stage_xunit(2, xu2);
        lds_barrier();
        {
            // the history this verify used, for the next step's commit-verify;
            // with a commit pending, the committed history also goes to the
            // pool (q/k units by the key head's first pair only)
            const int k = tid % UPR;
            if (tid < (kWidth - 1) * UPR && (k >= 32 || owner)) {
                const size_t hoff = (size_t)(tid / UPR) * p.C + unit_channel(k);
                out_store(reinterpret_cast<uint4 *>(p.xh + (size_t)b * (kWidth - 1) * p.C + hoff), hu);
                if (FUSED && n > 0)
                    out_store(reinterpret_cast<uint4 *>(p.hist_out + (size_t)slot * (kWidth - 1) * p.C + hoff), hu);
            }
        }
        const T *Xt = reinterpret_cast<const T *>(P);
        auto tap = [](uint2 w, int k) {
            return T{(uint16_t)(((k < 2 ? w.x : w.y) >> (16 * (k & 1))) & 0xffffu)};
        };
#pragma unroll
        for (int k = 0; k < kWidth; ++k) {
            cinA.w[k] = tap(wA, k);
            cinV.w[k] = tap(wV, k);
        }
#pragma unroll
        for (int r = 0; r < kWidth - 1; ++r) {
            cinA.hist[r] = Xt[r * 512 + tid];
            cinV.hist[r] = Xt[r * 512 + 256 + tid];
        }
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            cinA.x[t] = Xt[(kWidth - 1 + t) * 512 + tid];
            cinV.x[t] = Xt[(kWidth - 1 + t) * 512 + 256 + tid];
        }
    }
    float v[NR];   // value channel tid = row rb + lane of head h0 + hh
    {
        float y[NR];
        conv_rows(cinA, p.act, y);
#pragma unroll
        for (int t = 0; t < NR; ++t)
            Mt[jc * MS + (isq ? NR + t : t)] = y[t];
        if (isq) {
#pragma unroll
            for (int c = NC; c < MS; ++c)
                Mt[jc * MS + c] = 0.0f;
        }
        conv_rows(cinV, p.act, v);
    }
    // raw row inputs for the commit's conv history (staged inputs were stored
    // above); with more than two value heads per key head the first pair
    // stores the key head's q/k channels
    if constexpr (!STAGED) {
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            if (owner)
                out_store(&p.xs[((size_t)b * NR + t) * p.C + chA], cinA.x[t]);
            out_store(&p.xs[((size_t)b * NR + t) * p.C + chV], cinV.x[t]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (DEPTH == 3)
        load_chunk(c2, rs, soff, 2);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();   // the column table and the gates are complete

    // commit-verify: the previous step's stash of this key head and value-head
    // pair (n rows of k^_t, e_t, a_t) goes straight from HBM into P, which is
    // free until the product tables: k^ rows at P[t*D], e rows at
    // P[NR*D + (2t + pair head)*D] (a row's two heads are contiguous in the
    // stash as well), in 1 KiB pieces, one per wave instruction, with no
    // registers held across the Gram matrix. The gates come through one
    // register (a zero-size resource when nothing is pending: zeros).
    float sa = 0.0f;
    if constexpr (FUSED) {
        const int sr = src < 0 ? 0 : src;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.pas + (size_t)sr * HV * NR, n > 0 ? HV * NR * 4 : 0);
        sa = buf_load<float>(ra, (uint32_t)((h0 + min(tid / NR, 1)) * NR + tid % NR) * 4, 0);
        if (n > 0) {
            const float *kb = p.pks + ((size_t)src * HK + kh) * NR * D;
            const int nk = (n * D + 255) / 256;
            for (int i = wave; i < nk + n; i += 4) {
                if (i < nk) {
                    const int f = i * 256 + lane * 4;
                    if (f < n * D)
                        lds_dma16(kb + f, P + i * 256);
                } else {
                    const int t = i - nk;
                    lds_dma16(p.pes + (((size_t)src * NR + t) * HV + h0) * D + lane * 4, P + NR * D + t * 2 * D);
                }
            }
        }
    }

    float *Pw = P + wave * 64 * PS;
    float *invw = invs[wave];
    const float *alw = al[hh], *bew = be[hh];

    // M^T M, each wave a quarter of the key indices; then every wave adds the
    // four shares in the same order, so all waves hold the same bits
    {
        f32x4 accg = {0.0f, 0.0f, 0.0f, 0.0f};
        float gv[2] = {0.0f, 0.0f}, dv[2] = {0.0f, 0.0f};
        gram_share<NVL, MS>(wave, kg, m, Mt, accg, gv, dv);
        float *g = gp[wave];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int u = 4 * kg + q;
            if (u < NR && m < NMF)
                g[u * NC + m] = accg[q];
            if (u == m && m >= NR && m < NMF)
                g[NR * NC + m - NR] = accg[q];   // |q_{m-NR}|^2
        }
        if (NVL) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                float x = gv[c], y = dv[c];
                x += __shfl_xor(x, 16, 64);
                x += __shfl_xor(x, 32, 64);
                y += __shfl_xor(y, 16, 64);
                y += __shfl_xor(y, 32, 64);
                gv[c] = x;
                dv[c] = y;
            }
            if (kg == 0 && m < NR) {
                g[m * NC + NMF] = gv[0];
                g[m * NC + NMF + 1] = gv[1];
            }
            if (lane == 0) {
                g[NR * NC + NMF - NR] = dv[0];
                g[NR * NC + NMF - NR + 1] = dv[1];
            }
        }
    }
    if constexpr (FUSED) {
        if (tid < 2 * NR)
            alo[tid / NR][tid % NR] = sa;
        // vmcnt(0): this wave's stash pieces are in LDS (the state chunks
        // requested before them have arrived too, as loads return in order)
        __builtin_amdgcn_s_waitcnt(0x0f70);
    }
    lds_barrier();   // from here on each wave finishes its rows alone
    auto gram = [&](int idx) { return (gp[0][idx] + gp[1][idx]) + (gp[2][idx] + gp[3][idx]); };
    auto inv_norm = [&](int c) {
        const float nn = c < NR ? gram(c * NC + c) : gram(NR * NC + c - NR);
        return 1.0f / sqrtf(nn + p.eps);
    };
    if (lane < NC)
        invw[lane] = inv_norm(lane);

    // This head's scalar coefficients, one pair per lane and kept in
    // registers (the solve broadcasts them with readlane). Lane i < NT holds
    // the pair (t, u), u <= t, of the row-by-row enumeration:
    //   cA = b_t g(t,u) k_u.k_t (u < t; 0 when u = t), cB = g(t,u) k_u.q_t;
    // lane t < NR holds cG = g(t,-1) and cb = b_t. The decay products
    // multiply a_{u+1} .. a_t in order (factors outside are 1).
    float cA, cB, cG, cb;
    {
        int t, u;
        tri_decode(min(lane, NT - 1), t, u);
        float gtu = 1.0f;
#pragma unroll
        for (int q = 1; q < NR; ++q)
            gtu *= (q > u && q <= t) ? alw[q] : 1.0f;
        // the norms this wave just stored (the same bits inv_norm gives; a
        // wave's LDS accesses stay in order, so no sync is needed)
        const float iu = invw[u];
        cA = (u < t) ? bew[t] * (gtu * (gram(u * NC + t) * iu * invw[t])) : 0.0f;
        cB = gtu * (gram(u * NC + NR + t) * iu * invw[NR + t]);
        const int tt = min(lane, NR - 1);
        float gt = 1.0f;
#pragma unroll
        for (int q = 0; q < NR; ++q)
            gt *= q <= tt ? alw[q] : 1.0f;
        cG = gt;
        cb = bew[tt];
    }
    // parked in LDS while the state streams (registers are the limit there)
    cpark[wave][lane] = float4{cA, cB, cG, cb};

    f32x4 acc[4];
    float pv[4][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        pv[q][0] = pv[q][1] = 0.0f;
    }
    // commit-verify: each chunk takes the n accepted rows (the replay
    // commit's update, in its order) and goes back to the pool before its
    // products, so the verify reads the committed state
    // (stores through a resource that is empty when nothing is pending: no
    // branch around them)
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(FUSED ? p.ssm_out + ((size_t)slot * HV + h0 + hh) * D * D : nullptr, FUSED && n > 0 ? D * D * 4 : 0);
    auto commit_chunk = [&](f32x4 (&sc)[CK], int c) {
        if constexpr (FUSED) {
            {
                const float *Pe = P + NR * D + hh * D;
#pragma unroll 1
                for (int t = 0; t < n; ++t) {
                    const float a = alo[hh][t];
                    const float4 ev = *reinterpret_cast<const float4 *>(&Pe[t * 2 * D + rb + 4 * m]);
#pragma unroll
                    for (int k = 0; k < CK; ++k) {
                        const float kk = P[t * D + 4 * (c * CK + k) + kg];
                        sc[k][0] = row_update(sc[k][0], a, ev.x, kk);
                        sc[k][1] = row_update(sc[k][1], a, ev.y, kk);
                        sc[k][2] = row_update(sc[k][2], a, ev.z, kk);
                        sc[k][3] = row_update(sc[k][3], a, ev.w, kk);
                    }
                }
#pragma unroll
                for (int k = 0; k < CK; ++k)
                    buf_stream_store_f4(rw, soff, (uint32_t)(c * CK + k) * 4 * D * 4, sc[k]);
            }
        }
    };
    if constexpr (FUSED) {
        // the loads past the last chunk fall outside the state's resource:
        // they return zeros and move no bytes
        static_assert(NCHUNK % 2 == 0, "chunks go in pairs");
#pragma unroll 1
        for (int c = 0; c < NCHUNK; c += 2) {
            commit_chunk(c0, c);
            mfma_chunk<CK, NVL, MS>(c0, c, kg, m, Mt, acc, pv);
            load_chunk_checked(c0, rs, soff, c + 2);
            commit_chunk(c1, c + 1);
            mfma_chunk<CK, NVL, MS>(c1, c + 1, kg, m, Mt, acc, pv);
            load_chunk_checked(c1, rs, soff, c + 3);
        }
    } else {
#pragma unroll
    for (int c = 0; c < NCHUNK; ++c) {
        if (c % 3 == 0) {
            commit_chunk(c0, c);
            mfma_chunk<CK, NVL, MS>(c0, c, kg, m, Mt, acc, pv);
            if (c + 3 < NCHUNK)
                load_chunk(c0, rs, soff, c + 3);
        } else if (c % 3 == 1) {
            commit_chunk(c1, c);
            mfma_chunk<CK, NVL, MS>(c1, c, kg, m, Mt, acc, pv);
            if (c + 3 < NCHUNK)
                load_chunk(c1, rs, soff, c + 3);
        } else {
            commit_chunk(c2, c);
            mfma_chunk<CK, NVL, MS>(c2, c, kg, m, Mt, acc, pv);
            if (c + 3 < NCHUNK)
                load_chunk(c2, rs, soff, c + 3);
        }
    }
    }
    if constexpr (FUSED)
        lds_barrier();   // every wave is done with the staged stash before the product tables overwrite it

    // (S_0 M^)[i][c] = (S_0 M)[i][c] inv_c. Tile v, register q of lane (kg, m):
    // row 16kg + 4q + v of the block, column m.
    if (m < NMF) {
        const float ic = invw[m];
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                Pw[(16 * kg + 4 * q + v4) * PS + m] = acc[v4][q] * ic;
    }
    if (NVL) {
        // the four key-index groups kg hold partial sums: add lanes l^16 and l^32
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                float x = pv[v4][c];
                x += __shfl_xor(x, 16, 64);
                x += __shfl_xor(x, 32, 64);
                pv[v4][c] = x;
            }
        if (kg == 0) {
            const float i0 = invw[NMF], i1 = invw[NMF + 1];
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                Pw[(4 * m + v4) * PS + NMF] = pv[v4][0] * i0;
                Pw[(4 * m + v4) * PS + NMF + 1] = pv[v4][1] * i1;
            }
        }
    }
    wave_lds_sync();

    // row rb + lane, by forward substitution with the broadcast coefficients:
    // e_t = b_t (v_t - g(t,-1) (S_0 k^_t)) - sum_{u<t} cA(t,u) e_u,
    // o_t = scale (g(t,-1) (S_0 q^_t) + sum_{u<=t} cB(t,u) e_u)
    {
        float *Pr = Pw + lane * PS;
        const float4 cc = cpark[wave][lane];
        cA = cc.x;
        cB = cc.y;
        cG = cc.z;
        cb = cc.w;
        float e[NR];
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            const float r = __builtin_fmaf(-lane_value(cG, t), Pr[t], v[t]);
            float s = lane_value(cb, t) * r;
#pragma unroll
            for (int u = 0; u < t; ++u)
                s = __builtin_fmaf(-lane_value(cA, t * (t + 1) / 2 + u), e[u], s);
            e[t] = s;
        }
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            float s = lane_value(cG, t) * Pr[NR + t];
#pragma unroll
            for (int u = 0; u <= t; ++u)
                s = __builtin_fmaf(lane_value(cB, t * (t + 1) / 2 + u), e[u], s);
            const size_t oi = (((size_t)b * NR + t) * HV + h0 + hh) * D + rb + lane;
            out_store(&p.out[oi], from_f32<T>(p.scale * s));
            out_store(&p.es[oi], e[t]);
        }
        if (SNAP) {
            // this row of the product table is read only by this lane: reuse it for e_t
#pragma unroll
            for (int t = 0; t < NR; ++t)
                Pr[t] = e[t];
        }
    }

    // normalised keys for the commit (the key head's first pair of value heads)
    if (owner) {
        float *ks = p.ks + ((size_t)b * HK + kh) * NR * D;
        for (int idx = tid; idx < NR * D; idx += kThreads)
            out_store(&ks[idx], Mt[(idx % D) * MS + idx / D] * invw[idx / D]);
    }

    if (SNAP) {
        wave_lds_sync();
        // S_t for every row, by the same update the replay commit applies,
        // chunk by chunk from a second read of S_0; the next chunk loads
        // while this one's snapshots are stored
        float *snap_h = p.snap + ((size_t)b * HV + h0 + hh) * NR * D * D;   // a head's S_1..S_R are contiguous
        auto snap_chunk = [&](f32x4 (&sc)[CK], int c) {
#pragma unroll 1
            for (int t = 0; t < NR; ++t) {
                const float a = alw[t];
                const float it = invw[t];
                float ev[4];
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4)
                    ev[v4] = Pw[(4 * m + v4) * PS + t];
                float *dst = snap_h + (size_t)t * D * D;
#pragma unroll
                for (int k = 0; k < CK; ++k) {
                    const int j = 4 * (c * CK + k) + kg;
                    const float kk = Mt[j * MS + t] * it;
#pragma unroll
                    for (int v4 = 0; v4 < 4; ++v4)
                        sc[k][v4] = row_update(sc[k][v4], a, ev[v4], kk);
                    stream_store(dst + (size_t)j * D + rb + 4 * m, sc[k]);
                }
            }
        };
        static_assert(NCHUNK % 2 == 0, "chunks go in pairs");
        load_chunk(c0, rs, soff, 0);
        load_chunk(c1, rs, soff, 1);
#pragma unroll 1
        for (int c = 0; c < NCHUNK; c += 2) {
            snap_chunk(c0, c);
            if (c + 2 < NCHUNK)
                load_chunk(c0, rs, soff, c + 2);
            snap_chunk(c1, c + 1);
            if (c + 3 < NCHUNK)
                load_chunk(c1, rs, soff, c + 3);
        }
    }
}

// ---- verify, d = 128, small batches: a unit split over several workgroups ----
//
// With fewer (request, pair of value heads) units than compute units, one
// workgroup per unit leaves most of the chip idle and each
// workgroup streams 128 KiB in a long dependent chain. Here a workgroup takes
// one block of RB = 16 RPL rows of one value head (RPL state rows per lane:
// 64-row blocks, four workgroups per unit, down to 16-row blocks, sixteen per
// unit, on the smallest batches), and its four waves split the block's 128
// key indices: wave w streams K-steps 8w..8w+7 (both chunks requested at the
// start) into partial products of all the block's rows, which are summed
// through LDS before wave 0 solves them. Each workgroup repeats the unit's
// conv of the key head and its Gram matrix: more arithmetic, no more HBM
// traffic (the repeated input loads hit the caches). From the column table
// on, each phase runs at the rate of one SIMD, so smaller blocks on more
// compute units shorten it. In snapshot mode each wave then applies every
// row's update to its two chunks, still in registers, and stores its part of
// S_1..S_R. Every result element takes the same operations in the same order
// whatever the block size and the mode, so all of them agree bit for bit.
template <int RPL> struct RowBits;
template <> struct RowBits<4> {
    static __device__ __forceinline__ void load(float (&d)[4], __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
    {
        const f32x4 v = buf_stream_load_f4(r, voff, soff);
        d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
    }
    static __device__ __forceinline__ void store(const float (&s)[4], __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
    {
        buf_stream_store_f4(r, voff, soff, f32x4{s[0], s[1], s[2], s[3]});
    }
    static __device__ __forceinline__ void put(float *dst, const float (&s)[4])
    {
        *reinterpret_cast<f32x4 *>(dst) = f32x4{s[0], s[1], s[2], s[3]};
    }
};
template <> struct RowBits<2> {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ void load(float (&d)[2], __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
    {
        const f2 v = __builtin_bit_cast(f2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, kStreamPolicy));
        d[0] = v[0]; d[1] = v[1];
    }
    static __device__ __forceinline__ void store(const float (&s)[2], __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
    {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, f2{s[0], s[1]}), r, (int)voff, (int)soff,
                                              kStreamPolicy);
    }
    static __device__ __forceinline__ void put(float *dst, const float (&s)[2])
    {
        *reinterpret_cast<f2 *>(dst) = f2{s[0], s[1]};
    }
};
template <> struct RowBits<1> {
    static __device__ __forceinline__ void load(float (&d)[1], __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
    {
        d[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, kStreamPolicy));
    }
    static __device__ __forceinline__ void store(const float (&s)[1], __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
    {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, s[0]), r, (int)voff, (int)soff, kStreamPolicy);
    }
    static __device__ __forceinline__ void put(float *dst, const float (&s)[1]) { *dst = s[0]; }
};

template <int NR, bool SNAP, bool FUSED, int RPL>
__global__ __launch_bounds__(kThreads) void gdn_verify_d128_split_kernel(const VerifyParams<bf16_t> p)
{
    using T = bf16_t;
    constexpr int D = 128;
    constexpr int NC = 2 * NR;
    constexpr int NMF = NC < 16 ? NC : 16;
    constexpr int NVL = NC - NMF;
    static_assert(NVL == 0 || NVL == 2, "unsupported row count");
    constexpr int MS = NVL ? 20 : 16;
    constexpr int PS = NC + 1;
    constexpr int CK = 4;
    constexpr int NT = NR * (NR + 1) / 2;
    static_assert(NT <= 64, "one coefficient pair per lane");
    static_assert(RPL == 1 || RPL == 2 || RPL == 4, "state rows per lane");
    constexpr int RB = 16 * RPL;          // rows per block
    constexpr int BPH = D / RB;           // blocks per value head
    constexpr int WPU = 2 * BPH;          // workgroups per unit
    constexpr int LPRW = RB / 4;          // lanes per e row in the stash copy
    constexpr int NROWS = kWidth - 1 + NR;
    constexpr int UPR = 32 + RB / 8;   // 16-byte units per staged row: q 16 | k 16 | v RB / 8 (RB channels)
    constexpr int NU = NROWS * UPR;
    constexpr int NUT = (NU + kThreads - 1) / kThreads;   // staged units per thread
    static_assert(NUT <= 2, "staged units per thread");
    constexpr int XFLOATS = NROWS * UPR * 4;               // staged rows, as floats
    constexpr int RFLOATS = 4 * RB * PS;                    // per-wave partial products
    // commit-verify: the previous step's stash (k^ [t][j] for the key head,
    // then e [t][RB] of the block's rows), loaded through registers with the
    // staged inputs, SQ float4 per thread
    constexpr int SFLOATS = FUSED && !SNAP ? NR * D + NR * RB : 0;
    constexpr int SQ = (SFLOATS / 4 + kThreads - 1) / kThreads;
    constexpr int PFLOATS = XFLOATS > RFLOATS ? XFLOATS : RFLOATS;

    __shared__ __align__(16) float Mt[D * MS];
    __shared__ __align__(16) float P[PFLOATS];   // staged inputs; then the four waves' partial products
    __shared__ __align__(16) float Sst[SFLOATS > 0 ? SFLOATS : 4];   // commit-verify: the stash
    __shared__ float invs[NC];
    __shared__ float gp[4][NR * NC + NR];
    __shared__ float al[NR], be[NR];
    __shared__ float eb[SNAP ? NR * RB : 1];   // e_t of the block's rows, for the snapshots
    __shared__ float alo[FUSED ? NR : 1];      // commit-verify: the previous step's a_t of head h

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int HV = p.HV, HK = p.HK;
    const int G = HV / HK;
    const int npair = HV / 2;
    const int b = blockIdx.x / (npair * WPU);
    const int rem = blockIdx.x % (npair * WPU);
    const int h0 = 2 * (rem / WPU);
    const int blk = rem % WPU;
    const int h = h0 + blk / BPH;        // this workgroup's value head
    const int rb = RB * (blk % BPH);     // and its block of rows
    const int kh = h0 / G;
    const bool owner = (h0 % G) == 0;    // the key head's first pair stores its q/k inputs
    const int slot_in = p.slot_ids[b];
    int src = -1;
    if constexpr (FUSED)
        src = p.src_row[b];

    // staged unit k of a row: q units 0..15, k units 16..31, then the block's
    // value channels rb..rb+RB-1 of head h; unit k starts at local channel 8k
    auto unit_channel = [&](int k) {
        return k < 16 ? kh * D + 8 * k : (k < 32 ? HK * D + kh * D + 8 * (k - 16) : 2 * HK * D + h * D + rb + 8 * (k - 32));
    };
    const int gt_ = min(tid, NR - 1);
    const size_t gi = ((size_t)b * NR + gt_) * HV + h;
    const T ga = p.alpha[gi], gb = p.beta[gi];
    const int jc = tid & (D - 1);
    const bool isq = tid < D;
    const int chA = isq ? kh * D + jc : HK * D + kh * D + jc;
    const int chV = 2 * HK * D + h * D + rb + min(tid, RB - 1);
    const uint2 wA = *reinterpret_cast<const uint2 *>(p.conv_w + (size_t)chA * kWidth);
    const uint2 wV = *reinterpret_cast<const uint2 *>(p.conv_w + (size_t)chV * kWidth);
    bool bad = slot_in < 0 || slot_in >= p.P;
    int errbits = bad && slot_in != -1 ? 1 : 0;
    // commit-verify: n accepted rows of the previous step's row src go into
    // the state before it is read (a padding request ignores src)
    int n = 0;
    if constexpr (FUSED) {
        if (!bad && src != -1) {
            if (src < 0 || src >= p.Bp || p.prev_slots[src] != slot_in) {
                bad = true;
                errbits |= 4;
            } else {
                n = p.prev_accept[src];
                if (n < 0 || n > NR) {
                    bad = true;
                    errbits |= 2;
                    n = 0;
                }
            }
        }
    }
    const int slot = bad ? 0 : slot_in;
    // staged rows: history then the verify rows. The history is the pool's,
    // or with n > 0 pending rows the committed one, entry n + r of [the
    // history the previous verify read | its rows], from the previous step's
    // scratch (the pool's history of this slot is being rewritten)
    uint4 su[NUT];
#pragma unroll
    for (int q = 0; q < NUT; ++q) {
        const int uu = min(q * kThreads + tid, NU - 1);
        const int r = uu / UPR, k = uu % UPR;
        const int e = r + n;
        const T *row = r >= kWidth - 1 ? p.x + ((size_t)b * NR + (r - (kWidth - 1))) * p.C
            : n == 0                   ? p.conv + ((size_t)slot * (kWidth - 1) + r) * p.C
            : e < kWidth - 1           ? p.pxh + ((size_t)src * (kWidth - 1) + e) * p.C
                                       : p.pxs + ((size_t)src * NR + e - (kWidth - 1)) * p.C;
        su[q] = *reinterpret_cast<const uint4 *>(row + unit_channel(k));
    }
    // commit-verify: the n pending rows' stash (k^ rows of the key head, e of
    // the block's rows) and the gates of head h, requested with the inputs
    // (plain loads: a copy straight into LDS, pending beside ordinary loads,
    // makes the compiler wait for every load in flight at the next use of
    // any of them, the state chunks included)
    float sa = 0.0f;
    float4 stv[SQ > 0 ? SQ : 1];
    if constexpr (FUSED && !SNAP) {
        const int sr = src < 0 ? 0 : src;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.pas + (size_t)sr * HV * NR, n > 0 ? HV * NR * 4 : 0);
        sa = buf_load<float>(ra, (uint32_t)(h * NR + min(tid, NR - 1)) * 4, 0);
        const float *kb = p.pks + ((size_t)sr * HK + kh) * NR * D;
#pragma unroll
        for (int q = 0; q < SQ; ++q) {
            const int f = 4 * (q * kThreads + tid);   // float index in [k^ rows | e rows]
            stv[q] = float4{0.0f, 0.0f, 0.0f, 0.0f};
            if (f < n * D) {
                stv[q] = *reinterpret_cast<const float4 *>(kb + f);
            } else if (f >= NR * D && f - NR * D < n * RB) {
                const int t = (f - NR * D) / RB, c = (f - NR * D) % RB;
                stv[q] = *reinterpret_cast<const float4 *>(p.pes + (((size_t)src * NR + t) * HV + h) * D + rb + c);
            }
        }
    }
    if (bad) {
        if (errbits && tid == 0 && blk == 0 && p.err)
            atomicOr(p.err, errbits);
        for (int idx = tid; idx < NR * RB; idx += kThreads) {
            const int t = idx / RB, i = idx % RB;
            out_store(&p.out[(((size_t)b * NR + t) * HV + h) * D + rb + i], from_f32<T>(0.0f));
        }
        return;
    }

    // this wave's two chunks: K-steps 8w .. 8w + 7 of the block
    const int kg = lane >> 4;
    const int m = lane & 15;
    // (commit-verify in snapshot mode: with n > 0 pending rows, S_0 is the
    // previous step's S_n of this head, which also goes to the pool)
    const __amdgpu_buffer_rsrc_t rs =
        FUSED && SNAP && n > 0 ? make_rsrc(p.psnap + (((size_t)src * HV + h) * NR + (n - 1)) * D * D, D * D * 4)
                               : make_rsrc(p.ssm + ((size_t)slot * HV + h) * D * D, D * D * 4);
    const uint32_t soff = (kg * D + rb + RPL * m) * 4;
    // lane (kg, m) holds rows rb + RPL m .. + RPL - 1 of key index 4 K-step + kg
    float c0[CK][RPL], c1[CK][RPL];
    auto load_rows = [&](float (&sc)[CK][RPL], int c) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < CK; ++k)
            RowBits<RPL>::load(sc[k], rs, soff, (uint32_t)(c * CK + k) * 4 * D * 4);
        asm volatile("" ::: "memory");
    };
    load_rows(c0, 2 * wave);
    load_rows(c1, 2 * wave + 1);
    __builtin_amdgcn_sched_barrier(0);

    float *const Sk = Sst;
    float *const Se = Sst + NR * D;
    if constexpr (FUSED && !SNAP) {
#pragma unroll
        for (int q = 0; q < SQ; ++q)
            if (4 * (q * kThreads + tid) < SFLOATS)
                reinterpret_cast<float4 *>(Sst)[q * kThreads + tid] = stv[q];
        if (tid < NR)
            alo[tid] = sa;
    }
    if (tid < NR) {
        al[tid] = to_f32(ga);
        be[tid] = to_f32(gb);
        if (rb == 0)
            out_store(&p.as[((size_t)b * HV + h) * NR + tid], to_f32(ga));
    }
    uint4 *Xs = reinterpret_cast<uint4 *>(P);
#pragma unroll
    for (int q = 0; q < NUT; ++q) {
        const int uu = q * kThreads + tid;
        if (uu < NU) {
            Xs[uu] = su[q];
            const int r = uu / UPR, k = uu % UPR;
            // verify rows to the raw-row stash: the block's value channels, and
            // the key head's q/k channels from the first block of its first pair
            if (r >= kWidth - 1 && (k >= 32 || (owner && blk == 0)))
                out_store(reinterpret_cast<uint4 *>(p.xs + ((size_t)b * NR + r - (kWidth - 1)) * p.C + unit_channel(k)), su[q]);
        }
    }
    lds_barrier();
    {
        // the history this verify used, for the next step's commit-verify
        // (the block's value channels; the key head's q/k channels from the
        // first block of its first pair); with a commit pending, the
        // committed history goes to the pool by the same writers
        static_assert((kWidth - 1) * UPR <= kThreads, "history units in the first pass");
        const int k = tid % UPR;
        if (tid < (kWidth - 1) * UPR && (k >= 32 || (owner && blk == 0))) {
            const size_t hoff = (size_t)(tid / UPR) * p.C + unit_channel(k);
            out_store(reinterpret_cast<uint4 *>(p.xh + (size_t)b * (kWidth - 1) * p.C + hoff), su[0]);
            if (FUSED && n > 0)
                out_store(reinterpret_cast<uint4 *>(p.hist_out + (size_t)slot * (kWidth - 1) * p.C + hoff), su[0]);
        }
    }
    float v[NR];   // value channel rb + tid of head h (threads < RB)
    {
        ChanIn<NR, T> cinA, cinV;
        const T *Xt = reinterpret_cast<const T *>(P);
        auto tap = [](uint2 w, int k) {
            return T{(uint16_t)(((k < 2 ? w.x : w.y) >> (16 * (k & 1))) & 0xffffu)};
        };
#pragma unroll
        for (int k = 0; k < kWidth; ++k) {
            cinA.w[k] = tap(wA, k);
            cinV.w[k] = tap(wV, k);
        }
        const int cv = 256 + min(tid, RB - 1);   // local channel of the value input
#pragma unroll
        for (int r = 0; r < kWidth - 1; ++r) {
            cinA.hist[r] = Xt[r * UPR * 8 + tid];
            cinV.hist[r] = Xt[r * UPR * 8 + cv];
        }
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            cinA.x[t] = Xt[(kWidth - 1 + t) * UPR * 8 + tid];
            cinV.x[t] = Xt[(kWidth - 1 + t) * UPR * 8 + cv];
        }
        float y[NR];
        conv_rows(cinA, p.act, y);
#pragma unroll
        for (int t = 0; t < NR; ++t)
            Mt[jc * MS + (isq ? NR + t : t)] = y[t];
        if (isq) {
#pragma unroll
            for (int c = NC; c < MS; ++c)
                Mt[jc * MS + c] = 0.0f;
        }
        conv_rows(cinV, p.act, v);
    }
    lds_barrier();   // the column table and the gates are complete

    // M^T M, each wave a quarter of the key indices (as in the one-round kernel)
    {
        f32x4 accg = {0.0f, 0.0f, 0.0f, 0.0f};
        float gv[2] = {0.0f, 0.0f}, dv[2] = {0.0f, 0.0f};
        gram_share<NVL, MS>(wave, kg, m, Mt, accg, gv, dv);
        float *g = gp[wave];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int uq = 4 * kg + q;
            if (uq < NR && m < NMF)
                g[uq * NC + m] = accg[q];
            if (uq == m && m >= NR && m < NMF)
                g[NR * NC + m - NR] = accg[q];
        }
        if (NVL) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                float x = gv[c], y = dv[c];
                x += __shfl_xor(x, 16, 64);
                x += __shfl_xor(x, 32, 64);
                y += __shfl_xor(y, 16, 64);
                y += __shfl_xor(y, 32, 64);
                gv[c] = x;
                dv[c] = y;
            }
            if (kg == 0 && m < NR) {
                g[m * NC + NMF] = gv[0];
                g[m * NC + NMF + 1] = gv[1];
            }
            if (lane == 0) {
                g[NR * NC + NMF - NR] = dv[0];
                g[NR * NC + NMF - NR + 1] = dv[1];
            }
        }
    }

    // partial products of this wave's K-steps: all the block's rows, every
    // column (tile v holds rows rb + RPL m + v)
    f32x4 acc[RPL];
    float pv[RPL][2];
#pragma unroll
    for (int q = 0; q < RPL; ++q) {
        acc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        pv[q][0] = pv[q][1] = 0.0f;
    }
    auto mfma_rows = [&](const float (&sc)[CK][RPL], int c) {
#pragma unroll
        for (int k = 0; k < CK; ++k) {
            const int j = 4 * (c * CK + k) + kg;
            const float bm = Mt[j * MS + m];
#pragma unroll
            for (int v = 0; v < RPL; ++v)
                acc[v] = __builtin_amdgcn_mfma_f32_16x16x4f32(sc[k][v], bm, acc[v], 0, 0, 0);
            if (NVL) {
                const float2 mv = *reinterpret_cast<const float2 *>(&Mt[j * MS + 16]);
#pragma unroll
                for (int v = 0; v < RPL; ++v) {
                    pv[v][0] = __builtin_fmaf(sc[k][v], mv.x, pv[v][0]);
                    pv[v][1] = __builtin_fmaf(sc[k][v], mv.y, pv[v][1]);
                }
            }
        }
    };
    if constexpr (FUSED) {
        // this wave's two chunks take the n accepted rows (replay: the
        // commit's update, in its order; snapshot: they are S_n already) and
        // go back to the pool before their products; stores through a
        // resource that is empty when nothing is pending
        const __amdgpu_buffer_rsrc_t rw =
            make_rsrc(p.ssm_out + ((size_t)slot * HV + h) * D * D, n > 0 ? D * D * 4 : 0);
        auto commit_chunk = [&](float (&sc)[CK][RPL], int c) {
#pragma unroll 1
            for (int t = 0; t < (SNAP ? 0 : n); ++t) {
                const float a = alo[t];
                float ev[RPL];
#pragma unroll
                for (int v = 0; v < RPL; ++v)
                    ev[v] = Se[t * RB + RPL * m + v];
#pragma unroll
                for (int kk4 = 0; kk4 < CK; ++kk4) {
                    const float kk = Sk[t * D + 4 * (c * CK + kk4) + kg];
#pragma unroll
                    for (int v = 0; v < RPL; ++v)
                        sc[kk4][v] = row_update(sc[kk4][v], a, ev[v], kk);
                }
            }
#pragma unroll
            for (int kk4 = 0; kk4 < CK; ++kk4)
                RowBits<RPL>::store(sc[kk4], rw, soff, (uint32_t)(c * CK + kk4) * 4 * D * 4);
        };
        commit_chunk(c0, 2 * wave);
        commit_chunk(c1, 2 * wave + 1);
    }
    mfma_rows(c0, 2 * wave);
    mfma_rows(c1, 2 * wave + 1);
    lds_barrier();   // the Gram shares are in; the staged inputs are no longer read
    float *Pw = P + wave * RB * PS;
    if (m < NMF) {
        // tile v, register q of lane (kg, m): row RPL (4 kg + q) + v of the block, column m
#pragma unroll
        for (int v4 = 0; v4 < RPL; ++v4)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                Pw[(RPL * (4 * kg + q) + v4) * PS + m] = acc[v4][q];
    }
    if (NVL) {
#pragma unroll
        for (int v4 = 0; v4 < RPL; ++v4)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                float x = pv[v4][c];
                x += __shfl_xor(x, 16, 64);
                x += __shfl_xor(x, 32, 64);
                pv[v4][c] = x;
            }
        if (kg == 0) {
#pragma unroll
            for (int v4 = 0; v4 < RPL; ++v4) {
                Pw[(RPL * m + v4) * PS + NMF] = pv[v4][0];
                Pw[(RPL * m + v4) * PS + NMF + 1] = pv[v4][1];
            }
        }
    }
    auto gram = [&](int idx) { return (gp[0][idx] + gp[1][idx]) + (gp[2][idx] + gp[3][idx]); };
    if (tid < NC) {
        const float nn = tid < NR ? gram(tid * NC + tid) : gram(NR * NC + tid - NR);
        invs[tid] = 1.0f / sqrtf(nn + p.eps);
    }
    lds_barrier();   // partial products and norms are complete

    if (wave == 0) {
        // coefficients, one pair (t, u) per lane, as in the one-round kernel
        float cA, cB, cG, cb;
        {
            int t, uu;
            tri_decode(min(lane, NT - 1), t, uu);
            float gtu = 1.0f;
#pragma unroll
            for (int q = 1; q < NR; ++q)
                gtu *= (q > uu && q <= t) ? al[q] : 1.0f;
            const float iu = invs[uu];
            cA = (uu < t) ? be[t] * (gtu * (gram(uu * NC + t) * iu * invs[t])) : 0.0f;
            cB = gtu * (gram(uu * NC + NR + t) * iu * invs[NR + t]);
            const int tt = min(lane, NR - 1);
            float g = 1.0f;
#pragma unroll
            for (int q = 0; q < NR; ++q)
                g *= q <= tt ? al[q] : 1.0f;
            cG = g;
            cb = be[tt];
        }
        // row rb + lane (lanes < RB; the others only hold coefficients): the
        // four waves' partial products, scaled by the norms
        const int lr = min(lane, RB - 1);
        float pr[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                s += P[(w * RB + lr) * PS + c];
            pr[c] = s * invs[c];
        }
        float e[NR];
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            const float r = __builtin_fmaf(-lane_value(cG, t), pr[t], v[t]);
            float s = lane_value(cb, t) * r;
#pragma unroll
            for (int uu = 0; uu < t; ++uu)
                s = __builtin_fmaf(-lane_value(cA, t * (t + 1) / 2 + uu), e[uu], s);
            e[t] = s;
        }
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            float s = lane_value(cG, t) * pr[NR + t];
#pragma unroll
            for (int uu = 0; uu <= t; ++uu)
                s = __builtin_fmaf(lane_value(cB, t * (t + 1) / 2 + uu), e[uu], s);
            if (lane < RB) {
                const size_t oi = (((size_t)b * NR + t) * HV + h) * D + rb + lane;
                out_store(&p.out[oi], from_f32<T>(p.scale * s));
                out_store(&p.es[oi], e[t]);
                if (SNAP)
                    eb[t * RB + lane] = e[t];
            }
        }
    } else if (owner && blk == 0) {
        // normalised keys for the commit (three waves of the key head's first block)
        float *ks = p.ks + ((size_t)b * HK + kh) * NR * D;
        for (int idx = tid - 64; idx < NR * D; idx += kThreads - 64)
            out_store(&ks[idx], Mt[(idx % D) * MS + idx / D] * invs[idx / D]);
    }
    if (SNAP) {
        lds_barrier();   // e_t of every row of the block
        // S_t for every row by the update the replay commit applies: this
        // wave's K-steps of the block, from the S_0 still in registers
        float *snap_h = p.snap + ((size_t)b * HV + h) * NR * D * D;
#pragma unroll 1
        for (int t = 0; t < NR; ++t) {
            const float a = al[t];
            const float it = invs[t];
            float ev[RPL];
#pragma unroll
            for (int v4 = 0; v4 < RPL; ++v4)
                ev[v4] = eb[t * RB + RPL * m + v4];
            float *dst = snap_h + (size_t)t * D * D;
            auto snap_chunk = [&](float (&sc)[CK][RPL], int c) {
#pragma unroll
                for (int k = 0; k < CK; ++k) {
                    const int j = 4 * (c * CK + k) + kg;
                    const float kk = Mt[j * MS + t] * it;
#pragma unroll
                    for (int v4 = 0; v4 < RPL; ++v4)
                        sc[k][v4] = row_update(sc[k][v4], a, ev[v4], kk);
                    RowBits<RPL>::put(dst + (size_t)j * D + rb + RPL * m, sc[k]);
                }
            };
            snap_chunk(c0, 2 * wave);
            snap_chunk(c1, 2 * wave + 1);
        }
    }
}

// ---- verify, d = 128, snapshot mode: the state held in registers ------------
//
// The arithmetic of gdn_verify_d128_kernel (bf16 inputs), plus the snapshots
// S_t = a_t S_{t-1} + e_t k_t^T of every row. Those need S_0 once more after
// the solve, when e_t is known. Here each wave keeps its whole 32 KiB share of
// a unit's S_0 in registers (8 chunks of 4 K-steps, 128 VGPRs) from the
// products through the snapshot stores, so S_0 is read from HBM once.
//
// With that many registers a compute unit holds one or two workgroups, too few
// for a one-round grid, so the grid is fixed (one or two workgroups per
// compute unit) and each workgroup walks a list of (request, pair of value
// heads) units: w, w + grid, w + 2 grid, ... The next unit's inputs are
// requested as soon as the current unit's conv has consumed its own, and all
// 8 chunks of its state as soon as the current unit's snapshots are stored.
//
// A unit whose slot id is padding or outside the pool streams nothing: its
// state resource has size 0, so its chunk loads return zeros without touching
// memory, the pipeline keeps its shape, and its outputs are stored as zeros.
//
// (Replay mode keeps the one-round kernel: measured, walking units with this
// register-resident stream was slower there, 55.0 against 32.2 us for 64
// requests x 9 rows at one workgroup per compute unit, and 61 against 57 us for
// 128 requests x 4 rows at two. The per-unit chain of barriers, LDS round
// trips and broadcasts needs four resident workgroups to overlap.)

constexpr int kComputeUnits = 256;   // MI355X

// Resident workgroups per compute unit: two while the registers allow (up to
// 256 per lane), one where more are needed (up to 512).
template <int NR> __host__ __device__ constexpr int snapshot_groups_per_cu() { return (NR >= 3 && NR <= 6) ? 2 : 1; }

__device__ __forceinline__ int load_uniform(const int32_t *ptr, int idx)
{
    // a scalar load: its wait does not drain the vector loads in flight
    return ((const __attribute__((address_space(4))) int32_t *)ptr)[idx];
}

template <int NR, bool FUSED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(snapshot_groups_per_cu<NR>())))
void gdn_verify_d128_snapshot_kernel(const VerifyParams<bf16_t> p, int units)
{
    using T = bf16_t;
    constexpr int D = 128;
    constexpr int NC = 2 * NR;
    constexpr int NMF = NC < 16 ? NC : 16;
    constexpr int NVL = NC - NMF;
    static_assert(NVL == 0 || NVL == 2, "unsupported row count");
    constexpr int MS = NVL ? 20 : 16;
    constexpr int PS = NC + 1;
    constexpr int CK = 4;
    constexpr int NCHUNK = D / 4 / CK;
    constexpr int NT = NR * (NR + 1) / 2;
    static_assert(NT <= 64, "one coefficient pair per lane");
    constexpr int NROWS = kWidth - 1 + NR;
    constexpr int UPR = 64;
    constexpr int NXU = (NR * UPR + kThreads - 1) / kThreads;
    static_assert(NXU <= 3 && (kWidth - 1) * UPR <= kThreads, "staged units per thread");
    constexpr int PFLOATS = 4 * 64 * PS > NROWS * 256 ? 4 * 64 * PS : NROWS * 256;

    __shared__ __align__(16) float Mt[D * MS];
    __shared__ __align__(16) float P[PFLOATS];
    __shared__ float invs[4][NC];
    __shared__ float4 cpark[4][64];
    __shared__ float gp[4][NR * NC + NR];
    __shared__ float al[2][NR], be[2][NR];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int HV = p.HV, HK = p.HK;
    const int G = HV / HK;
    const int npair = HV / 2;
    const int kg = lane >> 4;
    const int m = lane & 15;
    const int hh = wave >> 1;
    const int rb = 64 * (wave & 1);
    const uint32_t soff = (kg * D + rb + 4 * m) * 4;
    const int jc = tid & (D - 1);
    const bool isq = tid < D;
    const int gidx = min(tid, 2 * NR - 1);
    const int ghh = gidx / NR, gtt = gidx % NR;

    // staged units: unit k of a row starts at local channel 8k; units 0..15
    // q, 16..31 k, 32..63 v channels of the pair
    auto unit_channel = [&](int kh, int h0, int k) {
        return k < 16 ? kh * D + 8 * k : (k < 32 ? HK * D + kh * D + 8 * (k - 16) : 2 * HK * D + h0 * D + 8 * (k - 32));
    };

    // one unit's inputs, held in registers from their request to the conv;
    // with a commit pending (commit-verify), its source row src_in, its n_in
    // accepted rows and any error bits
    int slot_in, src_in = -1, n_in = 0, err_in = 0;
    T ga, gb;
    uint4 xu0 = {}, xu1 = {}, xu2 = {}, hu = {};
    uint2 wA = {}, wV = {};
    auto load_inputs = [&](int u) {
        const int b = u / npair, h0 = 2 * (u % npair), kh = h0 / G;
        slot_in = load_uniform(p.slot_ids, b);
        err_in = (slot_in < -1 || slot_in >= p.P) ? 1 : 0;
        n_in = 0;
        if constexpr (FUSED) {
            src_in = load_uniform(p.src_row, b);
            if (err_in == 0 && slot_in != -1 && src_in != -1) {
                if (src_in < 0 || src_in >= p.Bp || load_uniform(p.prev_slots, src_in) != slot_in) {
                    err_in = 4;
                } else {
                    n_in = load_uniform(p.prev_accept, src_in);
                    if (n_in < 0 || n_in > NR) {
                        err_in = 2;
                        n_in = 0;
                    }
                }
            }
        }
        const size_t gi = ((size_t)b * NR + gtt) * HV + h0 + ghh;
        ga = p.alpha[gi];
        gb = p.beta[gi];
        const T *xbase = p.x + (size_t)b * NR * p.C;
        auto xunit = [&](int q) {
            const int uu = min(q * kThreads + tid, NR * UPR - 1);
            return *reinterpret_cast<const uint4 *>(xbase + (size_t)(uu / UPR) * p.C + unit_channel(kh, h0, uu % UPR));
        };
        xu0 = xunit(0);
        if constexpr (NXU > 1)
            xu1 = xunit(1);
        if constexpr (NXU > 2)
            xu2 = xunit(2);
        const int chA = isq ? kh * D + jc : HK * D + kh * D + jc;
        const int chV = 2 * HK * D + h0 * D + tid;
        wA = *reinterpret_cast<const uint2 *>(p.conv_w + (size_t)chA * kWidth);
        wV = *reinterpret_cast<const uint2 *>(p.conv_w + (size_t)chV * kWidth);
        // a slot id outside the pool reads slot 0's history (inside the pool);
        // with n_in > 0 pending rows the committed history, entry n_in + r of
        // [the history the previous verify read | its rows], from the previous
        // step's scratch
        const int sl = (slot_in < 0 || slot_in >= p.P) ? 0 : slot_in;
        const int uh = min(tid, (kWidth - 1) * UPR - 1);
        const int r = uh / UPR, e = r + n_in;
        const T *from = n_in == 0 ? p.conv + ((size_t)sl * (kWidth - 1) + r) * p.C
            : e < kWidth - 1      ? p.pxh + ((size_t)src_in * (kWidth - 1) + e) * p.C
                                  : p.pxs + ((size_t)src_in * NR + e - (kWidth - 1)) * p.C;
        hu = *reinterpret_cast<const uint4 *>(from + unit_channel(kh, h0, uh % UPR));
    };
    // this wave's head of unit u; an empty resource for a unit that streams
    // nothing; with n > 0 pending rows, the previous step's S_n
    auto state_rsrc = [&](int u, bool valid, int slot, int src, int n) {
        const int h0 = 2 * (u % npair);
        if (FUSED && valid && n > 0)
            return make_rsrc(p.psnap + (((size_t)src * HV + h0 + hh) * NR + (n - 1)) * D * D, D * D * 4);
        return valid ? make_rsrc(p.ssm + ((size_t)slot * HV + h0 + hh) * D * D, D * D * 4)
                     : make_rsrc(p.ssm, 0);
    };

    int u = blockIdx.x;
    if (u >= units)
        return;
    f32x4 S[NCHUNK][CK];
    load_inputs(u);
    bool valid = slot_in >= 0 && slot_in < p.P && err_in == 0;
    int slot = slot_in, n = n_in, errs = err_in;
    {
        const __amdgpu_buffer_rsrc_t rs = state_rsrc(u, valid, slot_in, src_in, n_in);
#pragma unroll
        for (int c = 0; c < NCHUNK; ++c)
            load_chunk(S[c], rs, soff, c);
    }

    while (true) {
        const int b = u / npair, h0 = 2 * (u % npair), kh = h0 / G;
        const bool owner = (h0 % G) == 0;
        const int nxt = u + (int)gridDim.x;
        const bool has_next = nxt < units;
        if (errs && tid == 0 && p.err)
            atomicOr(p.err, errs);

        if (tid < 2 * NR) {
            al[ghh][gtt] = to_f32(ga);
            be[ghh][gtt] = to_f32(gb);
            if (valid)
                out_store(&p.as[((size_t)b * HV + h0 + ghh) * NR + gtt], to_f32(ga));
        }
        // inputs to LDS (history rows, then the verify rows), and the verify
        // rows' units straight to the raw-row stash
        uint4 *Xs = reinterpret_cast<uint4 *>(P);
        if (tid < (kWidth - 1) * UPR)
            Xs[tid] = hu;
        auto stage_xunit = [&](int q, uint4 val) {
            const int uu = q * kThreads + tid;
            if (uu < NR * UPR) {
                const int r = uu / UPR, k = uu % UPR;
                Xs[(kWidth - 1) * UPR + uu] = val;
                if (valid && (k >= 32 || owner))
                    out_store(reinterpret_cast<uint4 *>(p.xs + ((size_t)b * NR + r) * p.C + unit_channel(kh, h0, k)), val);
            }
        };
        stage_xunit(0, xu0);
        if constexpr (NXU > 1)
            stage_xunit(1, xu1);
        if constexpr (NXU > 2)
            stage_xunit(2, xu2);
        lds_barrier();
        {
            // the history this verify used, for the next step's commit-verify;
            // with a commit pending, the committed history also goes to the
            // pool (q/k units by the key head's first pair only)
            const int k = tid % UPR;
            if (valid && tid < (kWidth - 1) * UPR && (k >= 32 || owner)) {
                const size_t hoff = (size_t)(tid / UPR) * p.C + unit_channel(kh, h0, k);
                out_store(reinterpret_cast<uint4 *>(p.xh + (size_t)b * (kWidth - 1) * p.C + hoff), hu);
                if (FUSED && n > 0)
                    out_store(reinterpret_cast<uint4 *>(p.hist_out + (size_t)slot * (kWidth - 1) * p.C + hoff), hu);
            }
        }

        float v[NR];   // value channel tid = row rb + lane of head h0 + hh
        {
            ChanIn<NR, T> cinA, cinV;
            const T *Xt = reinterpret_cast<const T *>(P);
            auto tap = [](uint2 w, int k) {
                return T{(uint16_t)(((k < 2 ? w.x : w.y) >> (16 * (k & 1))) & 0xffffu)};
            };
#pragma unroll
            for (int k = 0; k < kWidth; ++k) {
                cinA.w[k] = tap(wA, k);
                cinV.w[k] = tap(wV, k);
            }
#pragma unroll
            for (int r = 0; r < kWidth - 1; ++r) {
                cinA.hist[r] = Xt[r * 512 + tid];
                cinV.hist[r] = Xt[r * 512 + 256 + tid];
            }
#pragma unroll
            for (int t = 0; t < NR; ++t) {
                cinA.x[t] = Xt[(kWidth - 1 + t) * 512 + tid];
                cinV.x[t] = Xt[(kWidth - 1 + t) * 512 + 256 + tid];
            }
            float y[NR];
            conv_rows(cinA, p.act, y);
#pragma unroll
            for (int t = 0; t < NR; ++t)
                Mt[jc * MS + (isq ? NR + t : t)] = y[t];
            if (isq) {
#pragma unroll
                for (int c = NC; c < MS; ++c)
                    Mt[jc * MS + c] = 0.0f;
            }
            conv_rows(cinV, p.act, v);
        }
        // the next unit's inputs load while this one is finished
        if (has_next)
            load_inputs(nxt);
        const bool nvalid = has_next && slot_in >= 0 && slot_in < p.P && err_in == 0;
        lds_barrier();   // the column table and the gates are complete

        float *Pw = P + wave * 64 * PS;
        float *invw = invs[wave];
        const float *alw = al[hh], *bew = be[hh];
        {
            f32x4 accg = {0.0f, 0.0f, 0.0f, 0.0f};
            float gv[2] = {0.0f, 0.0f}, dv[2] = {0.0f, 0.0f};
            gram_share<NVL, MS>(wave, kg, m, Mt, accg, gv, dv);
            float *g = gp[wave];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int uq = 4 * kg + q;
                if (uq < NR && m < NMF)
                    g[uq * NC + m] = accg[q];
                if (uq == m && m >= NR && m < NMF)
                    g[NR * NC + m - NR] = accg[q];
            }
            if (NVL) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    float x = gv[c], y = dv[c];
                    x += __shfl_xor(x, 16, 64);
                    x += __shfl_xor(x, 32, 64);
                    y += __shfl_xor(y, 16, 64);
                    y += __shfl_xor(y, 32, 64);
                    gv[c] = x;
                    dv[c] = y;
                }
                if (kg == 0 && m < NR) {
                    g[m * NC + NMF] = gv[0];
                    g[m * NC + NMF + 1] = gv[1];
                }
                if (lane == 0) {
                    g[NR * NC + NMF - NR] = dv[0];
                    g[NR * NC + NMF - NR + 1] = dv[1];
                }
            }
        }
        lds_barrier();   // from here on each wave finishes its rows alone
        auto gram = [&](int idx) { return (gp[0][idx] + gp[1][idx]) + (gp[2][idx] + gp[3][idx]); };
        if (lane < NC) {
            const float nn = lane < NR ? gram(lane * NC + lane) : gram(NR * NC + lane - NR);
            invw[lane] = 1.0f / sqrtf(nn + p.eps);
        }
        {
            int t, uu;
            tri_decode(min(lane, NT - 1), t, uu);
            float gtu = 1.0f;
#pragma unroll
            for (int q = 1; q < NR; ++q)
                gtu *= (q > uu && q <= t) ? alw[q] : 1.0f;
            const float iu = invw[uu];
            const float cA = (uu < t) ? bew[t] * (gtu * (gram(uu * NC + t) * iu * invw[t])) : 0.0f;
            const float cB = gtu * (gram(uu * NC + NR + t) * iu * invw[NR + t]);
            const int tt = min(lane, NR - 1);
            float gt = 1.0f;
#pragma unroll
            for (int q = 0; q < NR; ++q)
                gt *= q <= tt ? alw[q] : 1.0f;
            cpark[wave][lane] = float4{cA, cB, gt, bew[tt]};
        }

        // commit-verify: S_n goes to the pool (stores through a resource that
        // is empty when nothing is pending)
        if constexpr (FUSED) {
            const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.ssm_out + ((size_t)slot * HV + h0 + hh) * D * D,
                                                        valid && n > 0 ? D * D * 4 : 0);
#pragma unroll
            for (int c = 0; c < NCHUNK; ++c)
#pragma unroll
                for (int kk4 = 0; kk4 < CK; ++kk4)
                    buf_stream_store_f4(rw, soff, (uint32_t)(c * CK + kk4) * 4 * D * 4, S[c][kk4]);
        }
        // products with the column table
        const __amdgpu_buffer_rsrc_t nrs = state_rsrc(nxt, nvalid, slot_in, src_in, n_in);
        f32x4 acc[4];
        float pv[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            pv[q][0] = pv[q][1] = 0.0f;
        }
#pragma unroll
        for (int c = 0; c < NCHUNK; ++c) {
            mfma_chunk<CK, NVL, MS>(S[c], c, kg, m, Mt, acc, pv);
            __builtin_amdgcn_sched_barrier(0);   // keeps each chunk's column-table reads next to its products
        }

        if (m < NMF) {
            const float ic = invw[m];
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    Pw[(16 * kg + 4 * q + v4) * PS + m] = acc[v4][q] * ic;
        }
        if (NVL) {
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    float x = pv[v4][c];
                    x += __shfl_xor(x, 16, 64);
                    x += __shfl_xor(x, 32, 64);
                    pv[v4][c] = x;
                }
            if (kg == 0) {
                const float i0 = invw[NMF], i1 = invw[NMF + 1];
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    Pw[(4 * m + v4) * PS + NMF] = pv[v4][0] * i0;
                    Pw[(4 * m + v4) * PS + NMF + 1] = pv[v4][1] * i1;
                }
            }
        }
        wave_lds_sync();

        // row rb + lane by forward substitution with the broadcast coefficients
        {
            float *Pr = Pw + lane * PS;
            const float4 cc = cpark[wave][lane];
            float e[NR];
            // one row at a time: each row's broadcasts are issued where they are used
#pragma unroll
            for (int t = 0; t < NR; ++t) {
                const float r = __builtin_fmaf(-lane_value(cc.z, t), Pr[t], v[t]);
                float s = lane_value(cc.w, t) * r;
#pragma unroll
                for (int uu = 0; uu < t; ++uu)
                    s = __builtin_fmaf(-lane_value(cc.x, t * (t + 1) / 2 + uu), e[uu], s);
                e[t] = s;
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int t = 0; t < NR; ++t) {
                float s = lane_value(cc.z, t) * Pr[NR + t];
#pragma unroll
                for (int uu = 0; uu <= t; ++uu)
                    s = __builtin_fmaf(lane_value(cc.y, t * (t + 1) / 2 + uu), e[uu], s);
                const size_t oi = (((size_t)b * NR + t) * HV + h0 + hh) * D + rb + lane;
                out_store(&p.out[oi], from_f32<T>(valid ? p.scale * s : 0.0f));
                if (valid)
                    out_store(&p.es[oi], e[t]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // this row of the product table is read only by this lane: reuse it for e_t
#pragma unroll
            for (int t = 0; t < NR; ++t)
                Pr[t] = e[t];
        }
        if (owner && valid) {
            float *ks = p.ks + ((size_t)b * HK + kh) * NR * D;
            for (int idx = tid; idx < NR * D; idx += kThreads)
                out_store(&ks[idx], Mt[(idx % D) * MS + idx / D] * invw[idx / D]);
        }

        {
            wave_lds_sync();
            if (valid) {
                // S_t for every row, by the update the replay commit applies, from
                // the S_0 still in registers; a head's S_1..S_R are contiguous.
                // Plain stores: for this volume (R states per request) they
                // measured faster than nontemporal ones (270 against 285 us for
                // 64 requests x 9 rows)
                float *snap_h = p.snap + ((size_t)b * HV + h0 + hh) * NR * D * D;
#pragma unroll 1
                for (int t = 0; t < NR; ++t) {
                    const float a = alw[t];
                    const float it = invw[t];
                    float ev[4];
#pragma unroll
                    for (int v4 = 0; v4 < 4; ++v4)
                        ev[v4] = Pw[(4 * m + v4) * PS + t];
                    float *dst = snap_h + (size_t)t * D * D;
#pragma unroll
                    for (int c = 0; c < NCHUNK; ++c)
#pragma unroll
                        for (int k = 0; k < CK; ++k) {
                            const int j = 4 * (c * CK + k) + kg;
                            const float kk = Mt[j * MS + t] * it;
#pragma unroll
                            for (int v4 = 0; v4 < 4; ++v4)
                                S[c][k][v4] = row_update(S[c][k][v4], a, ev[v4], kk);
                            *reinterpret_cast<f32x4 *>(dst + (size_t)j * D + rb + 4 * m) = S[c][k];
                        }
                }
            }
            if (has_next) {
#pragma unroll
                for (int c = 0; c < NCHUNK; ++c)
                    load_chunk(S[c], nrs, soff, c);
            }
        }
        if (!has_next)
            break;
        u = nxt;
        valid = nvalid;
        slot = slot_in;
        n = n_in;
        errs = err_in;
        lds_barrier();   // every wave is done with this unit's LDS
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
    int HK, HV, C, P, R, B;
};

// Workgroups per head: each streams one part of at most 8 KiB of the head's
// state (key rows j0 .. j0 + D/parts - 1, contiguous in the pool), in two
// 16-byte accesses per lane. Small read-modify-write pieces keep enough
// workgroups in flight to cover HBM latency with loads and stores interleaved
// (8 KiB measured faster than 4, 16, 32 or 64 KiB parts).
template <int D> __host__ __device__ constexpr int commit_parts() { return D * D * 4 > 8192 ? D * D * 4 / 8192 : 1; }

template <int D, typename T, bool SNAP, int NPART>
__device__ __forceinline__ void commit_body(const CommitParams<T> &p)
{
    constexpr int JW = D / NPART;          // key rows of this part
    constexpr int LPJ = D / 4;             // lanes per key row, 4 state rows each
    constexpr int GJ = kThreads / LPJ;     // key rows per pass
    constexpr int JPER = JW / GJ;          // passes
    static_assert(JPER >= 1 && JW % GJ == 0, "part must cover whole passes");

    __shared__ __align__(16) float eb[kMaxRows * D];   // e_t[i]
    __shared__ float kb[kMaxRows * JW];                // k_t[j0 + jl]
    __shared__ float al[kMaxRows];

    const int tid = threadIdx.x;
    const int HV = p.HV, HK = p.HK, R = p.R;
    const int G = HV / HK;
    // Workgroups are dealt to the 8 XCDs round-robin by index: the parts of
    // head bh take indices congruent to bh mod 8, so all of them run on one
    // XCD and share its L2 copy of the head's stashed rows.
    const int grp = blockIdx.x / (kXcds * NPART), rem = blockIdx.x % (kXcds * NPART);
    const int part = rem / kXcds;
    const int bh = grp * kXcds + rem % kXcds;
    if (bh >= p.B * HV)
        return;
    const int b = bh / HV;
    const int h = bh % HV;
    const int kh = h / G;
    const int slot = p.slot_ids[b];
    const int n = p.accept[b];
    const bool report = tid == 0 && part == 0 && p.err;

    if (slot < -1 || slot >= p.P) {
        if (report)
            atomicOr(p.err, 1);
        return;
    }
    if (n < 0 || n > R) {
        if (report)
            atomicOr(p.err, 2);
        return;
    }
    if (slot == -1 || n == 0)
        return;

    // Conv history: the last W-1 entries of [history | rows 0..n-1]. The value
    // channels belong to this head, the key head's q/k channels to its first
    // value head; one 16-byte unit of channels per thread, the parts of the
    // head sharing the units out. Loaded first, stored last: each unit is
    // read and written by its thread alone.
    constexpr int EPU = 16 / sizeof(T);   // channels per unit
    static_assert(D % EPU == 0, "units must not straddle channel groups");
    const bool owner = (h % G) == 0;
    const int nunit = (owner ? 3 * D : D) / EPU;
    const int hu = part * kThreads + tid;
    static_assert(kWidth == 4, "the history unit holds three rows");
    T *hist = nullptr;
    uint4 win0 = {}, win1 = {}, win2 = {};
    if (hu < nunit) {
        const int idx = hu * EPU;
        int c;
        if (idx < D)
            c = 2 * HK * D + h * D + idx;
        else if (idx < 2 * D)
            c = kh * D + (idx - D);
        else
            c = HK * D + kh * D + (idx - 2 * D);
        hist = p.conv + (size_t)slot * (kWidth - 1) * p.C + c;
        // entry src of [history (W-1) | rows]
        auto entry = [&](int src) {
            const T *from = src < kWidth - 1 ? hist + (size_t)src * p.C
                                             : p.xs + ((size_t)b * R + (src - (kWidth - 1))) * p.C + c;
            return *reinterpret_cast<const uint4 *>(from);
        };
        win0 = entry(n);
        win1 = entry(n + 1);
        win2 = entry(n + 2);
    }

    const int j0 = part * JW;
    const int rq = tid % LPJ;
    const int g = tid / LPJ;
    float *Sd = p.ssm + ((size_t)slot * HV + h) * D * D + (size_t)j0 * D;

    if (SNAP) {
        const float *src = p.snap + (((size_t)b * HV + h) * R + (n - 1)) * D * D + (size_t)j0 * D;
        constexpr int NV = JW * D / 4 / kThreads;
        float4 v[NV];
#pragma unroll
        for (int q = 0; q < NV; ++q)
            v[q] = stream_load(src + 4 * (q * kThreads + tid));
#pragma unroll
        for (int q = 0; q < NV; ++q)
            stream_store(Sd + 4 * (q * kThreads + tid), v[q]);
    } else {
        // staging loads first (fixed count, clamped indices, no branches),
        // then the state stream
        constexpr int NSE = (kMaxRows * D + kThreads - 1) / kThreads;
        constexpr int NSK = (kMaxRows * JW + kThreads - 1) / kThreads;
        const float *kt = p.ks + ((size_t)b * HK + kh) * R * D;  // k_t at kt[t*D + j]
        float ev_in[NSE], kv_in[NSK];
#pragma unroll
        for (int q = 0; q < NSE; ++q) {
            const int idx = min(q * kThreads + tid, n * D - 1);
            const int t = idx / D, i = idx % D;
            ev_in[q] = p.es[(((size_t)b * R + t) * HV + h) * D + i];
        }
#pragma unroll
        for (int q = 0; q < NSK; ++q) {
            const int idx = min(q * kThreads + tid, n * JW - 1);
            const int t = idx / JW, jl = idx % JW;
            kv_in[q] = kt[t * D + j0 + jl];
        }
        const float a_in = p.as[((size_t)b * HV + h) * R + min(tid, n - 1)];
        float4 s[JPER];
#pragma unroll
        for (int jj = 0; jj < JPER; ++jj)
            s[jj] = stream_load(Sd + (size_t)(jj * GJ + g) * D + 4 * rq);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < NSE; ++q) {
            const int idx = q * kThreads + tid;
            if (idx < n * D)
                eb[idx] = ev_in[q];
        }
#pragma unroll
        for (int q = 0; q < NSK; ++q) {
            const int idx = q * kThreads + tid;
            if (idx < n * JW)
                kb[idx] = kv_in[q];
        }
        if (tid < n)
            al[tid] = a_in;
        lds_barrier();
        for (int t = 0; t < n; ++t) {
            const float a = al[t];
            const float4 ev = *reinterpret_cast<const float4 *>(&eb[t * D + 4 * rq]);
#pragma unroll
            for (int jj = 0; jj < JPER; ++jj) {
                const float k = kb[t * JW + jj * GJ + g];
                s[jj].x = row_update(s[jj].x, a, ev.x, k);
                s[jj].y = row_update(s[jj].y, a, ev.y, k);
                s[jj].z = row_update(s[jj].z, a, ev.z, k);
                s[jj].w = row_update(s[jj].w, a, ev.w, k);
            }
        }
#pragma unroll
        for (int jj = 0; jj < JPER; ++jj)
            stream_store(Sd + (size_t)(jj * GJ + g) * D + 4 * rq, s[jj]);
    }

    // conv history, stored after the state
    if (hu < nunit) {
        *reinterpret_cast<uint4 *>(hist) = win0;
        *reinterpret_cast<uint4 *>(hist + (size_t)p.C) = win1;
        *reinterpret_cast<uint4 *>(hist + 2 * (size_t)p.C) = win2;
    }
}

template <int D, typename T, bool SNAP, int NPART>
__global__ __launch_bounds__(kThreads) void gdn_commit_kernel(const CommitParams<T> p)
{
    commit_body<D, T, SNAP, NPART>(p);
}

// A hybrid stack commits every GDN layer in one launch: grid row y is layer
// y, whose pool and scratch pointers arrive as kernel arguments (so a
// captured launch keeps them); slot ids and accept lengths are shared.
constexpr int kMaxLayers = 64;

struct StackLayer {
    float *ssm;
    void *conv;
    const char *scratch;
    int P;
};

struct CommitStack {
    StackLayer l[kMaxLayers];
    size_t xs, es, ks, as, snap;   // scratch part offsets, the same in every layer
    int layers;
};

// Other per-slot states committed in the same launch: windows of the last L
// entries of a stream, rolled by the accept length over the rows the verify
// staged (FreeToken PR #844, Design: the commit restores every slot state as
// it stands after the accepted rows, all of them with one upload of the slot
// and count indices).
constexpr int kMaxWindows = 16;

struct WindowSet {
    gdn_slot_window w[kMaxWindows];
    int count;
};

// Request b's window in window state w: new word u (of L * entry words) is
// word u + n * entry of [old window | staged rows], so every source lies ahead
// of its destination. The roll runs in chunks of one word per thread, each
// chunk read completely before any of it is written (a barrier between), and
// a chunk's sources lie beyond every word written before it: in place with no
// staging buffer. Whole-workgroup path (barriers inside).
__device__ __forceinline__ void commit_window(const gdn_slot_window &w, const int32_t *slot_ids,
                                              const int32_t *accept, int R, int32_t *err, int b)
{
    const int slot = slot_ids[b], n = accept[b];
    if (slot == -1)
        return;
    if (slot < -1 || slot >= w.num_slots || n < 0 || n > R) {
        if (threadIdx.x == 0 && err)
            atomicOr(err, (slot < -1 || slot >= w.num_slots) ? 1 : 2);
        return;
    }
    if (n == 0)
        return;
    const int ew = w.entry_bytes / 4;
    const int words = w.length * ew, shift = n * ew;
    uint32_t *state = static_cast<uint32_t *>(w.state) + (size_t)slot * words;
    const uint32_t *rows = static_cast<const uint32_t *>(w.rows) + (size_t)b * R * ew;
    for (int c = 0; c < words; c += kThreads) {
        const int u = c + (int)threadIdx.x;
        uint32_t v = 0;
        if (u < words) {
            const int src = u + shift;   // < words + n * ew <= words + R * ew
            v = src < words ? state[src] : rows[src - words];
        }
        __syncthreads();
        if (u < words)
            state[u] = v;
        __syncthreads();
    }
}

__device__ __forceinline__ void commit_windows(const WindowSet &ws, const int32_t *slot_ids, const int32_t *accept,
                                               int B, int R, int32_t *err)
{
    const int items = ws.count * B;
    for (int i = blockIdx.x; i < items; i += gridDim.x)
        commit_window(ws.w[i / B], slot_ids, accept, R, err, i % B);
}

__global__ __launch_bounds__(kThreads) void gdn_commit_windows_kernel(const WindowSet ws, const int32_t *slot_ids,
                                                                      const int32_t *accept, int B, int R,
                                                                      int32_t *err)
{
    commit_windows(ws, slot_ids, accept, B, R, err);
}

template <int D, typename T, bool SNAP, int NPART>
__global__ __launch_bounds__(kThreads) void gdn_commit_stack_kernel(const CommitParams<T> p0, const CommitStack st,
                                                                    const WindowSet ws)
{
    if ((int)blockIdx.y == st.layers) {   // the grid row after the layers: the window states
        commit_windows(ws, p0.slot_ids, p0.accept, p0.B, p0.R, p0.err);
        return;
    }
    CommitParams<T> p = p0;
    const StackLayer &l = st.l[blockIdx.y];
    p.ssm = l.ssm;
    p.conv = static_cast<T *>(l.conv);
    p.P = l.P;
    p.xs = reinterpret_cast<const T *>(l.scratch + st.xs);
    p.es = reinterpret_cast<const float *>(l.scratch + st.es);
    p.ks = reinterpret_cast<const float *>(l.scratch + st.ks);
    p.as = reinterpret_cast<const float *>(l.scratch + st.as);
    p.snap = SNAP ? reinterpret_cast<const float *>(l.scratch + st.snap) : nullptr;
    commit_body<D, T, SNAP, NPART>(p);
}

// ---- greedy acceptance --------------------------------------------------------

// One thread per request: the first row whose draft differs from the target's
// greedy token ends the accepted run.
__global__ __launch_bounds__(kThreads) void gdn_accept_greedy_kernel(const int32_t *draft, const int32_t *target,
                                                                     const int32_t *slot_ids, int B, int R,
                                                                     int32_t *accept, int32_t *next)
{
    const int b = blockIdx.x * kThreads + threadIdx.x;
    if (b >= B)
        return;
    if (slot_ids && slot_ids[b] == -1) {
        accept[b] = 0;
        if (next)
            next[b] = -1;
        return;
    }
    const int32_t *d = draft + (size_t)b * (R - 1);
    const int32_t *g = target + (size_t)b * R;
    int n = 1;
    while (n < R && d[n - 1] == g[n - 1])
        ++n;
    accept[b] = n;
    if (next)
        next[b] = g[n - 1];
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
    if (d->conv_width != kWidth || d->num_v_heads / d->num_k_heads > kMaxGroup)
        return GDN_ERR_UNSUPPORTED;
    c->HK = d->num_k_heads;
    c->HV = d->num_v_heads;
    c->D = d->d_k;
    c->C = 2 * c->HK * c->D + c->HV * c->D;
    c->esize = d->dtype == GDN_F32 ? 4 : 2;
    return GDN_OK;
}

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

struct VerifyLaunch {
    int batch, HK, HV;
    hipStream_t st;
};

// The split kernel's block size: 16- or 32-row blocks while the grid stays
// within one workgroup per compute unit (the phases after the column table
// run at one SIMD's rate, so more, smaller blocks finish sooner), 64-row
// blocks above that. Results do not depend on the choice.
template <int NR, bool SNAP, bool FUSED>
void launch_split(const VerifyParams<bf16_t> &vp, int units, hipStream_t st)
{
    if (units * 16 <= kComputeUnits)
        hipLaunchKernelGGL((gdn_verify_d128_split_kernel<NR, SNAP, FUSED, 1>), dim3(units * 16), dim3(kThreads), 0, st,
                           vp);
    else if (units * 8 <= kComputeUnits)
        hipLaunchKernelGGL((gdn_verify_d128_split_kernel<NR, SNAP, FUSED, 2>), dim3(units * 8), dim3(kThreads), 0, st,
                           vp);
    else
        hipLaunchKernelGGL((gdn_verify_d128_split_kernel<NR, SNAP, FUSED, 4>), dim3(units * 4), dim3(kThreads), 0, st,
                           vp);
}

template <int D, int NR, typename T, bool SNAP>
hipError_t launch_verify(const VerifyParams<T> &vp, const VerifyLaunch &l)
{
    if (D == 128 && (l.HV / l.HK) % 2 == 0) {
        const int units = l.batch * (l.HV / 2);
        bool done = false;
        if constexpr (sizeof(T) == 2) {
            // fewer units than compute units: split each over 4 to 16 workgroups
            // (measured: 1 request, replay 7.3 -> 6.1 us with four; at 16 requests,
            // one unit per compute unit, the split was slower in replay mode, 12.0
            // against 11.0 us). One threshold for both modes keeps their products
            // in the same order, so replay and snapshot agree bit for bit
            if (units < kComputeUnits) {
                launch_split<NR, SNAP, false>(vp, units, l.st);
                done = true;
            } else if constexpr (SNAP) {
                const int cap = kComputeUnits * snapshot_groups_per_cu<NR>();
                const int grid = units < cap ? units : cap;
                hipLaunchKernelGGL((gdn_verify_d128_snapshot_kernel<NR, false>), dim3(grid), dim3(kThreads), 0, l.st,
                                   vp, units);
                done = true;
            }
        }
        if (!done)
            hipLaunchKernelGGL((gdn_verify_d128_kernel<NR, T, SNAP, false>), dim3(units), dim3(kThreads), 0, l.st,
                               vp);
    } else {
        hipLaunchKernelGGL((gdn_verify_kernel<D, NR, T, SNAP>), dim3(l.batch * l.HV), dim3(kThreads),
                           0, l.st, vp);
    }
    return hipGetLastError();
}

template <int D, typename T, bool SNAP>
hipError_t verify_rows(int rows, const VerifyParams<T> &vp, const VerifyLaunch &l)
{
    switch (rows) {
    case 1: return launch_verify<D, 1, T, SNAP>(vp, l);
    case 2: return launch_verify<D, 2, T, SNAP>(vp, l);
    case 3: return launch_verify<D, 3, T, SNAP>(vp, l);
    case 4: return launch_verify<D, 4, T, SNAP>(vp, l);
    case 5: return launch_verify<D, 5, T, SNAP>(vp, l);
    case 6: return launch_verify<D, 6, T, SNAP>(vp, l);
    case 7: return launch_verify<D, 7, T, SNAP>(vp, l);
    case 8: return launch_verify<D, 8, T, SNAP>(vp, l);
    case 9: return launch_verify<D, 9, T, SNAP>(vp, l);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, bool SNAP>
hipError_t verify_dim(int D, int rows, const VerifyParams<T> &vp, const VerifyLaunch &l)
{
    switch (D) {
    case 32: return verify_rows<32, T, SNAP>(rows, vp, l);
    case 64: return verify_rows<64, T, SNAP>(rows, vp, l);
    case 128: return verify_rows<128, T, SNAP>(rows, vp, l);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
VerifyParams<T> verify_params(const Checked &c, const gdn_layer_desc *d, const gdn_pool *pool, const void *conv_w,
                              const void *x, const void *alpha, const void *beta, const int32_t *slot_ids,
                              bool snapshot, void *scratch, const ScratchLayout &L, void *out, int32_t *err)
{
    VerifyParams<T> vp = {};
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
    vp.xh = reinterpret_cast<T *>(base + L.xh);
    vp.snap = snapshot ? reinterpret_cast<float *>(base + L.snap) : nullptr;
    vp.HK = c.HK;
    vp.HV = c.HV;
    vp.C = c.C;
    vp.P = pool->num_slots;
    vp.act = d->act;
    vp.scale = d->scale;
    vp.eps = d->l2_eps;
    return vp;
}

template <typename T>
hipError_t verify_typed(const Checked &c, const gdn_layer_desc *d, const gdn_pool *pool,
                        const void *conv_w, const void *x, const void *alpha, const void *beta,
                        const int32_t *slot_ids, int batch, int rows, bool snapshot, void *scratch,
                        const ScratchLayout &L, void *out, int32_t *err, hipStream_t st)
{
    const VerifyParams<T> vp =
        verify_params<T>(c, d, pool, conv_w, x, alpha, beta, slot_ids, snapshot, scratch, L, out, err);
    const VerifyLaunch l{batch, c.HK, c.HV, st};
    return snapshot ? verify_dim<T, true>(c.D, rows, vp, l) : verify_dim<T, false>(c.D, rows, vp, l);
}

// Commit-verify: the d = 128 verify kernels of the same batch sizes (the
// split kernel below one unit per compute unit, the one-round kernel from
// there), with the previous step's commit applied to each state chunk on its
// way in.
template <int NR, bool SNAP>
hipError_t launch_commit_verify(const VerifyParams<bf16_t> &vp, int batch, int HV, hipStream_t st)
{
    const int units = batch * (HV / 2);
    if (units < kComputeUnits) {
        launch_split<NR, SNAP, true>(vp, units, st);
    } else if constexpr (SNAP) {
        const int cap = kComputeUnits * snapshot_groups_per_cu<NR>();
        hipLaunchKernelGGL((gdn_verify_d128_snapshot_kernel<NR, true>), dim3(units < cap ? units : cap),
                           dim3(kThreads), 0, st, vp, units);
    } else {
        hipLaunchKernelGGL((gdn_verify_d128_kernel<NR, bf16_t, false, true>), dim3(units), dim3(kThreads), 0, st, vp);
    }
    return hipGetLastError();
}

template <bool SNAP>
hipError_t commit_verify_rows(int rows, const VerifyParams<bf16_t> &vp, int batch, int HV, hipStream_t st)
{
    switch (rows) {
    case 1: return launch_commit_verify<1, SNAP>(vp, batch, HV, st);
    case 2: return launch_commit_verify<2, SNAP>(vp, batch, HV, st);
    case 3: return launch_commit_verify<3, SNAP>(vp, batch, HV, st);
    case 4: return launch_commit_verify<4, SNAP>(vp, batch, HV, st);
    case 5: return launch_commit_verify<5, SNAP>(vp, batch, HV, st);
    case 6: return launch_commit_verify<6, SNAP>(vp, batch, HV, st);
    case 7: return launch_commit_verify<7, SNAP>(vp, batch, HV, st);
    case 8: return launch_commit_verify<8, SNAP>(vp, batch, HV, st);
    case 9: return launch_commit_verify<9, SNAP>(vp, batch, HV, st);
    default: return hipErrorInvalidValue;
    }
}

template <int D, typename T, bool SNAP, int NPART>
hipError_t launch_commit_parts(const CommitParams<T> &cp, const CommitStack *stack, int layers, int blocks,
                               hipStream_t st, const WindowSet *ws)
{
    const int groups = (blocks + kXcds - 1) / kXcds;
    const dim3 grid(groups * kXcds * NPART, layers + (ws && ws->count > 0 ? 1 : 0));
    if (stack) {
        WindowSet none = {};
        hipLaunchKernelGGL((gdn_commit_stack_kernel<D, T, SNAP, NPART>), grid, dim3(kThreads), 0, st, cp, *stack,
                           ws ? *ws : none);
    } else
        hipLaunchKernelGGL((gdn_commit_kernel<D, T, SNAP, NPART>), grid, dim3(kThreads), 0, st, cp);
    return hipGetLastError();
}

template <int D, typename T, bool SNAP>
hipError_t launch_commit(const CommitParams<T> &cp, const CommitStack *stack, int layers, int blocks,
                         hipStream_t st, const WindowSet *ws)
{
    // 8 KiB parts at every batch size: 16 KiB parts for 16 requests and 4 KiB
    // parts for one request measured no faster
    return launch_commit_parts<D, T, SNAP, commit_parts<D>()>(cp, stack, layers, blocks, st, ws);
}

template <typename T, bool SNAP>
hipError_t commit_dim(int D, const CommitParams<T> &cp, const CommitStack *stack, int layers, int blocks,
                      hipStream_t st, const WindowSet *ws)
{
    switch (D) {
    case 32: return launch_commit<32, T, SNAP>(cp, stack, layers, blocks, st, ws);
    case 64: return launch_commit<64, T, SNAP>(cp, stack, layers, blocks, st, ws);
    case 128: return launch_commit<128, T, SNAP>(cp, stack, layers, blocks, st, ws);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t commit_typed(const Checked &c, const gdn_pool *pool, const int32_t *slot_ids,
                        const int32_t *accept, int batch, int rows, bool snapshot,
                        const void *scratch, const ScratchLayout &L, int32_t *err, hipStream_t st,
                        const CommitStack *stack = nullptr, int layers = 1, const WindowSet *ws = nullptr)
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
    cp.B = batch;
    const int blocks = batch * c.HV;
    return snapshot ? commit_dim<T, true>(c.D, cp, stack, layers, blocks, st, ws)
                    : commit_dim<T, false>(c.D, cp, stack, layers, blocks, st, ws);
}

gdn_status check_common(const gdn_layer_desc *desc, const gdn_pool *pool, int32_t batch,
                        int32_t rows, gdn_commit_mode mode, const void *scratch,
                        size_t scratch_bytes, Checked *c, ScratchLayout *L)
{
    gdn_status s = check_desc(desc, c);
    if (s != GDN_OK)
        return s;
    if (!pool || !pool->ssm || !pool->conv || pool->num_slots < 1 || !aligned16(pool->ssm) ||
        !aligned16(pool->conv))
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
    if (!conv_w || !x || !alpha || !beta || !slot_ids || !out || !aligned16(conv_w) || !aligned16(x))
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

gdn_status gdn_spec_commit_verify(const gdn_layer_desc *desc, const gdn_pool *pool, const void *conv_w,
                                  const void *x, const void *alpha, const void *beta,
                                  const int32_t *slot_ids, int32_t batch, int32_t rows, gdn_commit_mode mode,
                                  void *scratch, size_t scratch_bytes, const int32_t *src_row,
                                  const void *prev_scratch, size_t prev_scratch_bytes, const int32_t *prev_slot_ids,
                                  const int32_t *prev_accept_len, int32_t prev_batch, void *out, int32_t *err_flag,
                                  void *stream)
{
    Checked c;
    ScratchLayout L;
    gdn_status s = check_common(desc, pool, batch, rows, mode, scratch, scratch_bytes, &c, &L);
    if (s != GDN_OK)
        return s;
    if (prev_batch < 0)
        return GDN_ERR_INVALID_ARG;
    if (desc->dtype != GDN_BF16 || c.D != 128 || (c.HV / c.HK) % 2 != 0)
        return GDN_ERR_UNSUPPORTED;
    if ((size_t)prev_batch * c.HV > 0x7fffffffu)
        return GDN_ERR_UNSUPPORTED;
    const bool snap = mode == GDN_COMMIT_SNAPSHOT;
    const ScratchLayout Lp = scratch_layout(c.HK, c.HV, c.D, c.C, c.esize, prev_batch, rows, snap);
    if (prev_batch > 0) {
        if (!prev_scratch || !aligned16(prev_scratch) || !prev_slot_ids || !prev_accept_len)
            return GDN_ERR_INVALID_ARG;
        if (prev_scratch_bytes < Lp.total)
            return GDN_ERR_SCRATCH_TOO_SMALL;
        // this step's stash must not land on the one being committed
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(scratch), a1 = a0 + L.total;
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(prev_scratch), b1 = b0 + Lp.total;
        if (batch > 0 && a0 < b1 && b0 < a1)
            return GDN_ERR_INVALID_ARG;
    }
    if (batch == 0)
        return GDN_OK;
    if (!conv_w || !x || !alpha || !beta || !slot_ids || !src_row || !out || !aligned16(conv_w) || !aligned16(x))
        return GDN_ERR_INVALID_ARG;
    VerifyParams<bf16_t> vp =
        verify_params<bf16_t>(c, desc, pool, conv_w, x, alpha, beta, slot_ids, snap, scratch, L, out, err_flag);
    const char *pb = static_cast<const char *>(prev_scratch);
    vp.ssm_out = pool->ssm;
    vp.hist_out = static_cast<bf16_t *>(pool->conv);
    vp.src_row = src_row;
    vp.prev_slots = prev_slot_ids;
    vp.prev_accept = prev_accept_len;
    vp.pxs = prev_batch > 0 ? reinterpret_cast<const bf16_t *>(pb + Lp.xs) : nullptr;
    vp.pes = prev_batch > 0 ? reinterpret_cast<const float *>(pb + Lp.es) : nullptr;
    vp.pks = prev_batch > 0 ? reinterpret_cast<const float *>(pb + Lp.ks) : nullptr;
    vp.pas = prev_batch > 0 ? reinterpret_cast<const float *>(pb + Lp.as) : nullptr;
    vp.pxh = prev_batch > 0 ? reinterpret_cast<const bf16_t *>(pb + Lp.xh) : nullptr;
    vp.psnap = prev_batch > 0 && snap ? reinterpret_cast<const float *>(pb + Lp.snap) : nullptr;
    vp.Bp = prev_batch;
    const hipError_t e = snap ? commit_verify_rows<true>(rows, vp, batch, c.HV, static_cast<hipStream_t>(stream))
                              : commit_verify_rows<false>(rows, vp, batch, c.HV, static_cast<hipStream_t>(stream));
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

gdn_status gdn_spec_commit_layers(const gdn_layer_desc *desc, const gdn_pool *pools,
                                  void *const *scratch, int32_t layers, const int32_t *slot_ids,
                                  const int32_t *accept_len, int32_t batch, int32_t rows,
                                  gdn_commit_mode mode, size_t scratch_bytes, int32_t *err_flag,
                                  void *stream)
{
    if (layers < 1)
        return GDN_ERR_INVALID_ARG;
    return gdn_spec_commit_all(desc, pools, scratch, layers, nullptr, 0, slot_ids, accept_len, batch, rows, mode,
                               scratch_bytes, err_flag, stream);
}

gdn_status gdn_spec_commit_all(const gdn_layer_desc *desc, const gdn_pool *pools, void *const *scratch,
                               int32_t layers, const gdn_slot_window *windows, int32_t num_windows,
                               const int32_t *slot_ids, const int32_t *accept_len, int32_t batch, int32_t rows,
                               gdn_commit_mode mode, size_t scratch_bytes, int32_t *err_flag, void *stream)
{
    if (layers < 0 || layers > kMaxLayers || num_windows < 0 || num_windows > kMaxWindows ||
        layers + num_windows < 1 || (layers > 0 && (!pools || !scratch)) || (num_windows > 0 && !windows))
        return GDN_ERR_INVALID_ARG;
    if (batch < 0 || rows < 1 || rows > kMaxRows)
        return GDN_ERR_INVALID_ARG;
    WindowSet ws = {};
    for (int i = 0; i < num_windows; ++i) {
        const gdn_slot_window &w = windows[i];
        if (!w.state || !w.rows || w.num_slots < 1 || w.length < 1 || w.entry_bytes < 4 || w.entry_bytes % 4 ||
            (reinterpret_cast<uintptr_t>(w.state) & 3) || (reinterpret_cast<uintptr_t>(w.rows) & 3))
            return GDN_ERR_INVALID_ARG;
        if ((int64_t)w.length * w.entry_bytes + (int64_t)kMaxRows * w.entry_bytes > 0x7fffffff)
            return GDN_ERR_UNSUPPORTED;
        ws.w[i] = w;
    }
    ws.count = num_windows;
    Checked c;
    ScratchLayout L;
    for (int l = 0; l < layers; ++l) {
        const gdn_status s = check_common(desc, &pools[l], batch, rows, mode, scratch[l], scratch_bytes, &c, &L);
        if (s != GDN_OK)
            return s;
    }
    if (batch == 0)
        return GDN_OK;
    if (!slot_ids || !accept_len)
        return GDN_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (layers == 0) {
        const int items = num_windows * batch;
        hipLaunchKernelGGL(gdn_commit_windows_kernel, dim3(items < 4096 ? items : 4096), dim3(kThreads), 0, st, ws,
                           slot_ids, accept_len, batch, rows, err_flag);
        return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    }
    CommitStack stack = {};
    for (int l = 0; l < layers; ++l)
        stack.l[l] = StackLayer{pools[l].ssm, pools[l].conv, static_cast<const char *>(scratch[l]),
                                pools[l].num_slots};
    stack.xs = L.xs;
    stack.es = L.es;
    stack.ks = L.ks;
    stack.as = L.as;
    stack.snap = L.snap;
    stack.layers = layers;
    const bool snap = mode == GDN_COMMIT_SNAPSHOT;
    // layer 0's pointers fill the shared parameters; each grid row swaps in its own
    hipError_t e = desc->dtype == GDN_F32
        ? commit_typed<float>(c, &pools[0], slot_ids, accept_len, batch, rows, snap, scratch[0], L, err_flag, st,
                              &stack, layers, &ws)
        : commit_typed<bf16_t>(c, &pools[0], slot_ids, accept_len, batch, rows, snap, scratch[0], L, err_flag, st,
                               &stack, layers, &ws);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_spec_accept_greedy(const int32_t *draft, const int32_t *target,
                                  const int32_t *slot_ids, int32_t batch, int32_t rows,
                                  int32_t *accept_len, int32_t *next_token, void *stream)
{
    if (batch < 0 || rows < 1 || rows > kMaxRows)
        return GDN_ERR_INVALID_ARG;
    if (batch == 0)
        return GDN_OK;
    if (!target || !accept_len || (rows > 1 && !draft))
        return GDN_ERR_INVALID_ARG;
    hipLaunchKernelGGL(gdn_accept_greedy_kernel, dim3((batch + kThreads - 1) / kThreads), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), draft, target, slot_ids, batch, rows, accept_len,
                       next_token);
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
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
