// spec_attention.hip -- verification attention over a paged KV cache for
// MI355X (gfx950): the C ABI of include/spec_attention.h.
//
// The k+1 verify rows of a request and the Hq/Hkv query heads that share a
// KV head form a block of R*G queries; every key and value of that KV head is
// read once per block (lmdeploy PR #5006, What's included, Verification path:
// verification attention over paged KV with a cross-workgroup reduce).
//
// Split kernel: one workgroup per (request, KV head, key split, group of 4
// query tiles); wave w takes 16 queries. Splits are long enough for about
// 2048 workgroups per launch, in multiples of 256 positions. Per tile of 32
// keys:
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16: the key rows are the A operand
//   (16 bytes of one key per lane, straight from the page), the wave's
//   queries the B operand (held in registers). Lane (kg, n) ends with the
//   scores of keys 4kg..4kg+3 (and 16 + the same) for query n.
//   Online softmax per query: the max and sum over a query's 32 keys are
//   within the lane and across lanes n, n^16, n^32, n^48.
//   O += P V on the same instruction: the lane's 8 probabilities, in that key
//   order, are exactly its A operand; V is the B operand, read from a
//   transposed copy of the tile in LDS whose key order matches.
// Combine kernel: per (request, KV head) the splits' partial results merge
// with their running maxima into o.

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "spec_attention.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreadsA = 256;   // 4 waves, one query tile each
constexpr int kTilesPerGroup = 4;
constexpr int kKeyTile = 32;
constexpr int kSplitUnit = 256;  // split lengths are multiples of this
constexpr int kTargetGroups = 2048;  // workgroups a launch aims for
constexpr int kMaxRowsA = 9;
constexpr float kNeg = -1.0e30f;  // masked score: finite, so a fully masked row stays NaN-free

struct AttnParams {
    const uint16_t *q;
    const uint16_t *kc;
    const uint16_t *vc;
    const int32_t *bt;
    const int32_t *seq;
    float *opart;     // [B*Hkv][S][QG*64][D]
    float *mpart;     // [B*Hkv][S][QG*64]
    float *lpart;     // [B*Hkv][S][QG*64]
    int32_t *flags;   // [B*Hkv][S][QG]: a page id was out of range
    uint16_t *out;
    int32_t *err;
    int B, R, Hq, Hkv, G, PS, NP, MB, S, QG, KC;   // KC: positions per split
    float scale;
};

__device__ __forceinline__ uint16_t bf16_bits(float v)
{
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bool request_refused(int L, const AttnParams &p)
{
    return L < 0 || (L != 0 && (L < p.R || L > p.MB * p.PS));
}

// LDS position of key k (0..31) of a tile: keys 4c..4c+3 and 16+4c..16+4c+3
// sit together at 8c..8c+7, the order in which lane group c holds their
// probabilities.
__device__ __forceinline__ int key_slot(int k)
{
    return 8 * ((k & 15) >> 2) + 4 * (k >> 4) + (k & 3);
}

template <int D>
__global__ __launch_bounds__(kThreadsA) __attribute__((amdgpu_waves_per_eu(2))) void gdn_attn_split_kernel(const AttnParams p)
{
    constexpr int DS = D / 32;   // K-steps of Q K^T
    constexpr int DT = D / 16;   // output tiles of P V
    constexpr int NVU = kKeyTile * D / 8 / kThreadsA;   // 16-byte V units per thread per tile
    static_assert(NVU * kThreadsA * 8 == kKeyTile * D, "V tile splits evenly");

    __shared__ __align__(16) uint16_t vt[D * kKeyTile];   // [d][slot]: V^T of the tile

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int kg = lane >> 4, n = lane & 15;
    const int qg = blockIdx.x % p.QG;
    const int rest = blockIdx.x / p.QG;
    const int s = rest % p.S;
    const int bg = rest / p.S;
    const int g = bg % p.Hkv, b = bg / p.Hkv;
    const int L = p.seq[b];
    const int k0 = s * p.KC;

    if (request_refused(L, p) || L == 0 || k0 >= L) {
        if (request_refused(L, p) && s == 0 && qg == 0 && tid == 0 && p.err)
            atomicOr(p.err, 4);
        return;   // the combine counts the splits that ran from seq_len alone
    }
    const int k1 = min(k0 + p.KC, L);
    const int ntile = (k1 - k0 + kKeyTile - 1) / kKeyTile;

    // this wave's queries: column n of query tile 4 qg + wave
    const int nq = p.R * p.G;
    const int qi = 16 * (kTilesPerGroup * qg + wave) + n;
    const bool qok = qi < nq;
    const bool active = 16 * (kTilesPerGroup * qg + wave) < nq;   // wave has any query
    const int qc = qok ? qi : 0;
    const int t = qc / p.G, h = g * p.G + qc % p.G;
    const int last = qok ? L - p.R + t : -1;   // the last position this query sees

    bf16x8 qv[DS];
    {
        const uint16_t *qrow = p.q + (((size_t)b * p.R + t) * p.Hq + h) * D + 8 * kg;
#pragma unroll
        for (int ks = 0; ks < DS; ++ks)
            qv[ks] = *reinterpret_cast<const bf16x8 *>(qrow + 32 * ks);
    }
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        o[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float mrun = kNeg, lrun = 0.0f;
    int badpage = 0;

    for (int it = 0; it < ntile; ++it) {
        const int p0 = k0 + it * kKeyTile;   // a multiple of 32: the tile lies in one page
        int page = p.bt[(size_t)b * p.MB + p0 / p.PS];
        if (page < 0 || page >= p.NP) {
            badpage = 1;
            page = 0;
        }
        const size_t row0 = (size_t)page * p.PS + p0 % p.PS;   // cache row of position p0

        // V units of the tile, loaded first so they arrive under Q K^T
        uint4 vu[NVU];
#pragma unroll
        for (int i = 0; i < NVU; ++i) {
            const int u = i * kThreadsA + tid;
            const int k = u % kKeyTile, d0 = 8 * (u / kKeyTile);
            vu[i] = *reinterpret_cast<const uint4 *>(p.vc + ((row0 + k) * p.Hkv + g) * D + d0);
        }

        float pv[8];
        if (active) {
            f32x4 sacc[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                sacc[st] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                const uint16_t *krow = p.kc + ((row0 + 16 * st + n) * p.Hkv + g) * D + 8 * kg;
#pragma unroll
                for (int ks = 0; ks < DS; ++ks)
                    sacc[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        *reinterpret_cast<const bf16x8 *>(krow + 32 * ks), qv[ks], sacc[st], 0, 0, 0);
            }
            // lane (kg, n): sacc[st][v] is the score of position p0 + 16 st + 4 kg + v, query n
            float sv[8];
            float tmax = kNeg;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int pos = p0 + 16 * st + 4 * kg + v;
                    const float x = pos <= last ? sacc[st][v] * p.scale : kNeg;
                    sv[4 * st + v] = x;
                    tmax = fmaxf(tmax, x);
                }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float mnew = fmaxf(mrun, tmax);
            const float alpha = __expf(mrun - mnew);
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                pv[i] = __expf(sv[i] - mnew);
                psum += pv[i];
            }
            psum += __shfl_xor(psum, 16, 64);
            psum += __shfl_xor(psum, 32, 64);
            lrun = lrun * alpha + psum;
            mrun = mnew;
            // o[dt][v] belongs to query 4 kg + v, whose factor lane 4 kg + v holds
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float a = __shfl(alpha, 4 * kg + v, 64);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    o[dt][v] *= a;
            }
        }

        __syncthreads();   // the previous tile's V is no longer read
#pragma unroll
        for (int i = 0; i < NVU; ++i) {
            const int u = i * kThreadsA + tid;
            const int k = u % kKeyTile, d0 = 8 * (u / kKeyTile);
            const int slot = key_slot(k);
            const uint32_t w[4] = {vu[i].x, vu[i].y, vu[i].z, vu[i].w};
#pragma unroll
            for (int j = 0; j < 8; ++j)
                vt[(d0 + j) * kKeyTile + slot] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
        }
        __syncthreads();

        if (active) {
            bf16x8 pa;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                pa[i] = __builtin_bit_cast(__bf16, bf16_bits(pv[i]));
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8 vb = *reinterpret_cast<const bf16x8 *>(&vt[(16 * dt + n) * kKeyTile + 8 * kg]);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[dt], 0, 0, 0);
            }
        }
    }

    // partial results: lane (kg, n) holds o of queries 4 kg + v, dims 16 dt + n
    const int QP = p.QG * 64;
    const size_t part = (size_t)bg * p.S + s;
    if (active) {
        const int qbase = 16 * (kTilesPerGroup * qg + wave);
        float *op = p.opart + (part * QP + qbase) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                op[(size_t)(4 * kg + v) * D + 16 * dt + n] = o[dt][v];
        if (kg == 0) {
            p.mpart[part * QP + qbase + n] = mrun;
            p.lpart[part * QP + qbase + n] = lrun;
        }
    }
    if (tid == 0)
        p.flags[part * p.QG + qg] = badpage;
}

// One workgroup per (request, KV head): o = sum_s e^{m_s - M} O_s / sum_s e^{m_s - M} l_s.
template <int D>
__global__ __launch_bounds__(kThreadsA) void gdn_attn_combine_kernel(const AttnParams p)
{
    const int bg = blockIdx.x;
    const int g = bg % p.Hkv, b = bg / p.Hkv;
    const int L = p.seq[b];
    const int nq = p.R * p.G;
    const int QP = p.QG * 64;
    bool zero = L == 0 || request_refused(L, p);
    const int ns = zero ? 0 : (L + p.KC - 1) / p.KC;
    if (!zero) {
        int bad = 0;
        for (int i = 0; i < ns * p.QG; ++i)
            bad |= p.flags[(size_t)bg * p.S * p.QG + i];
        if (bad) {
            zero = true;
            if (threadIdx.x == 0 && p.err)
                atomicOr(p.err, 1);
        }
    }
    for (int idx = threadIdx.x; idx < nq * D; idx += kThreadsA) {
        const int qi = idx / D, d = idx % D;
        const int t = qi / p.G, h = g * p.G + qi % p.G;
        float r = 0.0f;
        if (!zero) {
            float M = kNeg;
            for (int s = 0; s < ns; ++s)
                M = fmaxf(M, p.mpart[((size_t)bg * p.S + s) * QP + qi]);
            float num = 0.0f, den = 0.0f;
            for (int s = 0; s < ns; ++s) {
                const size_t part = (size_t)bg * p.S + s;
                const float w = __expf(p.mpart[part * QP + qi] - M);
                num += w * p.opart[(part * QP + qi) * D + d];
                den += w * p.lpart[part * QP + qi];
            }
            r = num / den;
        }
        p.out[(((size_t)b * p.R + t) * p.Hq + h) * D + d] = bf16_bits(r);
    }
}

struct AttnLayout {
    size_t opart, mpart, lpart, flags, total;
    int S, QG, KC;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

gdn_status attn_layout(const gdn_attn_desc *d, int batch, int rows, int max_blocks, AttnLayout *l)
{
    if (!d || batch < 0 || rows < 1 || rows > kMaxRowsA || max_blocks < 1)
        return GDN_ERR_INVALID_ARG;
    if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->num_q_heads % d->num_kv_heads != 0 ||
        d->page_size < 1)
        return GDN_ERR_INVALID_ARG;
    if ((d->head_dim != 128 && d->head_dim != 256) || d->page_size % kKeyTile != 0 ||
        (d->num_q_heads / d->num_kv_heads) * rows > 128)
        return GDN_ERR_UNSUPPORTED;
    const size_t maxpos = (size_t)max_blocks * d->page_size;
    if (maxpos > (size_t)1 << 30)
        return GDN_ERR_UNSUPPORTED;
    const int nq = (d->num_q_heads / d->num_kv_heads) * rows;
    l->QG = (nq + 16 * kTilesPerGroup - 1) / (16 * kTilesPerGroup);
    // enough splits to fill the chip, in whole units: long splits for a
    // large batch keep the partial results small
    const size_t units = (maxpos + kSplitUnit - 1) / kSplitUnit;
    const size_t per_split_groups = (size_t)(batch > 0 ? batch : 1) * d->num_kv_heads * l->QG;
    size_t want = (kTargetGroups + per_split_groups - 1) / per_split_groups;
    want = want < 1 ? 1 : (want > units ? units : want);
    l->KC = (int)((units + want - 1) / want) * kSplitUnit;
    l->S = (int)((maxpos + l->KC - 1) / l->KC);
    const size_t parts = (size_t)batch * d->num_kv_heads * l->S;
    const size_t QP = (size_t)l->QG * 64;
    size_t off = 0;
    l->opart = off;
    off = align256(off + parts * QP * d->head_dim * sizeof(float));
    l->mpart = off;
    off = align256(off + parts * QP * sizeof(float));
    l->lpart = off;
    off = align256(off + parts * QP * sizeof(float));
    l->flags = off;
    off = align256(off + parts * l->QG * sizeof(int32_t));
    l->total = off;
    return GDN_OK;
}

bool aligned16a(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

}  // namespace

extern "C" {

gdn_status gdn_spec_attn_scratch_bytes(const gdn_attn_desc *desc, int32_t batch, int32_t rows,
                                       int32_t max_blocks, size_t *bytes)
{
    AttnLayout l;
    const gdn_status s = attn_layout(desc, batch, rows, max_blocks, &l);
    if (s != GDN_OK)
        return s;
    if (!bytes)
        return GDN_ERR_INVALID_ARG;
    *bytes = l.total;
    return GDN_OK;
}

gdn_status gdn_spec_attn_verify(const gdn_attn_desc *desc, const void *q, const void *k_cache,
                                const void *v_cache, int32_t num_pages, const int32_t *block_table,
                                int32_t max_blocks, const int32_t *seq_lens, int32_t batch,
                                int32_t rows, void *scratch, size_t scratch_bytes, void *out,
                                int32_t *err_flag, void *stream)
{
    AttnLayout l;
    gdn_status s = attn_layout(desc, batch, rows, max_blocks, &l);
    if (s != GDN_OK)
        return s;
    if (batch == 0)
        return GDN_OK;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !scratch || !out || num_pages < 1 ||
        !aligned16a(q) || !aligned16a(k_cache) || !aligned16a(v_cache) || !aligned16a(scratch))
        return GDN_ERR_INVALID_ARG;
    if (scratch_bytes < l.total)
        return GDN_ERR_SCRATCH_TOO_SMALL;
    if ((size_t)batch * desc->num_kv_heads * l.S * l.QG > 0x7fffffffu)
        return GDN_ERR_UNSUPPORTED;
    char *base = static_cast<char *>(scratch);
    AttnParams p;
    p.q = static_cast<const uint16_t *>(q);
    p.kc = static_cast<const uint16_t *>(k_cache);
    p.vc = static_cast<const uint16_t *>(v_cache);
    p.bt = block_table;
    p.seq = seq_lens;
    p.opart = reinterpret_cast<float *>(base + l.opart);
    p.mpart = reinterpret_cast<float *>(base + l.mpart);
    p.lpart = reinterpret_cast<float *>(base + l.lpart);
    p.flags = reinterpret_cast<int32_t *>(base + l.flags);
    p.out = static_cast<uint16_t *>(out);
    p.err = err_flag;
    p.B = batch;
    p.R = rows;
    p.Hq = desc->num_q_heads;
    p.Hkv = desc->num_kv_heads;
    p.G = desc->num_q_heads / desc->num_kv_heads;
    p.PS = desc->page_size;
    p.NP = num_pages;
    p.MB = max_blocks;
    p.S = l.S;
    p.QG = l.QG;
    p.KC = l.KC;
    p.scale = desc->scale;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 split_grid((unsigned)(batch * p.Hkv * l.S * l.QG));
    const dim3 combine_grid((unsigned)(batch * p.Hkv));
    if (desc->head_dim == 128) {
        hipLaunchKernelGGL(gdn_attn_split_kernel<128>, split_grid, dim3(kThreadsA), 0, st, p);
        hipLaunchKernelGGL(gdn_attn_combine_kernel<128>, combine_grid, dim3(kThreadsA), 0, st, p);
    } else {
        hipLaunchKernelGGL(gdn_attn_split_kernel<256>, split_grid, dim3(kThreadsA), 0, st, p);
        hipLaunchKernelGGL(gdn_attn_combine_kernel<256>, combine_grid, dim3(kThreadsA), 0, st, p);
    }
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"
