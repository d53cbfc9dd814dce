// spec_attention.hip -- verification attention over a paged KV cache for
// MI355X (gfx950): the C ABI of include/spec_attention.h.
//
// The k+1 verify rows of a request and the Hq/Hkv query heads that share a
// KV head form a block of R*G queries (at most 128: eight tiles of 16); every
// key and value of that KV head is read from HBM once for the whole block
// (lmdeploy PR #5006, What's included, Verification path: verification
// attention over paged KV with a cross-workgroup reduce).
//
// Split kernel. The batch's key tiles (32 positions, inside one page) are
// laid end to end over all (request, KV head) pairs and cut into equal
// ranges, one per workgroup of a fixed grid, so every workgroup streams the
// same number of bytes whatever the mix of sequence lengths. A workgroup's
// range is one stream of tiles, whatever pairs it crosses: cursors for the
// loads (two tiles ahead, nontemporal, following the block table page by
// page), the LDS stores (one tile ahead) and the arithmetic each move one
// tile per step, with one workgroup barrier per tile. One wave per query
// tile (16 queries) does the arithmetic on each tile staged in LDS:
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16, K rows in their cache layout
//     as the A operand, the queries (in registers) as B. Lane (kg, n) ends
//     with the scores of keys 4kg..4kg+3 and 16+4kg..16+4kg+3 for query n.
//   online softmax per query in base 2: its 32 scores sit in lanes n, n^16,
//     n^32, n^48.
//   O^T += V^T P^T on the same instruction: the lane's 8 probabilities are
//     the B operand as they stand; the V operand (8 keys of one head-dim
//     column) comes from V rows in LDS through ds_read_b64_tr_b16, whose
//     16-lane transpose hands lane n the column it needs, so V is never
//     rearranged.
// Each (range, pair) piece leaves a partial result (its running max, sum and
// unnormalised output per query) in a record; cutting at both range and
// pair boundaries numbers the records range + pair, so no index table is
// needed.
// Combine kernel. Per (pair, query tile) the pair's records merge, weighted
// by their running maxima, into o.

#include <hip/hip_runtime.h>

#include <mutex>
#include <stddef.h>
#include <stdint.h>

#include "spec_attention.h"

// Scratch of gdn_spec_attn_verify_static: the split records and pair starts
// of one call, on every GPU the library runs on, for the life of the process.
// Host code never uses this name as an address (on the host it is only a
// stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[GDN_SPEC_ATTN_STATIC_SCRATCH_BYTES];

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kKeyTile = 32;      // positions per tile; page sizes are multiples of it
constexpr int kMaxRowsA = 9;
constexpr int kMaxQTiles = 8;     // at most 128 queries per KV head
constexpr int kMaxKvHeads = 1024; // a tile's per-thread byte offsets stay 32-bit
constexpr int kSplitGroups = 256; // split-kernel workgroups on a large batch: one per compute unit
constexpr int kMinGroupTiles = 4; // a small batch gets fewer workgroups, each at least this many tiles
constexpr int kThreadsS = 512;    // split kernel: eight waves, one per query tile, all loading tiles
constexpr float kNeg = -1.0e30f;  // starting softmax reference: below any score, and finite
constexpr float kSlack = 8.0f;    // how far (log2 units) a score may pass the running softmax reference
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kVmcnt0 = 0x0F70;   // s_waitcnt operand: vector memory count 0, the other counters untouched

// LDS tile geometry: K rows, then V rows, 2D bytes each plus 128 spare.
// Row r starts its units (r & 7) positions in: the 16 rows one operand read
// touches (16 keys of K for the A operand; 16 keys x 4 column groups of V
// for the transposing reads) then fall evenly on the banks, every write of
// a row stays one contiguous run, and a lane's addresses for successive
// column or K steps differ by constants (instruction offsets, no per-step
// address arithmetic).
template <int D> struct Tile {
    static constexpr int RS = D * 2 + 128;               // row stride, bytes
    static constexpr int KB = kKeyTile * RS;
    static constexpr int BUF = 2 * KB;                   // one K + V tile
    static constexpr int UPR = D / 8;                    // 16-byte units per row
    static constexpr int UNITS = 2 * kKeyTile * UPR;     // units of a K + V tile
    static constexpr int NU = UNITS / kThreadsS;         // units per thread
    static constexpr int PD = D == 256 ? 2 : 4;          // tiles whose loads are in flight
    static_assert(UNITS % kThreadsS == 0, "tile units spread evenly");
    static_assert(RS % 16 == 0, "rows stay 16-byte aligned");
};

struct AttnParams {
    const uint16_t *q;
    const uint16_t *kc;
    const uint16_t *vc;
    const int32_t *bt;
    const int32_t *seq;
    float *rec;       // records: [NW + B*Hkv][RECF] (O [QP][D], m [QP] in log2 units, l [QP], flag)
    int32_t *starts;  // [B*Hkv + 1]: key tiles before each pair, then the total (from the split kernel)
    uint16_t *out;
    int32_t *err;
    int B, R, Hq, Hkv, G, PS, NP, MB, NQ, QT, NW, RECF, TPP;   // TPP: key tiles per page
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

// Lengths and block-table entries are read-only for the whole launch: read
// through the constant address space, a uniform index becomes a scalar load,
// whose wait does not hold back the tile loads in flight.
typedef const __attribute__((address_space(4))) int32_t cint32;

__device__ __forceinline__ int seq_len(int b, const AttnParams &p) { return ((cint32 *)p.seq)[b]; }

__device__ __forceinline__ int table_entry(size_t i, const AttnParams &p) { return ((cint32 *)p.bt)[i]; }

__device__ __forceinline__ bool request_refused(int L, const AttnParams &p)
{
    return L < 0 || (L != 0 && (L < p.R || L > p.MB * p.PS));
}

// Key tiles of pair pr = (request pr / Hkv, KV head pr % Hkv); padding and
// refused requests have none.
__device__ __forceinline__ int pair_tiles(int pr, const AttnParams &p)
{
    const int L = seq_len(pr / p.Hkv, p);
    return (L <= 0 || request_refused(L, p)) ? 0 : (L + kKeyTile - 1) / kKeyTile;
}

// Inclusive prefix sum over the workgroup (blockDim.x a multiple of 64, at
// most 512); `total` gets the sum over all threads.
__device__ int block_scan(int x, int *wsum, int &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o)
            x += y;
    }
    if (lane == 63)
        wsum[wave] = x;
    __syncthreads();
    int before = 0;
    total = 0;
    for (int i = 0; i < nw; ++i) {
        const int v = wsum[i];
        before += i < wave ? v : 0;
        total += v;
    }
    __syncthreads();
    return x + before;
}

// Total key tiles T of the batch, the pair holding tile lo = w ceil(T / NW)
// (the first of range w) and the tiles before it; pair -1 when the range is
// empty. Workgroup 0 also writes each pair's first tile, then T, to starts[]
// for the combine kernel.
struct Located {
    int T, pair, start;
};

__device__ Located locate(const AttnParams &p, int w, int *wsum, int *loc)
{
    const int np = p.B * p.Hkv;
    const int tid = threadIdx.x, nthr = blockDim.x;
    if (tid == 0)
        loc[0] = -1;
    int T = 0, x0 = 0, incl0 = 0;
    for (int c0 = 0; c0 < np; c0 += nthr) {
        const int pr = c0 + tid;
        const int x = pr < np ? pair_tiles(pr, p) : 0;
        int tot;
        const int incl = block_scan(x, wsum, tot) + T;
        if (w == 0 && pr < np)
            p.starts[pr] = incl - x;
        if (c0 == 0) {
            x0 = x;
            incl0 = incl;
        }
        T += tot;
    }
    if (w == 0 && tid == 0)
        p.starts[np] = T;
    T = __builtin_amdgcn_readfirstlane(T);
    const int lo = w * ((T + p.NW - 1) / p.NW);
    Located r{T, -1, 0};
    if (lo >= T)
        return r;
    if (np <= nthr) {
        // the one scan already placed every pair
        if (tid < np && x0 > 0 && incl0 > lo && incl0 - x0 <= lo) {
            loc[0] = tid;
            loc[1] = incl0 - x0;
        }
        __syncthreads();
    } else {
        int base = 0;
        for (int c0 = 0; c0 < np; c0 += nthr) {
            const int pr = c0 + tid;
            const int x = pr < np ? pair_tiles(pr, p) : 0;
            int tot;
            const int incl = block_scan(x, wsum, tot) + base;
            if (pr < np && x > 0 && incl > lo && incl - x <= lo) {
                loc[0] = pr;
                loc[1] = incl - x;
            }
            base += tot;
            __syncthreads();
            if (loc[0] >= 0)
                break;
        }
    }
    // the same for every thread: kept in scalar registers, so the loads that
    // depend on it (lengths, block-table entries) are scalar loads
    r.pair = __builtin_amdgcn_readfirstlane(loc[0]);
    r.start = __builtin_amdgcn_readfirstlane(loc[1]);
    __syncthreads();
    return r;
}

// A walk along the batch's run of key tiles, at most one tile per step: the
// pair holding the current tile (its request, KV head, length and tile
// count) and the tile's index t within the pair. Every field is the same for
// the whole workgroup, so it lives in scalar registers.
struct Cursor {
    int pr, b, g, L, nt, t;
};

__device__ __forceinline__ void set_pair(Cursor &c, int pr, const AttnParams &p)
{
    c.pr = pr;
    c.b = pr / p.Hkv;
    c.g = pr - c.b * p.Hkv;
    c.L = seq_len(c.b, p);
    c.nt = (c.L <= 0 || request_refused(c.L, p)) ? 0 : (c.L + kKeyTile - 1) / kKeyTile;
}

// To tile 0 of the next pair that has tiles (the caller knows one remains).
__device__ __forceinline__ void next_pair(Cursor &c, const AttnParams &p)
{
    do
        set_pair(c, c.pr + 1, p);
    while (c.nt == 0);
    c.t = 0;
}

__device__ __forceinline__ void step(Cursor &c, const AttnParams &p)
{
    if (++c.t == c.nt)
        next_pair(c, p);
}

// The load side's walk also follows the pages: the block of the request
// that holds the tile, the tile's place in its page, and the addresses of
// the tile's first key in the K and V caches for KV head g. The block
// table is read once per page. A page id outside the pool is read as page 0
// and flagged in `bad`, which goes into the piece's record when the walk
// leaves the pair.
struct PageWalk {
    Cursor c;
    int blk, tip;
    const char *kt, *vt;
    bool bad;
};

template <int D>
__device__ __forceinline__ void set_page(PageWalk &pw, const AttnParams &p)
{
    int page = table_entry((size_t)pw.c.b * p.MB + pw.blk, p);
    if (page < 0 || page >= p.NP) {
        pw.bad = true;
        page = 0;
    }
    const size_t off = (((size_t)page * p.PS + pw.tip * kKeyTile) * p.Hkv + pw.c.g) * D;
    pw.kt = reinterpret_cast<const char *>(p.kc + off);
    pw.vt = reinterpret_cast<const char *>(p.vc + off);
}

template <int D>
__device__ __forceinline__ void record_flag(const PageWalk &pw, const AttnParams &p, int w)
{
    if (threadIdx.x == 0)
        p.rec[(size_t)(w + pw.c.pr) * p.RECF + (size_t)p.QT * 16 * (D + 2)] = pw.bad ? 1.0f : 0.0f;
}

template <int D>
__device__ __forceinline__ void step_pages(PageWalk &pw, const AttnParams &p, int w)
{
    if (pw.c.t + 1 == pw.c.nt) {
        record_flag<D>(pw, p, w);   // leaving the pair
        next_pair(pw.c, p);
        pw.blk = 0;
        pw.tip = 0;
        pw.bad = false;
        set_page<D>(pw, p);
    } else {
        ++pw.c.t;
        if (++pw.tip == p.TPP) {
            pw.tip = 0;
            ++pw.blk;
            set_page<D>(pw, p);
        } else {
            const size_t rows = (size_t)kKeyTile * p.Hkv * D * 2;   // the page's next 32 positions
            pw.kt += rows;
            pw.vt += rows;
        }
    }
}

// This thread's units of a K + V tile, k < NU/2 in K and the rest the same
// units of V: byte offsets from the tile's first key (fixed for the launch).
template <int D>
__device__ __forceinline__ void unit_offsets(const AttnParams &p, uint32_t (&off)[Tile<D>::NU / 2])
{
    using TL = Tile<D>;
#pragma unroll
    for (int k = 0; k < TL::NU / 2; ++k) {
        const int u = threadIdx.x + k * kThreadsS;
        const int key = u / TL::UPR, du = u % TL::UPR;
        off[k] = (uint32_t)key * (uint32_t)p.Hkv * (uint32_t)(D * 2) + 16u * (uint32_t)du;
    }
}

// A step past the end of the range loads nothing it needs; it still issues
// its loads (so every step counts the same loads), from `spare`, 8 KiB of
// this workgroup's own scratch that stays in the cache, rather than reading
// the last tile from memory again.
constexpr uint32_t kSpareMask = 0x1FF0;
static_assert(16 * (128 + 2) * 4 >= kSpareMask + 16, "a record (one query tile, D >= 128) covers the spare reads");

template <int D>
__device__ __forceinline__ void load_tile(const PageWalk &pw, const uint32_t (&off)[Tile<D>::NU / 2], bool past,
                                          const char *spare, uint4 (&pre)[Tile<D>::NU])
{
    using TL = Tile<D>;
#pragma unroll
    for (int k = 0; k < TL::NU; ++k) {
        const uint32_t o = off[k % (TL::NU / 2)];
        const char *src = past ? spare + (o & kSpareMask) : (k < TL::NU / 2 ? pw.kt : pw.vt) + o;
        // read once per call: streamed past the caches
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src));
        pre[k] = uint4{x[0], x[1], x[2], x[3]};
    }
}

// Keys past the sequence are stored as zeros: their slots may hold anything,
// and 0 * NaN would reach o through P V. (Applied here, not at the load, so
// that nothing waits for the loads before the tile is needed; only the tile
// that holds position L - 1 can reach past it.)
template <int D>
__device__ __forceinline__ void store_tile(char *buf, const uint4 (&pre)[Tile<D>::NU], int p0, int L)
{
    using TL = Tile<D>;
    const bool tail = p0 + kKeyTile > L;
#pragma unroll
    for (int k = 0; k < TL::NU; ++k) {
        const int u = threadIdx.x + k * kThreadsS;   // K units, then V units
        const int row = u / TL::UPR, du = u % TL::UPR;   // row: key (K) or 32 + key (V)
        const int key = row % kKeyTile;
        uint4 val = pre[k];
        if (tail && p0 + key >= L)
            val = uint4{0u, 0u, 0u, 0u};
        *reinterpret_cast<uint4 *>(buf + row * TL::RS + 16 * (du + (key & 7))) = val;
    }
}

// Reductions over the four lanes n, n^16, n^32, n^48 that hold one query's
// scores. v_permlane16_swap / v_permlane32_swap (with the value as both
// operands) leave x[l] and x[l^16] (or x[l^32]) in the two results, in lane
// order, on every lane: no LDS round trip as a shuffle would take.
__device__ __forceinline__ float max_xor16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One key tile against this wave's 16 queries: scores, online softmax, and
// the tile's P V added into o. `buf` holds the tile's K and V rows, `p0` is
// its first position, `last` the last position the lane's query n sees, and
// `full` says every query of the workgroup sees the whole tile. The softmax
// runs in base 2: c2 = scale log2(e), and mrun is in units of log2.
template <int D>
__device__ __forceinline__ void attend(const char *buf, int p0, int last, bool full, float c2, int kg, int n,
                                       const bf16x8 (&qv)[D / 32], f32x4 (&o)[D / 16], float &mrun, float &lrun)
{
    using TL = Tile<D>;
    constexpr int DS = D / 32;
    constexpr int DT = D / 16;
    f32x4 sacc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        sacc[st] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        // key 16 st + n, unit 4 ks + kg (at position 4 ks + kg + (n & 7))
        const char *krow = buf + (16 * st + n) * TL::RS + 16 * (kg + (n & 7));
#pragma unroll
        for (int ks = 0; ks < DS; ++ks)
            sacc[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8 *>(krow + 64 * ks),
                                                               qv[ks], sacc[st], 0, 0, 0);
    }
    // lane (kg, n): sacc[st][v] is the (unscaled) score of position
    // p0 + 16 st + 4 kg + v, query n
    float sv[8];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            sv[4 * st + v] = sacc[st][v];
    if (!full) {
        // only a pair's last tile or two hold positions that some verify row
        // does not see. Masked scores are -inf: if a row sees none of the
        // tile, its maximum stays -inf, the reference does not move, and every
        // probability is exp2(-inf) = 0, so a piece the row cannot see leaves
        // l = 0, o = 0 (a finite masked score would become the reference and
        // its scaled rounding error could reach exp2 as a huge argument)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (p0 + 16 * st + 4 * kg + v > last)
                    sv[4 * st + v] = -__builtin_inff();
    }
    float tmax = sv[0];
#pragma unroll
    for (int j = 1; j < 8; ++j)
        tmax = fmaxf(tmax, sv[j]);
    tmax = max_xor32(max_xor16(tmax)) * c2;   // scale > 0: the maximum commutes with it
    // The running reference mrun moves only when a score passes it by more
    // than kSlack: softmax does not depend on the reference, and probabilities
    // up to 2^kSlack are exact in fp32 and as relative in bf16 as any other,
    // so the rescale of o is rare once the first tile has set mrun.
    const float mnew = tmax > mrun + kSlack ? tmax : mrun;
    const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
    float psum = 0.0f;
    bf16x8 pa;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float pj = __builtin_amdgcn_exp2f(fmaf(sv[j], c2, -mnew));
        psum += pj;
        pa[j] = (__bf16)pj;   // nearest, ties to even (v_cvt_pk_bf16_f32)
    }
    psum = sum_xor32(sum_xor16(psum));
    lrun = lrun * alpha + psum;
    mrun = mnew;
    // o holds O^T: o[dt][v] is column 16 dt + 4 kg + v of query n, this lane's own
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                o[dt][v] *= alpha;
    }
    // O^T += V^T P^T. V operand (A) of column tile dt: lane r of group kg
    // names a row (key 4 kg + r/4, columns 16 dt + 4 (r%4) ..) and the
    // transpose gives lane n keys 4 kg .. 4 kg + 3 of column 16 dt + n; the
    // second read does keys 16 + 4 kg ..: the key order of the probabilities
    // in pa, which are the B operand as they stand
    // (rows 4 kg + r/4 and 16 rows further start their units equally far in)
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const int vr = 4 * kg + (n >> 2);
    const char *vrow = buf + TL::KB + vr * TL::RS + 16 * (vr & 7) + 8 * (n & 3);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vrow + 32 * dt));
        const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vrow + 16 * TL::RS + 32 * dt));
        const bf16x8 vb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pa, o[dt], 0, 0, 0);
    }
}

template <int D>
__global__ __launch_bounds__(kThreadsS) __attribute__((amdgpu_waves_per_eu(2))) void gdn_attn_split_kernel(const AttnParams p)
{
    using TL = Tile<D>;
    constexpr int DS = D / 32;   // K-steps of Q K^T
    constexpr int DT = D / 16;   // output column tiles of P V

    __shared__ __align__(16) char smem[2 * TL::BUF];
    __shared__ int wsum[8];
    __shared__ int loc[2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = lane >> 4, n = lane & 15;
    const int w = blockIdx.x;

    // this workgroup's range lo .. hi-1 of the batch's key tiles
    const Located first = locate(p, w, wsum, loc);
    if (first.pair < 0)
        return;
    const int per = (first.T + p.NW - 1) / p.NW;
    const int lo = w * per, hi = min(first.T, lo + per);
    const int ntot = hi - lo;

    // this wave's queries: query qi = 16 wave + n is verify row qi / G of
    // query head g G + qi % G, which sees positions 0 .. L - R + row
    const bool computes = wave < p.QT;   // one wave per query tile; the others only load
    const int qi = 16 * wave + n;
    const bool qok = computes && qi < p.NQ;
    const int qc = qok ? qi : 0;
    const int qrow = qc / p.G, qhead = qc % p.G;
    auto load_q = [&](const Cursor &c, bf16x8 (&qv)[DS]) {
        const uint16_t *src = p.q + (((size_t)c.b * p.R + qrow) * p.Hq + c.g * p.G + qhead) * D + 8 * kg;
#pragma unroll
        for (int ks = 0; ks < DS; ++ks)
            qv[ks] = *reinterpret_cast<const bf16x8 *>(src + 32 * ks);
    };

    // The range is one stream of tiles, whatever pairs it crosses: the
    // loads run PD tiles ahead of the arithmetic and LDS stores one tile
    // ahead, each with its own cursor, so the pipeline never drains at a
    // pair boundary. The compute cursor cc ends a piece (its record) at the
    // pair's last tile or the range's.
    Cursor c0;
    set_pair(c0, first.pair, p);
    c0.t = lo - first.start;
    Cursor cs = c0, cc = c0;   // LDS stores, arithmetic
    PageWalk pw;               // loads
    pw.c = c0;
    pw.blk = c0.t / p.TPP;
    pw.tip = c0.t - pw.blk * p.TPP;
    pw.bad = false;
    set_page<D>(pw, p);
    uint32_t off[TL::NU / 2];
    unit_offsets<D>(p, off);
    bf16x8 qv[DS];
    if (computes)
        load_q(cc, qv);
    int last = qok ? cc.L - p.R + qrow : -1;
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        o[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float mrun = kNeg, lrun = 0.0f;
    const int QP = p.QT * 16;
    const float c2 = p.scale * kLog2e;

    // Tile j of the range is consumed from LDS buffer j & 1. Its loads went
    // out PD tiles earlier, into register set j % PD, which is stored to its
    // buffer one tile ahead. Every step issues the same loads and stores
    // (past the range the loads read `spare` and the stores go to a buffer
    // no step consumes; the steps past its end skip only the arithmetic), so
    // each wait for a register set covers just that set's loads. Each cursor
    // moves on one tile per step while its tile is inside the range.
    uint4 pre[TL::PD][TL::NU];
    // record w of the scratch: at least 8 KiB (one query tile, D >= 128)
    const char *spare = reinterpret_cast<const char *>(p.rec + (size_t)w * p.RECF);
#pragma unroll
    for (int s = 0; s < TL::PD; ++s) {
        if (s > 0 && s < ntot)
            step_pages<D>(pw, p, w);
        load_tile<D>(pw, off, s >= ntot, spare, pre[s]);
    }
    store_tile<D>(smem, pre[0], cs.t * kKeyTile, cs.L);
    __syncthreads();
    const int nsteps = (ntot + TL::PD - 1) / TL::PD * TL::PD;
    for (int j0 = 0; j0 < nsteps; j0 += TL::PD) {
#pragma unroll
        for (int s = 0; s < TL::PD; ++s) {
            const int j = j0 + s;
            if (j + TL::PD < ntot)
                step_pages<D>(pw, p, w);
            load_tile<D>(pw, off, j + TL::PD >= ntot, spare, pre[s]);
            if (j < ntot) {
                if (computes)
                    attend<D>(smem + (j & 1) * TL::BUF, cc.t * kKeyTile, last,
                              cc.t * kKeyTile + kKeyTile - 1 <= cc.L - p.R, c2, kg, n, qv, o, mrun, lrun);
                if (cc.t == cc.nt - 1 || j == ntot - 1) {
                    // the piece of pair cc in this range ends: its record, in
                    // which lane (kg, n) holds columns 16 dt + 4 kg .. + 3 of query
                    // 16 wave + n (rows of the query slots past NQ are not written)
                    float *rec = p.rec + (size_t)(w + cc.pr) * p.RECF;
                    if (qok) {
                        const int qb = 16 * wave;
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt)
                            *reinterpret_cast<f32x4 *>(&rec[(size_t)(qb + n) * D + 16 * dt + 4 * kg]) = o[dt];
                        if (kg == 0) {
                            rec[(size_t)QP * D + qb + n] = mrun;
                            rec[(size_t)QP * D + QP + qb + n] = lrun;
                        }
                    }
                    if (j < ntot - 1) {
                        // on to the next pair: its queries (the first tile of the
                        // new piece waits for them, and so for the tile loads in
                        // flight: one memory latency per switch)
                        next_pair(cc, p);
                        last = qok ? cc.L - p.R + qrow : -1;
                        if (computes)
                            load_q(cc, qv);
                        // wait for them here, on this path only: otherwise the
                        // queries would count as possibly in flight at every
                        // step, and each step's products would first wait for
                        // the previous step's tile loads
                        __builtin_amdgcn_s_waitcnt(kVmcnt0);
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt)
                            o[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                        mrun = kNeg;
                        lrun = 0.0f;
                    }
                } else {
                    ++cc.t;
                }
            }
            if (j + 1 < ntot)
                step(cs, p);
            store_tile<D>(smem + ((j + 1) & 1) * TL::BUF, pre[(s + 1) % TL::PD], cs.t * kKeyTile, cs.L);
            __syncthreads();
        }
    }
    record_flag<D>(pw, p, w);   // the range's last piece
}

// One workgroup per (pair, query tile): o = sum_r 2^{m_r - M} O_r / sum_r 2^{m_r - M} l_r
// over the pair's records r (maxima in units of log2). Each load instruction
// of a wave reads whole record rows (lane l: columns 4 l .. 4 l + 3 of a row
// of D floats); wave v of eight takes queries 2 v and 2 v + 1 of the tile.
// The records come in chunks of kChunk: every load of a chunk is issued
// before any arithmetic and the chunks merge online, so a pair spread over
// up to kChunk records costs one round trip to memory once its range is
// known.
constexpr int kChunk = 8;
constexpr int kThreadsC = 512;

template <int D>
__global__ __launch_bounds__(kThreadsC) void gdn_attn_combine_kernel(const AttnParams p)
{
    constexpr int LPR = D / 4;            // lanes per row
    constexpr int RPI = 64 / LPR;         // rows per load instruction
    constexpr int QPT = 2 / RPI;          // queries per thread
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pr = blockIdx.x, qt = blockIdx.y;
    const int np = p.B * p.Hkv;
    const int b = pr / p.Hkv, g = pr % p.Hkv;
    const int L = seq_len(b, p);
    const int QP = p.QT * 16;
    typedef const __attribute__((address_space(4))) float cfloat;

    const int total = ((cint32 *)p.starts)[np], start = ((cint32 *)p.starts)[pr];
    const int nt = pair_tiles(pr, p);
    if (request_refused(L, p) && g == 0 && qt == 0 && tid == 0 && p.err)
        atomicOr(p.err, 4);
    const int c0 = 4 * (lane % LPR);
    const int q0 = 16 * qt + 2 * wave + lane / LPR;   // this thread's queries: q0 + RPI k
    f32x4 acc[QPT];
    float mrun[QPT], den[QPT];
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
        acc[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        mrun[k] = kNeg;
        den[k] = 0.0f;
    }
    bool bad = false;
    if (nt > 0) {
        const int per = (total + p.NW - 1) / p.NW;
        const int w0 = start / per, w1 = (start + nt - 1) / per;
        for (int c = w0; c <= w1; c += kChunk) {
            f32x4 ov[kChunk][QPT];
            float mv[kChunk][QPT], lv[kChunk][QPT], fl[kChunk];
#pragma unroll
            for (int r = 0; r < kChunk; ++r) {
                const float *rec = p.rec + (size_t)(min(c + r, w1) + pr) * p.RECF;   // past w1: w1 again, unused
#pragma unroll
                for (int k = 0; k < QPT; ++k) {
                    const int qi = q0 + RPI * k;
                    // (a query slot past NQ has no row: its result is never stored)
                    ov[r][k] = qi < p.NQ ? *reinterpret_cast<const f32x4 *>(&rec[(size_t)qi * D + c0])
                                         : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    if (RPI == 1) {
                        // the wave's queries are uniform: scalar loads, no vector registers
                        mv[r][k] = ((const cfloat *)rec)[(size_t)QP * D + qi];
                        lv[r][k] = ((const cfloat *)rec)[(size_t)QP * D + QP + qi];
                    } else {
                        mv[r][k] = rec[(size_t)QP * D + qi];
                        lv[r][k] = rec[(size_t)QP * D + QP + qi];
                    }
                }
                fl[r] = ((const cfloat *)rec)[(size_t)QP * (D + 2)];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < kChunk; ++r)
                bad |= c + r <= w1 && fl[r] != 0.0f;
#pragma unroll
            for (int k = 0; k < QPT; ++k) {
                float m = mrun[k];
#pragma unroll
                for (int r = 0; r < kChunk; ++r)
                    m = c + r <= w1 ? fmaxf(m, mv[r][k]) : m;
                const float alpha = __builtin_amdgcn_exp2f(mrun[k] - m);
                float dsum = den[k] * alpha;
                f32x4 a = acc[k] * alpha;
#pragma unroll
                for (int r = 0; r < kChunk; ++r) {
                    const float wr = c + r <= w1 ? __builtin_amdgcn_exp2f(mv[r][k] - m) : 0.0f;
                    dsum = fmaf(wr, lv[r][k], dsum);
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        a[v] = fmaf(wr, ov[r][k][v], a[v]);
                }
                mrun[k] = m;
                den[k] = dsum;
                acc[k] = a;
            }
        }
        if (bad && g == 0 && qt == 0 && tid == 0 && p.err)
            atomicOr(p.err, 1);
    }
    const bool zero = nt == 0 || bad;
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
        const int qi = q0 + RPI * k;
        if (qi < p.NQ) {
            const float inv = zero ? 0.0f : 1.0f / den[k];
            const int t = qi / p.G, h = g * p.G + qi % p.G;
            uint32_t wd[2];
#pragma unroll
            for (int v = 0; v < 2; ++v)
                wd[v] = (uint32_t)bf16_bits(zero ? 0.0f : acc[k][2 * v] * inv) |
                        ((uint32_t)bf16_bits(zero ? 0.0f : acc[k][2 * v + 1] * inv) << 16);
            // nontemporal: written back as it goes, not by the release at the
            // kernel's end (the partial records above stay write-back: this
            // kernel reads them right after the split kernel wrote them)
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            __builtin_nontemporal_store(u32x2{wd[0], wd[1]},
                                        reinterpret_cast<u32x2 *>(p.out + (((size_t)b * p.R + t) * p.Hq + h) * D + c0));
        }
    }
}

struct AttnLayout {
    size_t starts, total;
    int QT, NW, RECF;
};

gdn_status attn_layout(const gdn_attn_desc *d, int batch, int rows, int max_blocks, AttnLayout *l)
{
    if (!d || batch < 0 || rows < 1 || rows > kMaxRowsA || max_blocks < 1)
        return GDN_ERR_INVALID_ARG;
    if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->num_q_heads % d->num_kv_heads != 0 ||
        d->page_size < 1 || !(d->scale > 0.0f && d->scale <= 3.0e38f))
        return GDN_ERR_INVALID_ARG;
    if ((d->head_dim != 128 && d->head_dim != 256) || d->page_size % kKeyTile != 0 || d->num_kv_heads > kMaxKvHeads ||
        (d->num_q_heads / d->num_kv_heads) * rows > 16 * kMaxQTiles)
        return GDN_ERR_UNSUPPORTED;
    const size_t maxpos = (size_t)max_blocks * d->page_size;
    if (maxpos > (size_t)1 << 30)
        return GDN_ERR_UNSUPPORTED;
    // every tile index of the batch fits an int
    const size_t pairs = (size_t)batch * d->num_kv_heads;
    const size_t max_tiles = pairs * ((maxpos + kKeyTile - 1) / kKeyTile);
    if (max_tiles > 0x7fffffffu || pairs > 0x7fffffffu)
        return GDN_ERR_UNSUPPORTED;
    const int nq = (d->num_q_heads / d->num_kv_heads) * rows;
    l->QT = (nq + 15) / 16;
    const size_t groups = (max_tiles + kMinGroupTiles - 1) / kMinGroupTiles;
    l->NW = (int)(groups < (size_t)kSplitGroups ? (groups > 0 ? groups : 1) : kSplitGroups);
    l->RECF = l->QT * 16 * (d->head_dim + 2) + 4;
    l->starts = ((size_t)l->NW + pairs) * (size_t)l->RECF * sizeof(float);
    l->total = l->starts + (pairs + 1) * sizeof(int32_t);
    return GDN_OK;
}

bool aligned16a(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Checks that need no scratch, then the launch of both kernels on `buf`.
gdn_status attn_check(const gdn_attn_desc *desc, const void *q, const void *k_cache, const void *v_cache,
                      int32_t num_pages, const int32_t *block_table, const int32_t *seq_lens, void *out)
{
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out || num_pages < 1 || !aligned16a(q) ||
        !aligned16a(k_cache) || !aligned16a(v_cache) || !aligned16a(out))
        return GDN_ERR_INVALID_ARG;
    return GDN_OK;
}

gdn_status attn_launch(const gdn_attn_desc *desc, const AttnLayout &l, const void *q, const void *k_cache,
                       const void *v_cache, int32_t num_pages, const int32_t *block_table, int32_t max_blocks,
                       const int32_t *seq_lens, int32_t batch, int32_t rows, void *buf, void *out,
                       int32_t *err_flag, hipStream_t st)
{
    AttnParams p;
    p.q = static_cast<const uint16_t *>(q);
    p.kc = static_cast<const uint16_t *>(k_cache);
    p.vc = static_cast<const uint16_t *>(v_cache);
    p.bt = block_table;
    p.seq = seq_lens;
    p.rec = static_cast<float *>(buf);
    p.starts = reinterpret_cast<int32_t *>(static_cast<char *>(buf) + l.starts);
    p.out = static_cast<uint16_t *>(out);
    p.err = err_flag;
    p.B = batch;
    p.R = rows;
    p.Hq = desc->num_q_heads;
    p.Hkv = desc->num_kv_heads;
    p.G = desc->num_q_heads / desc->num_kv_heads;
    p.PS = desc->page_size;
    p.TPP = desc->page_size / kKeyTile;
    p.NP = num_pages;
    p.MB = max_blocks;
    p.NQ = p.G * rows;
    p.QT = l.QT;
    p.NW = l.NW;
    p.RECF = l.RECF;
    p.scale = desc->scale;
    const dim3 split_grid((unsigned)l.NW);
    const dim3 combine_grid((unsigned)(batch * p.Hkv), (unsigned)l.QT);
    if (desc->head_dim == 128) {
        hipLaunchKernelGGL(gdn_attn_split_kernel<128>, split_grid, dim3(kThreadsS), 0, st, p);
        hipLaunchKernelGGL(gdn_attn_combine_kernel<128>, combine_grid, dim3(kThreadsC), 0, st, p);
    } else {
        hipLaunchKernelGGL(gdn_attn_split_kernel<256>, split_grid, dim3(kThreadsS), 0, st, p);
        hipLaunchKernelGGL(gdn_attn_combine_kernel<256>, combine_grid, dim3(kThreadsC), 0, st, p);
    }
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// Device address of `scratch` on the device of `st` (the current device for
// the null stream), looked up on the first call on that device with the
// device current, and kept for the life of the process.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

gdn_status static_scratch(hipStream_t st, void **ptr)
{
    int dev = 0;
    if ((st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev)) != hipSuccess)
        return GDN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices)
        return GDN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess)
            return GDN_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess)
            return GDN_ERR_HIP;
        void *addr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (cur != dev)
            (void)hipSetDevice(cur);
        if (e != hipSuccess || !addr)
            return GDN_ERR_HIP;
        g_scratch_ptr[dev] = addr;
    }
    *ptr = g_scratch_ptr[dev];
    return GDN_OK;
}

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
                                int32_t rows, void *scratch_buf, size_t scratch_bytes, void *out,
                                int32_t *err_flag, void *stream)
{
    AttnLayout l;
    gdn_status s = attn_layout(desc, batch, rows, max_blocks, &l);
    if (s != GDN_OK)
        return s;
    if (batch == 0)
        return GDN_OK;
    s = attn_check(desc, q, k_cache, v_cache, num_pages, block_table, seq_lens, out);
    if (s != GDN_OK)
        return s;
    if (!scratch_buf || !aligned16a(scratch_buf))
        return GDN_ERR_INVALID_ARG;
    if (scratch_bytes < l.total)
        return GDN_ERR_SCRATCH_TOO_SMALL;
    return attn_launch(desc, l, q, k_cache, v_cache, num_pages, block_table, max_blocks, seq_lens, batch, rows,
                       scratch_buf, out, err_flag, static_cast<hipStream_t>(stream));
}

gdn_status gdn_spec_attn_verify_static(const gdn_attn_desc *desc, const void *q, const void *k_cache,
                                       const void *v_cache, int32_t num_pages, const int32_t *block_table,
                                       int32_t max_blocks, const int32_t *seq_lens, int32_t batch,
                                       int32_t rows, void *out, int32_t *err_flag, void *stream)
{
    AttnLayout l;
    gdn_status s = attn_layout(desc, batch, rows, max_blocks, &l);
    if (s != GDN_OK)
        return s;
    if (batch == 0)
        return GDN_OK;
    s = attn_check(desc, q, k_cache, v_cache, num_pages, block_table, seq_lens, out);
    if (s != GDN_OK)
        return s;
    if (l.total > GDN_SPEC_ATTN_STATIC_SCRATCH_BYTES)
        return GDN_ERR_SCRATCH_TOO_SMALL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    void *buf = nullptr;
    s = static_scratch(st, &buf);
    if (s != GDN_OK)
        return s;
    return attn_launch(desc, l, q, k_cache, v_cache, num_pages, block_table, max_blocks, seq_lens, batch, rows,
                       buf, out, err_flag, st);
}

}  // extern "C"
