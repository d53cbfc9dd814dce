/*
 * spec_attention.h -- C ABI of the verification attention in libgdn_spec.so:
 * the full-attention layers of a hybrid model score the same k+1 verify rows
 * as its GatedDeltaNet layers, against each request's KV cache kept in pages
 * (lmdeploy PR #5006, What's included, Verification path: dedicated
 * verification attention kernels over paged KV, with a cross-workgroup
 * reduce).
 *
 * For request b with seq_len L (keys and values of all L positions already
 * in the cache, the verify rows' own at positions L-rows .. L-1), verify row t
 * and query head h:
 *     o[b][t][h] = sum_{p <= L-rows+t} softmax_p(scale * q[b][t][h] . k_p) v_p
 * where k_p, v_p are KV head h / (Hq/Hkv) at position p, found in page
 * block_table[b][p / page_size], slot p % page_size. Readings the page leaves
 * open: causal within the verify rows (row t sees what decoding would), the
 * contiguous query-head groups, and seq_len 0 for a padding request.
 *
 * Inputs are bf16 with fp32 arithmetic: scores and softmax in fp32, the
 * probabilities rounded to bf16 for the product with V, fp32 accumulation,
 * o rounded once to bf16 (nearest, ties to even).
 *
 * Ownership as for gdn_spec.h: the caller allocates every buffer (device
 * memory), the library allocates nothing, keeps no state, never
 * synchronises and never reads device memory on the host; all work is
 * enqueued on `stream`.
 */
#ifndef SPEC_ATTENTION_H
#define SPEC_ATTENTION_H

#include <stddef.h>
#include <stdint.h>

#include "gdn_spec.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t num_q_heads;    /* Hq */
    int32_t num_kv_heads;   /* Hkv, dividing Hq, at most 1024; (Hq/Hkv) * rows <= 128 */
    int32_t head_dim;       /* D: 128 or 256 */
    int32_t page_size;      /* positions per page: a multiple of 32 */
    float scale;            /* score scale, finite and > 0; usually 1/sqrt(D) */
} gdn_attn_desc;

/* Scratch bytes gdn_spec_attn_verify needs for this batch: the per-split
 * partial results of the cross-workgroup reduce. */
gdn_status gdn_spec_attn_scratch_bytes(const gdn_attn_desc *desc, int32_t batch, int32_t rows,
                                       int32_t max_blocks, size_t *bytes);

/*
 * Verification attention of `rows` rows (1..9) of `batch` requests.
 *  q            bf16 [batch][rows][Hq][D], 16-byte aligned
 *  k_cache      bf16 [num_pages][page_size][Hkv][D], 16-byte aligned
 *  v_cache      bf16 [num_pages][page_size][Hkv][D], 16-byte aligned
 *  block_table  int32 [batch][max_blocks]: page of each block of each request
 *  seq_lens     int32 [batch]: positions in the cache including the verify
 *               rows, in [rows, max_blocks * page_size]; 0 = padding
 *  scratch      scratch_bytes >= gdn_spec_attn_scratch_bytes(), 16-byte aligned
 *  out          bf16 [batch][rows][Hq][D], 16-byte aligned (zeros for padding and
 *               refused requests)
 *  err_flag     int32, nullable: bit 0 is OR-ed in when a page id is outside
 *               [0, num_pages), bit 2 when a seq_len is outside the range
 *               above; that request's output is zero.
 * Host-checkable problems return a status before any launch.
 */
gdn_status gdn_spec_attn_verify(const gdn_attn_desc *desc, const void *q, const void *k_cache,
                                const void *v_cache, int32_t num_pages, const int32_t *block_table,
                                int32_t max_blocks, const int32_t *seq_lens, int32_t batch,
                                int32_t rows, void *scratch, size_t scratch_bytes, void *out,
                                int32_t *err_flag, void *stream);

/*
 * gdn_spec_attn_verify with no scratch argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc. It allocates nothing and calls no
 * allocating routine. The partial results go to a file-scope device array of
 * GDN_SPEC_ATTN_STATIC_SCRATCH_BYTES (64 MiB) that every GPU the library runs
 * on holds until the process ends; its address is looked up on the first call
 * on each device. Nothing in it needs to start at zero: each call writes every
 * record it reads back.
 *
 * A call whose gdn_spec_attn_scratch_bytes() exceeds the array returns
 * GDN_ERR_SCRATCH_TOO_SMALL before anything is launched; all other arguments,
 * results and errors are those of gdn_spec_attn_verify. Every call on one GPU
 * uses that GPU's array and leaves the last call's contents in it: calls that
 * may overlap on one GPU (other streams, other host threads) race and must be
 * ordered by the caller. GDN_ERR_HIP if the array's address cannot be found.
 */
#define GDN_SPEC_ATTN_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

gdn_status gdn_spec_attn_verify_static(const gdn_attn_desc *desc, const void *q, const void *k_cache,
                                       const void *v_cache, int32_t num_pages, const int32_t *block_table,
                                       int32_t max_blocks, const int32_t *seq_lens, int32_t batch,
                                       int32_t rows, void *out, int32_t *err_flag, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_ATTENTION_H */
