/*
 * attn.h -- C ABI of the MI355X (gfx950) exact-attention library (libattn.so).
 *
 * The library computes exact scaled-dot-product attention with the tiled,
 * online-softmax method (FlashAttention): O = softmax(scale * Q K^T + mask) V,
 * without ever writing the N x N score matrix to device memory, and saves the
 * per-row log-sum-exp so that the backward can rebuild P by recomputation.
 *
 * Sources (cited below as P1..P4 with their sections):
 *   P1  ai6s.net/6af30f4d40858c2d8819b6d5.html -- generic FlashAttention ideas
 *       (tiling §2.2, online softmax §2.3, recomputation §2.4, CUDA teaching
 *       kernel §2.5) and the Ascend NPU implementation (§3).
 *   P2  aicoding.csdn.net/6a69d3ff10ee7a33f2941f44.html -- FlashAttention in
 *       ops-transformer (block loop, online softmax, calling interface,
 *       pitfalls: ragged lengths, causal mask, precision).
 *   P3  jsqmd.com/news/1148352 -- porting FlashAttention (online softmax
 *       state m, l, O_acc §2; head_dim 64/128 and backward notes §4).
 *   P4  ai6s.net/6a0ed07b662f9a54cb761aa2.html -- FlashAttention under the
 *       catlass templates ("usage": mask None / causal / (window_left,
 *       window_right) selecting variants of one kernel).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense and contiguous, layout [B, H, N, d] with d innermost
 *    (P2 memory table; P4 "usage" example tensors), element type `dt`.
 *    lse is dense float32 [B, H, N], natural-log units: lse_i = m_i + ln(l_i)
 *    with m_i the row maximum of scale * q_i . k_j over allowed keys and l_i
 *    the row sum of exp(scale * q_i . k_j - m_i)  (P1 §2.4 keeps m and l).
 *  - Masks (P4 "usage"; bounds are this library's reading, both inclusive):
 *      ATTN_MASK_NONE     every key j < N is allowed;
 *      ATTN_MASK_CAUSAL   key j is allowed for query i iff j <= i;
 *      ATTN_MASK_SLIDING  allowed iff i - window_left <= j <= i + window_right.
 *    Windows are read only for SLIDING, must be >= 0, and values >= N act as
 *    unbounded.  CAUSAL equals SLIDING(N-1, 0); NONE equals SLIDING(N-1, N-1).
 *    Because the diagonal is always allowed, no row is ever empty.
 *  - Supported: dt in {F16, BF16}; d in {64, 128} (P3 §4: the head sizes the
 *    tiling is built for); N >= 1 with one head's rows below 2^31 bytes
 *    (N * d * 2 < 2^31, i.e. N < 8,388,608 at d = 128); B, H >= 1 with
 *    B * H < 2^31 and B * H * N * d / 8 below 2^32 - 2^11 (every launch stays
 *    under 2^32 threads); any finite scale (negative and zero allowed).  Any N is
 *    handled (ragged tails are masked in-kernel, P2 "pitfall 1"), not padded.
 *  - Ownership: the caller allocates and owns every buffer.  The library never
 *    allocates, frees or retains device memory and keeps no state between
 *    calls; it is thread-safe.  Inputs are read only.  Outputs must not overlap
 *    any input or each other (ATTN_E_ALIAS, checked by address range).
 *  - Device pointers must be 16-byte aligned (ATTN_E_ALIGN).  All device
 *    buffers and `stream` must belong to the calling thread's current HIP
 *    device, on which the kernels are launched (the library cannot tell a
 *    host pointer or another device's pointer from a valid one).
 *  - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL is the
 *    default stream) and the call returns without synchronising.
 *  - Errors: every argument is validated on the host before any HIP call; on
 *    any error nothing is launched and no output is written.  A launch failure
 *    reported by the runtime returns ATTN_E_HIP; a fault inside a kernel
 *    surfaces at the caller's next synchronisation.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_dtype {
  ATTN_F16 = 0,  /* IEEE binary16 storage, fp32 accumulation */
  ATTN_BF16 = 1  /* bfloat16 storage, fp32 accumulation */
} attn_dtype;

typedef enum attn_mask_mode {
  ATTN_MASK_NONE = 0,
  ATTN_MASK_CAUSAL = 1,
  ATTN_MASK_SLIDING = 2
} attn_mask_mode;

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_E_NULLPTR = 1,     /* a required pointer is NULL */
  ATTN_E_SHAPE = 2,       /* B, H or N < 1, sizes too large to index, H not a multiple
                             of H_kv, or max_seqlen outside [1, T] */
  ATTN_E_UNSUPPORTED = 3, /* dtype or head size d not supported */
  ATTN_E_MASK = 4,        /* unknown mask mode or negative window */
  ATTN_E_SCALE = 5,       /* scale is NaN or infinite */
  ATTN_E_ALIGN = 6,       /* a device pointer is not 16-byte aligned */
  ATTN_E_ALIAS = 7,       /* an output overlaps an input or another output */
  ATTN_E_WORKSPACE = 8,   /* workspace missing or smaller than required */
  ATTN_E_HIP = 9,         /* the HIP runtime reported an error at launch */
  ATTN_E_SCRATCH = 10     /* attn_bwd_noalloc: the sizes need more than its fixed scratch */
} attn_status;

/*
 * attn_fwd -- forward pass (P1 §2.2 tiling, §2.3 online softmax; P3 §2).
 *
 *   Q, K, V  in:  [B, H, N, d] of `dt`.
 *   O        out: [B, H, N, d] of `dt`, O = P V with P = softmax(scale Q K^T
 *                 + mask) row-wise, rounded once from fp32 to `dt`.
 *   lse      out: [B, H, N] float32, as in the conventions above.
 *   scale    multiplies the scores before the softmax (P1 §1 uses 1/sqrt(d)).
 *   mode, window_left, window_right: the mask, as above.
 *   stream   hipStream_t to enqueue on.
 * Returns ATTN_OK or the first validation error; see the conventions.
 */
attn_status attn_fwd(attn_dtype dt, const void* Q, const void* K, const void* V, void* O,
                     float* lse, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                     attn_mask_mode mode, int64_t window_left, int64_t window_right,
                     void* stream);

/* Size of the fixed device scratch of attn_bwd_noalloc, per GPU. */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * attn_fwd_persistent -- attn_fwd_gqa with persistent scheduling (the pages'
 * AI cores looping over their share of Q blocks, P1 §3.2 and §3.3 "AI Core
 * count"): the grid holds only the workgroups the GPU runs at once, and each
 * claims its next query block from a work queue per accelerator die until
 * none is left, in the same die-local, heaviest-first order as attn_fwd.
 * Same arguments, layouts, results (bit for bit) and errors as attn_fwd_gqa
 * (H_kv = H: standard attention).  The queues are counters inside the
 * library's code object, one set per GPU, which every launch leaves at zero:
 * nothing to allocate or clear, but two attn_fwd_persistent launches must
 * not run at the same time on one GPU (e.g. on two streams).
 */
attn_status attn_fwd_persistent(attn_dtype dt, const void* Q, const void* K, const void* V,
                                void* O, float* lse, int64_t B, int64_t H, int64_t H_kv,
                                int64_t N, int64_t d, float scale, attn_mask_mode mode,
                                int64_t window_left, int64_t window_right, void* stream);

/*
 * attn_bwd_workspace_bytes -- size in bytes of the device workspace attn_bwd
 * needs for these sizes: two float32 values per row (-D_i with
 * D_i = dO_i . O_i, and the row's lse rescaled to the score units the
 * kernels use), each array padded to 256 B.
 * Returns 0 if the sizes are invalid.  Pure host function, no HIP call.
 */
size_t attn_bwd_workspace_bytes(attn_dtype dt, int64_t B, int64_t H, int64_t N, int64_t d);

/*
 * attn_bwd -- recomputation backward (P1 §2.4; P3 §4): rebuilds P tile by
 * tile from the saved lse, never storing it, and returns the exact gradients
 * of O with respect to Q, K and V for the upstream gradient dO:
 *   dV = P^T dO;  dP = dO V^T;  D_i = dO_i . O_i (from the stored O);
 *   dS = P * (dP - D);  dQ = scale dS K;  dK = scale dS^T Q.
 *
 *   Q, K, V, O, dO  in:  [B, H, N, d] of `dt` (O as written by attn_fwd).
 *   lse             in:  [B, H, N] float32 as written by attn_fwd.
 *   dQ, dK, dV      out: [B, H, N, d] of `dt`, fp32-accumulated, rounded once.
 *   workspace       device scratch of at least attn_bwd_workspace_bytes(...)
 *                   bytes, 16-byte aligned, owned by the caller; its contents
 *                   on entry are ignored and on return are unspecified.
 *   Other arguments as for attn_fwd (same scale and mask as the forward).
 * The result is deterministic (no atomics).
 */
attn_status attn_bwd(attn_dtype dt, const void* Q, const void* K, const void* V, const void* O,
                     const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                     void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t N,
                     int64_t d, float scale, attn_mask_mode mode, int64_t window_left,
                     int64_t window_right, void* stream);

/*
 * Grouped-query and variable-length variants (P1 §5 names both among
 * FlashAttention's extensions; the pages give no formulas, so the readings
 * below are this library's).
 *
 * Grouped-query attention (GQA; multi-query attention is H_kv = 1): the H
 * query heads share H_kv key/value heads, H a multiple of H_kv, and query
 * head h reads key/value head h / (H / H_kv) -- consecutive query heads
 * share one.  With H_kv = H these calls equal attn_fwd / attn_bwd.
 *
 * Packed variable-length batch: n_seqs sequences are stored one after the
 * other along the row axis, T rows in all: Q, O (and dO, dQ) are [H, T, d],
 * K, V (and dK, dV) are [H_kv, T, d], lse is [H, T]; sequence s occupies
 * rows [cu_seqlens[s], cu_seqlens[s+1]).  Each sequence attends only to
 * itself, and the mask applies to positions counted from the sequence's
 * first row (causal: key j <= query i within the sequence).
 *   cu_seqlens  in: int32 device array of n_seqs + 1 row offsets, 4-byte
 *               aligned, caller-owned.  The caller guarantees
 *               0 = cu[0] <= cu[1] <= ... <= cu[n_seqs] <= T and
 *               cu[s+1] - cu[s] <= max_seqlen.  These values live on the
 *               device and are not validated; the kernels clamp every
 *               sequence to rows [0, T), so malformed offsets never make
 *               them access memory outside the tensors, but the results for
 *               such offsets are unspecified.  Rows outside every sequence
 *               are not written.  Empty sequences are allowed.
 *   n_seqs      >= 1;  max_seqlen in [1, T];  total = T >= 1.
 * The size rules of the conventions apply with B*H*N replaced by
 * n_seqs*H*max_seqlen for the thread bound and by H*T for the tensor sizes.
 */

/* attn_fwd_gqa -- attn_fwd with K, V of shape [B, H_kv, N, d]. */
attn_status attn_fwd_gqa(attn_dtype dt, const void* Q, const void* K, const void* V, void* O,
                         float* lse, int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                         float scale, attn_mask_mode mode, int64_t window_left,
                         int64_t window_right, void* stream);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc): the same computation with the same kernels, but the workspace
 * is a fixed array of ATTN_NOALLOC_SCRATCH_BYTES inside the library's code
 * object, one per GPU, which the library holds until the process ends.
 *
 *   Arguments as for attn_bwd, without workspace and workspace_bytes; every
 *   buffer still belongs to the caller and to the current device.
 * Validates every argument like attn_bwd, then returns ATTN_E_SCRATCH without
 * launching anything if attn_bwd_workspace_bytes(dt, B, H, N, d) exceeds
 * ATTN_NOALLOC_SCRATCH_BYTES (two float32 values per row: up to 4,194,240
 * rows B*H*N).  Calls no allocating routine; the first call on a device looks
 * up that device's copy of the array (hipGetSymbolAddress), later calls reuse
 * the address.  The array needs no clearing: every value the second kernel
 * reads is written by the first kernel of the same call.  All calls on one GPU
 * share its array, so calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.
 */
attn_status attn_bwd_noalloc(attn_dtype dt, const void* Q, const void* K, const void* V,
                             const void* O, const float* lse, const void* dO, void* dQ, void* dK,
                             void* dV, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                             attn_mask_mode mode, int64_t window_left, int64_t window_right,
                             void* stream);

/*
 * attn_bwd_gqa -- attn_bwd with K, V, dK, dV of shape [B, H_kv, N, d]:
 * dK and dV of a key/value head sum the contributions of all the query
 * heads that read it (deterministic, no atomics: with few key/value heads
 * the query heads of a group are split into slices whose fp32 partial sums
 * are added in a fixed order).  Workspace: attn_bwd_gqa_workspace_bytes.
 */
attn_status attn_bwd_gqa(attn_dtype dt, const void* Q, const void* K, const void* V,
                         const void* O, const float* lse, const void* dO, void* dQ, void* dK,
                         void* dV, void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                         int64_t H_kv, int64_t N, int64_t d, float scale, attn_mask_mode mode,
                         int64_t window_left, int64_t window_right, void* stream);

/* attn_fwd_varlen -- forward over a packed variable-length batch (see above). */
attn_status attn_fwd_varlen(attn_dtype dt, const void* Q, const void* K, const void* V, void* O,
                            float* lse, const int32_t* cu_seqlens, int64_t n_seqs,
                            int64_t max_seqlen, int64_t total, int64_t H, int64_t H_kv,
                            int64_t d, float scale, attn_mask_mode mode, int64_t window_left,
                            int64_t window_right, void* stream);

/*
 * attn_bwd_gqa_workspace_bytes / attn_bwd_varlen_workspace_bytes -- device
 * workspace attn_bwd_gqa / attn_bwd_varlen need: the per-row arrays of
 * attn_bwd plus, when the library splits the query heads of a group, fp32
 * partial dK and dV.  Return 0 for invalid sizes.  Pure host functions.
 */
size_t attn_bwd_gqa_workspace_bytes(attn_dtype dt, int64_t B, int64_t H, int64_t H_kv, int64_t N,
                                    int64_t d);
size_t attn_bwd_varlen_workspace_bytes(attn_dtype dt, int64_t n_seqs, int64_t max_seqlen,
                                       int64_t total, int64_t H, int64_t H_kv, int64_t d);

/* attn_bwd_varlen -- backward over a packed variable-length batch (see above);
 * workspace: attn_bwd_varlen_workspace_bytes. */
attn_status attn_bwd_varlen(attn_dtype dt, const void* Q, const void* K, const void* V,
                            const void* O, const float* lse, const void* dO, void* dQ, void* dK,
                            void* dV, void* workspace, size_t workspace_bytes,
                            const int32_t* cu_seqlens, int64_t n_seqs, int64_t max_seqlen,
                            int64_t total, int64_t H, int64_t H_kv, int64_t d, float scale,
                            attn_mask_mode mode, int64_t window_left, int64_t window_right,
                            void* stream);

/*
 * Split-KV decoding over a paged K/V cache (P1 §5 names split-KV decoding
 * and paged caches among FlashAttention's extensions; the layout is this
 * library's).  Each of n_seqs sequences contributes n_q new query tokens,
 * which sit at the last n_q positions of its cache, and attends to its
 * seq_lens[s] cached keys.
 *
 *   Q            in:  [n_seqs, H, n_q, d] of `dt`.
 *   K_cache, V_cache  in: page pools [n_pages, H_kv, page_size, d] of `dt`;
 *                page_size a multiple of 64.
 *   block_table  in:  int32 [n_seqs, max_pages_per_seq], device, 4-byte
 *                aligned: key j of sequence s is row j % page_size of page
 *                block_table[s][j / page_size].
 *   seq_lens     in:  int32 [n_seqs], device: cache length L_s of each
 *                sequence, with n_q <= L_s <= max_seqlen <= max_pages_per_seq
 *                * page_size.
 *   O            out: [n_seqs, H, n_q, d] of `dt`; lse out: float32
 *                [n_seqs, H, n_q], natural-log units as for attn_fwd.
 *   workspace    device scratch of attn_decode_workspace_bytes(...) bytes
 *                (zero when the keys are not split; then it may be NULL).
 *   Query head h reads key/value head h / (H / H_kv) (grouped-query).
 *   Masks use cache positions: query token i of sequence s is at position
 *   p = L_s - n_q + i; NONE lets it see all L_s keys, CAUSAL keys j <= p,
 *   SLIDING keys p - window_left <= j <= p + window_right.
 * The keys are split over workgroups (chunks of whole 64-key tiles) when the
 * sequences alone do not fill the chip; the partial results are merged by
 * the online-softmax rule.  block_table and seq_lens live on the device and
 * are not validated: lengths are clamped to [0, max_pages_per_seq *
 * page_size] and page numbers to [0, n_pages), so malformed values never
 * make the kernels access memory outside the buffers, but give unspecified
 * results; so does L_s < n_q, or L_s > max_seqlen.  Other rules as in the
 * conventions (ATTN_E_UNSUPPORTED also for page_size).
 */
size_t attn_decode_workspace_bytes(attn_dtype dt, int64_t n_seqs, int64_t H, int64_t H_kv,
                                   int64_t n_q, int64_t d, int64_t max_seqlen);

attn_status attn_decode(attn_dtype dt, const void* Q, const void* K_cache, const void* V_cache,
                        const int32_t* block_table, const int32_t* seq_lens, void* O, float* lse,
                        void* workspace, size_t workspace_bytes, int64_t n_seqs, int64_t H,
                        int64_t H_kv, int64_t n_q, int64_t d, int64_t page_size, int64_t n_pages,
                        int64_t max_pages_per_seq, int64_t max_seqlen, float scale,
                        attn_mask_mode mode, int64_t window_left, int64_t window_right,
                        void* stream);

/* attn_status_str -- static, NUL-terminated description of a status code. */
const char* attn_status_str(attn_status s);

/*
 * Host-only planning queries.  They make no HIP call, need no GPU and exist
 * so that the host logic can be checked on its own.
 */

/* attn_fwd_check -- the exact validation attn_fwd performs, without launching. */
attn_status attn_fwd_check(attn_dtype dt, const void* Q, const void* K, const void* V,
                           const void* O, const float* lse, int64_t B, int64_t H, int64_t N,
                           int64_t d, float scale, attn_mask_mode mode, int64_t window_left,
                           int64_t window_right);

/* attn_bwd_check -- the exact validation attn_bwd performs, without launching. */
attn_status attn_bwd_check(attn_dtype dt, const void* Q, const void* K, const void* V,
                           const void* O, const float* lse, const void* dO, const void* dQ,
                           const void* dK, const void* dV, const void* workspace,
                           size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t d,
                           float scale, attn_mask_mode mode, int64_t window_left,
                           int64_t window_right);

/*
 * attn_fwd_tiles -- the forward's tile shape: *block_q query rows per
 * workgroup (Br) and *block_k key rows per streamed K/V tile (Bc) for head
 * size d and mask mode (P1 §2.2).  Br is 256 without a mask and 128 with a
 * causal or sliding mask; Bc is 64.  Returns ATTN_E_UNSUPPORTED for other d,
 * ATTN_E_MASK for an unknown mode.
 */
attn_status attn_fwd_tiles(int64_t d, attn_mask_mode mode, int64_t* block_q, int64_t* block_k);

/*
 * attn_kv_tile_range -- the half-open range [*lo, *hi) of key tiles (of
 * block_k rows) that the query block [q0, q0 + block_q) visits: every tile
 * holding at least one allowed (query, key) pair of that block and no other
 * (whole-tile skipping for causal and sliding masks, P1 §3.3 key optimisation
 * (4)).  Windows as in the conventions.  Returns ATTN_E_SHAPE / ATTN_E_MASK
 * on invalid arguments.
 */
attn_status attn_kv_tile_range(int64_t N, int64_t q0, int64_t block_q, int64_t block_k,
                               attn_mask_mode mode, int64_t window_left, int64_t window_right,
                               int64_t* lo, int64_t* hi);

/*
 * attn_fwd_workgroup -- which (head index b*H + h, query block) the forward's
 * workgroup `wg` of `n_wg` = B*H*n_qblk processes: workgroups are dealt to the
 * 8 accelerator dies round-robin, so consecutive ids are remapped to keep all
 * query blocks of one head on one die's L2; causal masks also run the longest
 * query blocks first, four heads at a time (the last block of each of the four,
 * then the second-to-last of each, ...).  Returns ATTN_E_SHAPE if wg is out of
 * range.
 */
attn_status attn_fwd_workgroup(int64_t wg, int64_t n_heads, int64_t n_qblk, attn_mask_mode mode,
                               int64_t* head, int64_t* qblk);

/*
 * attn_bwd_kv_workgroup -- which (head index b*H + h, key block) workgroup
 * `wg` of the backward's key-major dK/dV pass (n_wg = B*H*n_kblk) processes
 * for standard multi-head attention.  Workgroups are dealt to the 8
 * accelerator dies round-robin.  With a causal mask and a head count that is
 * a multiple of 32, die x runs the heads h with h % 8 == x, four at a time,
 * each group's heaviest key block (it sees every query tile) first; with a
 * causal mask otherwise the order is key-block-major over all heads;
 * without one it is the forward's head-major order.  Returns ATTN_E_SHAPE if
 * wg is out of range, ATTN_E_MASK for an unknown mode, ATTN_E_NULLPTR for
 * null outputs.
 */
attn_status attn_bwd_kv_workgroup(int64_t wg, int64_t n_heads, int64_t n_kblk,
                                  attn_mask_mode mode, int64_t* head, int64_t* kblk);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
