// plan.hpp -- tile geometry shared by the host planner and the device kernels.
//
// Everything here is plain integer arithmetic on sizes; it is compiled both
// into host code (validation, launch geometry, the host-only query functions)
// and into the kernels, so the two always agree on which key tiles a query
// block visits and which workgroup owns which query block.
//
// Sources: P1 = ai6s.net/6af30f4d40858c2d8819b6d5.html, P4 =
// ai6s.net/6a0ed07b662f9a54cb761aa2.html.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define ATTN_HD __host__ __device__ __forceinline__
#else
#define ATTN_HD inline
#endif

namespace attn {

enum MaskMode : int { kNone = 0, kCausal = 1, kSliding = 2 };

// Forward tile shape: 64-row K/V tiles; workgroups of 32-row wavefronts.
// Without a mask a workgroup has 8 wavefronts (256 query rows) so that each
// K/V tile is fetched once for more rows; with a causal or sliding mask it
// has 4 (128 rows), whose finer work items balance the unequal row lengths
// and waste fewer products on tiles past a wavefront's band.  The three are
// build parameters (ATTN_FWD_BLOCK_K: 32, 64 or 128; ATTN_FWD_WAVES_NONE,
// ATTN_FWD_WAVES_MASKED: 4 or 8) so that the tile-shape sweep can build other
// shapes; the defaults are the ones the sweep chose.
#ifndef ATTN_FWD_BLOCK_K
#define ATTN_FWD_BLOCK_K 64
#endif
#ifndef ATTN_FWD_WAVES_NONE
#define ATTN_FWD_WAVES_NONE 8
#endif
#ifndef ATTN_FWD_WAVES_MASKED
#define ATTN_FWD_WAVES_MASKED 4
#endif
static_assert(ATTN_FWD_BLOCK_K == 32 || ATTN_FWD_BLOCK_K == 64 || ATTN_FWD_BLOCK_K == 128,
              "key tile of 32, 64 or 128 rows");
static_assert((ATTN_FWD_WAVES_NONE == 4 || ATTN_FWD_WAVES_NONE == 8) &&
                  (ATTN_FWD_WAVES_MASKED == 4 || ATTN_FWD_WAVES_MASKED == 8),
              "4 or 8 wavefronts per workgroup");
constexpr int kFwdBlockK = ATTN_FWD_BLOCK_K;
ATTN_HD constexpr int fwd_waves(int mode) {
  return mode == 0 ? ATTN_FWD_WAVES_NONE : ATTN_FWD_WAVES_MASKED;
}
ATTN_HD constexpr int fwd_block_q(int mode) { return 32 * fwd_waves(mode); }

// Backward: the dQ pass mirrors the forward (query-major); the dK/dV pass is
// key-major with 4 wavefronts x 64 key rows and 64-row query tiles.
constexpr int kBwdDqBlockQ = 128;
constexpr int kBwdDqBlockK = 64;
constexpr int kBwdKvBlockK = 256;
constexpr int kBwdKvBlockQ = 64;
constexpr int kBwdThreads = 256;

constexpr int kNumXcd = 8;  // accelerator dies per MI355X, each with its own L2

ATTN_HD int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
ATTN_HD int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }
ATTN_HD int64_t imax(int64_t a, int64_t b) { return a > b ? a : b; }

// The allowed key interval [klo, khi) of the query rows [q0, q1) (q1 clipped
// to N): its union over the rows, per mask rule (P4 "usage" variants; the
// bounds are the inclusive reading documented in attn.h).  Windows must be
// clipped to [0, N] by the caller.
ATTN_HD void allowed_key_hull(int64_t N, int64_t q0, int64_t q1, int mode, int64_t wl, int64_t wr,
                              int64_t* klo, int64_t* khi) {
  q1 = imin(q1, N);
  int64_t lo = 0, hi = N;
  if (mode == kCausal) {
    hi = q1;  // last query q1-1 sees keys <= q1-1
  } else if (mode == kSliding) {
    lo = imax(0, q0 - wl);
    hi = imin(N, q1 - 1 + wr + 1);
  }
  *klo = lo;
  *khi = hi;
}

// Key tiles [lo, hi) of block_k rows that query rows [q0, q0 + block_q) visit
// (whole-tile skipping, P1 §3.3 optimisation (4)).  Every tile in range holds
// at least one allowed pair: the hull is an interval of allowed keys.
ATTN_HD void kv_tile_range(int64_t N, int64_t q0, int64_t block_q, int64_t block_k, int mode,
                           int64_t wl, int64_t wr, int64_t* lo, int64_t* hi) {
  int64_t klo, khi;
  allowed_key_hull(N, q0, q0 + block_q, mode, wl, wr, &klo, &khi);
  *lo = klo / block_k;
  *hi = ceil_div(khi, block_k);
}

// Query tiles [lo, hi) of block_q rows that key rows [k0, k0 + block_k) are
// visited by (the backward's key-major loop).  Mirror of kv_tile_range.
ATTN_HD void q_tile_range(int64_t N, int64_t k0, int64_t block_k, int64_t block_q, int mode,
                          int64_t wl, int64_t wr, int64_t* lo, int64_t* hi) {
  int64_t k1 = imin(k0 + block_k, N);
  int64_t qlo = 0, qhi = N;
  if (mode == kCausal) {
    qlo = k0;  // key k is seen by queries >= k
  } else if (mode == kSliding) {
    qlo = imax(0, k0 - wr);            // query i sees j iff j - wr <= i <= j + wl
    qhi = imin(N, k1 - 1 + wl + 1);
  }
  *lo = qlo / block_q;
  *hi = ceil_div(qhi, block_q);
}

// True if every (query, key) pair of query rows [q0, q0 + nq) x key rows
// [k0, k0 + nk) is allowed and every key is < N, so the tile needs no mask.
// Query rows >= N are padding whose results are never stored.
ATTN_HD bool tile_all_allowed(int64_t N, int64_t q0, int64_t nq, int64_t k0, int64_t nk, int mode,
                              int64_t wl, int64_t wr) {
  if (k0 + nk > N) return false;
  int64_t qlast = imin(q0 + nq, N) - 1;
  if (mode == kCausal) return k0 + nk - 1 <= q0;
  if (mode == kSliding) return k0 >= qlast - wl && k0 + nk - 1 <= q0 + wr;
  return true;
}

// True if no pair of query rows [q0, q0 + nq) x key rows [k0, k0 + nk) is
// allowed (a wavefront can then skip its share of the tile).
ATTN_HD bool tile_none_allowed(int64_t N, int64_t q0, int64_t nq, int64_t k0, int64_t nk, int mode,
                               int64_t wl, int64_t wr) {
  if (q0 >= N || k0 >= N) return true;
  int64_t qlast = imin(q0 + nq, N) - 1;
  int64_t klast = imin(k0 + nk, N) - 1;
  if (mode == kCausal) return k0 > qlast;
  if (mode == kSliding) return k0 > qlast + wr || klast < q0 - wl;
  return false;
}

// Query heads and their rows.  A launch's query heads are numbered
// x = outer * H + h, where outer is the batch index (fixed-length batches,
// [B, H, N, d]) or the sequence index (packed variable-length batches,
// [H, T, d]), and h the query head.  Query head h reads key/value head
// h / group (group = H / H_kv query heads share one; group = 1 is standard
// multi-head attention, H_kv = 1 multi-query attention), so a fixed-length
// query head x = b*H + h reads key/value head b*H_kv + h/group, and the
// query heads of one key/value head are consecutive.  q_row0 / kv_row0 are
// the indices of the head's first row in the [rows, d] view of the query
// side (Q, O, dO, dQ and the per-row lse and workspace arrays) and of the
// key/value side (K, V, dK, dV); len is the head's row count.  For a packed
// batch, seq_lo/seq_hi are the sequence's row offsets, which the caller
// supplies and which are clamped here to 0 <= seq_lo <= seq_hi <= rows, so
// a head never reaches outside its tensors whatever the offsets hold.
struct HeadRows {
  int64_t q_row0, kv_row0, len;
};

// The index arithmetic is a template on the integer type: the host checks use
// int64_t, the kernels uint32_t (all indices are below 2^31 after
// validation; 32-bit divisions are far shorter on the GPU than 64-bit ones,
// whose code measurably slowed the whole kernel).  Row offsets are 64-bit.
template <typename I>
ATTN_HD HeadRows query_head_rows(I x, I H, I group, I rows, bool packed, int64_t seq_lo,
                                 int64_t seq_hi) {
  const I outer = x / H, h = x - outer * H, kvh = h / group, H_kv = H / group;
  HeadRows r;
  if (!packed) {
    r.q_row0 = static_cast<int64_t>(x) * rows;
    r.kv_row0 = (static_cast<int64_t>(outer) * H_kv + kvh) * rows;
    r.len = rows;
  } else {
    const int64_t lo = imin(imax(seq_lo, 0), rows);
    const int64_t hi = imin(imax(seq_hi, lo), rows);
    r.q_row0 = static_cast<int64_t>(h) * rows + lo;
    r.kv_row0 = static_cast<int64_t>(kvh) * rows + lo;
    r.len = hi - lo;
  }
  return r;
}

// Key/value head y = outer * H_kv + kvh of the backward's key-major pass and
// its group of query heads: query head kvh*group + g (g < group) starts at
// row q_row0 + g * q_stride of the query side.
struct KvHeadRows {
  int64_t kv_row0, q_row0, q_stride, len;
};

template <typename I>
ATTN_HD KvHeadRows kv_head_rows(I y, I H_kv, I group, I rows, bool packed, int64_t seq_lo,
                                int64_t seq_hi) {
  const I outer = y / H_kv, kvh = y - outer * H_kv, H = H_kv * group;
  KvHeadRows r;
  if (!packed) {
    r.kv_row0 = static_cast<int64_t>(y) * rows;
    r.q_row0 = (static_cast<int64_t>(outer) * H + static_cast<int64_t>(kvh) * group) * rows;
    r.q_stride = rows;
    r.len = rows;
  } else {
    const int64_t lo = imin(imax(seq_lo, 0), rows);
    const int64_t hi = imin(imax(seq_hi, lo), rows);
    r.kv_row0 = static_cast<int64_t>(kvh) * rows + lo;
    r.q_row0 = static_cast<int64_t>(kvh) * group * rows + lo;
    r.q_stride = rows;
    r.len = hi - lo;
  }
  return r;
}

// Workgroup id -> work item.  The hardware deals consecutive workgroup ids
// round-robin to the kNumXcd dies; this bijection gives die x a contiguous
// run of work items, so all query blocks of a head share one die's L2.
template <typename I>
ATTN_HD I xcd_remap(I wg, I n_wg) {
  const I per = n_wg / kNumXcd, rem = n_wg % kNumXcd;
  const I xcd = wg % kNumXcd, slot = wg / kNumXcd;
  const I start = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return start + slot;
}

// Work item -> (head, query block).  With a causal mask the query blocks run
// last-first (they visit the most key tiles, so starting them first shortens
// the tail of the launch), over ATTN_FWD_CAUSAL_CHUNK consecutive heads (of
// one die's run) at a time: the last blocks of the chunk's heads, then their
// second-to-last blocks, and so on.  One head at a time left the long blocks
// of a die's last head to finish alone (a tail of about a tenth of the
// launch at 16 heads of 32 blocks per die and 64 workgroup slots); chunks of
// 4 heads measured 2-7% faster on causal forwards at N = 4096..16384, chunks
// of 8 or 16 up to 20% slower at long N (more distinct K/V per die's L2).
#ifndef ATTN_FWD_CAUSAL_CHUNK
#define ATTN_FWD_CAUSAL_CHUNK 4
#endif
constexpr int kFwdCausalChunk = ATTN_FWD_CAUSAL_CHUNK;
template <typename I>
ATTN_HD void fwd_work_item(I wg, I n_heads, I n_qblk, int mode, I* head, I* qblk) {
  const I item = xcd_remap<I>(wg, n_heads * n_qblk);
  if (mode != kCausal) {
    *head = item / n_qblk;
    *qblk = item - *head * n_qblk;
    return;
  }
  const I C = static_cast<I>(kFwdCausalChunk), per = C * n_qblk;
  const I c = item / per, r = item - c * per, h0 = c * C;
  const I nh = n_heads - h0 < C ? n_heads - h0 : C;  // the last chunk may be short
  const I rank = r / nh;
  *head = h0 + (r - rank * nh);
  *qblk = n_qblk - 1 - rank;
}

// Work item -> (head x = s * heads + h, block) for a packed variable-length
// batch of n_seqs sequences with `heads` heads each and n_blk blocks of the
// longest sequence.  Work per head varies with its sequence's length, so the
// equal-count runs of xcd_remap would leave the dies unevenly loaded.  With
// `heads` a multiple of kNumXcd, die x instead takes heads
// [x * heads/8, (x+1) * heads/8) of every sequence -- every die gets the same
// share of every sequence, and query heads that read one key/value head stay
// on one die's L2 -- and runs its items block by block, heaviest first:
// descending block index (a causal query block's work grows with its index,
// and without a mask only long sequences have high indices), or ascending
// when `ascending` (a causal key block's work shrinks with its index).  For
// other head counts the order is the same block by block, over all heads,
// dealt round-robin to the dies.
template <typename I>
ATTN_HD void packed_work_item(I wg, I heads, I n_seqs, I n_blk, bool ascending, I* head, I* blk) {
  const I per_blk = heads * n_seqs;
  I b, s, h;
  if (heads % kNumXcd == 0) {
    const I hp = heads / kNumXcd, xcd = wg % kNumXcd, slot = wg / kNumXcd;
    b = slot / (hp * n_seqs);
    const I rem = slot - b * (hp * n_seqs);
    s = rem / hp;
    h = xcd * hp + (rem - s * hp);
  } else {
    b = wg / per_blk;
    const I rem = wg - b * per_blk;
    s = rem / heads;
    h = rem - s * heads;
  }
  *head = s * heads + h;
  *blk = ascending ? b : n_blk - 1 - b;
}

// Work item -> (head, key block) of the backward's key-major pass.  Under a
// causal mask key block b sees every query tile from b on, so block 0 does
// up to 16 times the work of the last one at N = 4096: the order runs the
// heaviest blocks first.  Consecutive ids go to the dies in turn.  For
// standard multi-head attention (`grouped`) with the head count a multiple
// of kNumXcd * kBwdKvHeadGroup, die x takes the heads h with
// h % kNumXcd == x, kBwdKvHeadGroup of them at a time, block-major (heaviest
// block first) within each group, so that the workgroups running on a die
// at once read the Q/dO tiles of a few heads (+1.9% at B8 H40 N4096, groups
// of 4; groups of 1 and 2 measured -1.7% and 0%, and with key/value heads
// shared by several query heads grouping lost 0.6-18%).  Otherwise the order
// is block-major over all heads, with id % n_heads = head (which keeps a
// head on one die when the head count is a multiple of kNumXcd).
// Other masks give every key block about the same work and keep the
// head-major order of fwd_work_item, where the blocks of a head run side by
// side and share its streamed Q/dO tiles in L2.
constexpr int kBwdKvHeadGroup = 4;
template <typename I>
ATTN_HD void kv_work_item(I wg, I n_heads, I n_kblk, int mode, I* head, I* kblk,
                          bool grouped = true) {
  if (mode == kCausal) {
    const I G = static_cast<I>(kBwdKvHeadGroup);
    if (grouped && n_heads % (kNumXcd * G) == 0) {
      const I x = wg % kNumXcd, s = wg / kNumXcd;
      const I per_group = G * n_kblk;
      const I grp = s / per_group, r = s - grp * per_group;
      const I kb = r / G;
      *kblk = kb;
      *head = x + kNumXcd * (grp * G + (r - kb * G));
      return;
    }
    *kblk = wg / n_heads;
    *head = wg - *kblk * n_heads;
  } else {
    fwd_work_item<I>(wg, n_heads, n_kblk, kNone, head, kblk);
  }
}

}  // namespace attn
