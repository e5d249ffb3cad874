// validate.hpp -- host-side validation shared by the launch code.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "attn.h"

namespace attn {

// The tensors of one call.  Fixed-length batch: Q, O, dO, dQ are
// [B, H, N, d], K, V, dK, dV are [B, H_kv, N, d], lse is [B, H, N]
// (outer = B, rows = max_len = N).  Packed variable-length batch: Q, O, dO,
// dQ are [H, T, d], K, V, dK, dV are [H_kv, T, d], lse is [H, T]
// (outer = n_seqs, rows = T, max_len = the longest sequence).
struct Geometry {
  int64_t outer, H, H_kv, rows, max_len, d;
  bool packed;
  int64_t n_heads() const { return outer * H; }       // query heads of a launch
  int64_t n_kv_heads() const { return outer * H_kv; }
  // Rows of the query side (lse, workspace arrays) and element counts.
  int64_t q_rows() const { return packed ? H * rows : outer * H * rows; }
  int64_t kv_rows() const { return packed ? H_kv * rows : outer * H_kv * rows; }
};

inline Geometry fixed_geometry(int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d) {
  return Geometry{B, H, H_kv, N, N, d, false};
}

struct TensorArgs {
  int dt;
  Geometry g;
  float scale;
  int mode;
  int64_t wl, wr;
  int n_in, n_out;
  const void* in[8];
  uint64_t in_bytes[8];
  unsigned in_align[8];  // required alignment of each input (16 unless set)
  const void* out[8];
  uint64_t out_bytes[8];
};

attn_status check_sizes(int dt, int64_t B, int64_t H, int64_t N, int64_t d);
attn_status check_geometry(int dt, const Geometry& g);
attn_status check_mask(int mode, int64_t wl, int64_t wr);
attn_status check_common(const TensorArgs& a);
// Pointers, mask, scale, alignment and aliasing of a call (check_common
// without the geometry).
attn_status check_buffers(const TensorArgs& a);
// Bytes of one float32 value per row, padded to 256.
inline uint64_t row_array_bytes(int64_t B, int64_t H, int64_t N) {
  const uint64_t rows = static_cast<uint64_t>(B) * H * N;
  return (rows * 4u + 255u) / 256u * 256u;
}
uint64_t workspace_bytes(int64_t B, int64_t H, int64_t N);

// The backward's key-major pass runs one workgroup per (key/value head, key
// block) and walks the query heads of its group.  With few key/value heads
// (multi-query attention) that leaves the chip idle, so the group is split
// into kv_split(g) slices (a divisor of the group), one workgroup each, whose
// fp32 partial dK/dV a reduction sums in slice order.
int64_t kv_split(const Geometry& g);
// Workspace of a backward call: the per-row arrays, then (when split) the
// partial dK and dV, [kv_split][kv rows][d] float32 each.
uint64_t bwd_workspace_bytes(const Geometry& g);

// Validation of a forward / backward call on any geometry (cu_seqlens is
// read only for a packed batch).
attn_status fwd_check_g(int dt, const void* Q, const void* K, const void* V, const void* O,
                        const float* lse, const int32_t* cu_seqlens, const Geometry& g,
                        float scale, int mode, int64_t wl, int64_t wr);
attn_status bwd_check_g(int dt, const void* Q, const void* K, const void* V, const void* O,
                        const float* lse, const void* dO, const void* dQ, const void* dK,
                        const void* dV, const void* ws, size_t ws_bytes,
                        const int32_t* cu_seqlens, const Geometry& g, float scale, int mode,
                        int64_t wl, int64_t wr, bool check_ws = true);

// Split-KV decoding over a paged cache (decode.hpp): validation, and the
// workspace (fp32 partial O and lse per split) it needs.
struct DecodeGeometry {
  int64_t n_seqs, H, H_kv, n_q, d, page_size, n_pages, max_pages, max_seqlen;
};
attn_status decode_sizes(int dt, const DecodeGeometry& g);
uint64_t decode_workspace_bytes(int64_t n_seqs, int64_t H, int64_t H_kv, int64_t n_q, int64_t d,
                                int64_t max_seqlen);
attn_status decode_check(int dt, const void* Q, const void* K, const void* V,
                         const int32_t* block_table, const int32_t* seq_lens, const void* O,
                         const float* lse, const void* ws, size_t ws_bytes,
                         const DecodeGeometry& g, float scale, int mode, int64_t wl, int64_t wr);

attn_status fwd_check(int dt, const void* Q, const void* K, const void* V, const void* O,
                      const float* lse, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                      int mode, int64_t wl, int64_t wr);
attn_status bwd_check(int dt, const void* Q, const void* K, const void* V, const void* O,
                      const float* lse, const void* dO, const void* dQ, const void* dK,
                      const void* dV, const void* ws, size_t ws_bytes, int64_t B, int64_t H,
                      int64_t N, int64_t d, float scale, int mode, int64_t wl, int64_t wr);

}  // namespace attn
