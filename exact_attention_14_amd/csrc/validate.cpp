// validate.cpp -- host-only part of the C ABI: argument validation, status
// strings, workspace sizing and the planning queries declared in attn.h.
// Makes no HIP call; builds with any C++17 compiler (also the sanitizer build).
#include <cmath>
#include <cstdint>
#include <cstring>

#include "attn.h"
#include "decode.hpp"
#include "plan.hpp"
#include "validate.hpp"

namespace attn {
namespace {

constexpr int64_t kMaxI32 = 2147483647;

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

Range range_of(const void* p, uint64_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

}  // namespace

attn_status check_geometry(int dt, const Geometry& g) {
  if (dt != ATTN_F16 && dt != ATTN_BF16) return ATTN_E_UNSUPPORTED;
  if (g.d != 64 && g.d != 128) return ATTN_E_UNSUPPORTED;
  if (g.outer < 1 || g.H < 1 || g.H_kv < 1 || g.rows < 1 || g.max_len < 1) return ATTN_E_SHAPE;
  // Kernels index heads, rows and workgroups with 32-bit integers and
  // element offsets with 64-bit ones.
  if (g.outer > kMaxI32 || g.H > kMaxI32 || g.rows > kMaxI32) return ATTN_E_SHAPE;
  // Query heads share key/value heads in equal groups.
  if (g.H_kv > g.H || g.H % g.H_kv != 0) return ATTN_E_SHAPE;
  if (g.max_len > g.rows) return ATTN_E_SHAPE;
  if (g.outer * g.H > kMaxI32) return ATTN_E_SHAPE;
  // One head's rows are addressed through 32-bit buffer offsets.
  if (g.rows * g.d * 2 > kMaxI32) return ATTN_E_SHAPE;
  const int64_t heads = g.packed ? g.H : g.outer * g.H;
  if (heads > (int64_t(1) << 62) / (g.rows * g.d * 4)) return ATTN_E_SHAPE;
  // Grids: one workgroup per (head, 64-row block) at most, and at most 2^32
  // threads per launch (bounded as if every launch used d/8 threads per row
  // of the longest sequence).
  const int64_t nh = g.n_heads();
  if (nh * ceil_div(g.max_len, 64) > kMaxI32) return ATTN_E_SHAPE;
  if (nh * g.max_len > (int64_t(1) << 32) / (g.d / 8) - 256) return ATTN_E_SHAPE;
  return ATTN_OK;
}

attn_status check_sizes(int dt, int64_t B, int64_t H, int64_t N, int64_t d) {
  return check_geometry(dt, fixed_geometry(B, H, H, N, d));
}

attn_status check_mask(int mode, int64_t wl, int64_t wr) {
  if (mode != ATTN_MASK_NONE && mode != ATTN_MASK_CAUSAL && mode != ATTN_MASK_SLIDING)
    return ATTN_E_MASK;
  if (mode == ATTN_MASK_SLIDING && (wl < 0 || wr < 0)) return ATTN_E_MASK;
  return ATTN_OK;
}

attn_status check_common(const TensorArgs& a) {
  attn_status s = check_geometry(a.dt, a.g);
  if (s != ATTN_OK) return s;
  return check_buffers(a);
}

attn_status check_buffers(const TensorArgs& a) {
  attn_status s;
  for (int i = 0; i < a.n_in; ++i)
    if (a.in[i] == nullptr) return ATTN_E_NULLPTR;
  for (int i = 0; i < a.n_out; ++i)
    if (a.out[i] == nullptr) return ATTN_E_NULLPTR;
  s = check_mask(a.mode, a.wl, a.wr);
  if (s != ATTN_OK) return s;
  if (!std::isfinite(a.scale)) return ATTN_E_SCALE;
  for (int i = 0; i < a.n_in; ++i)
    if (a.in_align[i] == 4 ? !aligned4(a.in[i]) : !aligned16(a.in[i])) return ATTN_E_ALIGN;
  for (int i = 0; i < a.n_out; ++i)
    if (!aligned16(a.out[i])) return ATTN_E_ALIGN;
  Range in_r[8], out_r[8];
  for (int i = 0; i < a.n_in; ++i) in_r[i] = range_of(a.in[i], a.in_bytes[i]);
  for (int i = 0; i < a.n_out; ++i) out_r[i] = range_of(a.out[i], a.out_bytes[i]);
  for (int o = 0; o < a.n_out; ++o) {
    for (int i = 0; i < a.n_in; ++i)
      if (overlap(out_r[o], in_r[i])) return ATTN_E_ALIAS;
    for (int p = 0; p < o; ++p)
      if (overlap(out_r[o], out_r[p])) return ATTN_E_ALIAS;
  }
  return ATTN_OK;
}

// Two float32 arrays of one value per row, each padded to 256 bytes: -D_i
// and the row's score offset -lse_i * log2(e) / c (see BwdParams).
uint64_t workspace_bytes(int64_t B, int64_t H, int64_t N) {
  return 2u * row_array_bytes(B, H, N);
}

int64_t kv_split(const Geometry& g) {
  const int64_t group = g.H / g.H_kv;
  if (group == 1) return 1;
  // Key blocks that hold rows (for a packed batch at least the total rows'
  // worth) times key/value heads; aim for two workgroups per compute unit.
  constexpr int64_t kTarget = 512;
  const int64_t blocks = g.packed ? ceil_div(g.rows, kBwdKvBlockK) * g.H_kv
                                  : g.outer * g.H_kv * ceil_div(g.rows, kBwdKvBlockK);
  for (int64_t s = 1; s < group; ++s)
    if (group % s == 0 && blocks * s >= kTarget) return s;
  return group;
}

uint64_t bwd_workspace_bytes(const Geometry& g) {
  const uint64_t rows = 2u * row_array_bytes(1, 1, g.q_rows());
  const int64_t split = kv_split(g);
  if (split == 1) return rows;
  return rows + 2u * static_cast<uint64_t>(split) * g.kv_rows() * g.d * 4u;
}

namespace {

// Tensor sizes of a call: query side, key/value side, per-row float32.
struct Sizes {
  uint64_t q, kv, rows;
};

Sizes sizes_of(const Geometry& g) {
  return Sizes{static_cast<uint64_t>(g.q_rows()) * g.d * 2u,
               static_cast<uint64_t>(g.kv_rows()) * g.d * 2u,
               static_cast<uint64_t>(g.q_rows()) * 4u};
}

TensorArgs base_args(int dt, const Geometry& g, float scale, int mode, int64_t wl, int64_t wr) {
  TensorArgs a{};
  a.dt = dt; a.g = g; a.scale = scale;
  a.mode = mode; a.wl = wl; a.wr = wr;
  for (int i = 0; i < 8; ++i) a.in_align[i] = 16;
  return a;
}

// The packed batch's row offsets join the inputs (int32, 4-byte aligned).
void add_offsets(TensorArgs& a, const int32_t* cu_seqlens) {
  if (!a.g.packed) return;
  a.in[a.n_in] = cu_seqlens;
  a.in_bytes[a.n_in] = static_cast<uint64_t>(a.g.outer + 1) * 4u;
  a.in_align[a.n_in] = 4;
  ++a.n_in;
}

}  // namespace

attn_status fwd_check_g(int dt, const void* Q, const void* K, const void* V, const void* O,
                        const float* lse, const int32_t* cu_seqlens, const Geometry& g,
                        float scale, int mode, int64_t wl, int64_t wr) {
  attn_status s = check_geometry(dt, g);
  if (s != ATTN_OK) return s;
  const Sizes z = sizes_of(g);
  TensorArgs a = base_args(dt, g, scale, mode, wl, wr);
  a.n_in = 3;
  a.in[0] = Q; a.in[1] = K; a.in[2] = V;
  a.in_bytes[0] = z.q; a.in_bytes[1] = a.in_bytes[2] = z.kv;
  add_offsets(a, cu_seqlens);
  a.n_out = 2;
  a.out[0] = O; a.out[1] = lse;
  a.out_bytes[0] = z.q; a.out_bytes[1] = z.rows;
  return check_common(a);
}

attn_status bwd_check_g(int dt, const void* Q, const void* K, const void* V, const void* O,
                        const float* lse, const void* dO, const void* dQ, const void* dK,
                        const void* dV, const void* ws, size_t ws_bytes,
                        const int32_t* cu_seqlens, const Geometry& g, float scale, int mode,
                        int64_t wl, int64_t wr, bool check_ws) {
  attn_status s = check_geometry(dt, g);
  if (s != ATTN_OK) return s;
  const Sizes z = sizes_of(g);
  const uint64_t wb = bwd_workspace_bytes(g);
  TensorArgs a = base_args(dt, g, scale, mode, wl, wr);
  a.n_in = 6;
  a.in[0] = Q; a.in[1] = K; a.in[2] = V; a.in[3] = O; a.in[4] = lse; a.in[5] = dO;
  a.in_bytes[0] = a.in_bytes[3] = a.in_bytes[5] = z.q;
  a.in_bytes[1] = a.in_bytes[2] = z.kv;
  a.in_bytes[4] = z.rows;
  add_offsets(a, cu_seqlens);
  a.n_out = check_ws ? 4 : 3;
  a.out[0] = dQ; a.out[1] = dK; a.out[2] = dV; a.out[3] = ws;
  a.out_bytes[0] = z.q;
  a.out_bytes[1] = a.out_bytes[2] = z.kv;
  a.out_bytes[3] = wb;
  s = check_common(a);
  if (s != ATTN_OK) return s;
  if (check_ws && ws_bytes < wb) return ATTN_E_WORKSPACE;
  return ATTN_OK;
}

attn_status decode_sizes(int dt, const DecodeGeometry& g) {
  if (dt != ATTN_F16 && dt != ATTN_BF16) return ATTN_E_UNSUPPORTED;
  if (g.d != 64 && g.d != 128) return ATTN_E_UNSUPPORTED;
  // Pages hold whole 64-key tiles.
  if (g.page_size < kDecTileK || g.page_size % kDecTileK != 0) return ATTN_E_UNSUPPORTED;
  if (g.n_seqs < 1 || g.H < 1 || g.H_kv < 1 || g.n_q < 1 || g.n_pages < 1 || g.max_pages < 1 ||
      g.max_seqlen < 1)
    return ATTN_E_SHAPE;
  if (g.n_seqs > kMaxI32 || g.H > kMaxI32 || g.n_q > kMaxI32 || g.page_size > kMaxI32 ||
      g.n_pages > kMaxI32 || g.max_pages > kMaxI32)
    return ATTN_E_SHAPE;
  if (g.H_kv > g.H || g.H % g.H_kv != 0) return ATTN_E_SHAPE;
  // Positions within a sequence are 32-bit; the longest sequence fits its pages.
  if (g.max_pages > kMaxI32 / g.page_size) return ATTN_E_SHAPE;
  if (g.max_seqlen > g.max_pages * g.page_size) return ATTN_E_SHAPE;
  if (g.n_seqs > kMaxI32 / g.max_pages) return ATTN_E_SHAPE;
  // Tensor sizes stay far below 2^62 bytes.
  const int64_t group = g.H / g.H_kv;
  if (g.n_seqs * g.H > kMaxI32 / g.n_q) return ATTN_E_SHAPE;
  if (g.n_pages > (int64_t(1) << 62) / (g.H_kv * g.page_size * g.d * 2)) return ATTN_E_SHAPE;
  // Grid of the decode launch and thread count of the combine launch.
  const int64_t rt = dec_row_tiles(group, g.n_q);
  int64_t n_splits, chunk;
  dec_plan(g.n_seqs, g.H_kv, rt, g.max_seqlen, &n_splits, &chunk);
  if (g.n_seqs * g.H_kv * rt > kMaxI32 / n_splits) return ATTN_E_SHAPE;
  if (g.n_seqs * g.H_kv * rt * kDecRows * (g.d / 8) > (int64_t(1) << 32) - 256) return ATTN_E_SHAPE;
  return ATTN_OK;
}

uint64_t decode_workspace_bytes(int64_t n_seqs, int64_t H, int64_t H_kv, int64_t n_q, int64_t d,
                                int64_t max_seqlen) {
  const int64_t rt = dec_row_tiles(H / H_kv, n_q);
  int64_t n_splits, chunk;
  dec_plan(n_seqs, H_kv, rt, max_seqlen, &n_splits, &chunk);
  if (n_splits == 1) return 0;
  const uint64_t parts = static_cast<uint64_t>(n_seqs) * H_kv * rt * n_splits;
  // partial O [parts][32][d], then partial lse [parts][32], 256-byte aligned
  const uint64_t o_bytes = (parts * kDecRows * d * 4u + 255u) / 256u * 256u;
  return o_bytes + parts * kDecRows * 4u;
}

attn_status decode_check(int dt, const void* Q, const void* K, const void* V,
                         const int32_t* block_table, const int32_t* seq_lens, const void* O,
                         const float* lse, const void* ws, size_t ws_bytes,
                         const DecodeGeometry& g, float scale, int mode, int64_t wl, int64_t wr) {
  attn_status s = decode_sizes(dt, g);
  if (s != ATTN_OK) return s;
  const uint64_t q_bytes = static_cast<uint64_t>(g.n_seqs) * g.H * g.n_q * g.d * 2u;
  const uint64_t pool_bytes = static_cast<uint64_t>(g.n_pages) * g.H_kv * g.page_size * g.d * 2u;
  const uint64_t wb = decode_workspace_bytes(g.n_seqs, g.H, g.H_kv, g.n_q, g.d, g.max_seqlen);
  TensorArgs a{};
  a.dt = dt; a.scale = scale; a.mode = mode; a.wl = wl; a.wr = wr;
  for (int i = 0; i < 8; ++i) a.in_align[i] = 16;
  a.n_in = 5;
  a.in[0] = Q; a.in[1] = K; a.in[2] = V; a.in[3] = block_table; a.in[4] = seq_lens;
  a.in_bytes[0] = q_bytes; a.in_bytes[1] = a.in_bytes[2] = pool_bytes;
  a.in_bytes[3] = static_cast<uint64_t>(g.n_seqs) * g.max_pages * 4u;
  a.in_bytes[4] = static_cast<uint64_t>(g.n_seqs) * 4u;
  a.in_align[3] = a.in_align[4] = 4;
  a.n_out = 2;
  a.out[0] = O; a.out[1] = lse;
  a.out_bytes[0] = q_bytes;
  a.out_bytes[1] = static_cast<uint64_t>(g.n_seqs) * g.H * g.n_q * 4u;
  if (wb > 0) {  // the workspace is read only when the keys are split
    a.out[2] = ws;
    a.out_bytes[2] = wb;
    a.n_out = 3;
  }
  s = check_buffers(a);
  if (s != ATTN_OK) return s;
  if (ws_bytes < wb) return ATTN_E_WORKSPACE;
  return ATTN_OK;
}

attn_status fwd_check(int dt, const void* Q, const void* K, const void* V, const void* O,
                      const float* lse, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                      int mode, int64_t wl, int64_t wr) {
  return fwd_check_g(dt, Q, K, V, O, lse, nullptr, fixed_geometry(B, H, H, N, d), scale, mode, wl,
                     wr);
}

attn_status bwd_check(int dt, const void* Q, const void* K, const void* V, const void* O,
                      const float* lse, const void* dO, const void* dQ, const void* dK,
                      const void* dV, const void* ws, size_t ws_bytes, int64_t B, int64_t H,
                      int64_t N, int64_t d, float scale, int mode, int64_t wl, int64_t wr) {
  return bwd_check_g(dt, Q, K, V, O, lse, dO, dQ, dK, dV, ws, ws_bytes, nullptr,
                     fixed_geometry(B, H, H, N, d), scale, mode, wl, wr);
}

}  // namespace attn

extern "C" {

const char* attn_status_str(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULLPTR: return "a required pointer is NULL";
    case ATTN_E_SHAPE: return "B, H or N out of range";
    case ATTN_E_UNSUPPORTED: return "unsupported dtype or head size (d must be 64 or 128)";
    case ATTN_E_MASK: return "unknown mask mode or negative window";
    case ATTN_E_SCALE: return "scale is not finite";
    case ATTN_E_ALIGN: return "a device pointer is not 16-byte aligned";
    case ATTN_E_ALIAS: return "an output overlaps an input or another output";
    case ATTN_E_WORKSPACE: return "workspace missing or too small";
    case ATTN_E_SCRATCH:
      return "the sizes need more scratch than the allocation-free entry point holds";
    case ATTN_E_HIP: return "HIP runtime error at launch";
  }
  return "unknown status";
}

size_t attn_bwd_workspace_bytes(attn_dtype dt, int64_t B, int64_t H, int64_t N, int64_t d) {
  if (attn::check_sizes(dt, B, H, N, d) != ATTN_OK) return 0;
  return static_cast<size_t>(attn::workspace_bytes(B, H, N));
}

size_t attn_bwd_gqa_workspace_bytes(attn_dtype dt, int64_t B, int64_t H, int64_t H_kv, int64_t N,
                                    int64_t d) {
  const attn::Geometry g = attn::fixed_geometry(B, H, H_kv, N, d);
  if (attn::check_geometry(dt, g) != ATTN_OK) return 0;
  return static_cast<size_t>(attn::bwd_workspace_bytes(g));
}

size_t attn_bwd_varlen_workspace_bytes(attn_dtype dt, int64_t n_seqs, int64_t max_seqlen,
                                       int64_t total, int64_t H, int64_t H_kv, int64_t d) {
  const attn::Geometry g{n_seqs, H, H_kv, total, max_seqlen, d, true};
  if (attn::check_geometry(dt, g) != ATTN_OK) return 0;
  return static_cast<size_t>(attn::bwd_workspace_bytes(g));
}

size_t attn_decode_workspace_bytes(attn_dtype dt, int64_t n_seqs, int64_t H, int64_t H_kv,
                                   int64_t n_q, int64_t d, int64_t max_seqlen) {
  // The page parameters do not affect the split; any valid ones will do.
  const attn::DecodeGeometry g{n_seqs, H, H_kv, n_q, d, attn::kDecTileK, 1,
                               attn::ceil_div(max_seqlen, attn::kDecTileK), max_seqlen};
  if (attn::decode_sizes(dt, g) != ATTN_OK) return 0;
  return static_cast<size_t>(attn::decode_workspace_bytes(n_seqs, H, H_kv, n_q, d, max_seqlen));
}

attn_status attn_fwd_check(attn_dtype dt, const void* Q, const void* K, const void* V,
                           const void* O, const float* lse, int64_t B, int64_t H, int64_t N,
                           int64_t d, float scale, attn_mask_mode mode, int64_t window_left,
                           int64_t window_right) {
  return attn::fwd_check(dt, Q, K, V, O, lse, B, H, N, d, scale, mode, window_left, window_right);
}

attn_status attn_bwd_check(attn_dtype dt, const void* Q, const void* K, const void* V,
                           const void* O, const float* lse, const void* dO, const void* dQ,
                           const void* dK, const void* dV, const void* workspace,
                           size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t d,
                           float scale, attn_mask_mode mode, int64_t window_left,
                           int64_t window_right) {
  return attn::bwd_check(dt, Q, K, V, O, lse, dO, dQ, dK, dV, workspace, workspace_bytes, B, H, N,
                         d, scale, mode, window_left, window_right);
}

attn_status attn_fwd_tiles(int64_t d, attn_mask_mode mode, int64_t* block_q, int64_t* block_k) {
  if (block_q == nullptr || block_k == nullptr) return ATTN_E_NULLPTR;
  if (d != 64 && d != 128) return ATTN_E_UNSUPPORTED;
  if (attn::check_mask(mode, 0, 0) != ATTN_OK) return ATTN_E_MASK;
  *block_q = attn::fwd_block_q(mode);
  *block_k = attn::kFwdBlockK;
  return ATTN_OK;
}

attn_status attn_kv_tile_range(int64_t N, int64_t q0, int64_t block_q, int64_t block_k,
                               attn_mask_mode mode, int64_t window_left, int64_t window_right,
                               int64_t* lo, int64_t* hi) {
  if (lo == nullptr || hi == nullptr) return ATTN_E_NULLPTR;
  if (N < 1 || N > attn::kMaxI32 || block_q < 1 || block_k < 1 || q0 < 0 || q0 >= N)
    return ATTN_E_SHAPE;
  attn_status s = attn::check_mask(mode, window_left, window_right);
  if (s != ATTN_OK) return s;
  const int64_t wl = attn::imin(window_left, N), wr = attn::imin(window_right, N);
  attn::kv_tile_range(N, q0, block_q, block_k, mode, wl, wr, lo, hi);
  return ATTN_OK;
}

attn_status attn_fwd_workgroup(int64_t wg, int64_t n_heads, int64_t n_qblk, attn_mask_mode mode,
                               int64_t* head, int64_t* qblk) {
  if (head == nullptr || qblk == nullptr) return ATTN_E_NULLPTR;
  if (n_heads < 1 || n_qblk < 1 || n_heads > attn::kMaxI32 || n_qblk > attn::kMaxI32 ||
      n_heads * n_qblk > attn::kMaxI32 || wg < 0 || wg >= n_heads * n_qblk)
    return ATTN_E_SHAPE;
  if (attn::check_mask(mode, 0, 0) != ATTN_OK) return ATTN_E_MASK;
  attn::fwd_work_item<int64_t>(wg, n_heads, n_qblk, mode, head, qblk);
  return ATTN_OK;
}

attn_status attn_bwd_kv_workgroup(int64_t wg, int64_t n_heads, int64_t n_kblk,
                                  attn_mask_mode mode, int64_t* head, int64_t* kblk) {
  if (head == nullptr || kblk == nullptr) return ATTN_E_NULLPTR;
  if (n_heads < 1 || n_kblk < 1 || n_heads > attn::kMaxI32 || n_kblk > attn::kMaxI32 ||
      n_heads * n_kblk > attn::kMaxI32 || wg < 0 || wg >= n_heads * n_kblk)
    return ATTN_E_SHAPE;
  if (attn::check_mask(mode, 0, 0) != ATTN_OK) return ATTN_E_MASK;
  attn::kv_work_item<int64_t>(wg, n_heads, n_kblk, mode, head, kblk);
  return ATTN_OK;
}

}  // extern "C"
