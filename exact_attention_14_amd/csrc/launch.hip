// launch.hip -- the C ABI entry points that enqueue work: attn_fwd / attn_bwd and
// their grouped-query (_gqa) and packed variable-length (_varlen) variants, and
// split-KV decoding over a paged cache (attn_decode).
// Validation lives in validate.cpp and runs before any HIP call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "attn.h"
#include "kernels.hpp"
#include "plan.hpp"
#include "validate.hpp"

// Workspace of attn_bwd_noalloc: a fixed array in the code object, one copy
// per GPU.  In host code this name is only a handle for hipGetSymbolAddress,
// never a device address; kernels get the per-device address it returns.
static __device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace attn {
namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];  // device address of `scratch` on each device, once known

// The current device's copy of `scratch`, looked up once per device.
attn_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return ATTN_E_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return ATTN_OK;
}

// Scores enter the exp2 domain as s * c with c = |scale| * log2(e) > 0; a
// negative scale is folded into Q by flipping its sign bits.  A zero scale
// is replaced by c = 1e-30: every score then maps to |s * c| < 2^-24, whose
// exp2 rounds to exactly 1 in fp32 -- the uniform softmax that scale 0 gives
// -- while masked keys still map to exp2(-inf) = 0.
float exp2_coeff(float scale) {
  const float c = std::fabs(scale) * 1.4426950408889634f;
  return c < 1e-30f ? 1e-30f : c;
}

// Windows are read only for a sliding mask and act as unbounded from the
// head's row count on (for a packed batch, from T on: every sequence is
// shorter).
int clip_window(int64_t w, int64_t N) { return static_cast<int>(w < N ? w : N); }

HeadGeom head_geom(const Geometry& g, const int32_t* cu_seqlens) {
  HeadGeom h{};
  h.rows = static_cast<int>(g.rows);
  h.H = static_cast<int>(g.H);
  h.group = static_cast<int>(g.H / g.H_kv);
  h.cu_seqlens = g.packed ? cu_seqlens : nullptr;
  return h;
}

// Compute units of the current device, looked up once per device.
std::mutex g_cu_mu;
int g_cu_count[kMaxDevices];

attn_status compute_units(int* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_E_HIP;
  std::lock_guard<std::mutex> lock(g_cu_mu);
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      return ATTN_E_HIP;
    g_cu_count[dev] = n;
  }
  *out = g_cu_count[dev];
  return ATTN_OK;
}

attn_status fwd_impl(attn_dtype dt, const void* Q, const void* K, const void* V, void* O,
                     float* lse, const int32_t* cu_seqlens, const Geometry& g, float scale,
                     attn_mask_mode mode, int64_t wl, int64_t wr, void* stream,
                     bool persistent = false) {
  attn_status s = fwd_check_g(dt, Q, K, V, O, lse, cu_seqlens, g, scale, mode, wl, wr);
  if (s != ATTN_OK) return s;
  int n_cu = 0;
  if (persistent) {
    s = compute_units(&n_cu);
    if (s != ATTN_OK) return s;
  }
  FwdParams p{};
  p.Q = Q; p.K = K; p.V = V; p.O = O; p.lse = lse;
  p.g = head_geom(g, cu_seqlens);
  p.n_heads = static_cast<int>(g.n_heads());
  p.n_qblk = static_cast<int>(ceil_div(g.max_len, fwd_block_q(mode)));
  p.wl = mode == ATTN_MASK_SLIDING ? clip_window(wl, g.rows) : 0;
  p.wr = mode == ATTN_MASK_SLIDING ? clip_window(wr, g.rows) : 0;
  p.c = exp2_coeff(scale);
  p.qsign = scale < 0.0f ? 0x80008000u : 0u;
  const int64_t n_wg = g.n_heads() * p.n_qblk;
  hipError_t e = launch_fwd(p, dt == ATTN_BF16, static_cast<int>(g.d), mode, n_wg, n_cu,
                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

attn_status bwd_impl(attn_dtype dt, const void* Q, const void* K, const void* V, const void* O,
                     const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                     void* workspace, size_t workspace_bytes, const int32_t* cu_seqlens,
                     const Geometry& g, float scale, attn_mask_mode mode, int64_t wl, int64_t wr,
                     void* stream) {
  attn_status s = bwd_check_g(dt, Q, K, V, O, lse, dO, dQ, dK, dV, workspace, workspace_bytes,
                              cu_seqlens, g, scale, mode, wl, wr);
  if (s != ATTN_OK) return s;
  BwdParams p{};
  p.Q = Q; p.K = K; p.V = V; p.O = O; p.lse = lse; p.dO = dO;
  p.dQ = dQ; p.dK = dK; p.dV = dV;
  const uint64_t row_bytes = row_array_bytes(1, 1, g.q_rows());
  p.Dneg = static_cast<float*>(workspace);
  p.Loff = reinterpret_cast<float*>(static_cast<char*>(workspace) + row_bytes);
  p.kv_split = static_cast<int>(kv_split(g));
  p.kv_rows = g.kv_rows();
  if (p.kv_split > 1) {
    p.dK_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * row_bytes);
    p.dV_part = p.dK_part + static_cast<size_t>(p.kv_split) * g.kv_rows() * g.d;
  }
  p.g = head_geom(g, cu_seqlens);
  p.n_heads = static_cast<int>(g.n_heads());
  p.n_kv_heads = static_cast<int>(g.n_kv_heads());
  p.max_len = static_cast<int>(g.max_len);
  p.wl = mode == ATTN_MASK_SLIDING ? clip_window(wl, g.rows) : 0;
  p.wr = mode == ATTN_MASK_SLIDING ? clip_window(wr, g.rows) : 0;
  p.c = exp2_coeff(scale);
  p.scale = scale;
  p.qsign = scale < 0.0f ? 0x80008000u : 0u;
  p.lse_mul = -1.4426950408889634f / p.c;
  hipError_t e = launch_bwd(p, dt == ATTN_BF16, static_cast<int>(g.d), mode,
                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

Geometry packed_geometry(int64_t n_seqs, int64_t max_seqlen, int64_t total, int64_t H,
                         int64_t H_kv, int64_t d) {
  return Geometry{n_seqs, H, H_kv, total, max_seqlen, d, true};
}

}  // namespace
}  // namespace attn

extern "C" {

attn_status attn_fwd(attn_dtype dt, const void* Q, const void* K, const void* V, void* O,
                     float* lse, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                     attn_mask_mode mode, int64_t window_left, int64_t window_right,
                     void* stream) {
  return attn::fwd_impl(dt, Q, K, V, O, lse, nullptr, attn::fixed_geometry(B, H, H, N, d), scale,
                        mode, window_left, window_right, stream);
}

attn_status attn_fwd_gqa(attn_dtype dt, const void* Q, const void* K, const void* V, void* O,
                         float* lse, int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                         float scale, attn_mask_mode mode, int64_t window_left,
                         int64_t window_right, void* stream) {
  return attn::fwd_impl(dt, Q, K, V, O, lse, nullptr, attn::fixed_geometry(B, H, H_kv, N, d),
                        scale, mode, window_left, window_right, stream);
}

attn_status attn_fwd_persistent(attn_dtype dt, const void* Q, const void* K, const void* V,
                                void* O, float* lse, int64_t B, int64_t H, int64_t H_kv,
                                int64_t N, int64_t d, float scale, attn_mask_mode mode,
                                int64_t window_left, int64_t window_right, void* stream) {
  return attn::fwd_impl(dt, Q, K, V, O, lse, nullptr, attn::fixed_geometry(B, H, H_kv, N, d),
                        scale, mode, window_left, window_right, stream, true);
}

attn_status attn_fwd_varlen(attn_dtype dt, const void* Q, const void* K, const void* V, void* O,
                            float* lse, const int32_t* cu_seqlens, int64_t n_seqs,
                            int64_t max_seqlen, int64_t total, int64_t H, int64_t H_kv,
                            int64_t d, float scale, attn_mask_mode mode, int64_t window_left,
                            int64_t window_right, void* stream) {
  return attn::fwd_impl(dt, Q, K, V, O, lse, cu_seqlens,
                        attn::packed_geometry(n_seqs, max_seqlen, total, H, H_kv, d), scale,
                        mode, window_left, window_right, stream);
}

attn_status attn_bwd(attn_dtype dt, const void* Q, const void* K, const void* V, const void* O,
                     const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                     void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t N,
                     int64_t d, float scale, attn_mask_mode mode, int64_t window_left,
                     int64_t window_right, void* stream) {
  return attn::bwd_impl(dt, Q, K, V, O, lse, dO, dQ, dK, dV, workspace, workspace_bytes, nullptr,
                        attn::fixed_geometry(B, H, H, N, d), scale, mode, window_left,
                        window_right, stream);
}

attn_status attn_bwd_noalloc(attn_dtype dt, const void* Q, const void* K, const void* V,
                             const void* O, const float* lse, const void* dO, void* dQ, void* dK,
                             void* dV, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                             attn_mask_mode mode, int64_t window_left, int64_t window_right,
                             void* stream) {
  const attn::Geometry g = attn::fixed_geometry(B, H, H, N, d);
  // Every argument but the workspace first, before any HIP call.
  attn_status s = attn::bwd_check_g(dt, Q, K, V, O, lse, dO, dQ, dK, dV, nullptr, 0, nullptr, g,
                                    scale, mode, window_left, window_right, false);
  if (s != ATTN_OK) return s;
  if (attn::bwd_workspace_bytes(g) > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_E_SCRATCH;
  void* ws = nullptr;
  s = attn::scratch_address(&ws);
  if (s != ATTN_OK) return s;
  return attn::bwd_impl(dt, Q, K, V, O, lse, dO, dQ, dK, dV, ws, ATTN_NOALLOC_SCRATCH_BYTES,
                        nullptr, g, scale, mode, window_left, window_right, stream);
}

attn_status attn_bwd_gqa(attn_dtype dt, const void* Q, const void* K, const void* V,
                         const void* O, const float* lse, const void* dO, void* dQ, void* dK,
                         void* dV, void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                         int64_t H_kv, int64_t N, int64_t d, float scale, attn_mask_mode mode,
                         int64_t window_left, int64_t window_right, void* stream) {
  return attn::bwd_impl(dt, Q, K, V, O, lse, dO, dQ, dK, dV, workspace, workspace_bytes, nullptr,
                        attn::fixed_geometry(B, H, H_kv, N, d), scale, mode, window_left,
                        window_right, stream);
}

attn_status attn_bwd_varlen(attn_dtype dt, const void* Q, const void* K, const void* V,
                            const void* O, const float* lse, const void* dO, void* dQ, void* dK,
                            void* dV, void* workspace, size_t workspace_bytes,
                            const int32_t* cu_seqlens, int64_t n_seqs, int64_t max_seqlen,
                            int64_t total, int64_t H, int64_t H_kv, int64_t d, float scale,
                            attn_mask_mode mode, int64_t window_left, int64_t window_right,
                            void* stream) {
  return attn::bwd_impl(dt, Q, K, V, O, lse, dO, dQ, dK, dV, workspace, workspace_bytes,
                        cu_seqlens, attn::packed_geometry(n_seqs, max_seqlen, total, H, H_kv, d),
                        scale, mode, window_left, window_right, stream);
}

attn_status attn_decode(attn_dtype dt, const void* Q, const void* K_cache, const void* V_cache,
                        const int32_t* block_table, const int32_t* seq_lens, void* O, float* lse,
                        void* workspace, size_t workspace_bytes, int64_t n_seqs, int64_t H,
                        int64_t H_kv, int64_t n_q, int64_t d, int64_t page_size, int64_t n_pages,
                        int64_t max_pages_per_seq, int64_t max_seqlen, float scale,
                        attn_mask_mode mode, int64_t window_left, int64_t window_right,
                        void* stream) {
  const attn::DecodeGeometry g{n_seqs, H, H_kv, n_q, d, page_size, n_pages, max_pages_per_seq,
                               max_seqlen};
  attn_status s = attn::decode_check(dt, Q, K_cache, V_cache, block_table, seq_lens, O, lse,
                                     workspace, workspace_bytes, g, scale, mode, window_left,
                                     window_right);
  if (s != ATTN_OK) return s;
  attn::DecParams p{};
  p.Q = Q; p.K = K_cache; p.V = V_cache; p.O = O; p.lse = lse;
  p.block_table = block_table; p.seq_lens = seq_lens;
  p.n_seqs = static_cast<int>(n_seqs);
  p.H = static_cast<int>(H);
  p.H_kv = static_cast<int>(H_kv);
  p.group = static_cast<int>(H / H_kv);
  p.n_q = static_cast<int>(n_q);
  p.page_size = static_cast<int>(page_size);
  p.n_pages = static_cast<int>(n_pages);
  p.max_pages = static_cast<int>(max_pages_per_seq);
  const int64_t rt = attn::dec_row_tiles(H / H_kv, n_q);
  int64_t n_splits, chunk;
  attn::dec_plan(n_seqs, H_kv, rt, max_seqlen, &n_splits, &chunk);
  p.row_tiles = static_cast<int>(rt);
  p.n_splits = static_cast<int>(n_splits);
  p.chunk = static_cast<int>(chunk);
  if (n_splits > 1) {
    const uint64_t parts = static_cast<uint64_t>(n_seqs) * H_kv * rt * n_splits;
    p.part_o = static_cast<float*>(workspace);
    p.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          (parts * attn::kDecRows * d * 4u + 255u) / 256u * 256u);
  }
  const int64_t cap = max_pages_per_seq * page_size;
  p.wl = mode == ATTN_MASK_SLIDING ? attn::clip_window(window_left, cap) : 0;
  p.wr = mode == ATTN_MASK_SLIDING ? attn::clip_window(window_right, cap) : 0;
  p.c = attn::exp2_coeff(scale);
  p.qsign = scale < 0.0f ? 0x80008000u : 0u;
  hipError_t e = attn::launch_decode(p, dt == ATTN_BF16, static_cast<int>(d), mode,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

}  // extern "C"
