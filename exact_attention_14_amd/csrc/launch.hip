// launch.hip -- the C ABI entry points that enqueue work (attn_fwd, attn_bwd).
// Validation lives in validate.cpp and runs before any HIP call.
#include <hip/hip_runtime.h>

#include <cmath>

#include "attn.h"
#include "kernels.hpp"
#include "plan.hpp"
#include "validate.hpp"

namespace attn {
namespace {

// Scores enter the exp2 domain as s * c with c = |scale| * log2(e) > 0; a
// negative scale is folded into Q by flipping its sign bits.  A zero scale
// is replaced by c = 1e-30: every score then maps to |s * c| < 2^-24, whose
// exp2 rounds to exactly 1 in fp32 -- the uniform softmax that scale 0 gives
// -- while masked keys still map to exp2(-inf) = 0.
float exp2_coeff(float scale) {
  const float c = std::fabs(scale) * 1.4426950408889634f;
  return c < 1e-30f ? 1e-30f : c;
}

int clip_window(int64_t w, int64_t N) { return static_cast<int>(w < N ? w : N); }

}  // namespace
}  // namespace attn

extern "C" {

attn_status attn_fwd(attn_dtype dt, const void* Q, const void* K, const void* V, void* O,
                     float* lse, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                     attn_mask_mode mode, int64_t window_left, int64_t window_right,
                     void* stream) {
  attn_status s = attn::fwd_check(dt, Q, K, V, O, lse, B, H, N, d, scale, mode, window_left,
                                  window_right);
  if (s != ATTN_OK) return s;
  attn::FwdParams p{};
  p.Q = Q; p.K = K; p.V = V; p.O = O; p.lse = lse;
  p.N = static_cast<int>(N);
  p.n_heads = static_cast<int>(B * H);
  p.n_qblk = static_cast<int>(attn::ceil_div(N, attn::fwd_block_q(mode)));
  p.wl = mode == ATTN_MASK_SLIDING ? attn::clip_window(window_left, N) : 0;
  p.wr = mode == ATTN_MASK_SLIDING ? attn::clip_window(window_right, N) : 0;
  p.c = attn::exp2_coeff(scale);
  p.qsign = scale < 0.0f ? 0x80008000u : 0u;
  const int64_t n_wg = B * H * p.n_qblk;
  hipError_t e = attn::launch_fwd(p, dt == ATTN_BF16, static_cast<int>(d), mode, n_wg,
                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

attn_status attn_bwd(attn_dtype dt, const void* Q, const void* K, const void* V, const void* O,
                     const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                     void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t N,
                     int64_t d, float scale, attn_mask_mode mode, int64_t window_left,
                     int64_t window_right, void* stream) {
  attn_status s = attn::bwd_check(dt, Q, K, V, O, lse, dO, dQ, dK, dV, workspace, workspace_bytes,
                                  B, H, N, d, scale, mode, window_left, window_right);
  if (s != ATTN_OK) return s;
  attn::BwdParams p{};
  p.Q = Q; p.K = K; p.V = V; p.O = O; p.lse = lse; p.dO = dO;
  p.dQ = dQ; p.dK = dK; p.dV = dV;
  p.Dneg = static_cast<float*>(workspace);
  p.Loff = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    attn::row_array_bytes(B, H, N));
  p.N = static_cast<int>(N);
  p.n_heads = static_cast<int>(B * H);
  p.wl = mode == ATTN_MASK_SLIDING ? attn::clip_window(window_left, N) : 0;
  p.wr = mode == ATTN_MASK_SLIDING ? attn::clip_window(window_right, N) : 0;
  p.c = attn::exp2_coeff(scale);
  p.scale = scale;
  p.qsign = scale < 0.0f ? 0x80008000u : 0u;
  p.lse_mul = -1.4426950408889634f / p.c;
  hipError_t e = attn::launch_bwd(p, dt == ATTN_BF16, static_cast<int>(d), mode,
                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

}  // extern "C"
