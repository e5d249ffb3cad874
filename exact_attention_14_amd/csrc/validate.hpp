// validate.hpp -- host-side validation shared by the launch code.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "attn.h"

namespace attn {

struct TensorArgs {
  int dt;
  int64_t B, H, N, d;
  float scale;
  int mode;
  int64_t wl, wr;
  int n_in, n_out;
  const void* in[8];
  uint64_t in_bytes[8];
  const void* out[8];
  uint64_t out_bytes[8];
};

attn_status check_sizes(int dt, int64_t B, int64_t H, int64_t N, int64_t d);
attn_status check_mask(int mode, int64_t wl, int64_t wr);
attn_status check_common(const TensorArgs& a);
// Bytes of one float32 value per row, padded to 256.
inline uint64_t row_array_bytes(int64_t B, int64_t H, int64_t N) {
  const uint64_t rows = static_cast<uint64_t>(B) * H * N;
  return (rows * 4u + 255u) / 256u * 256u;
}
uint64_t workspace_bytes(int64_t B, int64_t H, int64_t N);

attn_status fwd_check(int dt, const void* Q, const void* K, const void* V, const void* O,
                      const float* lse, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                      int mode, int64_t wl, int64_t wr);
attn_status bwd_check(int dt, const void* Q, const void* K, const void* V, const void* O,
                      const float* lse, const void* dO, const void* dQ, const void* dK,
                      const void* dV, const void* ws, size_t ws_bytes, int64_t B, int64_t H,
                      int64_t N, int64_t d, float scale, int mode, int64_t wl, int64_t wr);

}  // namespace attn
