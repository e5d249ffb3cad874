// kernels.hpp -- kernel parameter blocks and host-side launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct FwdParams {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* lse;
  int N;          // rows per head
  int n_heads;    // B * H
  int n_qblk;     // ceil(N / fwd_block_q(mode))
  int wl, wr;     // windows clipped to [0, N] (sliding only)
  float c;        // |scale| * log2(e), at least 1e-30 (see launch code)
  uint32_t qsign; // 0x80008000 flips the sign of both 16-bit halves of a word
};

struct BwdParams {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const float* lse;
  const void* dO;
  void* dQ;
  void* dK;
  void* dV;
  float* Dneg;    // workspace: -D_i = -(dO_i . O_i), [n_heads * N]
  float* Loff;    // workspace: lse_i * lse_mul, a row's score offset, [n_heads * N]
  int N;
  int n_heads;
  int wl, wr;
  float c;        // |scale| * log2(e), at least 1e-30
  float scale;    // the signed scale (applied to dQ and dK)
  uint32_t qsign; // sign flip folded into Q for negative scales
  float lse_mul;  // -log2(e) / c: exp2(c * (s + lse * lse_mul)) = exp(scale * q.k - lse)
};

hipError_t launch_fwd(const FwdParams& p, int dt_bf16, int d, int mode, int64_t n_wg,
                      hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, int dt_bf16, int d, int mode, hipStream_t stream);

}  // namespace attn
