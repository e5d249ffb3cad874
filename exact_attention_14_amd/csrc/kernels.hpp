// kernels.hpp -- kernel parameter blocks and host-side launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace attn {

// Head geometry shared by both passes (see query_head_rows in plan.hpp).
struct HeadGeom {
  int rows;       // rows per head: N of a fixed-length batch, T of a packed one
  int H;          // query heads per batch entry or sequence
  int group;      // H / H_kv, query heads per key/value head
  const int32_t* cu_seqlens;  // packed batch: n_seqs + 1 row offsets; else null
};

struct FwdParams {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* lse;
  HeadGeom g;
  int n_heads;    // query heads of the launch: B * H, or n_seqs * H
  int n_qblk;     // ceil(longest sequence / fwd_block_q(mode))
  int wl, wr;     // windows clipped to [0, rows] (sliding only)
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
  float* Dneg;    // workspace: -D_i = -(dO_i . O_i), one per query-side row
  float* Loff;    // workspace: lse_i * lse_mul, a row's score offset, likewise
  HeadGeom g;
  int n_heads;    // query heads of the dQ launch: B * H, or n_seqs * H
  int n_kv_heads; // key/value heads of the dK/dV launch: B * H_kv, or n_seqs * H_kv
  int max_len;    // longest sequence (N of a fixed-length batch)
  int wl, wr;
  float c;        // |scale| * log2(e), at least 1e-30
  float scale;    // the signed scale (applied to dQ and dK)
  uint32_t qsign; // sign flip folded into Q for negative scales
  float lse_mul;  // -log2(e) / c: exp2(c * (s + lse * lse_mul)) = exp(scale * q.k - lse)
};

hipError_t launch_fwd(const FwdParams& p, int dt_bf16, int d, int mode, int64_t n_wg,
                      hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, int dt_bf16, int d, int mode, hipStream_t stream);

// The rows of query head x (device side: reads the packed batch's offsets).
__device__ __forceinline__ HeadRows query_rows(const HeadGeom& g, int64_t x) {
  if (g.cu_seqlens == nullptr) return query_head_rows(x, g.H, g.group, g.rows, false, 0, 0);
  const int64_t s = x / g.H;
  return query_head_rows(x, g.H, g.group, g.rows, true, g.cu_seqlens[s], g.cu_seqlens[s + 1]);
}

// The rows of key/value head y and its query heads (device side).
__device__ __forceinline__ KvHeadRows kv_rows(const HeadGeom& g, int64_t y) {
  const int H_kv = g.H / g.group;
  if (g.cu_seqlens == nullptr) return kv_head_rows(y, H_kv, g.group, g.rows, false, 0, 0);
  const int64_t s = y / H_kv;
  return kv_head_rows(y, H_kv, g.group, g.rows, true, g.cu_seqlens[s], g.cu_seqlens[s + 1]);
}

}  // namespace attn
