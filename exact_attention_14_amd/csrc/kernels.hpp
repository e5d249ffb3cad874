// kernels.hpp -- kernel parameter blocks and host-side launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode.hpp"
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
  int kv_split;   // slices of each group of query heads in the dK/dV pass
  float* dK_part; // kv_split > 1: fp32 partial dK, [kv_split][kv_rows][d] (workspace)
  float* dV_part; // likewise for dV
  int64_t kv_rows;  // rows of the key/value side (B*H_kv*N, or H_kv*T)
  int wl, wr;
  float c;        // |scale| * log2(e), at least 1e-30
  float scale;    // the signed scale (applied to dQ and dK)
  uint32_t qsign; // sign flip folded into Q for negative scales
  float lse_mul;  // -log2(e) / c: exp2(c * (s + lse * lse_mul)) = exp(scale * q.k - lse)
};

// persist_cus > 0: persistent launch on a device with that many compute units.
hipError_t launch_fwd(const FwdParams& p, int dt_bf16, int d, int mode, int64_t n_wg,
                      int persist_cus, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, int dt_bf16, int d, int mode, hipStream_t stream);
hipError_t launch_decode(const DecParams& p, int dt_bf16, int d, int mode, hipStream_t stream);

// The rows of query head x (device side: reads the packed batch's offsets).
__device__ __forceinline__ HeadRows query_rows(const HeadGeom& g, uint32_t x) {
  const uint32_t H = g.H, group = g.group, rows = g.rows;
  if (g.cu_seqlens == nullptr) return query_head_rows<uint32_t>(x, H, group, rows, false, 0, 0);
  const uint32_t s = x / H;
  return query_head_rows<uint32_t>(x, H, group, rows, true, g.cu_seqlens[s], g.cu_seqlens[s + 1]);
}

// The rows of key/value head y and its query heads (device side).
__device__ __forceinline__ KvHeadRows kv_rows(const HeadGeom& g, uint32_t y) {
  const uint32_t group = g.group, H_kv = g.H / g.group, rows = g.rows;
  if (g.cu_seqlens == nullptr) return kv_head_rows<uint32_t>(y, H_kv, group, rows, false, 0, 0);
  const uint32_t s = y / H_kv;
  return kv_head_rows<uint32_t>(y, H_kv, group, rows, true, g.cu_seqlens[s], g.cu_seqlens[s + 1]);
}

// Work items of fixed-length batches (device side, 32-bit arithmetic).
__device__ __forceinline__ void fwd_item(uint32_t wg, uint32_t n_heads, uint32_t n_blk, int mode,
                                         int64_t* head, int64_t* blk) {
  uint32_t h, b;
  fwd_work_item<uint32_t>(wg, n_heads, n_blk, mode, &h, &b);
  *head = h;
  *blk = b;
}

__device__ __forceinline__ void kv_item(uint32_t wg, uint32_t n_heads, uint32_t n_blk, int mode,
                                        bool grouped, int64_t* head, int64_t* blk) {
  uint32_t h, b;
  kv_work_item<uint32_t>(wg, n_heads, n_blk, mode, &h, &b, grouped);
  *head = h;
  *blk = b;
}

// Work item of a packed batch (device side, 32-bit arithmetic).
__device__ __forceinline__ void packed_item(uint32_t wg, uint32_t heads, uint32_t n_seqs,
                                            uint32_t n_blk, bool ascending, int64_t* head,
                                            int64_t* blk) {
  uint32_t h, b;
  packed_work_item<uint32_t>(wg, heads, n_seqs, n_blk, ascending, &h, &b);
  *head = h;
  *blk = b;
}

}  // namespace attn
