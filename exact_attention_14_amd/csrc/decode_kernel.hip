// decode_kernel.hip -- split-KV decoding over a paged K/V cache for gfx950.
//
// P1 = ai6s.net/6af30f4d40858c2d8819b6d5.html §5 (split-KV decoding and the
// paged cache as FlashAttention extensions), §2.3 (the online-softmax update
// that also merges the splits) and §2.2 (tiling); layout and split rules in
// decode.hpp.
//
// Decoding reads every cached key and value once per key/value head and does
// 4*d FLOP per (query row, key) with only group * n_q query rows: the work is
// bound by HBM, not by the matrix cores.  The kernel is organised for that:
//
// * One workgroup per (sequence, key/value head, 32-row query tile, key
//   split).  The query tile holds all rows that read the key/value head
//   (its group's query heads times the n_q new tokens), so every cached K/V
//   byte is fetched once per tile; unused rows of the 32 are padding.
// * K and V travel in 64-key tiles from the paged pool straight into LDS
//   (direct HBM-to-LDS buffer loads, one buffer resource per tile built from
//   the page's 64-bit address, so the pool may exceed 4 GiB), double
//   buffered so that one tile's loads are in flight while the other is
//   consumed.  K rows are padded and V rows swizzled as in the forward.
// * Two wavefronts per workgroup, each taking 32 keys of every tile, keep
//   their own online-softmax state (exact per-tile row max; m, l, l~, the
//   output accumulator) for the same 32 rows; at the end wavefront 1 hands
//   its state to wavefront 0 through LDS, which merges them by the same rule.
// * Scores S^T = K Q^T and the output O^T += V^T P^T run on the 32x32x16
//   matrix cores exactly as in the forward (Q in registers as the B
//   operand, V^T read with the transposing ds_read_b64_tr_b16).
// * With one split the workgroup writes O (normalised by l~, the sum of the
//   rounded probabilities) and lse directly; otherwise it writes its fp32
//   partial O and base-2 lse to the workspace and decode_combine_kernel
//   merges the splits.
// * Sequence lengths and page numbers come from device memory and are
//   clamped (lengths to the pages a sequence may own, page numbers to the
//   pool), so malformed values never move an access outside the buffers.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "decode.hpp"
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

template <int D>
struct DecLayout {
  static constexpr int BC = kDecTileK;
  static constexpr int NW = kDecWaves;
  static constexpr int NCH = D / 8;               // 16-byte chunks per row
  static constexpr int K_PITCH = D * 2 + 16;      // padded K row
  static constexpr int V_PITCH = D * 2;
  static constexpr int K_BYTES = BC * K_PITCH;
  static constexpr int V_BYTES = BC * V_PITCH;
  static constexpr int K_SLOTS = BC * (NCH + 1);
  static constexpr int K_INSTR = K_SLOTS / 64;
  static constexpr int K_INSTR_PER_WAVE = (K_INSTR + NW - 1) / NW;
  static constexpr int V_WAVE_LOADS = V_BYTES / NW / 1024;
  static constexpr int V_ROWS_PER_1K = 1024 / (D * 2);
  static constexpr int VSWZ_MASK = NCH / 4 - 1;
  static __device__ __forceinline__ int vswz(int row) { return (row & VSWZ_MASK) << 2; }
};

template <typename T, int D, int MASK>
__global__ __launch_bounds__(64 * kDecWaves) void decode_kernel(DecParams p) {
  using L = DecLayout<D>;
  constexpr int BC = kDecTileK, NW = kDecWaves;
  constexpr int KSTEPS = D / 16, DBLK = D / 32;
  constexpr uint32_t ROWB = D * 2;
  constexpr bool kOneSum = std::is_same<T, _Float16>::value;
  static_assert(L::K_SLOTS % 64 == 0 && NW == 2, "decode tile geometry");

  __shared__ __attribute__((aligned(16))) char k_lds0[L::K_BYTES], k_lds1[L::K_BYTES];
  __shared__ __attribute__((aligned(16))) char v_lds0[L::V_BYTES], v_lds1[L::V_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Work item: row tile fastest (the row tiles of one split read the same
  // keys), then split, key/value head, sequence.
  uint32_t rest = blockIdx.x;
  const uint32_t rt = rest % p.row_tiles;
  rest /= p.row_tiles;
  const uint32_t split = rest % p.n_splits;
  rest /= p.n_splits;
  const uint32_t kvh = rest % p.H_kv;
  const uint32_t s = rest / p.H_kv;

  // The sequence's cache length, clamped to what its pages and the splits
  // can hold; this split's keys [k_begin, k_end).
  int Lk = p.seq_lens[s];
  const int cap = p.max_pages * p.page_size;
  const int cover = p.n_splits * p.chunk;
  Lk = Lk < 0 ? 0 : (Lk > cap ? cap : Lk);
  Lk = Lk > cover ? cover : Lk;
  const int n_rows = p.group * p.n_q;
  // Query rows of the tile: row r = rt*32 + r32 is token r % n_q of query
  // head kvh*group + r / n_q, at cache position Lk - n_q + r % n_q.
  const int r = static_cast<int>(rt) * kDecRows + r32;
  const int pos = Lk - p.n_q + r % p.n_q;
  const int min_pos = Lk - p.n_q;

  int k_begin = static_cast<int>(split) * p.chunk;
  int k_end = k_begin + p.chunk < Lk ? k_begin + p.chunk : Lk;
  if (MASK == kSliding) {
    const int lo = min_pos - p.wl;
    if (k_begin < lo) k_begin = lo < 0 ? 0 : lo;
  }
  const int t_lo = k_begin / BC;
  const int t_hi = k_end > k_begin ? (k_end + BC - 1) / BC : t_lo;

  // Outputs of the tile: rows of the key/value head's group are contiguous.
  const size_t qrow0 = (static_cast<size_t>(s) * p.H + static_cast<size_t>(kvh) * p.group) * p.n_q;
  const size_t part = ((static_cast<size_t>(s) * p.H_kv + kvh) * p.row_tiles + rt) * p.n_splits + split;

  if (t_hi <= t_lo) {
    // Nothing to attend in this split: an empty partial (lse = -inf, which
    // the combine skips).  With a single split the rows are left unwritten
    // (only a malformed cache length of zero gets here).
    if (p.n_splits > 1 && wave == 0 && half == 0) p.part_lse[part * kDecRows + r32] = -INFINITY;
    return;
  }

  const auto rQ = make_rsrc(reinterpret_cast<const char*>(p.Q) + qrow0 * ROWB,
                            static_cast<uint32_t>(n_rows) * ROWB);
  u32x4_t qf[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk)
    qf[kk] = buf_load16(rQ, static_cast<uint32_t>(r) * ROWB + kk * 32 + half * 16, 0) ^ p.qsign;

  f32x16_t acc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) acc[b] = f32x16_t{};
  float m = -INFINITY, l = 0.0f, lr = 0.0f;
  const float c = p.c;

  // Direct-load slots, as in the forward with NW = 2 wavefronts; the
  // resource of a tile covers its 64 rows, so padding slots (offset past
  // the tile) read as zeros.
  constexpr uint32_t TILE_BYTES = BC * ROWB;
  uint32_t kg_off[L::K_INSTR_PER_WAVE];
#pragma unroll
  for (int i = 0; i < L::K_INSTR_PER_WAVE; ++i) {
    const int slot = (wave + NW * i) * 64 + lane;
    const int row = slot / (L::NCH + 1), ch = slot % (L::NCH + 1);
    kg_off[i] = ch == L::NCH ? TILE_BYTES : static_cast<uint32_t>(row) * ROWB + ch * 16;
  }
  const int vs_slot = wave * 64 + lane;
  const int vs_row = vs_slot / L::NCH, vs_phys = vs_slot % L::NCH;
  const uint32_t vg_off = static_cast<uint32_t>(vs_row) * ROWB + ((vs_phys ^ L::vswz(vs_row)) << 4);

  // Readers: this wavefront's 32 keys are rows 32*wave .. +31 of a tile.
  const int kr_off = (wave * 32 + r32) * L::K_PITCH + half * 16;
  const int G = lane >> 4, tt = (lane >> 2) & 3, cc = lane & 3;
  int vr_off[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
    const int row = 4 * half + tt;
    const int chunk = 4 * db + 2 * (G & 1) + (cc >> 1);
    vr_off[db] = (wave * 32 + row) * L::V_PITCH + ((chunk ^ L::vswz(row)) << 4) + (cc & 1) * 8;
  }

  // The page of tile t (clamped into the pool) and its K / V resources,
  // bounded to the tile's rows below the cache length: rows past it may hold
  // stale values (even NaN) and read as zeros instead, since a masked key's
  // zero probability would not cancel a NaN in the output product.
  const int32_t* table = p.block_table + static_cast<size_t>(s) * p.max_pages;
  auto tile_rsrc = [&](int t, const void* pool) {
    const int key0 = t * BC;
    int page = table[key0 / p.page_size];
    page = page < 0 ? 0 : (page >= p.n_pages ? p.n_pages - 1 : page);
    const size_t row0 = (static_cast<size_t>(page) * p.H_kv + kvh) * p.page_size + key0 % p.page_size;
    const int valid = Lk - key0 < BC ? Lk - key0 : BC;
    return make_rsrc(reinterpret_cast<const char*>(pool) + row0 * ROWB,
                     static_cast<uint32_t>(valid) * ROWB);
  };
  auto load_tile = [&](int t, char* kd, char* vd) {
    const auto rK = tile_rsrc(t, p.K);
    const auto rV = tile_rsrc(t, p.V);
#pragma unroll
    for (int i = 0; i < L::K_INSTR_PER_WAVE; ++i) {
      const int j = wave + NW * i;
      if (j < L::K_INSTR) buf_load16_lds(rK, kd + j * 1024, kg_off[i], 0);
    }
#pragma unroll
    for (int j = 0; j < L::V_WAVE_LOADS; ++j)
      buf_load16_lds(rV, vd + (NW * j + wave) * 1024, vg_off,
                     static_cast<uint32_t>(NW * j * L::V_ROWS_PER_1K) * ROWB);
  };

  // One tile: scores of this wavefront's 32 keys, mask, exact row max and
  // rescale, probabilities, and the output product.
  auto tile = [&](int t, const char* kb_, const char* vb_) {
    const int k0 = t * BC;
    f32x16_t sc = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) sc = Elem<T>::mma(ld_lds16(kb_ + kr_off + kk * 32), qf[kk], sc);
    bool full = k0 + BC <= Lk;
    if (MASK == kCausal) full = full && k0 + BC - 1 <= min_pos;
    if (MASK == kSliding) full = full && k0 >= Lk - 1 - p.wl && k0 + BC - 1 <= min_pos + p.wr;
    if (!full) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + wave * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
        bool ok = key < k_end;
        if (MASK == kCausal) ok = ok && key <= pos;
        if (MASK == kSliding) ok = ok && key >= pos - p.wl && key <= pos + p.wr;
        if (!ok) sc[i] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[i]);
    mx = halves_max(mx);
    const float mt = mx == -INFINITY ? -INFINITY : mx * c;
    const float mnew = fmaxf(m, mt);
    const float base = mnew == -INFINITY ? 0.0f : mnew;
    const float corr = mnew == -INFINITY ? 1.0f : fast_exp2(m - mnew);
    m = mnew;
#pragma unroll
    for (int b = 0; b < DBLK; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][i] *= corr;
    uint32_t pk[8];
    float rs = 0.0f, rr = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e0 = fast_exp2(fmaf(sc[2 * j], c, -base));
      const float e1 = fast_exp2(fmaf(sc[2 * j + 1], c, -base));
      pk[j] = Elem<T>::pack2(e0, e1);
      if (kOneSum) {
        rs = Elem<T>::add_pair(pk[j], rs);
      } else {
        rs += e0 + e1;
        rr = Elem<T>::add_pair(pk[j], rr);
      }
    }
    l = l * corr + rs;
    lr = kOneSum ? l : lr * corr + rr;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4_t b = {pk[ks * 4 + 0], pk[ks * 4 + 1], pk[ks * 4 + 2], pk[ks * 4 + 3]};
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const char* va = vb_ + vr_off[db] + ks * 16 * L::V_PITCH;
        const u32x2_t lo2 = ld_lds_tr8(va);
        const u32x2_t hi2 = ld_lds_tr8(va + 8 * L::V_PITCH);
        acc[db] = Elem<T>::mma(u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]}, b, acc[db]);
      }
    }
  };

  // Two-stage pipeline: tile t+1 loads into the other stage while tile t is
  // consumed; the step ends when both wavefronts' loads of t+1 have landed
  // and both are done reading stage t (a stage is refilled only after the
  // barrier that follows its last read).
  load_tile(t_lo, k_lds0, v_lds0);
  wait_vmem();
  __syncthreads();
  for (int t = t_lo; t < t_hi; t += 2) {
    if (t + 1 < t_hi) load_tile(t + 1, k_lds1, v_lds1);
    tile(t, k_lds0, v_lds0);
    wait_vmem();
    __syncthreads();
    if (t + 1 >= t_hi) break;
    if (t + 2 < t_hi) load_tile(t + 2, k_lds0, v_lds0);
    tile(t + 1, k_lds1, v_lds1);
    wait_vmem();
    __syncthreads();
  }

  // Merge the two wavefronts' states (same lanes, same rows) in LDS; the
  // loop's last barrier has retired every read of the stages.
  const float lt = halves_sum(l);
  const float lrt = kOneSum ? lt : halves_sum(lr);
  float* xch = reinterpret_cast<float*>(k_lds0);  // [DBLK*16 + 3][64] floats
  if (wave == 1) {
#pragma unroll
    for (int b = 0; b < DBLK; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) xch[(b * 16 + i) * 64 + lane] = acc[b][i];
    xch[(DBLK * 16 + 0) * 64 + lane] = m;
    xch[(DBLK * 16 + 1) * 64 + lane] = lt;
    xch[(DBLK * 16 + 2) * 64 + lane] = lrt;
  }
  __syncthreads();
  if (wave == 1) return;
  const float m1 = xch[(DBLK * 16 + 0) * 64 + lane];
  const float mm = fmaxf(m, m1);
  const float f0 = mm == -INFINITY ? 0.0f : fast_exp2(m - mm);
  const float f1 = mm == -INFINITY ? 0.0f : fast_exp2(m1 - mm);
  const float lsum = lt * f0 + xch[(DBLK * 16 + 1) * 64 + lane] * f1;
  const float lrsum = lrt * f0 + xch[(DBLK * 16 + 2) * 64 + lane] * f1;
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = acc[b][i] * f0 + xch[(b * 16 + i) * 64 + lane] * f1;
  // A row with no allowed key in this split (possible only at a window's
  // edge or past a short sequence's end) leaves O = 0 and lse = -inf.
  const float inv = lrsum > 0.0f ? 1.0f / lrsum : 0.0f;
  const float lse2 = lsum > 0.0f ? mm + __log2f(lsum) : -INFINITY;

  if (p.n_splits == 1) {
    const auto rO = make_rsrc(reinterpret_cast<char*>(p.O) + qrow0 * ROWB,
                              static_cast<uint32_t>(n_rows) * ROWB);
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2_t v = {Elem<T>::pack2(acc[db][g * 4 + 0] * inv, acc[db][g * 4 + 1] * inv),
                           Elem<T>::pack2(acc[db][g * 4 + 2] * inv, acc[db][g * 4 + 3] * inv)};
        buf_store8(v, rO, static_cast<uint32_t>(r) * ROWB + (db * 32 + g * 8 + half * 4) * 2);
      }
    if (half == 0 && r < n_rows) p.lse[qrow0 + r] = lse2 * 0.6931471805599453f;
    return;
  }
  const auto rP = make_rsrc(p.part_o + part * kDecRows * D, kDecRows * D * 4);
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      buf_store16(u32x4_t{__float_as_uint(acc[db][g * 4 + 0] * inv),
                          __float_as_uint(acc[db][g * 4 + 1] * inv),
                          __float_as_uint(acc[db][g * 4 + 2] * inv),
                          __float_as_uint(acc[db][g * 4 + 3] * inv)},
                  rP, (static_cast<uint32_t>(r32) * D + db * 32 + g * 8 + half * 4) * 4);
  if (half == 0) p.part_lse[part * kDecRows + r32] = lse2;
}

// Merges the splits of one query row: weights 2^(lse_k - max), skipping
// empty splits (lse_k = -inf).  One thread per 8 output elements.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecParams p, uint32_t n_threads) {
  constexpr int CH = D / 8;
  const uint32_t gid = blockIdx.x * 256 + threadIdx.x;
  if (gid >= n_threads) return;
  const uint32_t ch = gid % CH;
  uint32_t rest = gid / CH;
  const uint32_t r32 = rest % kDecRows;
  rest /= kDecRows;
  const uint32_t rt = rest % p.row_tiles;
  rest /= p.row_tiles;
  const uint32_t kvh = rest % p.H_kv;
  const uint32_t s = rest / p.H_kv;
  const int r = static_cast<int>(rt) * kDecRows + static_cast<int>(r32);
  if (r >= p.group * p.n_q) return;
  const size_t part0 = ((static_cast<size_t>(s) * p.H_kv + kvh) * p.row_tiles + rt) * p.n_splits;
  float mx = -INFINITY;
  for (int k = 0; k < p.n_splits; ++k) mx = fmaxf(mx, p.part_lse[(part0 + k) * kDecRows + r32]);
  float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float wsum = 0.0f;
  if (mx != -INFINITY) {
    for (int k = 0; k < p.n_splits; ++k) {
      const float lk = p.part_lse[(part0 + k) * kDecRows + r32];
      if (lk == -INFINITY) continue;
      const float w = fast_exp2(lk - mx);
      const float4* src =
          reinterpret_cast<const float4*>(p.part_o + ((part0 + k) * kDecRows + r32) * D + ch * 8);
      const float4 a = src[0], b = src[1];
      o[0] += w * a.x; o[1] += w * a.y; o[2] += w * a.z; o[3] += w * a.w;
      o[4] += w * b.x; o[5] += w * b.y; o[6] += w * b.z; o[7] += w * b.w;
      wsum += w;
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  const size_t row = (static_cast<size_t>(s) * p.H + static_cast<size_t>(kvh) * p.group) * p.n_q + r;
  u32x4_t out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = Elem<T>::pack2(o[2 * i] * inv, o[2 * i + 1] * inv);
  *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(p.O) + (row * D + ch * 8) * 2) = out;
  if (ch == 0) p.lse[row] = wsum > 0.0f ? (mx + __log2f(wsum)) * 0.6931471805599453f : -INFINITY;
}

template <typename T, int D, int MASK>
hipError_t launch_mask(const DecParams& p, hipStream_t stream) {
  const int64_t n_wg = static_cast<int64_t>(p.n_seqs) * p.H_kv * p.row_tiles * p.n_splits;
  hipLaunchKernelGGL((decode_kernel<T, D, MASK>), dim3(static_cast<unsigned>(n_wg)),
                     dim3(64 * kDecWaves), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_splits == 1) return e;
  const int64_t n_threads =
      static_cast<int64_t>(p.n_seqs) * p.H_kv * p.row_tiles * kDecRows * (D / 8);
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(static_cast<unsigned>(ceil_div(n_threads, 256))),
                     dim3(256), 0, stream, p, static_cast<uint32_t>(n_threads));
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const DecParams& p, int mode, hipStream_t stream) {
  switch (mode) {
    case kCausal: return launch_mask<T, D, kCausal>(p, stream);
    case kSliding: return launch_mask<T, D, kSliding>(p, stream);
    default: return launch_mask<T, D, kNone>(p, stream);
  }
}

}  // namespace

hipError_t launch_decode(const DecParams& p, int dt_bf16, int d, int mode, hipStream_t stream) {
  if (dt_bf16)
    return d == 64 ? launch_d<__bf16, 64>(p, mode, stream) : launch_d<__bf16, 128>(p, mode, stream);
  return d == 64 ? launch_d<_Float16, 64>(p, mode, stream) : launch_d<_Float16, 128>(p, mode, stream);
}

}  // namespace attn
