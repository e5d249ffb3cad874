// bwd_kernels.hip -- recomputation backward for gfx950 (MI355X).
//
// P1 = ai6s.net/6af30f4d40858c2d8819b6d5.html §2.4 (the backward rebuilds S
// and P from the saved statistics instead of storing P) and P3 =
// jsqmd.com/news/1148352 §4 (the backward is several times the forward's work
// and relies on recomputation).  With lse saved by the forward, a tile of P
// is exp(scale * q.k - lse) directly -- no running max is needed.
//
// Two launches (three with split groups), no atomics, so the result is
// deterministic:
//   1. bwd_dq:      query-major like the forward.  D_i = dO_i . O_i from the
//                   forward's stored O (fp32), written negated for the
//                   second pass together with each row's score offset
//                   lse_i * lse_mul.  Per 64-key tile, 32 keys
//                   at a time: S^T = K Q^T, P^T, dP^T = V dO^T,
//                   dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.  Q and dO stay
//                   in registers; two wavefronts per SIMD.
//   2. bwd_dkdv:    key-major.  Per 64-query tile, 32 queries at a time:
//                   S = Q K^T, P, dP = dO V^T, dS = P (dP - D) (the rows'
//                   offsets and -D are the accumulators' starting values),
//                   dV^T += dO^T P, dK^T += Q^T dS.  K and V stay in
//                   registers; each wavefront owns 64 keys (two blocks that
//                   share every operand read from LDS) with its dV and dK
//                   accumulators in AGPRs, one wavefront per SIMD.
//                   With grouped-query heads a key/value head's workgroup
//                   walks the query heads of its group (P1 §5 names
//                   grouped-query attention).  When there are too few
//                   key/value heads to fill the chip, each group is split
//                   into slices with one workgroup each, and
//   3. bwd_kv_reduce: sums the slices' fp32 partial dK/dV in slice order.
// Tiles stream through double-buffered LDS stages filled by direct
// HBM-to-LDS loads (one array per stage, so reading one stage never waits
// for the loads into the other).  Each 64-row tile is stored once, row-major
// with its 16-byte chunks permuted per row, and read both ways: as rows with
// 16-byte reads (operands whose reduction index is d) and transposed with
// ds_read_b64_tr_b16 (operands whose reduction index is the tile's rows).
// The permutation is chosen so that both read patterns are free of LDS bank
// conflicts.  All products accumulate in fp32; P and dS are rounded to the
// storage type before they enter a product.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace attn {
namespace {

// A 64-row tile of a [rows][D] 16-bit matrix in LDS: row-major, 16-byte
// chunk c of row r stored at chunk position c ^ swz(r).
//  * Row reads (lane r of a 16-lane group reads one chunk of row r0 + r):
//    swz takes 16 distinct values over any 16 consecutive rows (d = 128) or
//    8 over the rows of one parity (d = 64, two rows per 256-byte bank line),
//    so the 16 lanes cover all 64 banks.
//  * Transposing reads (32 lanes read four consecutive rows x four aligned
//    chunks): the four rows' swz values differ in the bits that select the
//    aligned group of four chunks, so the rows land in disjoint banks.
template <int D>
struct BwdTile {
  static constexpr int NCH = D / 8;         // 16-byte chunks per row
  static constexpr int ROWB = D * 2;        // bytes per row
  static constexpr int BYTES = 64 * ROWB;
  static constexpr int INSTR = BYTES / 1024;  // 1 KiB direct loads per tile
  static constexpr int R1K = 1024 / ROWB;     // rows per direct load
  static __device__ __forceinline__ int swz(int r) {
    return NCH == 16 ? (((r & 3) << 2) | ((r >> 2) & 3))
                     : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
  static __device__ __forceinline__ int off(int row, int chunk) {
    return row * ROWB + ((chunk ^ swz(row)) << 4);
  }
};

// Direct loads of one tile by NW wavefronts: instruction j = w + NW*i fills
// LDS bytes [j KiB, +1 KiB), i.e. rows j*R1K + lane/NCH at chunk position
// lane % NCH, fetching the logical chunk stored there.  swz depends on the
// row's low four bits only, which the NW*R1K-row stride between a
// wavefront's instructions leaves unchanged, so one per-lane offset serves.
template <int D, int NW>
struct TileLoader {
  using L = BwdTile<D>;
  static constexpr int PER_WAVE = L::INSTR / NW;
  static_assert(L::INSTR % NW == 0 && (NW * L::R1K) % 16 == 0, "loader geometry");
  uint32_t voff;
  int wave;
  __device__ TileLoader(int wave_, int lane) : wave(wave_) {
    const int row = wave_ * L::R1K + lane / L::NCH;
    voff = static_cast<uint32_t>(row) * L::ROWB +
           static_cast<uint32_t>(((lane % L::NCH) ^ L::swz(row)) << 4);
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, char* dst, int row0) const {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i)
      buf_load16_lds(r, dst + (wave + NW * i) * 1024, voff,
                     static_cast<uint32_t>(row0 + NW * i * L::R1K) * L::ROWB);
  }
};

// Per-lane offsets of the two read patterns (relative to a tile and to the
// 32-row block / 16-row step selected by an immediate added by the caller).
template <int D>
struct TileReaders {
  using L = BwdTile<D>;
  static constexpr int KSTEPS = D / 16, DBLK = D / 32;
  // Row reads, A operand of a product reducing over d: lane (r, half) reads
  // row r, chunk 2kk + half.
  int row[KSTEPS];
  // Transposing reads, A operand of a product reducing over the tile's rows:
  // lane (group G, t, cc) reads rows 4*half + t and 4*half + t + 8 of a 16-row
  // step, columns 32db + 16(G%2) + 4cc .. +3.
  int tr[DBLK][2];
  __device__ TileReaders(int lane) {
    const int half = lane >> 5, r32 = lane & 31;
    const int G = lane >> 4, tt = (lane >> 2) & 3, cc = lane & 3;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) row[kk] = L::off(r32, 2 * kk + half);
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        tr[db][h] = L::off(4 * half + tt + 8 * h, 4 * db + 2 * (G & 1) + (cc >> 1)) + (cc & 1) * 8;
  }
  // 32 x 16 A operand, rows blk*32 .., chunk pair kk.
  __device__ __forceinline__ u32x4_t rows(const char* tile, int blk, int kk) const {
    return ld_lds16(tile + row[kk] + blk * 32 * L::ROWB);
  }
  // 32 x 16 A operand of the transpose: d block db, tile rows 16*st .. +15.
  __device__ __forceinline__ u32x4_t trans(const char* tile, int db, int st) const {
    const u32x2_t lo2 = ld_lds_tr8(tile + tr[db][0] + st * 16 * L::ROWB);
    const u32x2_t hi2 = ld_lds_tr8(tile + tr[db][1] + st * 16 * L::ROWB);
    return u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
  }
};

// ------------------------------------------------------------------ dQ
// PAIR (fixed-length batches with an even number of query heads per
// key/value head): eight wavefronts, the first four on query head 2x and the
// last four on head 2x+1 of the same key/value head, over the same 128-row
// block, so every K/V tile brought into LDS serves both heads.
template <typename T, int D, int MASK, bool PAIR>
__global__ __launch_bounds__(PAIR ? 2 * kBwdThreads : kBwdThreads)
__attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdParams p, int n_qblk) {
  using L = BwdTile<D>;
  constexpr int BQ = kBwdDqBlockQ, BK = kBwdDqBlockK;
  constexpr int NW = (PAIR ? 2 : 1) * kBwdThreads / 64;
  static_assert(BK == 64 && BQ == 32 * (PAIR ? NW / 2 : NW), "dQ tile geometry");
  constexpr int KSTEPS = D / 16, DBLK = D / 32;
  constexpr uint32_t ROWB = L::ROWB;
  __shared__ __attribute__((aligned(16))) char k_lds0[L::BYTES], k_lds1[L::BYTES];
  __shared__ __attribute__((aligned(16))) char v_lds0[L::BYTES], v_lds1[L::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // With PAIR the wavefront's rows start at 32 * (wave % 4) within the block.
  const int wrow = PAIR ? wave % 4 : wave;
  int64_t head, qblk;
  if (p.g.cu_seqlens == nullptr)
    fwd_item(blockIdx.x, p.n_heads / (PAIR ? 2 : 1), n_qblk, MASK, &head, &qblk);
  else
    packed_item(blockIdx.x, p.g.H, p.n_heads / p.g.H, n_qblk, false, &head, &qblk);
  if (PAIR) {
    // item (outer, pair) -> query head outer*H + 2*pair + wave/4
    const int64_t hp = p.g.H / 2;
    head = (head / hp) * p.g.H + 2 * (head % hp) + wave / 4;
  }
  // The query head's rows (a packed sequence's blocks past its end exit) and
  // its key/value head.
  const HeadRows hr = query_rows(p.g, head);
  const int N = static_cast<int>(hr.len);
  const int q0 = static_cast<int>(qblk) * BQ;
  if (q0 >= N) return;
  const size_t qoff = static_cast<size_t>(hr.q_row0) * ROWB;
  const size_t kvoff = static_cast<size_t>(hr.kv_row0) * ROWB;
  const uint32_t head_bytes = static_cast<uint32_t>(N) * ROWB;
  const auto rQ = make_rsrc(reinterpret_cast<const char*>(p.Q) + qoff, head_bytes);
  const auto rK = make_rsrc(reinterpret_cast<const char*>(p.K) + kvoff, head_bytes);
  const auto rV = make_rsrc(reinterpret_cast<const char*>(p.V) + kvoff, head_bytes);
  const auto rG = make_rsrc(reinterpret_cast<const char*>(p.dO) + qoff, head_bytes);
  const auto rO = make_rsrc(reinterpret_cast<const char*>(p.O) + qoff, head_bytes);

  // Q and dO of this lane's row stay in registers (B operands); the lane
  // holds elements kk*16 + half*8 .. +7 of the row for every kk.
  const int wq0 = q0 + wrow * 32;
  const int qrow = wq0 + r32;
  u32x4_t qf[KSTEPS], gf[KSTEPS];
  float dsum = 0.0f;
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    const uint32_t off = static_cast<uint32_t>(qrow) * ROWB + kk * 32 + half * 16;
    qf[kk] = buf_load16(rQ, off, 0) ^ p.qsign;
    gf[kk] = buf_load16(rG, off, 0);
    const u32x4_t of = buf_load16(rO, off, 0);
    const T* ov = reinterpret_cast<const T*>(&of);
    const T* gv = reinterpret_cast<const T*>(&gf[kk]);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      dsum = fmaf(static_cast<float>(ov[e]), static_cast<float>(gv[e]), dsum);
  }
  // D = dO . O over the whole row (the two halves of the wavefront hold its
  // two halves); rows past N read as zeros.  The dK/dV pass, launched next on
  // the same stream, starts its accumulators from -D and the row's score
  // offset, written here once per row.
  dsum = halves_sum(dsum);
  const size_t srow = static_cast<size_t>(hr.q_row0) + qrow;
  const float lse = qrow < N ? p.lse[srow] : 0.0f;
  if (half == 0 && qrow < N) {
    p.Dneg[srow] = -dsum;
    p.Loff[srow] = lse * p.lse_mul;
  }
  const float lse2 = qrow < N ? lse * kLog2e : INFINITY;
  const float Dq = -dsum;
  const float c = p.c;

  f32x16_t acc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) acc[b] = f32x16_t{};

  int64_t lo64, hi64;
  kv_tile_range(N, q0, BQ, BK, MASK, p.wl, p.wr, &lo64, &hi64);
  const int lo = static_cast<int>(lo64), hi = static_cast<int>(hi64);
  const TileLoader<D, NW> ld(wave, lane);
  const TileReaders<D> rd(lane);

  // One key tile from a pair of stages: 32 keys at a time, S^T and dP^T,
  // then dS^T, then dQ^T += K^T dS^T over the block's two 16-key steps.
  auto tile = [&](int t, const char* kt, const char* vt) {
    const int k0 = t * BK;
    if (MASK != kNone && tile_none_allowed(N, wq0, 32, k0, BK, MASK, p.wl, p.wr)) return;
    const bool full = tile_all_allowed(N, wq0, 32, k0, BK, MASK, p.wl, p.wr);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        s = Elem<T>::mma(rd.rows(kt, kb, kk), qf[kk], s);
        dp = Elem<T>::mma(rd.rows(vt, kb, kk), gf[kk], dp);
      }
      // Boundary tiles only: masked scores become -inf, so P = 0 there.
      if (!full) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
          bool ok = key < N;
          if (MASK == kCausal) ok = ok && key <= qrow;
          if (MASK == kSliding) ok = ok && key >= qrow - p.wl && key <= qrow + p.wr;
          if (!ok) s[i] = -INFINITY;
        }
      }
      uint32_t ds[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float e[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = 2 * j + u;
          e[u] = fast_exp2(fmaf(s[i], c, -lse2)) * (dp[i] + Dq);
        }
        ds[j] = Elem<T>::pack2(e[0], e[1]);
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const u32x4_t b = {ds[h2 * 4 + 0], ds[h2 * 4 + 1], ds[h2 * 4 + 2], ds[h2 * 4 + 3]};
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
          acc[db] = Elem<T>::mma(rd.trans(kt, db, kb * 2 + h2), b, acc[db]);
      }
      // Keeps the two 32-key blocks from being interleaved (register
      // pressure: each block holds its own S^T, dP^T and operand reads).
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  ld.load(rK, k_lds0, lo * BK);
  ld.load(rV, v_lds0, lo * BK);
  wait_vmem();
  __syncthreads();
  for (int t = lo; t < hi; t += 2) {
    if (t + 1 < hi) {
      ld.load(rK, k_lds1, (t + 1) * BK);
      ld.load(rV, v_lds1, (t + 1) * BK);
    }
    tile(t, k_lds0, v_lds0);
    wait_vmem();
    __syncthreads();
    if (t + 1 >= hi) break;
    if (t + 2 < hi) {
      ld.load(rK, k_lds0, (t + 2) * BK);
      ld.load(rV, v_lds0, (t + 2) * BK);
    }
    tile(t + 1, k_lds1, v_lds1);
    wait_vmem();
    __syncthreads();
  }

  // dQ = scale * dS K; stores past N are dropped by the buffer bound.
  const auto rdQ = make_rsrc(reinterpret_cast<char*>(p.dQ) + qoff, head_bytes);
  const float sc = p.scale;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2_t v = {Elem<T>::pack2(acc[db][g * 4 + 0] * sc, acc[db][g * 4 + 1] * sc),
                         Elem<T>::pack2(acc[db][g * 4 + 2] * sc, acc[db][g * 4 + 3] * sc)};
      buf_store8(v, rdQ, static_cast<uint32_t>(qrow) * ROWB + (db * 32 + g * 8 + half * 4) * 2);
    }
}

// ---------------------------------------------------------------- dK, dV
// Each wavefront owns KB = 2 blocks of 32 keys, so every Q / dO operand read
// from LDS feeds the products of both blocks.
template <typename T, int D, int MASK>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdParams p, int n_kblk) {
  using L = BwdTile<D>;
  constexpr int BK = kBwdKvBlockK, BQ = kBwdKvBlockQ, NW = kBwdThreads / 64;
  constexpr int KB = BK / (32 * NW);
  static_assert(BQ == 64 && KB == 2, "dK/dV tile geometry");
  constexpr int KSTEPS = D / 16, DBLK = D / 32;
  constexpr uint32_t ROWB = L::ROWB;
  __shared__ __attribute__((aligned(16))) char q_lds0[L::BYTES], q_lds1[L::BYTES];
  __shared__ __attribute__((aligned(16))) char g_lds0[L::BYTES], g_lds1[L::BYTES];
  __shared__ __attribute__((aligned(16))) float s_off0[BQ], s_off1[BQ], s_dn0[BQ], s_dn1[BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The kv_split slices of one (key/value head, key block) item are
  // consecutive workgroups, so the item order (heaviest first) holds across
  // slices, and die wg % 8 keeps a fixed share of the query heads.
  const uint32_t slice = blockIdx.x % p.kv_split, item = blockIdx.x / p.kv_split;
  int64_t head, kblk;
  if (p.g.cu_seqlens == nullptr) {
    kv_item(item, p.n_kv_heads, n_kblk, MASK, p.g.group == 1, &head, &kblk);
  } else {
    const int H_kv = p.g.H / p.g.group;
    packed_item(item, H_kv, p.n_kv_heads / H_kv, n_kblk, MASK == kCausal, &head, &kblk);
  }
  const int g_per = p.g.group / p.kv_split;
  const int g0 = static_cast<int>(slice) * g_per, g1 = g0 + g_per;
  // The key/value head's rows (a packed sequence's blocks past its end exit)
  // and its query heads g0 .. g1-1, whose contributions accumulate here.
  const KvHeadRows kr = kv_rows(p.g, head);
  const int N = static_cast<int>(kr.len);
  const int k0 = static_cast<int>(kblk) * BK;
  if (k0 >= N) return;
  const size_t kvoff = static_cast<size_t>(kr.kv_row0) * ROWB;
  const uint32_t head_bytes = static_cast<uint32_t>(N) * ROWB;
  const auto rK = make_rsrc(reinterpret_cast<const char*>(p.K) + kvoff, head_bytes);
  const auto rV = make_rsrc(reinterpret_cast<const char*>(p.V) + kvoff, head_bytes);

  // K (with a negative scale's sign flip folded in) and V as B operands of
  // S = Q K^T and dP = dO V^T: lane (key r32 of block kb, half).
  const int wk0 = k0 + wave * 32 * KB;
  int kcol[KB];
  u32x4_t kf[KB][KSTEPS], vf[KB][KSTEPS];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    kcol[kb] = wk0 + kb * 32 + r32;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const uint32_t off = static_cast<uint32_t>(kcol[kb]) * ROWB + kk * 32 + half * 16;
      kf[kb][kk] = buf_load16(rK, off, 0) ^ p.qsign;
      vf[kb][kk] = buf_load16(rV, off, 0);
    }
  }
  const float c = p.c;

  // dV^T and dK^T accumulate in AGPRs (inline-asm matrix instructions); the
  // score and dP tiles stay in VGPRs where the vector code reads them.
  f32x16_t dv[KB * DBLK], dk[KB * DBLK];
#pragma unroll
  for (int b = 0; b < KB * DBLK; ++b) {
    dv[b] = f32x16_t{};
    dk[b] = f32x16_t{};
  }
  acc_fence(dv);
  acc_fence(dk);

  int64_t lo64, hi64;
  q_tile_range(N, k0, BK, BQ, MASK, p.wl, p.wr, &lo64, &hi64);
  const int lo = static_cast<int>(lo64), hi = static_cast<int>(hi64);
  const TileLoader<D, NW> ld(wave, lane);
  const TileReaders<D> rd(lane);

  // The score offsets and -D of a query tile (the starting values of the
  // score and dP accumulators), one 4-byte direct load each by wavefront 0;
  // rows past N read as zero and are masked.
  auto load_stats = [&](__amdgpu_buffer_rsrc_t rL, __amdgpu_buffer_rsrc_t rD, int q0, float* sl,
                        float* sd) {
    if (wave == 0) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rL, (__attribute__((address_space(3))) void*)(sl), 4,
                                               lane * 4, q0 * 4, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rD, (__attribute__((address_space(3))) void*)(sd), 4,
                                               lane * 4, q0 * 4, 0, 0);
    }
  };

  // 32 per-row values of a query block in the layout of the score tile's
  // rows: element 4*g4 + u of a lane is row g4*8 + half*4 + u.
  auto row_tile = [&](const float* v, int qb) {
    f32x16_t t;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(v + qb * 32 + g4 * 8 + half * 4);
#pragma unroll
      for (int u = 0; u < 4; ++u) t[g4 * 4 + u] = __uint_as_float(x[u]);
    }
    return t;
  };

  // One query tile: 32 queries at a time, S and dP for both key blocks (the
  // accumulators start from -lse * log2(e) / c and -D, so the products
  // deliver exp2's argument divided by c and dP - D), then P and dS, then the
  // two 16-query steps of dV^T += dO^T P and dK^T += Q^T dS.
  auto tile = [&](int t, const char* qt, const char* gt, const float* sl, const float* sd) {
    const int q0 = t * BQ;
    if (MASK != kNone && tile_none_allowed(N, q0, BQ, wk0, 32 * KB, MASK, p.wl, p.wr)) return;
    const bool full = tile_all_allowed(N, q0, BQ, wk0, 32 * KB, MASK, p.wl, p.wr);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16_t s[KB], dp[KB];
      {
        const f32x16_t lt = row_tile(sl, qb), dt = row_tile(sd, qb);
        const u32x4_t aq = rd.rows(qt, qb, 0), ag = rd.rows(gt, qb, 0);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          s[kb] = Elem<T>::mma(aq, kf[kb][0], lt);
          dp[kb] = Elem<T>::mma(ag, vf[kb][0], dt);
        }
      }
#pragma unroll
      for (int kk = 1; kk < KSTEPS; ++kk) {
        const u32x4_t aq = rd.rows(qt, qb, kk), ag = rd.rows(gt, qb, kk);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          s[kb] = Elem<T>::mma(aq, kf[kb][kk], s[kb]);
          dp[kb] = Elem<T>::mma(ag, vf[kb][kk], dp[kb]);
        }
      }
      // Boundary tiles only: masked scores become -inf, so P = 0 there.
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int q = q0 + qb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
            bool ok = kcol[kb] < N && q < N;
            if (MASK == kCausal) ok = ok && kcol[kb] <= q;
            if (MASK == kSliding) ok = ok && kcol[kb] >= q - p.wl && kcol[kb] <= q + p.wr;
            if (!ok) s[kb][i] = -INFINITY;
          }
      }
      uint32_t pk[KB][8], dsk[KB][8];
      auto form = [&](int kb, int j) {
        const float p0 = fast_exp2(s[kb][2 * j] * c), p1 = fast_exp2(s[kb][2 * j + 1] * c);
        pk[kb][j] = Elem<T>::pack2(p0, p1);
        dsk[kb][j] = Elem<T>::pack2(p0 * dp[kb][2 * j], p1 * dp[kb][2 * j + 1]);
      };
      // Block 0's P and dS first; block 1's are formed a pair or two at a
      // time between block 0's products, so that this vector work runs
      // beside the matrix cores (with one wavefront per SIMD nothing else
      // would fill them).
#pragma unroll
      for (int j = 0; j < 8; ++j) form(0, j);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        u32x4_t ag[DBLK], aq[DBLK];
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          ag[db] = rd.trans(gt, db, qb * 2 + h2);
          aq[db] = rd.trans(qt, db, qb * 2 + h2);
        }
        const u32x4_t bp0 = {pk[0][h2 * 4 + 0], pk[0][h2 * 4 + 1], pk[0][h2 * 4 + 2],
                             pk[0][h2 * 4 + 3]};
        const u32x4_t bs0 = {dsk[0][h2 * 4 + 0], dsk[0][h2 * 4 + 1], dsk[0][h2 * 4 + 2],
                             dsk[0][h2 * 4 + 3]};
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          if (db == 0) {
            Elem<T>::template mma_acc<true>(dv[db], ag[db], bp0);
            Elem<T>::template mma_acc<true>(dk[db], aq[db], bs0);
          } else {
            Elem<T>::template mma_acc<false>(dv[db], ag[db], bp0);
            Elem<T>::template mma_acc<false>(dk[db], aq[db], bs0);
          }
#pragma unroll
          for (int u = 0; u < 4 / DBLK; ++u) form(1, h2 * 4 + db * (4 / DBLK) + u);
          __builtin_amdgcn_sched_barrier(0);
        }
        const u32x4_t bp1 = {pk[1][h2 * 4 + 0], pk[1][h2 * 4 + 1], pk[1][h2 * 4 + 2],
                             pk[1][h2 * 4 + 3]};
        const u32x4_t bs1 = {dsk[1][h2 * 4 + 0], dsk[1][h2 * 4 + 1], dsk[1][h2 * 4 + 2],
                             dsk[1][h2 * 4 + 3]};
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          if (db == 0) {
            Elem<T>::template mma_acc<true>(dv[DBLK + db], ag[db], bp1);
            Elem<T>::template mma_acc<true>(dk[DBLK + db], aq[db], bs1);
          } else {
            Elem<T>::template mma_acc<false>(dv[DBLK + db], ag[db], bp1);
            Elem<T>::template mma_acc<false>(dk[DBLK + db], aq[db], bs1);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The query tiles of each query head of the group in turn (one head
  // without grouping); every tile ends with a barrier, so the next head's
  // first loads may refill stage 0.
  for (int gq = g0; gq < g1; ++gq) {
    const size_t qoff = static_cast<size_t>(kr.q_row0 + gq * kr.q_stride) * ROWB;
    const size_t soff = static_cast<size_t>(kr.q_row0 + gq * kr.q_stride);
    const auto rQ = make_rsrc(reinterpret_cast<const char*>(p.Q) + qoff, head_bytes);
    const auto rG = make_rsrc(reinterpret_cast<const char*>(p.dO) + qoff, head_bytes);
    const auto rL = make_rsrc(p.Loff + soff, static_cast<uint32_t>(N) * 4);
    const auto rD = make_rsrc(p.Dneg + soff, static_cast<uint32_t>(N) * 4);
    ld.load(rQ, q_lds0, lo * BQ);
    ld.load(rG, g_lds0, lo * BQ);
    load_stats(rL, rD, lo * BQ, s_off0, s_dn0);
    wait_vmem();
    __syncthreads();
    for (int t = lo; t < hi; t += 2) {
      if (t + 1 < hi) {
        ld.load(rQ, q_lds1, (t + 1) * BQ);
        ld.load(rG, g_lds1, (t + 1) * BQ);
        load_stats(rL, rD, (t + 1) * BQ, s_off1, s_dn1);
      }
      tile(t, q_lds0, g_lds0, s_off0, s_dn0);
      wait_vmem();
      __syncthreads();
      if (t + 1 >= hi) break;
      if (t + 2 < hi) {
        ld.load(rQ, q_lds0, (t + 2) * BQ);
        ld.load(rG, g_lds0, (t + 2) * BQ);
        load_stats(rL, rD, (t + 2) * BQ, s_off0, s_dn0);
      }
      tile(t + 1, q_lds1, g_lds1, s_off1, s_dn1);
      wait_vmem();
      __syncthreads();
    }
  }

  // K entered the products with a negative scale's sign flip, so
  // dK = scale * dS^T Q with the signed scale; dV = P^T dO.  A split group
  // leaves its fp32 partial sums (unscaled) for the reduction instead.
  acc_fence(dv);
  if (p.kv_split > 1) {
    acc_fence(dk);
    const size_t part = (static_cast<size_t>(slice) * p.kv_rows + kr.kv_row0) * D;
    const uint32_t part_bytes = static_cast<uint32_t>(N) * D * 4;
    const auto rpK = make_rsrc(p.dK_part + part, part_bytes);
    const auto rpV = make_rsrc(p.dV_part + part, part_bytes);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16_t& a_ = dk[kb * DBLK + db];
          const f32x16_t& b_ = dv[kb * DBLK + db];
          const uint32_t off = (static_cast<uint32_t>(kcol[kb]) * D + db * 32 + g * 8 + half * 4) * 4;
          buf_store16(u32x4_t{__float_as_uint(a_[g * 4 + 0]), __float_as_uint(a_[g * 4 + 1]),
                              __float_as_uint(a_[g * 4 + 2]), __float_as_uint(a_[g * 4 + 3])},
                      rpK, off);
          buf_store16(u32x4_t{__float_as_uint(b_[g * 4 + 0]), __float_as_uint(b_[g * 4 + 1]),
                              __float_as_uint(b_[g * 4 + 2]), __float_as_uint(b_[g * 4 + 3])},
                      rpV, off);
        }
    return;
  }
  const float sc = p.scale;
  const auto rdK = make_rsrc(reinterpret_cast<char*>(p.dK) + kvoff, head_bytes);
  const auto rdV = make_rsrc(reinterpret_cast<char*>(p.dV) + kvoff, head_bytes);
  // dV first, then dK (fenced only now): fewer values are live at once.
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16_t& b_ = dv[kb * DBLK + db];
        const uint32_t off =
            static_cast<uint32_t>(kcol[kb]) * ROWB + (db * 32 + g * 8 + half * 4) * 2;
        const u32x2_t b = {Elem<T>::pack2(b_[g * 4 + 0], b_[g * 4 + 1]),
                           Elem<T>::pack2(b_[g * 4 + 2], b_[g * 4 + 3])};
        buf_store8(b, rdV, off);
      }
  acc_fence(dk);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16_t& a_ = dk[kb * DBLK + db];
        const uint32_t off =
            static_cast<uint32_t>(kcol[kb]) * ROWB + (db * 32 + g * 8 + half * 4) * 2;
        const u32x2_t a = {Elem<T>::pack2(a_[g * 4 + 0] * sc, a_[g * 4 + 1] * sc),
                           Elem<T>::pack2(a_[g * 4 + 2] * sc, a_[g * 4 + 3] * sc)};
        buf_store8(a, rdK, off);
      }
}

// ------------------------------------------------------ split reduction
// dK = scale * sum of the slices' partial dK, dV = sum of the partial dV,
// added in slice order (deterministic), rounded once.  Eight consecutive
// elements per thread; the key/value side is [kv_rows, D] row-major.
template <typename T>
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(BwdParams p, int64_t n_elems) {
  const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (e0 >= n_elems) return;
  float k[8], v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) k[i] = v[i] = 0.0f;
  for (int s = 0; s < p.kv_split; ++s) {
    const float4* pk = reinterpret_cast<const float4*>(p.dK_part + s * n_elems + e0);
    const float4* pv = reinterpret_cast<const float4*>(p.dV_part + s * n_elems + e0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 a = pk[h], b = pv[h];
      k[4 * h + 0] += a.x; k[4 * h + 1] += a.y; k[4 * h + 2] += a.z; k[4 * h + 3] += a.w;
      v[4 * h + 0] += b.x; v[4 * h + 1] += b.y; v[4 * h + 2] += b.z; v[4 * h + 3] += b.w;
    }
  }
  const float sc = p.scale;
  u32x4_t ok, ov;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ok[i] = Elem<T>::pack2(k[2 * i] * sc, k[2 * i + 1] * sc);
    ov[i] = Elem<T>::pack2(v[2 * i], v[2 * i + 1]);
  }
  *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(p.dK) + e0 * 2) = ok;
  *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(p.dV) + e0 * 2) = ov;
}

template <typename T, int D, int MASK>
hipError_t launch_all(const BwdParams& p, hipStream_t stream) {
  const int n_qblk = static_cast<int>(ceil_div(p.max_len, kBwdDqBlockQ));
  const int64_t n_dq = static_cast<int64_t>(p.n_heads) * n_qblk;
  if (p.g.group % 2 == 0 && p.g.cu_seqlens == nullptr)
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, MASK, true>), dim3(static_cast<unsigned>(n_dq / 2)),
                       dim3(2 * kBwdThreads), 0, stream, p, n_qblk);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, MASK, false>), dim3(static_cast<unsigned>(n_dq)),
                       dim3(kBwdThreads), 0, stream, p, n_qblk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int n_kblk = static_cast<int>(ceil_div(p.max_len, kBwdKvBlockK));
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, MASK>),
                     dim3(static_cast<unsigned>(static_cast<int64_t>(p.n_kv_heads) * n_kblk *
                                                p.kv_split)),
                     dim3(kBwdThreads), 0, stream, p, n_kblk);
  e = hipGetLastError();
  if (e != hipSuccess || p.kv_split == 1) return e;

  const int64_t n_elems = p.kv_rows * D;
  hipLaunchKernelGGL((bwd_kv_reduce_kernel<T>),
                     dim3(static_cast<unsigned>(ceil_div(n_elems, 8 * 256))), dim3(256), 0, stream,
                     p, n_elems);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_mask(const BwdParams& p, int mode, hipStream_t stream) {
  switch (mode) {
    case kCausal: return launch_all<T, D, kCausal>(p, stream);
    case kSliding: return launch_all<T, D, kSliding>(p, stream);
    default: return launch_all<T, D, kNone>(p, stream);
  }
}

template <typename T>
hipError_t launch_d(const BwdParams& p, int d, int mode, hipStream_t stream) {
  return d == 64 ? launch_mask<T, 64>(p, mode, stream) : launch_mask<T, 128>(p, mode, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int dt_bf16, int d, int mode, hipStream_t stream) {
  return dt_bf16 ? launch_d<__bf16>(p, d, mode, stream) : launch_d<_Float16>(p, d, mode, stream);
}

}  // namespace attn
