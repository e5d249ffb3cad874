// bwd_kernels.hip -- recomputation backward for gfx950 (MI355X).
//
// P1 = ai6s.net/6af30f4d40858c2d8819b6d5.html §2.4 (the backward rebuilds S
// and P from the saved statistics instead of storing P) and P3 =
// jsqmd.com/news/1148352 §4 (the backward is several times the forward's work
// and relies on recomputation).  With lse saved by the forward, a tile of P
// is exp(scale * q.k - lse) directly -- no running max is needed.
//
// Three launches, no atomics, so the result is deterministic:
//   1. bwd_rowdot:  D_i = dO_i . O_i from the forward's stored O (fp32).
//   2. bwd_dq:      query-major like the forward.  Per 64-key tile:
//                   S^T = K Q^T, P^T, dP^T = V dO^T, dS^T = P^T (dP^T - D),
//                   dQ^T += K^T dS^T.  Q and dO stay in registers.
//   3. bwd_dkdv:    key-major.  Per 64-query tile: S = Q K^T, P,
//                   dP = dO V^T, dS = P (dP - D), dV^T += dO^T P,
//                   dK^T += Q^T dS.  K and V stay in registers.
// The matrix-core layouts are those of device_common.hpp: a 32x32 result
// tile feeds the next product as its B operand when its rows are the next
// reduction index, and operands read along that index are stored transposed
// in LDS in the matching perm16 order.  All products accumulate in fp32; P
// and dS are rounded to the storage type before they enter a product.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace attn {
namespace {

// ------------------------------------------------------------------ D_i
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(BwdParams p, int64_t rows) {
  constexpr int NCH = D / 8;
  constexpr int ROWS_PER_WG = 256 / NCH;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * ROWS_PER_WG + threadIdx.x / NCH;
  const int ch = threadIdx.x % NCH;
  float acc = 0.0f;
  if (row < rows) {
    const size_t off = (static_cast<size_t>(row) * D + ch * 8) * 2;
    const u32x4_t o = ld_global16(reinterpret_cast<const char*>(p.O) + off);
    const u32x4_t g = ld_global16(reinterpret_cast<const char*>(p.dO) + off);
    const T* ov = reinterpret_cast<const T*>(&o);
    const T* gv = reinterpret_cast<const T*>(&g);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(static_cast<float>(ov[e]), static_cast<float>(gv[e]), acc);
  }
#pragma unroll
  for (int w = NCH / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, NCH);
  if (row < rows && ch == 0) p.Dsum[row] = acc;
}

// Shared loaders --------------------------------------------------------
// A 64-row tile of [rows][D] elements is loaded by threads tid < 16 * NCH,
// each owning 4 consecutive rows of one 16-byte chunk, and written to LDS
// either as rows (XOR-swizzled chunks) or transposed (one LDS row per d
// index, the 64 rows at perm16 positions, chunks swizzled by the d index).
template <int D>
struct Tile64 {
  static constexpr int NCH = D / 8;
  static constexpr int KSWZ = NCH < 16 ? NCH : 16;
  static constexpr int BYTES = 64 * D * 2;
  static constexpr int T_PITCH = 64 * 2;
  static constexpr int LOADERS = 16 * NCH;

  static __device__ __forceinline__ int row_off(int row, int ch) {
    return (row * NCH + (ch ^ (row & (KSWZ - 1)))) * 16;
  }
  static __device__ __forceinline__ int tr_off(int drow, int chunk) {
    return drow * T_PITCH + ((chunk ^ (drow & 7)) << 4);
  }
  // Loads rows r0 + 4*rg .. +3, chunk ch of a [N][D] matrix (zeros past N).
  static __device__ __forceinline__ void load(u32x4_t v[4], const char* base, int r0, int N,
                                              int rg, int ch, uint32_t sign = 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = r0 + rg * 4 + r;
      v[r] = row < N ? (ld_global16(base + (static_cast<size_t>(row) * D + ch * 8) * 2) ^ sign)
                     : u32x4_t{0, 0, 0, 0};
    }
  }
  static __device__ __forceinline__ void store_rows(char* lds, const u32x4_t v[4], int rg, int ch) {
#pragma unroll
    for (int r = 0; r < 4; ++r) st_lds16(lds + row_off(rg * 4 + r, ch), v[r]);
  }
  static __device__ __forceinline__ void store_transposed(char* lds, const u32x4_t v[4], int rg,
                                                          int ch) {
    const int pos = perm16(rg * 4);
    const int chunk = pos >> 3, sub = (pos & 7) * 2;
    write_transposed_4x8(lds, v, ch * 8, [&](int drow) {
      return drow * T_PITCH + ((chunk ^ (drow & 7)) << 4) + sub;
    });
  }
};

// ------------------------------------------------------------------ dQ
template <typename T, int D, int MASK>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dq_kernel(BwdParams p, int n_qblk) {
  using L = Tile64<D>;
  constexpr int BQ = kBwdDqBlockQ, BK = kBwdDqBlockK;
  static_assert(BK == 64, "tile loader assumes 64-row tiles");
  constexpr int KSTEPS = D / 16, DBLK = D / 32, NCH = D / 8;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* k_rows = smem;
  char* k_tr = smem + L::BYTES;
  char* v_rows = smem + 2 * L::BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, r32 = lane & 31;
  const int N = p.N;
  int64_t head, qblk;
  fwd_work_item(blockIdx.x, p.n_heads, n_qblk, MASK, &head, &qblk);
  const int q0 = static_cast<int>(qblk) * BQ;
  const size_t hoff = static_cast<size_t>(head) * N * D;
  const char* Qh = reinterpret_cast<const char*>(p.Q) + hoff * 2;
  const char* Kh = reinterpret_cast<const char*>(p.K) + hoff * 2;
  const char* Vh = reinterpret_cast<const char*>(p.V) + hoff * 2;
  const char* dOh = reinterpret_cast<const char*>(p.dO) + hoff * 2;

  const int wq0 = q0 + wave * 32;
  const int qrow = wq0 + r32;
  u32x4_t qf[KSTEPS], gf[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    const size_t off = (static_cast<size_t>(qrow) * D + kk * 16 + half * 8) * 2;
    qf[kk] = qrow < N ? (ld_global16(Qh + off) ^ p.qsign) : u32x4_t{0, 0, 0, 0};
    gf[kk] = qrow < N ? ld_global16(dOh + off) : u32x4_t{0, 0, 0, 0};
  }
  const float lse2 = qrow < N ? p.lse[static_cast<size_t>(head) * N + qrow] * kLog2e : INFINITY;
  const float Dq = qrow < N ? p.Dsum[static_cast<size_t>(head) * N + qrow] : 0.0f;
  const float c = p.c;

  f32x16_t acc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) acc[b] = f32x16_t{};

  int64_t lo, hi;
  kv_tile_range(N, q0, BQ, BK, MASK, p.wl, p.wr, &lo, &hi);
  const bool loader = tid < L::LOADERS;
  const int rg = tid / NCH, ch = tid % NCH;

  for (int t = static_cast<int>(lo); t < static_cast<int>(hi); ++t) {
    const int k0 = t * BK;
    u32x4_t kv[4], vv[4];
    if (loader) {
      L::load(kv, Kh, k0, N, rg, ch);
      L::load(vv, Vh, k0, N, rg, ch);
    }
    __syncthreads();
    if (loader) {
      L::store_rows(k_rows, kv, rg, ch);
      L::store_transposed(k_tr, kv, rg, ch);
      L::store_rows(v_rows, vv, rg, ch);
    }
    __syncthreads();
    if (tile_none_allowed(N, wq0, 32, k0, BK, MASK, p.wl, p.wr)) continue;
    const bool full = tile_all_allowed(N, wq0, 32, k0, BK, MASK, p.wl, p.wr);

    uint32_t ds[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
      const int row = kb * 32 + r32;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        s = Elem<T>::mma(ld_lds16(k_rows + L::row_off(row, kk * 2 + half)), qf[kk], s);
        dp = Elem<T>::mma(ld_lds16(v_rows + L::row_off(row, kk * 2 + half)), gf[kk], dp);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float e[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = 2 * j + u;
          bool ok = true;
          if (!full) {
            const int key = k0 + kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
            ok = key < N;
            if (MASK == kCausal) ok = ok && key <= qrow;
            if (MASK == kSliding) ok = ok && key >= qrow - p.wl && key <= qrow + p.wr;
          }
          const float pr = ok ? fast_exp2(fmaf(s[i], c, -lse2)) : 0.0f;
          e[u] = pr * (dp[i] - Dq);
        }
        ds[kb][j] = Elem<T>::pack2(e[0], e[1]);
      }
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4_t b = {ds[kk >> 1][(kk & 1) * 4 + 0], ds[kk >> 1][(kk & 1) * 4 + 1],
                         ds[kk >> 1][(kk & 1) * 4 + 2], ds[kk >> 1][(kk & 1) * 4 + 3]};
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
        acc[db] = Elem<T>::mma(ld_lds16(k_tr + L::tr_off(db * 32 + r32, kk * 2 + half)), b, acc[db]);
    }
  }

  if (qrow < N) {
    char* dQh = reinterpret_cast<char*>(p.dQ) + hoff * 2;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2_t v = {Elem<T>::pack2(acc[db][g * 4 + 0] * sc, acc[db][g * 4 + 1] * sc),
                           Elem<T>::pack2(acc[db][g * 4 + 2] * sc, acc[db][g * 4 + 3] * sc)};
        st_global8(dQh + (static_cast<size_t>(qrow) * D + db * 32 + g * 8 + half * 4) * 2, v);
      }
  }
}

// ---------------------------------------------------------------- dK, dV
template <typename T, int D, int MASK>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdParams p, int n_kblk) {
  using L = Tile64<D>;
  constexpr int BK = kBwdKvBlockK, BQ = kBwdKvBlockQ;
  static_assert(BQ == 64, "tile loader assumes 64-row tiles");
  constexpr int KSTEPS = D / 16, DBLK = D / 32, NCH = D / 8;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* q_rows = smem;
  char* q_tr = smem + L::BYTES;
  char* g_rows = smem + 2 * L::BYTES;
  char* g_tr = smem + 3 * L::BYTES;
  float* lse_t = reinterpret_cast<float*>(smem + 4 * L::BYTES);
  float* D_t = lse_t + 64;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, r32 = lane & 31;
  const int N = p.N;
  int64_t head, kblk;
  fwd_work_item(blockIdx.x, p.n_heads, n_kblk, kNone, &head, &kblk);
  const int k0 = static_cast<int>(kblk) * BK;
  const size_t hoff = static_cast<size_t>(head) * N * D;
  const char* Qh = reinterpret_cast<const char*>(p.Q) + hoff * 2;
  const char* Kh = reinterpret_cast<const char*>(p.K) + hoff * 2;
  const char* Vh = reinterpret_cast<const char*>(p.V) + hoff * 2;
  const char* dOh = reinterpret_cast<const char*>(p.dO) + hoff * 2;
  const float* lse_h = p.lse + static_cast<size_t>(head) * N;
  const float* D_h = p.Dsum + static_cast<size_t>(head) * N;

  const int wk0 = k0 + wave * 32;
  const int kcol = wk0 + r32;
  u32x4_t kf[KSTEPS], vf[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    const size_t off = (static_cast<size_t>(kcol) * D + kk * 16 + half * 8) * 2;
    kf[kk] = kcol < N ? ld_global16(Kh + off) : u32x4_t{0, 0, 0, 0};
    vf[kk] = kcol < N ? ld_global16(Vh + off) : u32x4_t{0, 0, 0, 0};
  }
  const float c = p.c;

  f32x16_t dv[DBLK], dk[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) {
    dv[b] = f32x16_t{};
    dk[b] = f32x16_t{};
  }

  int64_t lo, hi;
  q_tile_range(N, k0, BK, BQ, MASK, p.wl, p.wr, &lo, &hi);
  const bool loader = tid < L::LOADERS;
  const int rg = tid / NCH, ch = tid % NCH;

  for (int t = static_cast<int>(lo); t < static_cast<int>(hi); ++t) {
    const int q0 = t * BQ;
    u32x4_t qv[4], gv[4];
    if (loader) {
      L::load(qv, Qh, q0, N, rg, ch, p.qsign);
      L::load(gv, dOh, q0, N, rg, ch);
    }
    float lse_v = INFINITY, D_v = 0.0f;
    if (tid < 64 && q0 + tid < N) {
      lse_v = lse_h[q0 + tid] * kLog2e;
      D_v = D_h[q0 + tid];
    }
    __syncthreads();
    if (loader) {
      L::store_rows(q_rows, qv, rg, ch);
      L::store_transposed(q_tr, qv, rg, ch);
      L::store_rows(g_rows, gv, rg, ch);
      L::store_transposed(g_tr, gv, rg, ch);
    }
    if (tid < 64) {
      lse_t[tid] = lse_v;
      D_t[tid] = D_v;
    }
    __syncthreads();
    if (tile_none_allowed(N, q0, BQ, wk0, 32, MASK, p.wl, p.wr)) continue;
    const bool full = tile_all_allowed(N, q0, BQ, wk0, 32, MASK, p.wl, p.wr);

    // One 32-query block at a time: S, dP -> P, dS -> two 16-query steps of
    // dV^T += dO^T P and dK^T += Q^T dS.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
      const int row = qb * 32 + r32;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        s = Elem<T>::mma(ld_lds16(q_rows + L::row_off(row, kk * 2 + half)), kf[kk], s);
        dp = Elem<T>::mma(ld_lds16(g_rows + L::row_off(row, kk * 2 + half)), vf[kk], dp);
      }
      uint32_t pk[8], dsk[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float pr[2], e[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = 2 * j + u;
          const int ql = qb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
          bool ok = true;
          if (!full) {
            const int q = q0 + ql;
            ok = kcol < N && q < N;
            if (MASK == kCausal) ok = ok && kcol <= q;
            if (MASK == kSliding) ok = ok && kcol >= q - p.wl && kcol <= q + p.wr;
          }
          pr[u] = ok ? fast_exp2(fmaf(s[i], c, -lse_t[ql])) : 0.0f;
          e[u] = pr[u] * (dp[i] - D_t[ql]);
        }
        pk[j] = Elem<T>::pack2(pr[0], pr[1]);
        dsk[j] = Elem<T>::pack2(e[0], e[1]);
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int st = qb * 2 + h2;
        const u32x4_t bp = {pk[h2 * 4 + 0], pk[h2 * 4 + 1], pk[h2 * 4 + 2], pk[h2 * 4 + 3]};
        const u32x4_t bs = {dsk[h2 * 4 + 0], dsk[h2 * 4 + 1], dsk[h2 * 4 + 2], dsk[h2 * 4 + 3]};
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          const int drow = db * 32 + r32;
          dv[db] = Elem<T>::mma(ld_lds16(g_tr + L::tr_off(drow, st * 2 + half)), bp, dv[db]);
          dk[db] = Elem<T>::mma(ld_lds16(q_tr + L::tr_off(drow, st * 2 + half)), bs, dk[db]);
        }
      }
    }
  }

  if (kcol < N) {
    // Q entered the products with its sign flipped for a negative scale, so
    // dK = |scale| dS^T Q' with Q' the stored (flipped) rows.
    const float sc = fabsf(p.scale);
    char* dKh = reinterpret_cast<char*>(p.dK) + hoff * 2;
    char* dVh = reinterpret_cast<char*>(p.dV) + hoff * 2;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const size_t off = (static_cast<size_t>(kcol) * D + db * 32 + g * 8 + half * 4) * 2;
        const u32x2_t a = {Elem<T>::pack2(dk[db][g * 4 + 0] * sc, dk[db][g * 4 + 1] * sc),
                           Elem<T>::pack2(dk[db][g * 4 + 2] * sc, dk[db][g * 4 + 3] * sc)};
        const u32x2_t b = {Elem<T>::pack2(dv[db][g * 4 + 0], dv[db][g * 4 + 1]),
                           Elem<T>::pack2(dv[db][g * 4 + 2], dv[db][g * 4 + 3])};
        st_global8(dKh + off, a);
        st_global8(dVh + off, b);
      }
  }
}

template <typename T, int D, int MASK>
hipError_t launch_all(const BwdParams& p, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(p.n_heads) * p.N;
  constexpr int rows_per_wg = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_rowdot_kernel<T, D>), dim3(static_cast<unsigned>(ceil_div(rows, rows_per_wg))),
                     dim3(256), 0, stream, p, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int n_qblk = static_cast<int>(ceil_div(p.N, kBwdDqBlockQ));
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, MASK>),
                     dim3(static_cast<unsigned>(static_cast<int64_t>(p.n_heads) * n_qblk)),
                     dim3(kBwdThreads), 3 * 64 * D * 2, stream, p, n_qblk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int n_kblk = static_cast<int>(ceil_div(p.N, kBwdKvBlockK));
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, MASK>),
                     dim3(static_cast<unsigned>(static_cast<int64_t>(p.n_heads) * n_kblk)),
                     dim3(kBwdThreads), 4 * 64 * D * 2 + 2 * 64 * 4, stream, p, n_kblk);
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
