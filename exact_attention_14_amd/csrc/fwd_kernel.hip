// fwd_kernel.hip -- exact attention forward for gfx950 (MI355X).
//
// The tiled online-softmax method (P1 = ai6s.net/6af30f4d40858c2d8819b6d5.html
// §2.2 tiling, §2.3 online softmax, §2.5 teaching kernel; P3 =
// jsqmd.com/news/1148352 §2 state m, l, O_acc), laid out for CDNA4:
//
// * One workgroup = 4 wavefronts = 128 query rows of one head; each wavefront
//   owns 32 query rows for the whole launch.  K/V are streamed in 64-row
//   tiles through a two-stage LDS ring (P1 §3.2 double-buffered queues): tile
//   t+1 is fetched from HBM into registers while tile t is consumed, then
//   written to the other stage.
// * Scores are computed transposed, S^T = K Q^T, on the 32x32x16 matrix
//   cores: K (A operand) comes from LDS, Q (B operand) stays in registers for
//   the whole launch.  In the result tile each lane owns one query row and 16
//   keys, so the row max is an in-lane reduction plus one swap between the
//   two halves of the wavefront (P3 §4: warp shuffles must be rewritten for
//   non-NVIDIA GPUs; here v_permlane32_swap).
// * The output is accumulated transposed too, O^T += V^T P^T: the score tile
//   converted to 16-bit is already the B operand, V^T (A operand) is stored
//   transposed in LDS in the matching permuted key order, and the per-row
//   rescale factor of the online softmax applies to the lane's own column.
// * Scores go straight to the exp2 domain with one FMA, s*c - m, where
//   c = |scale| * log2(e) (P1 §2.5 and §3.3 (2): exp2 instead of exp).  A
//   negative scale is folded into Q by flipping its sign bits (exact).
// * The running max only moves when a tile raises it by more than kTau
//   (2^kTau in the exp2 domain); otherwise the old max is kept, the
//   accumulator is not rescaled and probabilities may exceed 1 by at most
//   2^kTau.  The result is unchanged in exact arithmetic (m cancels between
//   numerator and l) and nearly all tiles skip the 64 multiplies per lane of
//   the rescale (P1 §2.3: the rescale corrects history when the max moves).
// * Whole key tiles outside the mask's band are never visited (P1 §3.3 (4));
//   only tiles that straddle the band edge or the ragged end of the sequence
//   evaluate the mask per element, with -inf (P2 "pitfall 1": ragged lengths;
//   P4 "performance data": NaN at window/tile boundaries, avoided here by
//   using 0 as the exponent base while a row has seen no allowed key).
// * Two row sums are kept: l of the fp32 probabilities (for lse) and l~ of
//   the 16-bit probabilities exactly as they enter the output product
//   (v_dot2 against ones).  O = acc / l~ is normalised once at the end and
//   rounded once to 16 bits, so O is a convex combination of V rows with the
//   rounded weights and a row dominated by one key reproduces that key's V
//   row up to the final rounding; lse = (m + log2 l) * ln 2.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace attn {
namespace {

constexpr float kTau = 8.0f;

template <typename T, int D, int MASK>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdParams p) {
  constexpr int BR = kFwdBlockQ, BC = kFwdBlockK;
  constexpr int NCH = D / 8;               // 16-byte chunks per row
  constexpr int KSTEPS = D / 16;           // reduction steps over d
  constexpr int DBLK = D / 32;             // 32-row blocks of O^T
  constexpr int KSWZ = NCH < 16 ? NCH : 16;
  constexpr int K_BYTES = BC * D * 2;
  constexpr int VT_PITCH = BC * 2;         // bytes per V^T row (one d index)
  constexpr int STAGE_BYTES = 2 * K_BYTES;
  constexpr int K_PER_THREAD = BC * NCH / kFwdThreads;
  static_assert(K_PER_THREAD >= 1, "K tile loader");
  static_assert((BC / 4) * NCH <= kFwdThreads, "V tile loader");

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, r32 = lane & 31;
  const int N = p.N;

  int64_t head, qblk;
  fwd_work_item(blockIdx.x, p.n_heads, p.n_qblk, MASK, &head, &qblk);
  const int q0 = static_cast<int>(qblk) * BR;
  const size_t hoff = static_cast<size_t>(head) * N * D;
  const char* Qh = reinterpret_cast<const char*>(p.Q) + hoff * 2;
  const char* Kh = reinterpret_cast<const char*>(p.K) + hoff * 2;
  const char* Vh = reinterpret_cast<const char*>(p.V) + hoff * 2;

  int64_t lo64, hi64;
  kv_tile_range(N, q0, BR, BC, MASK, p.wl, p.wr, &lo64, &hi64);
  const int lo = static_cast<int>(lo64), hi = static_cast<int>(hi64);

  // This lane's query row and its Q fragment (B operand of S^T = K Q^T).
  const int wq0 = q0 + wave * 32;
  const int qrow = wq0 + r32;
  u32x4_t qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    if (qrow < N) {
      qf[ks] = ld_global16(Qh + (static_cast<size_t>(qrow) * D + ks * 16 + half * 8) * 2);
      qf[ks] ^= p.qsign;
    } else {
      qf[ks] = u32x4_t{0, 0, 0, 0};
    }
  }

  f32x16_t acc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) acc[b] = f32x16_t{};
  float m = -INFINITY, l = 0.0f, lr = 0.0f;
  const float c = p.c;

  // Loader assignment.  K: thread owns chunks (row, ch) = divmod(tid + 256 j,
  // NCH).  V: thread owns 4 consecutive rows of one chunk, if tid < 16*NCH.
  u32x4_t kst[K_PER_THREAD];
  u32x4_t vst[4];
  const bool v_loader = tid < (BC / 4) * NCH;
  const int v_rg = tid / NCH, v_ch = tid % NCH;

  auto gload = [&](int t) {
    const int k0 = t * BC;
#pragma unroll
    for (int j = 0; j < K_PER_THREAD; ++j) {
      const int item = tid + kFwdThreads * j;
      const int key = k0 + item / NCH, ch = item % NCH;
      kst[j] = key < N ? ld_global16(Kh + (static_cast<size_t>(key) * D + ch * 8) * 2)
                       : u32x4_t{0, 0, 0, 0};
    }
    if (v_loader) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + v_rg * 4 + r;
        vst[r] = key < N ? ld_global16(Vh + (static_cast<size_t>(key) * D + v_ch * 8) * 2)
                         : u32x4_t{0, 0, 0, 0};
      }
    }
  };

  auto swrite = [&](int stage) {
    char* ks = smem + stage * STAGE_BYTES;
    char* vs = ks + K_BYTES;
#pragma unroll
    for (int j = 0; j < K_PER_THREAD; ++j) {
      const int item = tid + kFwdThreads * j;
      const int row = item / NCH, ch = item % NCH;
      st_lds16(ks + (row * NCH + (ch ^ (row & (KSWZ - 1)))) * 16, kst[j]);
    }
    if (v_loader) {
      // V^T row = d index; keys stored at perm16 positions, 16-byte chunks
      // XOR-swizzled by the row index.
      const int pos = perm16(v_rg * 4);  // 4 consecutive keys stay adjacent
      const int chunk = pos >> 3, sub = (pos & 7) * 2;
      write_transposed_4x8(vs, vst, v_ch * 8, [&](int drow) {
        return drow * VT_PITCH + ((chunk ^ (drow & 7)) << 4) + sub;
      });
    }
  };

  gload(lo);
  swrite(0);
  __syncthreads();

  for (int t = lo; t < hi; ++t) {
    const int stage = (t - lo) & 1;
    const bool more = t + 1 < hi;
    if (more) gload(t + 1);
    const char* ks = smem + stage * STAGE_BYTES;
    const char* vs = ks + K_BYTES;
    const int k0 = t * BC;

    if (!tile_none_allowed(N, wq0, 32, k0, BC, MASK, p.wl, p.wr)) {
      // S^T = K Q^T for two 32-key blocks.
      f32x16_t s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16_t{};
        const int row = kb * 32 + r32;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          const int ch = kk * 2 + half;
          const u32x4_t a = ld_lds16(ks + (row * NCH + (ch ^ (row & (KSWZ - 1)))) * 16);
          s[kb] = Elem<T>::mma(a, qf[kk], s[kb]);
        }
      }

      if (!tile_all_allowed(N, wq0, 32, k0, BC, MASK, p.wl, p.wr)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
            bool ok = key < N;
            if (MASK == kCausal) ok = ok && key <= qrow;
            if (MASK == kSliding) ok = ok && key >= qrow - p.wl && key <= qrow + p.wr;
            if (!ok) s[kb][i] = -INFINITY;
          }
        }
      }

      // Online softmax update (exp2 domain).
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = halves_max(mx);
      const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
      const float mnew = fmaxf(m, mt);
      const bool resc = mnew > m + kTau;
      float corr = 1.0f;
      if (resc) {
        corr = fast_exp2(m - mnew);
        m = mnew;
      }
      if (__any(resc)) {
#pragma unroll
        for (int b = 0; b < DBLK; ++b) acc[b] *= corr;
        l *= corr;
        lr *= corr;
      }
      const float base = (m == -INFINITY) ? 0.0f : m;

      uint32_t pk[2][8];
      float rs[2] = {0.0f, 0.0f}, rr[2] = {0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float e0 = fast_exp2(fmaf(s[kb][2 * j], c, -base));
          const float e1 = fast_exp2(fmaf(s[kb][2 * j + 1], c, -base));
          rs[kb] += e0 + e1;
          pk[kb][j] = Elem<T>::pack2(e0, e1);
          rr[kb] = Elem<T>::add_pair(pk[kb][j], rr[kb]);
        }
      }
      l += rs[0] + rs[1];
      lr += rr[0] + rr[1];

      // O^T += V^T P^T over four 16-key steps.
#pragma unroll
      for (int kk = 0; kk < BC / 16; ++kk) {
        const u32x4_t b = {pk[kk >> 1][(kk & 1) * 4 + 0], pk[kk >> 1][(kk & 1) * 4 + 1],
                           pk[kk >> 1][(kk & 1) * 4 + 2], pk[kk >> 1][(kk & 1) * 4 + 3]};
        const int chunk = kk * 2 + half;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          const int drow = db * 32 + r32;
          const u32x4_t a = ld_lds16(vs + drow * VT_PITCH + ((chunk ^ (drow & 7)) << 4));
          acc[db] = Elem<T>::mma(a, b, acc[db]);
        }
      }
    }

    if (more) swrite(stage ^ 1);
    __syncthreads();
  }

  // Epilogue: O = acc / l~ rounded once; lse in natural-log units.
  const float lt = halves_sum(l);
  const float lrt = halves_sum(lr);
  if (qrow < N) {
    const float inv = 1.0f / lrt;
    char* Oh = reinterpret_cast<char*>(p.O) + hoff * 2;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2_t v = {Elem<T>::pack2(acc[db][g * 4 + 0] * inv, acc[db][g * 4 + 1] * inv),
                           Elem<T>::pack2(acc[db][g * 4 + 2] * inv, acc[db][g * 4 + 3] * inv)};
        st_global8(Oh + (static_cast<size_t>(qrow) * D + db * 32 + g * 8 + half * 4) * 2, v);
      }
    }
    if (half == 0) p.lse[static_cast<size_t>(head) * N + qrow] = (m + log2f(lt)) * kLn2;
  }
}

template <typename T, int D, int MASK>
hipError_t launch_one(const FwdParams& p, int64_t n_wg, hipStream_t stream) {
  constexpr int lds = 2 * 2 * kFwdBlockK * D * 2;
  hipLaunchKernelGGL((fwd_kernel<T, D, MASK>), dim3(static_cast<unsigned>(n_wg)),
                     dim3(kFwdThreads), lds, stream, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_mask(const FwdParams& p, int mode, int64_t n_wg, hipStream_t stream) {
  switch (mode) {
    case kCausal: return launch_one<T, D, kCausal>(p, n_wg, stream);
    case kSliding: return launch_one<T, D, kSliding>(p, n_wg, stream);
    default: return launch_one<T, D, kNone>(p, n_wg, stream);
  }
}

template <typename T>
hipError_t launch_d(const FwdParams& p, int d, int mode, int64_t n_wg, hipStream_t stream) {
  return d == 64 ? launch_mask<T, 64>(p, mode, n_wg, stream)
                 : launch_mask<T, 128>(p, mode, n_wg, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int dt_bf16, int d, int mode, int64_t n_wg,
                      hipStream_t stream) {
  return dt_bf16 ? launch_d<__bf16>(p, d, mode, n_wg, stream)
                 : launch_d<_Float16>(p, d, mode, n_wg, stream);
}

}  // namespace attn
