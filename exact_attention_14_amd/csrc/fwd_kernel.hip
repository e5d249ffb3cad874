// fwd_kernel.hip -- exact attention forward for gfx950 (MI355X).
//
// The tiled online-softmax method (P1 = ai6s.net/6af30f4d40858c2d8819b6d5.html
// §2.2 tiling, §2.3 online softmax, §2.5 teaching kernel; P3 =
// jsqmd.com/news/1148352 §2 state m, l, O_acc), laid out for CDNA4:
//
// * Each wavefront owns 32 query rows of one head for the whole launch; a
//   workgroup has 8 of them (256 rows) without a mask and 4 (128 rows) with
//   a causal or sliding one, at two wavefronts per SIMD.  K/V are streamed
//   in 64-row tiles through two-stage LDS rings (P1 §3.2 double-buffered
//   queues), loaded by direct HBM-to-LDS buffer loads that need no
//   registers; each tile is fetched once for the whole workgroup.  Loads and
//   stores go through buffer resources bounded by the head's size, so rows
//   past N read as zeros and stores past N are dropped without branches.
//   Every LDS stage is an array of its own, so the compiler can tell that
//   reading one stage does not race the loads in flight into the other and
//   does not wait for them.
// * Scores are computed transposed, S^T = K Q^T, on the 32x32x16 matrix
//   cores: K (A operand) comes from LDS, Q (B operand) stays in registers for
//   the whole launch.  In the result tile each lane owns one query row and 16
//   keys, so the row max is an in-lane reduction plus one swap between the
//   two halves of the wavefront (P3 §4: warp shuffles must be rewritten for
//   non-NVIDIA GPUs; here v_permlane32_swap).
// * The output is accumulated transposed too, O^T += V^T P^T: the score tile
//   converted to 16-bit is already the B operand, and V^T (A operand) is read
//   from row-major V in LDS with the transposing ds_read_b64_tr_b16, in the
//   key order the score tile's layout implies.  The per-row rescale factor of
//   the online softmax applies to the lane's own column.
// * LDS layouts: K rows are padded by 16 bytes so that 16 lanes reading the
//   same 16-byte chunk of 16 consecutive rows hit distinct banks; V rows keep
//   their natural pitch with 16-byte chunks XOR-swizzled by (row mod 4) so
//   that the eight rows one transposing read touches spread over all banks.
//   The loop is unrolled over the two stages, so every LDS address is a
//   per-lane constant plus an immediate offset.
// * Scores go straight to the exp2 domain with one FMA, s*c - m, where
//   c = |scale| * log2(e) (P1 §2.5 and §3.3 (2): exp2 instead of exp).  A
//   negative scale is folded into Q by flipping its sign bits (exact).
// * Optimistic online softmax.  A tile's probabilities are first formed
//   against the running max m as it stands, without taking the tile's own
//   row max.  If none of them exceeds 2^kTau (checked through the lane's sum
//   of them, an upper bound) they are kept: m need not be the exact max, since
//   it cancels between the numerator and l.  kTau bounds what a kept
//   probability may add to the fp32 accumulators: 15 for fp16 (2^15 < 65504,
//   the largest fp16 probability), 32 for bf16 (whose rounding is 2^-9
//   relative at any magnitude): a tile then adds at most 2^33 |v| per row to
//   acc, so acc stays finite for |V| up to 2^78 at the longest head (2^17
//   tiles), where an exact max allows 2^105.  (A bound of 2^64 ran 0.6%
//   faster on causal attention with outlier keys but overflows for |V|
//   beyond 2^46.)  Otherwise (and while a row has no
//   m yet) the exact tile max is taken, m is raised to it, the accumulator, l
//   and l~ are rescaled (P1 §2.3: the rescale corrects history when the max
//   moves) and the tile's probabilities are formed again.  Nearly every tile
//   takes the first path and skips both the row max and the rescale; a large
//   kTau keeps it so when a few outlier keys raise the row max far above the
//   rest.
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

#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace attn {
namespace {

// 2^kTau, the bound on a probability formed against the running max (see the
// file comment): kTau = 15 for fp16, ATTN_FWD_BF16_TAU (32) for bf16.
#ifndef ATTN_FWD_BF16_TAU
#define ATTN_FWD_BF16_TAU 32
#endif
constexpr float pow2f(int n) { return n == 0 ? 1.0f : 2.0f * pow2f(n - 1); }
template <typename T>
constexpr float kSumBound = std::is_same<T, _Float16>::value ? pow2f(15) : pow2f(ATTN_FWD_BF16_TAU);

// Work queues of the persistent forward (fwd_kernel with PERSIST): the next unclaimed
// slot of each die's run of work items, and the number of workgroups that
// found every queue empty.  Zero when the code object loads; the last
// workgroup of every persistent launch sets them back to zero, so a launch
// needs no clearing beforehand (and two persistent launches must not run at
// the same time on one device).
__device__ uint32_t fwd_queue_next[kNumXcd];
__device__ uint32_t fwd_queue_done;

// A work item for a persistent workgroup (see fwd_kernel), as the id of the
// ordered launch's workgroup that would run it, or -1 when none is left
// (thread 0 only; vector atomics).
__device__ __forceinline__ int claim_item(uint32_t n_wg) {
  const uint32_t x0 = blockIdx.x % kNumXcd;
  int v = -1;
  for (uint32_t k = 0; k < kNumXcd && v < 0; ++k) {
    const uint32_t x = (x0 + k) % kNumXcd;
    // slots of die x: the ordered launch's workgroups w < n_wg with w % kNumXcd == x
    const uint32_t count = (n_wg + kNumXcd - 1 - x) / kNumXcd;
    const uint32_t slot = __hip_atomic_fetch_add(&fwd_queue_next[x], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (slot < count) v = static_cast<int>(slot * kNumXcd + x);
  }
  if (v < 0) {
    // Every queue is empty: the last workgroup to see it resets them.
    const uint32_t d = __hip_atomic_fetch_add(&fwd_queue_done, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (d == gridDim.x - 1) {
      for (uint32_t x = 0; x < kNumXcd; ++x)
        __hip_atomic_store(&fwd_queue_next[x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&fwd_queue_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  return v;
}

// Thread 0's claimed item passed on to the whole workgroup through LDS; the
// barriers also keep the next item's loads from overwriting LDS stages that
// the last item's wavefronts still read.
__device__ __forceinline__ int share_item(int v, int* slot_lds) {
  if (threadIdx.x == 0) *slot_lds = v;
  __syncthreads();
  const int w = *slot_lds;
  __syncthreads();
  return w;
}

template <int D, int NWAVES>
struct FwdLayout {
  static constexpr int BC = kFwdBlockK;
  static constexpr int NCH = D / 8;                  // 16-byte chunks per row
  static constexpr int K_PITCH = D * 2 + 16;         // padded K row
  static constexpr int V_PITCH = D * 2;
  static constexpr int K_BYTES = BC * K_PITCH;
  static constexpr int V_BYTES = BC * V_PITCH;
  // K and V go straight to LDS: each wavefront instruction fills 1 KiB.  K
  // rows have NCH + 1 slots of 16 bytes (the last one is padding).
  static constexpr int K_SLOTS = BC * (NCH + 1);
  // Whole 1 KiB loads: a K stage is rounded up to them (slots past the tile
  // are filled from past the buffer, i.e. with zeros, and never read).
  static constexpr int K_INSTR = (K_SLOTS + 63) / 64;          // 17 at d = 128, Bc = 64
  static constexpr int K_ALLOC = K_INSTR * 1024;
  static constexpr int NW = NWAVES;
  static constexpr int K_INSTR_PER_WAVE = (K_INSTR + NW - 1) / NW;
  static constexpr int V_INSTR = V_BYTES / 1024;
  static constexpr int V_WAVE_LOADS = (V_INSTR + NW - 1) / NW;
  static constexpr int V_ROWS_PER_1K = 1024 / (D * 2);
  static constexpr int VSWZ_MASK = NCH / 4 - 1;             // row bits used by the V swizzle
  static __device__ __forceinline__ int vswz(int row) { return (row & VSWZ_MASK) << 2; }
};

// PAIR (masked launches of fixed-length batches with an even number of
// query heads per key/value head): eight wavefronts, the first four on query head 2x and the last four
// on head 2x+1 of the same key/value head, over the same 128-row block.  Both
// halves visit the same key tiles, so every K/V tile brought into LDS serves
// 256 rows, as in the unmasked kernel, without the uneven tile counts that
// 256 consecutive rows have under a causal or sliding mask.
//
// PERSIST: the grid holds only as many workgroups as the chip runs at once;
// each claims work items from a queue per die (claim_item) until all are
// done.  A claimed slot s of die x is the item that workgroup s * kNumXcd + x
// runs in the ordered launch, so items keep their die and their
// heaviest-first order within it; a workgroup whose own die has run out takes
// items from the other dies' queues.  In the ordered launch the hardware
// dispatcher hands out the same workgroups, in id order, as compute-unit
// slots free up.
template <typename T, int D, int MASK, bool PAIR, bool PERSIST>
__global__ __launch_bounds__(64 * (PAIR ? 8 : fwd_waves(MASK))) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdParams p, uint32_t n_wg) {
  constexpr int NWAVES = PAIR ? 8 : fwd_waves(MASK);
  using L = FwdLayout<D, NWAVES>;
  constexpr int BR = fwd_block_q(MASK), BC = kFwdBlockK;
  constexpr int KSTEPS = D / 16;           // reduction steps over d
  constexpr int DBLK = D / 32;             // 32-row blocks of O^T
  constexpr int KB = BC / 32;              // 32-key blocks of a tile
  constexpr uint32_t ROW_BYTES = D * 2;
  constexpr bool kOneSum = std::is_same<T, _Float16>::value;

  __shared__ __attribute__((aligned(16))) char k_lds0[L::K_ALLOC], k_lds1[L::K_ALLOC];
  __shared__ __attribute__((aligned(16))) char v_lds0[L::V_BYTES], v_lds1[L::V_BYTES];
  __shared__ int slot_lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  // With PAIR the wavefront's query head is 2*item + sub and its rows start
  // at 32 * (wave % 4) within the block.
  const int sub = PAIR ? wave / 4 : 0, wrow = PAIR ? wave % 4 : wave;

  // A persistent workgroup claims its next item only when it has finished
  // the current one: claiming one ahead (so that the atomic's round trip
  // overlaps the work) measured 3-9% slower, since an item reserved early is
  // no longer available to a workgroup that frees up sooner.
  for (int wg = PERSIST ? share_item(threadIdx.x == 0 ? claim_item(n_wg) : -1, &slot_lds)
                        : static_cast<int>(blockIdx.x);
       wg >= 0; wg = PERSIST ? share_item(threadIdx.x == 0 ? claim_item(n_wg) : -1, &slot_lds) : -1) {
  int64_t head, qblk;
  const int hdiv = PAIR ? 2 : 1;
  if (p.g.cu_seqlens == nullptr)
    fwd_item(wg, p.n_heads / hdiv, p.n_qblk, MASK, &head, &qblk);
  else
    packed_item(wg, p.g.H / hdiv, p.n_heads / p.g.H, p.n_qblk, false, &head, &qblk);
  if (PAIR) {
    // item (outer, pair) -> query head outer*H + 2*pair + sub
    const int64_t hp = p.g.H / 2;
    head = (head / hp) * p.g.H + 2 * (head % hp) + sub;
  }
  // The head's rows: all N of a fixed-length batch, or one packed sequence
  // (whose query blocks past its end have nothing to do).  K and V come from
  // the head's key/value head.
  const HeadRows hr = query_rows(p.g, head);
  const int N = static_cast<int>(hr.len);
  const int q0 = static_cast<int>(qblk) * BR;
  if (q0 >= N) continue;
  const size_t qoff = static_cast<size_t>(hr.q_row0) * ROW_BYTES;
  const size_t kvoff = static_cast<size_t>(hr.kv_row0) * ROW_BYTES;
  const uint32_t head_bytes = static_cast<uint32_t>(N) * ROW_BYTES;
  const auto rQ = make_rsrc(reinterpret_cast<const char*>(p.Q) + qoff, head_bytes);
  const auto rK = make_rsrc(reinterpret_cast<const char*>(p.K) + kvoff, head_bytes);
  const auto rV = make_rsrc(reinterpret_cast<const char*>(p.V) + kvoff, head_bytes);

  int64_t lo64, hi64;
  kv_tile_range(N, q0, BR, BC, MASK, p.wl, p.wr, &lo64, &hi64);
  const int lo = static_cast<int>(lo64), hi = static_cast<int>(hi64);

  // This lane's query row and its Q fragment (B operand of S^T = K Q^T).
  const int wq0 = q0 + wrow * 32;
  const int qrow = wq0 + r32;
  u32x4_t qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    qf[ks] = buf_load16(rQ, static_cast<uint32_t>(qrow) * ROW_BYTES + ks * 32 + half * 16, 0) ^
             p.qsign;

  f32x16_t acc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) acc[b] = f32x16_t{};
  float m = -INFINITY, l = 0.0f, lr = 0.0f;
  const float c = p.c;

  static_assert(L::V_BYTES % 1024 == 0, "V tile must fill whole 1 KiB loads");
  // K direct loads: instruction j (= wave + NW*i, NW wavefronts) fills 16-byte slots
  // s = 64j + lane of the stage; slot s holds row s / (NCH+1), chunk
  // s % (NCH+1).  Padding slots point past the end of the head, so the
  // hardware fills them with zeros without touching memory.
  uint32_t kg_off[L::K_INSTR_PER_WAVE];
#pragma unroll
  for (int i = 0; i < L::K_INSTR_PER_WAVE; ++i) {
    const int slot = (wave + L::NW * i) * 64 + lane;
    const int row = slot / (L::NCH + 1), ch = slot % (L::NCH + 1);
    const bool pad = ch == L::NCH || (L::K_SLOTS % 64 != 0 && row >= BC);
    kg_off[i] = pad ? head_bytes : static_cast<uint32_t>(row) * ROW_BYTES + ch * 16;
  }
  // V direct loads: instruction j of wavefront w fills LDS bytes
  // [(NW*j + w) KiB, +1 KiB) of the stage, i.e. 16-byte slot s = 64*(NW*j+w) + lane
  // = (row, physical chunk); the lane fetches the logical chunk stored there.
  const int vs_slot = wave * 64 + lane;
  const int vs_row = vs_slot / L::NCH, vs_phys = vs_slot % L::NCH;
  const uint32_t vg_off = static_cast<uint32_t>(vs_row) * ROW_BYTES +
                          ((vs_phys ^ L::vswz(vs_row)) << 4);

  // Readers.  K (A of S^T): row kb*32 + r32, chunk 2kk + half.
  const int kr_off = r32 * L::K_PITCH + half * 16;
  // V^T (A of O^T) via transposing reads: lane (group G = lane/16, t, cc) of
  // the 16-lane group points at row 16ks + 4*half + t (+8 for the second
  // read), columns 32db + 16*(G%2) + 4cc .. +3.
  const int G = lane >> 4, tt = (lane >> 2) & 3, cc = lane & 3;
  int vr_off[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
    const int row = 4 * half + tt;
    const int chunk = 4 * db + 2 * (G & 1) + (cc >> 1);
    vr_off[db] = row * L::V_PITCH + ((chunk ^ L::vswz(row)) << 4) + (cc & 1) * 8;
  }

  auto gload_k_lds = [&](int t, char* dstb) {
    const uint32_t soff = static_cast<uint32_t>(t * BC) * ROW_BYTES;
#pragma unroll
    for (int i = 0; i < L::K_INSTR_PER_WAVE; ++i) {
      const int j = wave + L::NW * i;
      if (j < L::K_INSTR) buf_load16_lds(rK, dstb + j * 1024, kg_off[i], soff);
    }
  };
  auto gload_v_lds = [&](int t, char* dstb) {
#pragma unroll
    for (int j = 0; j < L::V_WAVE_LOADS; ++j)
      if (L::V_INSTR % L::NW == 0 || L::NW * j + wave < L::V_INSTR)
        buf_load16_lds(rV, dstb + (L::NW * j + wave) * 1024, vg_off,
                       static_cast<uint32_t>(t * BC + L::NW * j * L::V_ROWS_PER_1K) * ROW_BYTES);
  };

  // S^T = K Q^T of tile t from a K stage: two independent accumulation chains.
  auto scores = [&](const char* kb_, f32x16_t s[KB]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        s[kb] = Elem<T>::mma(ld_lds16(kb_ + kr_off + kb * 32 * L::K_PITCH + kk * 32),
                             qf[kk], s[kb]);
  };

  // Phase 1 of tile t: mask (boundary tiles only), row max, and the online
  // rescale (rare).  Returns the exponent base.
  auto apply_mask = [&](int t, f32x16_t s[KB]) {
    const int k0 = t * BC;
    if (!tile_all_allowed(N, wq0, 32, k0, BC, MASK, p.wl, p.wr)) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
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
  };
  // Exact row max of the tile (rare path): raises the running max to it and
  // rescales the accumulator, l and l~.
  auto raise_max = [&](f32x16_t s[KB]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = halves_max(mx);
    const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
    const float mnew = fmaxf(m, mt);
    const float corr = (mnew > m) ? fast_exp2(m - mnew) : 1.0f;
    m = mnew;
#pragma unroll
    for (int b = 0; b < DBLK; ++b) scale_in_place(acc[b], corr);
    l *= corr;
    lr *= corr;
  };

  // Phase 2: probabilities in the exp2 domain, rounded to 16 bits in
  // B-operand order, and the lane's sum of them.  For bf16 the sum is over
  // the fp32 values (bf16 rounding, up to 2^-8 relative, is too coarse for
  // lse); for fp16 it is over the rounded values (at most 2^-11 relative,
  // well inside lse's tolerance), so that one sum serves as both l and l~.
  // prob_pair handles pair pi (0 .. 8 KB - 1: block pi / 8, elements 2j, 2j + 1).
  auto prob_pair = [&](f32x16_t s[KB], float base, uint32_t pk[KB][8], float rsum[2], int pi) {
    const int kb = pi / 8, j = pi % 8;
    const float e0 = fast_exp2(fmaf(s[kb][2 * j], c, -base));
    const float e1 = fast_exp2(fmaf(s[kb][2 * j + 1], c, -base));
    pk[kb][j] = Elem<T>::pack2(e0, e1);
    if (kOneSum)
      rsum[kb % 2] = Elem<T>::add_pair(pk[kb][j], rsum[kb % 2]);
    else
      rsum[kb % 2] += e0 + e1;
  };
  auto softmax_exp = [&](f32x16_t s[KB], float base, uint32_t pk[KB][8]) -> float {
    float rsum[2] = {0.0f, 0.0f};
#pragma unroll
    for (int pi = 0; pi < 8 * KB; ++pi) prob_pair(s, base, pk, rsum, pi);
    return rsum[0] + rsum[1];
  };

  // Phases 1 and 2 of a pipeline step as one explicitly ordered stream: the
  // scores of the next tile (two chains, one per 32-key block) with the
  // probabilities of the current tile, one pair after each matrix
  // instruction.  K operands are read two reduction steps ahead from a
  // three-deep ring; the scheduling barrier after each step keeps the
  // compiler from regrouping (left to itself it read each operand one
  // instruction ahead and waited on most reads).
  auto scores_softmax = [&](const char* kb_, f32x16_t nxt[KB], f32x16_t cur[KB], float base,
                            uint32_t pk[KB][8]) -> float {
    constexpr int PAIRS_PER_MMA = (8 + KSTEPS - 1) / KSTEPS;
    float rsum[2] = {0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) nxt[kb] = f32x16_t{};
    u32x4_t kop[3][KB];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        kop[kk][kb] = ld_lds16(kb_ + kr_off + kb * 32 * L::K_PITCH + kk * 32);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      if (kk + 2 < KSTEPS) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          kop[(kk + 2) % 3][kb] = ld_lds16(kb_ + kr_off + kb * 32 * L::K_PITCH + (kk + 2) * 32);
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        nxt[kb] = Elem<T>::mma(kop[kk % 3][kb], qf[kk], nxt[kb]);
#pragma unroll
        for (int r = 0; r < PAIRS_PER_MMA; ++r) {
          const int pi = KB * kk + kb + r * KB * KSTEPS;
          if (pi < 8 * KB) prob_pair(cur, base, pk, rsum, pi);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return rsum[0] + rsum[1];
  };

  // Phase 3: O^T += V^T P^T over four 16-key steps, the DBLK chains
  // interleaved, with V^T operands read one step ahead (double-buffered), and
  // the row sum of the rounded probabilities.
  auto pv_sums = [&](const char* vb_, uint32_t pk[KB][8]) {
    auto vread = [&](int ks, int db) {
      const char* va = vb_ + vr_off[db] + ks * 16 * L::V_PITCH;
      const u32x2_t lo2 = ld_lds_tr8(va);
      const u32x2_t hi2 = ld_lds_tr8(va + 8 * L::V_PITCH);
      return u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
    };
    u32x4_t vop[2][DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) vop[0][db] = vread(0, db);
    float rr = 0.0f;
#pragma unroll
    for (int ks = 0; ks < BC / 16; ++ks) {
      if (ks + 1 < BC / 16) {
#pragma unroll
        for (int db = 0; db < DBLK; ++db) vop[(ks + 1) % 2][db] = vread(ks + 1, db);
      }
      const u32x4_t b = {pk[ks >> 1][(ks & 1) * 4 + 0], pk[ks >> 1][(ks & 1) * 4 + 1],
                         pk[ks >> 1][(ks & 1) * 4 + 2], pk[ks >> 1][(ks & 1) * 4 + 3]};
#pragma unroll
      for (int db = 0; db < DBLK; ++db) acc[db] = Elem<T>::mma(vop[ks % 2][db], b, acc[db]);
      if (!kOneSum) {
#pragma unroll
        for (int u = 0; u < 4; ++u) rr = Elem<T>::add_pair(b[u], rr);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!kOneSum) lr += rr;
  };

  // Software pipeline.  Iteration t computes the scores of tile t+1 (K stage
  // (t+1-lo)%2) interleaved with the softmax of tile t, then the output
  // product of tile t (V stage (t-lo)%2), so the matrix cores and the vector
  // ALUs have independent work in the same instruction stream (the order is
  // fixed in scores_softmax and pv_sums).  Meanwhile K of tile t+2
  // and V of tile t+1 travel from HBM straight into the LDS stages freed one
  // iteration ago.  The scores of the (nonexistent) tile after the last are
  // computed from whatever the stage holds and never used.
  f32x16_t sA[KB], sB[KB];
  gload_k_lds(lo, k_lds0);
  gload_v_lds(lo, v_lds0);
  if (lo + 1 < hi) gload_k_lds(lo + 1, k_lds1);
  wait_vmem();
  __syncthreads();
  scores(k_lds0, sA);
  // The first step refills stage 0 with K of tile lo+2: every wavefront must
  // have read tile lo's keys from it first.
  __syncthreads();

  // One pipeline step; P = (t - lo) % 2 selects the stages at compile time.
  auto step = [&](auto P_, int t, f32x16_t cur[KB], f32x16_t nxt[KB]) {
    constexpr int P = decltype(P_)::value;
    const bool has1 = t + 1 < hi, has2 = t + 2 < hi;
    if (has2) gload_k_lds(t + 2, P ? k_lds1 : k_lds0);
    if (has1) gload_v_lds(t + 1, P ? v_lds0 : v_lds1);
    apply_mask(t, cur);
    uint32_t pk[KB][8];
    float rs = scores_softmax(P ? k_lds0 : k_lds1, nxt, cur, m == -INFINITY ? 0.0f : m, pk);
    // Optimistic softmax: the probabilities used the running max; if one of
    // them exceeds 2^kTau (their sum does) or the row has no max yet, take
    // the exact tile max, rescale and recompute (rare).
    if (__any(!(rs <= kSumBound<T>) || m == -INFINITY)) {
      raise_max(cur);
      rs = softmax_exp(cur, m == -INFINITY ? 0.0f : m, pk);
    }
    l += rs;
    pv_sums(P ? v_lds1 : v_lds0, pk);
    wait_vmem();
    __syncthreads();
  };
  for (int t = lo; t < hi; t += 2) {
    step(std::integral_constant<int, 0>{}, t, sA, sB);
    if (t + 1 >= hi) break;
    step(std::integral_constant<int, 1>{}, t + 1, sB, sA);
  }

  // Epilogue: O = acc / l~ rounded once; lse in natural-log units.  Both
  // halves of the wavefront hold the same l, l~ and m; stores past N drop.
  const float lt = halves_sum(l);
  const float lrt = kOneSum ? lt : halves_sum(lr);
  const float inv = 1.0f / lrt;
  const auto rO = make_rsrc(reinterpret_cast<char*>(p.O) + qoff, head_bytes);
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2_t v = {Elem<T>::pack2(acc[db][g * 4 + 0] * inv, acc[db][g * 4 + 1] * inv),
                         Elem<T>::pack2(acc[db][g * 4 + 2] * inv, acc[db][g * 4 + 3] * inv)};
      buf_store8(v, rO, static_cast<uint32_t>(qrow) * ROW_BYTES + (db * 32 + g * 8 + half * 4) * 2);
    }
  }
  const auto rL = make_rsrc(p.lse + hr.q_row0, static_cast<uint32_t>(N) * 4);
  buf_store4((m + log2f(lt)) * kLn2, rL, static_cast<uint32_t>(qrow) * 4);
  }
}

// A persistent launch runs as many workgroups as the chip holds at once: two
// wavefronts per SIMD, four SIMDs per compute unit.
unsigned persistent_grid(int64_t n_wg, int waves, int n_cu) {
  const int64_t resident = static_cast<int64_t>(n_cu) * (8 / waves);
  return static_cast<unsigned>(n_wg < resident ? n_wg : resident);
}

template <typename T, int D, int MASK>
hipError_t launch_one(const FwdParams& p, int64_t n_wg, int persist_cus, hipStream_t stream) {
  // Pairs help fixed-length batches (+3.4% at B4 H32 H_kv8 N4096 causal); a
  // packed batch's many short items run better in four-wavefront workgroups.
  if (MASK != kNone && fwd_waves(MASK) == 4 && p.g.group % 2 == 0 && p.g.cu_seqlens == nullptr) {
    if (persist_cus > 0)
      hipLaunchKernelGGL((fwd_kernel<T, D, MASK, true, true>),
                         dim3(persistent_grid(n_wg / 2, 8, persist_cus)), dim3(64 * 8), 0, stream, p,
                         static_cast<uint32_t>(n_wg / 2));
    else
      hipLaunchKernelGGL((fwd_kernel<T, D, MASK, true, false>), dim3(static_cast<unsigned>(n_wg / 2)),
                         dim3(64 * 8), 0, stream, p, 0u);
  } else {
    if (persist_cus > 0)
      hipLaunchKernelGGL((fwd_kernel<T, D, MASK, false, true>),
                         dim3(persistent_grid(n_wg, fwd_waves(MASK), persist_cus)),
                         dim3(64 * fwd_waves(MASK)), 0, stream, p, static_cast<uint32_t>(n_wg));
    else
      hipLaunchKernelGGL((fwd_kernel<T, D, MASK, false, false>), dim3(static_cast<unsigned>(n_wg)),
                         dim3(64 * fwd_waves(MASK)), 0, stream, p, 0u);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_mask(const FwdParams& p, int mode, int64_t n_wg, int persist_cus,
                       hipStream_t stream) {
  switch (mode) {
    case kCausal: return launch_one<T, D, kCausal>(p, n_wg, persist_cus, stream);
    case kSliding: return launch_one<T, D, kSliding>(p, n_wg, persist_cus, stream);
    default: return launch_one<T, D, kNone>(p, n_wg, persist_cus, stream);
  }
}

template <typename T>
hipError_t launch_d(const FwdParams& p, int d, int mode, int64_t n_wg, int persist_cus,
                    hipStream_t stream) {
  return d == 64 ? launch_mask<T, 64>(p, mode, n_wg, persist_cus, stream)
                 : launch_mask<T, 128>(p, mode, n_wg, persist_cus, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int dt_bf16, int d, int mode, int64_t n_wg,
                      int persist_cus, hipStream_t stream) {
  return dt_bf16 ? launch_d<__bf16>(p, d, mode, n_wg, persist_cus, stream)
                 : launch_d<_Float16>(p, d, mode, n_wg, persist_cus, stream);
}

}  // namespace attn
