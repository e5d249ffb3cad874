// plan_check.cpp -- host-only brute-force checks of the tile geometry in
// plan.hpp and of the validation in validate.cpp.  Built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_native.py.
//
// For every small N, tile shape and mask it enumerates the allowed (query,
// key) pairs directly from the mask rule (none: all; causal: j <= i;
// sliding: i - wl <= j <= i + wr) and checks:
//   * kv_tile_range / q_tile_range visit exactly the tiles holding at least
//     one allowed pair (the allowed tiles of a block form one interval);
//   * tile_all_allowed / tile_none_allowed agree with the enumeration;
//   * xcd_remap is a bijection and gives each die a contiguous run;
//   * query_head_rows / kv_head_rows map grouped-query heads to their
//     key/value heads (query head h of a batch entry or sequence reads
//     key/value head h / group) and packed sequences to their rows, and keep
//     every head inside its tensor whatever row offsets they are given.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "attn.h"
#include "plan.hpp"
#include "validate.hpp"

using namespace attn;

static int failures = 0;
#define CHECK(cond, ...)                          \
  do {                                            \
    if (!(cond)) {                                \
      if (failures < 20) {                        \
        std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
        std::printf(__VA_ARGS__);                 \
        std::printf("\n");                        \
      }                                           \
      ++failures;                                 \
    }                                             \
  } while (0)

static bool allowed(int64_t i, int64_t j, int64_t N, int mode, int64_t wl, int64_t wr) {
  if (i < 0 || j < 0 || i >= N || j >= N) return false;
  if (mode == kCausal) return j <= i;
  if (mode == kSliding) return j >= i - wl && j <= i + wr;
  return true;
}

static void check_block(int64_t N, int64_t q0, int64_t nq, int64_t k0, int64_t nk, int mode,
                        int64_t wl, int64_t wr) {
  bool any = false, all = true;
  for (int64_t i = q0; i < q0 + nq; ++i) {
    for (int64_t j = k0; j < k0 + nk; ++j) {
      bool a = allowed(i, j, N, mode, wl, wr);
      if (i < N) {  // padding query rows never count
        any = any || a;
        all = all && a;
      }
    }
  }
  if (q0 >= N) all = false;  // no real rows: never claimed "all"
  bool none_k = tile_none_allowed(N, q0, nq, k0, nk, mode, wl, wr);
  bool all_k = tile_all_allowed(N, q0, nq, k0, nk, mode, wl, wr);
  CHECK(none_k == !any, "none N=%lld q0=%lld nq=%lld k0=%lld nk=%lld mode=%d wl=%lld wr=%lld",
        (long long)N, (long long)q0, (long long)nq, (long long)k0, (long long)nk, mode,
        (long long)wl, (long long)wr);
  if (q0 < N) {
    CHECK(all_k == all, "all N=%lld q0=%lld nq=%lld k0=%lld nk=%lld mode=%d wl=%lld wr=%lld got %d",
          (long long)N, (long long)q0, (long long)nq, (long long)k0, (long long)nk, mode,
          (long long)wl, (long long)wr, (int)all_k);
  }
}

int main() {
  const int modes[3] = {kNone, kCausal, kSliding};
  const int64_t windows[][2] = {{0, 0}, {1, 0}, {0, 1}, {3, 2}, {5, 40}, {63, 0}, {64, 0},
                                {65, 0}, {127, 1}, {128, 128}, {200, 0}, {1000, 1000}};
  const int64_t Ns[] = {1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 200, 257};
  const int64_t shapes[][2] = {{128, 64}, {64, 64}, {32, 32}, {16, 48}, {1, 1}, {128, 128}};
  for (int64_t N : Ns) {
    for (int mi = 0; mi < 3; ++mi) {
      const int mode = modes[mi];
      const int nw = mode == kSliding ? int(sizeof(windows) / sizeof(windows[0])) : 1;
      for (int wi = 0; wi < nw; ++wi) {
        const int64_t wl = imin(windows[wi][0], N), wr = imin(windows[wi][1], N);
        for (auto& sh : shapes) {
          const int64_t bq = sh[0], bk = sh[1];
          // kv_tile_range against enumeration
          for (int64_t q0 = 0; q0 < N; q0 += bq) {
            int64_t lo, hi;
            kv_tile_range(N, q0, bq, bk, mode, wl, wr, &lo, &hi);
            int64_t first = -1, last = -1;
            for (int64_t t = 0; t * bk < N; ++t) {
              bool any = false;
              for (int64_t i = q0; i < imin(q0 + bq, N); ++i)
                for (int64_t j = t * bk; j < imin(t * bk + bk, N); ++j)
                  any = any || allowed(i, j, N, mode, wl, wr);
              if (any) {
                if (first < 0) first = t;
                CHECK(last < 0 || last == t - 1, "allowed tiles not contiguous");
                last = t;
              }
            }
            CHECK(first == lo && last + 1 == hi,
                  "kv range N=%lld q0=%lld bq=%lld bk=%lld mode=%d wl=%lld wr=%lld: [%lld,%lld) vs [%lld,%lld]",
                  (long long)N, (long long)q0, (long long)bq, (long long)bk, mode, (long long)wl,
                  (long long)wr, (long long)lo, (long long)hi, (long long)first, (long long)last);
            for (int64_t t = lo; t < hi; ++t) check_block(N, q0, bq, t * bk, bk, mode, wl, wr);
            // a 32-row sub-block (one wavefront) against every tile
            for (int64_t t = 0; t * bk < N; ++t) check_block(N, q0, 32, t * bk, bk, mode, wl, wr);
          }
          // q_tile_range against enumeration
          for (int64_t k0 = 0; k0 < N; k0 += bk) {
            int64_t lo, hi;
            q_tile_range(N, k0, bk, bq, mode, wl, wr, &lo, &hi);
            int64_t first = -1, last = -1;
            for (int64_t t = 0; t * bq < N; ++t) {
              bool any = false;
              for (int64_t i = t * bq; i < imin(t * bq + bq, N); ++i)
                for (int64_t j = k0; j < imin(k0 + bk, N); ++j)
                  any = any || allowed(i, j, N, mode, wl, wr);
              if (any) {
                if (first < 0) first = t;
                last = t;
              }
            }
            CHECK(first == lo && last + 1 == hi, "q range N=%lld k0=%lld mode=%d",
                  (long long)N, (long long)k0, mode);
          }
        }
      }
    }
  }
  // xcd_remap: bijection with contiguous per-die runs
  for (int64_t n = 1; n <= 300; ++n) {
    std::vector<int> seen(n, 0);
    for (int64_t w = 0; w < n; ++w) {
      int64_t it = xcd_remap(w, n);
      CHECK(it >= 0 && it < n, "remap range");
      if (it >= 0 && it < n) seen[it]++;
      if (w >= kNumXcd) CHECK(xcd_remap(w, n) == xcd_remap(w - kNumXcd, n) + 1, "die run");
    }
    for (int64_t i = 0; i < n; ++i) CHECK(seen[i] == 1, "remap not a bijection n=%lld", (long long)n);
  }
  // packed_work_item: a bijection onto (head, block); with a head count that
  // is a multiple of 8 each die gets heads/8 consecutive heads of every
  // sequence, and every die's items run block by block in the stated order.
  for (int64_t heads : {1, 2, 3, 8, 16, 24, 40}) {
    for (int64_t n_seqs : {1, 2, 5}) {
      for (int64_t n_blk : {1, 3, 7}) {
        for (int asc = 0; asc < 2; ++asc) {
          const int64_t n = heads * n_seqs * n_blk;
          std::vector<int> seen(n, 0);
          std::vector<int64_t> last_blk(kNumXcd, asc ? -1 : n_blk);
          for (int64_t w = 0; w < n; ++w) {
            int64_t x, b;
            packed_work_item<int64_t>(w, heads, n_seqs, n_blk, asc != 0, &x, &b);
            CHECK(x >= 0 && x < heads * n_seqs && b >= 0 && b < n_blk, "packed item range");
            if (x < 0 || x >= heads * n_seqs || b < 0 || b >= n_blk) continue;
            seen[b * heads * n_seqs + x]++;
            const int64_t die = w % kNumXcd;
            if (heads % kNumXcd == 0)
              CHECK((x % heads) / (heads / kNumXcd) == die, "packed head on its die");
            CHECK(asc ? b >= last_blk[die] : b <= last_blk[die], "packed block order");
            last_blk[die] = b;
          }
          for (int64_t i = 0; i < n; ++i) CHECK(seen[i] == 1, "packed order not a bijection");
        }
      }
    }
  }
  // Head mapping, fixed-length batches: B x H query heads over B x H_kv
  // key/value heads, every row of a head.
  for (int64_t H = 1; H <= 12; ++H) {
    for (int64_t H_kv = 1; H_kv <= H; ++H_kv) {
      if (H % H_kv) continue;
      const int64_t group = H / H_kv, B = 3, rows = 5;
      for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h) {
          const HeadRows r = query_head_rows<int64_t>(b * H + h, H, group, rows, false, 0, 0);
          CHECK(r.q_row0 == (b * H + h) * rows && r.len == rows, "fixed q rows H=%lld", (long long)H);
          CHECK(r.kv_row0 == (b * H_kv + h / group) * rows, "fixed kv head H=%lld H_kv=%lld",
                (long long)H, (long long)H_kv);
        }
      for (int64_t y = 0; y < B * H_kv; ++y) {
        const KvHeadRows k = kv_head_rows<int64_t>(y, H_kv, group, rows, false, 0, 0);
        CHECK(k.kv_row0 == y * rows && k.len == rows, "fixed kv rows");
        for (int64_t g = 0; g < group; ++g) {
          // member g of the group is the query head that reads this key/value head
          const int64_t x = (y / H_kv) * H + (y % H_kv) * group + g;
          const HeadRows r = query_head_rows<int64_t>(x, H, group, rows, false, 0, 0);
          CHECK(r.kv_row0 == k.kv_row0 && r.q_row0 == k.q_row0 + g * k.q_stride, "fixed group");
        }
      }
    }
  }
  // Packed batches: sequence offsets, including malformed ones, stay inside
  // the head's T rows.
  {
    const int64_t T = 20;
    const int64_t offs[][2] = {{0, 20}, {0, 0}, {3, 9}, {19, 20}, {-5, 4}, {7, 3},
                               {15, 40}, {25, 30}, {-9, -2}, {20, 20}};
    for (auto& o : offs) {
      for (int64_t H = 1; H <= 6; ++H)
        for (int64_t H_kv = 1; H_kv <= H; ++H_kv) {
          if (H % H_kv) continue;
          const int64_t group = H / H_kv, n_seqs = 2;
          for (int64_t x = 0; x < n_seqs * H; ++x) {
            const HeadRows r = query_head_rows<int64_t>(x, H, group, T, true, o[0], o[1]);
            const int64_t h = x % H;
            CHECK(r.len >= 0 && r.q_row0 >= h * T && r.q_row0 + r.len <= (h + 1) * T,
                  "packed q rows inside head");
            CHECK(r.kv_row0 >= (h / group) * T && r.kv_row0 + r.len <= (h / group + 1) * T,
                  "packed kv rows inside head");
            CHECK(r.q_row0 - h * T == r.kv_row0 - (h / group) * T, "same sequence rows");
            if (o[0] >= 0 && o[0] <= o[1] && o[1] <= T)
              CHECK(r.q_row0 == h * T + o[0] && r.len == o[1] - o[0], "well-formed offsets");
          }
          for (int64_t y = 0; y < n_seqs * H_kv; ++y) {
            const KvHeadRows k = kv_head_rows<int64_t>(y, H_kv, group, T, true, o[0], o[1]);
            const int64_t kvh = y % H_kv;
            CHECK(k.len >= 0 && k.kv_row0 >= kvh * T && k.kv_row0 + k.len <= (kvh + 1) * T,
                  "packed kv-major rows inside head");
            for (int64_t g = 0; g < group; ++g) {
              const int64_t h = kvh * group + g;
              const HeadRows r = query_head_rows<int64_t>((y / H_kv) * H + h, H, group, T, true, o[0], o[1]);
              CHECK(r.q_row0 == k.q_row0 + g * k.q_stride && r.kv_row0 == k.kv_row0 &&
                        r.len == k.len, "packed group member");
            }
          }
        }
    }
  }
  // Validation: null, sizes, masks, scale, alignment, aliasing.
  char* base = static_cast<char*>(std::aligned_alloc(256, 1 << 17));
  const void *Q = base, *K = base + 4096, *V = base + 8192;
  void* O = base + 12288;
  float* L = reinterpret_cast<float*>(base + 16384);
  const int64_t B = 1, H = 2, N = 8, d = 64;  // 2 KiB per tensor
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, O, L, B, H, N, d, 0.125f, ATTN_MASK_NONE, 0, 0) == ATTN_OK, "ok");
  CHECK(attn_fwd_check(ATTN_BF16, nullptr, K, V, O, L, B, H, N, d, 0.1f, ATTN_MASK_NONE, 0, 0) == ATTN_E_NULLPTR, "null");
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, O, L, B, H, N, 96, 0.1f, ATTN_MASK_NONE, 0, 0) == ATTN_E_UNSUPPORTED, "d");
  CHECK(attn_fwd_check((attn_dtype)7, Q, K, V, O, L, B, H, N, d, 0.1f, ATTN_MASK_NONE, 0, 0) == ATTN_E_UNSUPPORTED, "dt");
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, O, L, 0, H, N, d, 0.1f, ATTN_MASK_NONE, 0, 0) == ATTN_E_SHAPE, "B");
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, O, L, B, H, INT64_MAX, d, 0.1f, ATTN_MASK_NONE, 0, 0) == ATTN_E_SHAPE, "N");
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, O, L, INT64_MAX / 2, INT64_MAX / 2, N, d, 0.1f, ATTN_MASK_NONE, 0, 0) == ATTN_E_SHAPE, "BH");
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, O, L, B, H, 8388608, 128, 0.1f, ATTN_MASK_NONE, 0, 0) == ATTN_E_SHAPE, "head bytes");
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, O, L, B, H, 8388607, 128, 0.1f, ATTN_MASK_NONE, 0, 0) == ATTN_E_ALIAS, "head bytes ok (then aliasing of the tiny test buffers)");
  // Launch width: B*H*N*d/8 threads (the backward's row dots) must stay below 2^32.
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, O, L, 64, 1, 4194304, 128, 0.1f, ATTN_MASK_NONE, 0, 0) == ATTN_E_SHAPE, "threads d128");
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, O, L, 63, 1, 4194304, 128, 0.1f, ATTN_MASK_NONE, 0, 0) == ATTN_E_ALIAS, "threads d128 ok");
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, O, L, 64, 1, 8388607, 64, 0.1f, ATTN_MASK_NONE, 0, 0) == ATTN_E_SHAPE, "threads d64");
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, O, L, B, H, N, d, 0.1f, ATTN_MASK_SLIDING, -1, 0) == ATTN_E_MASK, "wl");
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, O, L, B, H, N, d, 0.1f, (attn_mask_mode)9, 0, 0) == ATTN_E_MASK, "mode");
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, O, L, B, H, N, d, 0.1f, ATTN_MASK_CAUSAL, -5, -5) == ATTN_OK, "windows ignored");
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, O, L, B, H, N, d, 0.0f / 0.0f, ATTN_MASK_NONE, 0, 0) == ATTN_E_SCALE, "nan");
  CHECK(attn_fwd_check(ATTN_BF16, base + 8, K, V, O, L, B, H, N, d, 0.1f, ATTN_MASK_NONE, 0, 0) == ATTN_E_ALIGN, "align");
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, base + 4096 + 2048 - 16, L, B, H, N, d, 0.1f, ATTN_MASK_NONE, 0, 0) == ATTN_E_ALIAS, "alias O/K");
  CHECK(attn_fwd_check(ATTN_BF16, Q, K, V, O, reinterpret_cast<float*>(base + 12288 + 1024), B, H, N, d, 0.1f, ATTN_MASK_NONE, 0, 0) == ATTN_E_ALIAS, "alias O/lse");
  CHECK(attn_fwd_check(ATTN_BF16, Q, Q, Q, O, L, B, H, N, d, 0.1f, ATTN_MASK_NONE, 0, 0) == ATTN_OK, "inputs may alias");
  const size_t ws = attn_bwd_workspace_bytes(ATTN_F16, B, H, N, d);
  CHECK(ws == 512, "workspace %zu", ws);
  void *dQ = base + 20480, *dK = base + 24576, *dV = base + 28672, *W = base + 32768;
  CHECK(attn_bwd_check(ATTN_F16, Q, K, V, O, L, O, dQ, dK, dV, W, ws, B, H, N, d, 0.1f, ATTN_MASK_CAUSAL, 0, 0) == ATTN_OK, "bwd ok");
  CHECK(attn_bwd_check(ATTN_F16, Q, K, V, O, L, O, dQ, dK, dV, W, ws - 1, B, H, N, d, 0.1f, ATTN_MASK_CAUSAL, 0, 0) == ATTN_E_WORKSPACE, "bwd ws");
  CHECK(attn_bwd_check(ATTN_F16, Q, K, V, O, L, O, dQ, dK, dV, nullptr, ws, B, H, N, d, 0.1f, ATTN_MASK_CAUSAL, 0, 0) == ATTN_E_NULLPTR, "bwd ws null");
  CHECK(attn_bwd_check(ATTN_F16, Q, K, V, O, L, O, dQ, dQ, dV, W, ws, B, H, N, d, 0.1f, ATTN_MASK_CAUSAL, 0, 0) == ATTN_E_ALIAS, "bwd alias");
  CHECK(attn_bwd_check(ATTN_F16, Q, K, V, O, L, O, dQ, dK, dV, const_cast<void*>(Q), ws, B, H, N, d, 0.1f, ATTN_MASK_CAUSAL, 0, 0) == ATTN_E_ALIAS, "bwd ws alias");
  // Grouped-query and packed geometries (the validation every entry point runs).
  {
    // Fixed-length GQA: B = 1, H = 4, H_kv = 2, N = 8, d = 64: Q/O 4 KiB, K/V 2 KiB.
    const Geometry g = fixed_geometry(1, 4, 2, 8, 64);
    char* q = base + 4096 * 8;
    const void *gk = q + 4096, *gv = q + 6144;
    void* go = q + 8192;
    float* gl = reinterpret_cast<float*>(q + 12288);
    CHECK(fwd_check_g(ATTN_F16, q, gk, gv, go, gl, nullptr, g, 0.1f, 0, 0, 0) == ATTN_OK, "gqa ok");
    CHECK(fwd_check_g(ATTN_F16, q, gk, gv, q + 6144 + 1024, gl, nullptr, g, 0.1f, 0, 0, 0) == ATTN_E_ALIAS, "gqa V sized by H_kv");
    CHECK(fwd_check_g(ATTN_F16, q, gk, gv, q + 6144 + 2048, gl, nullptr, g, 0.1f, 0, 0, 0) == ATTN_OK, "gqa V ends where O starts");
    CHECK(fwd_check_g(ATTN_F16, q, gk, gv, go, gl, nullptr, fixed_geometry(1, 6, 4, 8, 64), 0.1f, 0, 0, 0) == ATTN_E_SHAPE, "H not a multiple of H_kv");
    CHECK(fwd_check_g(ATTN_F16, q, gk, gv, go, gl, nullptr, fixed_geometry(1, 2, 4, 8, 64), 0.1f, 0, 0, 0) == ATTN_E_SHAPE, "H_kv > H");
    CHECK(fwd_check_g(ATTN_F16, q, gk, gv, go, gl, nullptr, fixed_geometry(1, 4, 0, 8, 64), 0.1f, 0, 0, 0) == ATTN_E_SHAPE, "H_kv 0");
    // Packed: n_seqs = 3, T = 8, max_len 5, H = 4, H_kv = 1.
    const Geometry pg{3, 4, 1, 8, 5, 64, true};
    const int32_t* cu = reinterpret_cast<const int32_t*>(q + 16384);
    CHECK(fwd_check_g(ATTN_F16, q, gk, gv, go, gl, cu, pg, 0.1f, 1, 0, 0) == ATTN_OK, "packed ok");
    CHECK(fwd_check_g(ATTN_F16, q, gk, gv, go, gl, nullptr, pg, 0.1f, 1, 0, 0) == ATTN_E_NULLPTR, "packed cu null");
    CHECK(fwd_check_g(ATTN_F16, q, gk, gv, go, gl, reinterpret_cast<const int32_t*>(q + 16386), pg, 0.1f, 1, 0, 0) == ATTN_E_ALIGN, "packed cu align");
    CHECK(fwd_check_g(ATTN_F16, q, gk, gv, go, gl, reinterpret_cast<const int32_t*>(q + 16388), pg, 0.1f, 1, 0, 0) == ATTN_OK, "packed cu 4-byte aligned");
    CHECK(fwd_check_g(ATTN_F16, q, gk, gv, go, gl, reinterpret_cast<const int32_t*>(q + 12288), pg, 0.1f, 1, 0, 0) == ATTN_E_ALIAS, "packed cu under lse");
    CHECK(fwd_check_g(ATTN_F16, q, gk, gv, go, gl, cu, Geometry{3, 4, 1, 8, 9, 64, true}, 0.1f, 1, 0, 0) == ATTN_E_SHAPE, "max_len > T");
    CHECK(fwd_check_g(ATTN_F16, q, gk, gv, go, gl, cu, Geometry{0, 4, 1, 8, 5, 64, true}, 0.1f, 1, 0, 0) == ATTN_E_SHAPE, "no sequences");
    // H = 4 query heads on one key/value head with a single key block: the
    // group is split in 4, so the workspace adds 2 x 4 x 8 x 64 fp32 partials.
    const size_t pws = attn_bwd_varlen_workspace_bytes(ATTN_F16, 3, 5, 8, 4, 1, 64);
    CHECK(pws == 2 * 256 + 2 * 4 * 8 * 64 * 4, "packed split workspace %zu", pws);
    CHECK(attn_bwd_gqa_workspace_bytes(ATTN_F16, 1, 4, 4, 8, 64) == attn_bwd_workspace_bytes(ATTN_F16, 1, 4, 8, 64), "no split without groups");
    void* W2 = q + 40960;
    CHECK(bwd_check_g(ATTN_F16, q, gk, gv, go, gl, go, q + 24576, q + 28672, q + 30720, W2, pws, cu, pg, 0.1f, 1, 0, 0) == ATTN_OK, "packed bwd ok");
    CHECK(bwd_check_g(ATTN_F16, q, gk, gv, go, gl, go, q + 24576, q + 28672, q + 30720, W2, pws - 4, cu, pg, 0.1f, 1, 0, 0) == ATTN_E_WORKSPACE, "packed bwd ws");
    CHECK(bwd_check_g(ATTN_F16, q, gk, gv, go, gl, go, q + 24576, q + 28672, q + 28672 + 512, W2, pws, cu, pg, 0.1f, 1, 0, 0) == ATTN_E_ALIAS, "packed dK/dV overlap");
    CHECK(bwd_check_g(ATTN_F16, q, gk, gv, go, gl, go, q + 24576, q + 28672, q + 28672 + 1024, W2, pws, cu, pg, 0.1f, 1, 0, 0) == ATTN_OK, "packed dK/dV sized by H_kv");
  }
  for (int s = 0; s <= 9; ++s) CHECK(attn_status_str(static_cast<attn_status>(s)) != nullptr, "str");
  std::free(base);
  std::printf("plan_check: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
