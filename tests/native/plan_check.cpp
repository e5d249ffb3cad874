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
//   * xcd_remap is a bijection and gives each die a contiguous run.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "attn.h"
#include "plan.hpp"

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
  // Validation: null, sizes, masks, scale, alignment, aliasing.
  char* base = static_cast<char*>(std::aligned_alloc(256, 1 << 16));
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
  for (int s = 0; s <= 9; ++s) CHECK(attn_status_str(static_cast<attn_status>(s)) != nullptr, "str");
  std::free(base);
  std::printf("plan_check: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
