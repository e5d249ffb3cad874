// decode.hpp -- split-KV decoding over a paged K/V cache: parameters and the
// host/device planning arithmetic.
//
// P1 = ai6s.net/6af30f4d40858c2d8819b6d5.html §5 names split-KV decoding
// (Flash-Decoding) and the paged K/V cache among FlashAttention's
// extensions; the layout and split rules below are this library's.
//
// A decode call attends n_q new query tokens per sequence (the sequence's
// last n_q positions) to that sequence's cached keys.  The cache is a pool of
// pages, K and V each [n_pages, H_kv, page_size, d]; sequence s's key j lives
// in page block_table[s][j / page_size] at row j % page_size.  page_size is a
// multiple of the 64-key tile, so a tile never straddles two pages.  The
// query rows that read one key/value head (group * n_q of them: the group's
// query heads times the new tokens) are handled together in tiles of 32
// rows, and a sequence's keys are split into chunks processed by separate
// workgroups whose partial results a combine kernel merges by the
// online-softmax rule (P1 §2.3): lse = log2 sum 2^lse_k, O = sum 2^(lse_k -
// lse) O_k.
#pragma once

#include <stdint.h>

#include "plan.hpp"

namespace attn {

constexpr int kDecTileK = 64;      // keys per tile
constexpr int kDecWaves = 2;       // wavefronts per workgroup, 32 keys of each tile each
constexpr int kDecRows = 32;       // query rows per workgroup
constexpr int kDecTargetWg = 512;  // workgroups to aim for (two per compute unit)

// Query-row tiles per (sequence, key/value head).
ATTN_HD int64_t dec_row_tiles(int64_t group, int64_t n_q) {
  return ceil_div(group * n_q, kDecRows);
}

// Keys per split (a multiple of the tile) and the number of splits of the
// longest sequence: enough splits that the launch has about kDecTargetWg
// workgroups, never more than one per tile.
ATTN_HD void dec_plan(int64_t n_seqs, int64_t H_kv, int64_t row_tiles, int64_t max_seqlen,
                      int64_t* n_splits, int64_t* chunk) {
  const int64_t tiles = ceil_div(max_seqlen, kDecTileK);
  int64_t want = ceil_div(kDecTargetWg, n_seqs * H_kv * row_tiles);
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const int64_t per = ceil_div(tiles, want);
  *chunk = per * kDecTileK;
  *n_splits = ceil_div(tiles, per);
}

struct DecParams {
  const void* Q;     // [n_seqs, H, n_q, d]
  const void* K;     // [n_pages, H_kv, page_size, d]
  const void* V;
  void* O;           // [n_seqs, H, n_q, d]
  float* lse;        // [n_seqs, H, n_q]
  const int32_t* block_table;  // [n_seqs, max_pages]
  const int32_t* seq_lens;     // [n_seqs]
  float* part_o;     // n_splits > 1: [n_seqs * H_kv * row_tiles * n_splits][32][d]
  float* part_lse;   // likewise [..][32], base-2 units
  int n_seqs, H, H_kv, group, n_q;
  int page_size, n_pages, max_pages;
  int row_tiles, n_splits, chunk;
  int wl, wr;        // windows clipped to the largest cache length (sliding only)
  float c;           // |scale| * log2(e), at least 1e-30
  uint32_t qsign;    // sign flip folded into Q for negative scales
};

}  // namespace attn
