// Row and tile geometry of the sparse-query prefill, shared by the forward
// and backward kernels (see prefill.hip for the packing this describes).
#pragma once

#include "gqe_internal.h"

namespace gqe {

constexpr int kKeyBlock = 64;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

struct TileCoord {
  int b, v, tile;  // tile index within (b, v)
  bool valid;
};

// Block -> tile, longest causal extent first. Routed tile t of a group covers
// rows [256t, 256t+255], i.e. tokens up to (256t+255)/k; shared tile t covers
// tokens up to 256t+255, the same extent as routed tile k*t+k-1. Tiles are
// taken in "super-rounds" sr of decreasing extent (shared tile ts =
// tiles_s-1-sr): the shared tiles ts with the routed tiles t = k*ts+k-1 of
// the same extent, then routed tiles t = k*ts+k-2, ..., k*ts. Workgroups are
// dispatched in block order and go round-robin to the 8 XCDs (block i to XCD
// i % 8), so each XCD works through its own list, longest first.
//
// When G is a multiple of 8, XCD x's list holds the routed tiles of groups
// x, x+8, ... of every sequence, plus the shared tiles (sr, b) with
// (sr + b) % 8 == x: each XCD then streams K/V of one KV head (and now and
// then head 0) through its L2, and every 8 consecutive super-rounds give
// each XCD the same work. Otherwise the super-rounds are striped over all
// XCDs. A routed index past the last routed tile (S*k not a multiple of
// 256) and the unused tail of a shorter XCD list are invalid blocks, which
// exit at once.
// The map as a function of the block index i, for the host as well (the
// tests enumerate it); kernels call tile_of_block.
__host__ __device__ inline TileCoord tile_of_index(const PrefillParams& p, int tiles_r, int tiles_s, int i) {
  TileCoord c;
  int sr, rem;
  int nsh, sh_b0, sh_bstep;   // shared tiles first in rem: b = sh_b0 + sh_bstep*r, r < nsh
  int gsel, gstride, gcount;  // routed groups of this list: gsel + gstride*j, j < gcount
  if (p.G % 8 == 0) {
    const int x = i % 8, j = i / 8;
    const int gx = p.G / 8;
    const int per = p.K * p.B * gx;  // routed entries per super-round
    // shared tiles of XCD x in super-round r: b = (x - r) mod 8, +8, ... < B
    auto cnt = [&](int r) { return (p.B + 7 - ((x - r) & 7)) / 8; };
    // start(r) = r*per + shared tiles of super-rounds < r (B per 8 of them)
    auto start = [&](int r) {
      int n = r * per + p.B * (r / 8);
      for (int q = r & ~7; q < r; ++q) n += cnt(q);
      return n;
    };
    sr = (8 * j) / (8 * per + p.B);
    while (sr > 0 && start(sr) > j) --sr;
    while (start(sr + 1) <= j) ++sr;
    rem = j - start(sr);
    nsh = cnt(sr);
    sh_b0 = (x - sr) & 7;
    sh_bstep = 8;
    gsel = x;
    gstride = 8;
    gcount = gx;
  } else {
    const int per_round = p.K * p.B * p.G + p.B;
    sr = i / per_round;
    rem = i - sr * per_round;
    nsh = p.B;
    sh_b0 = 0;
    sh_bstep = 1;
    gsel = 0;
    gstride = 1;
    gcount = p.G;
  }
  const int ts = tiles_s - 1 - sr;
  c.valid = ts >= 0;
  if (rem < nsh) {
    c.b = sh_b0 + sh_bstep * rem;
    c.v = p.G;
    c.tile = ts;
  } else {
    rem -= nsh;
    const int per_step = p.B * gcount;
    const int step = rem / per_step;
    rem -= step * per_step;
    c.b = rem / gcount;
    c.v = gsel + gstride * (rem - c.b * gcount);
    c.tile = p.K * ts + p.K - 1 - step;
    if (step >= p.K || c.tile >= tiles_r) c.valid = false;
  }
  return c;
}

__device__ __forceinline__ TileCoord tile_of_block(const PrefillParams& p, int tiles_r, int tiles_s) {
  return tile_of_index(p, tiles_r, tiles_s, blockIdx.x);
}

// Grid size for tile_of_block: 8 lists of tiles_s super-rounds, or striped
// super-rounds (8 lists are at most this long).
inline int tile_grid_blocks(const PrefillParams& p, int tiles_s) {
  return (p.G % 8 == 0) ? 8 * (tiles_s * p.K * p.B * (p.G / 8) + p.B * ((tiles_s + 7) / 8))
                        : tiles_s * (p.K * p.B * p.G + p.B);
}

// Row r of (b, v) -> token position, slot, query head.
__device__ __forceinline__ void row_info(const PrefillParams& p, int b, int v, int r, int& pos,
                                         int& slot, int& head) {
  if (v == p.G) {
    pos = r;
    slot = 0;
    head = p.N;
  } else {
    pos = r / p.K;
    slot = r - pos * p.K;
    // (an index outside 0..M-1 breaks the caller's contract; clamping keeps
    // the row's query read inside q, the row's outputs are then unspecified)
    head = v * p.M + min(max(p.topk[(((int64_t)b * p.S + pos) * p.G + v) * p.K + slot], 0), p.M - 1);
  }
}

}  // namespace gqe
