// Host enumeration of the prefill's block -> tile map (prefill_tiles.h:
// tile_of_index and tile_grid_blocks, the functions the prefill kernels and
// the attention backward's dQ kernel use). For every shape in a grid of
// batch sizes, lengths, group counts and top-k values it checks that
//   - every (sequence, virtual group, tile) is produced by exactly one block
//     and every valid block names an existing tile;
//   - blocks come longest causal extent first: along each XCD's list
//     (blocks i, i + 8, ...) the last token position a tile covers never
//     increases;
//   - with G a multiple of 8, routed tiles of group v go to XCD v % 8.
// Prints one line per failing shape and "tile map ok: <n> shapes" at the end;
// exits 1 on any failure. Test infrastructure, built on the host only.
#include <climits>
#include <cstdio>
#include <vector>

#include "prefill_tiles.h"

using gqe::PrefillParams;
using gqe::TileCoord;

static int check(int B, int S, int G, int K) {
  PrefillParams p{};
  p.B = B;
  p.S = S;
  p.G = G;
  p.K = K;
  p.M = K;
  p.N = G * K;
  constexpr int TR = 256;
  const int tiles_r = (S * K + TR - 1) / TR, tiles_s = (S + TR - 1) / TR;
  const int nblk = gqe::tile_grid_blocks(p, tiles_s);
  const int tmax = tiles_r > tiles_s ? tiles_r : tiles_s;
  std::vector<int> cnt((size_t)B * (G + 1) * tmax, 0);
  // last token position a tile covers (its causal extent)
  auto extent = [&](int v, int tile) {
    if (v == G) return (TR * tile + TR - 1 < S - 1 ? TR * tile + TR - 1 : S - 1);
    const int last_row = TR * tile + TR - 1 < S * K - 1 ? TR * tile + TR - 1 : S * K - 1;
    return last_row / K;
  };
  int bad = 0;
  int last_ext[8];
  for (int x = 0; x < 8; ++x) last_ext[x] = INT_MAX;
  for (int i = 0; i < nblk; ++i) {
    const TileCoord c = gqe::tile_of_index(p, tiles_r, tiles_s, i);
    if (!c.valid) continue;
    const int lim = c.v == G ? tiles_s : tiles_r;
    if (c.b < 0 || c.b >= B || c.v < 0 || c.v > G || c.tile < 0 || c.tile >= lim) {
      if (bad++ < 3) printf("B=%d S=%d G=%d K=%d: block %d names (b=%d, v=%d, tile=%d) out of range\n", B, S, G, K, i,
                            c.b, c.v, c.tile);
      continue;
    }
    ++cnt[((size_t)c.b * (G + 1) + c.v) * tmax + c.tile];
    if (G % 8 == 0 && c.v < G && i % 8 != c.v % 8 && bad++ < 3)
      printf("B=%d S=%d G=%d K=%d: block %d (group %d) not on XCD %d\n", B, S, G, K, i, c.v, c.v % 8);
    const int e = extent(c.v, c.tile);
    if (e > last_ext[i % 8] && bad++ < 3)
      printf("B=%d S=%d G=%d K=%d: block %d extent %d after %d on XCD %d\n", B, S, G, K, i, e, last_ext[i % 8],
             i % 8);
    last_ext[i % 8] = e;
  }
  for (int b = 0; b < B; ++b)
    for (int v = 0; v <= G; ++v)
      for (int t = 0; t < (v == G ? tiles_s : tiles_r); ++t) {
        const int n = cnt[((size_t)b * (G + 1) + v) * tmax + t];
        if (n != 1 && bad++ < 3)
          printf("B=%d S=%d G=%d K=%d: tile (b=%d, v=%d, tile=%d) produced %d times\n", B, S, G, K, b, v, t, n);
      }
  return bad;
}

int main() {
  const int Bs[] = {1, 2, 3, 7, 8, 9, 16};
  const int Ss[] = {1, 2, 100, 255, 256, 257, 1000, 2048, 8205};
  const int Gs[] = {1, 2, 3, 5, 8, 16, 24};
  const int Ks[] = {1, 2, 3, 4};
  int shapes = 0, failed = 0;
  for (int B : Bs)
    for (int S : Ss)
      for (int G : Gs)
        for (int K : Ks) {
          ++shapes;
          if (check(B, S, G, K)) ++failed;
        }
  if (failed) {
    printf("tile map: %d of %d shapes failed\n", failed, shapes);
    return 1;
  }
  printf("tile map ok: %d shapes\n", shapes);
  return 0;
}
