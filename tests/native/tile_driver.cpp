// Host driver for the tile classifier in causal_attention_fa2_amd/csrc/tiles.h (CPU test only).
// stdin: lines "S BR BC causal window"; stdout per config: "R qt lo hi" for every query tile,
// "C kt lo hi" for every key tile, then one line of block classes (E empty / F full / P partial)
// for every (query tile, key tile) pair, row-major.
#include <cstdio>
#include "tiles.h"

int main() {
  int S, br, bc, causal, window;
  while (std::scanf("%d %d %d %d %d", &S, &br, &bc, &causal, &window) == 5) {
    const int nq = (S + br - 1) / br, nk = (S + bc - 1) / bc;
    std::printf("CFG %d %d %d %d %d\n", S, br, bc, causal, window);
    for (int qt = 0; qt < nq; ++qt) {
      int lo, hi;
      fa::kv_tile_range(qt * br, fa::imin_(qt * br + br - 1, S - 1), S, bc, causal, window, &lo, &hi);
      std::printf("R %d %d %d\n", qt, lo, hi);
    }
    for (int kt = 0; kt < nk; ++kt) {
      int lo, hi;
      fa::q_tile_range(kt * bc, fa::imin_(kt * bc + bc - 1, S - 1), S, br, causal, window, &lo, &hi);
      std::printf("C %d %d %d\n", kt, lo, hi);
    }
    std::printf("B ");
    for (int qt = 0; qt < nq; ++qt)
      for (int kt = 0; kt < nk; ++kt) {
        const int r0 = qt * br, r1 = r0 + br - 1, c0 = kt * bc, c1 = c0 + bc - 1;
        const bool e = fa::block_empty(r0, r1, c0, c1, S, causal, window);
        const bool f = fa::block_full(r0, r1, c0, c1, S, causal, window);
        std::putchar(e ? (f ? '!' : 'E') : (f ? 'F' : 'P'));
      }
    std::printf("\n");
  }
  return 0;
}
