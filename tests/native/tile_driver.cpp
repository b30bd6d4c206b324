// Host driver for the tile classifier in causal_attention_fa2_amd/csrc/tiles.h (CPU test only).
// stdin: lines "Sq Sk BR BC causal window sink"; the functions are called the way the kernels call
// them (query rows shifted to key positions by off = Sk - Sq). stdout per config: "R qt ns lo hi"
// for every query tile, "C kt lo hi" for every key tile, "V" and one character per (row, key) of visible(),
// then one line of block classes (E empty / F full / P partial) for every (query tile, key tile)
// pair, row-major.
#include <cstdio>
#include "tiles.h"

int main() {
  int sq, sk, br, bc, causal, window, sink;
  while (std::scanf("%d %d %d %d %d %d %d", &sq, &sk, &br, &bc, &causal, &window, &sink) == 7) {
    const int off = sk - sq;
    const int nq = (sq + br - 1) / br, nk = (sk + bc - 1) / bc;
    std::printf("CFG %d %d %d %d %d %d %d\n", sq, sk, br, bc, causal, window, sink);
    for (int qt = 0; qt < nq; ++qt) {
      int ns, lo, hi;
      fa::kv_tile_range(qt * br + off, fa::imin_(qt * br + br - 1, sq - 1) + off, sk, bc, causal, window,
                        sink, &ns, &lo, &hi);
      std::printf("R %d %d %d %d\n", qt, ns, lo, hi);
    }
    for (int kt = 0; kt < nk; ++kt) {
      int lo, hi;
      fa::q_tile_range(kt * bc, fa::imin_(kt * bc + bc - 1, sk - 1), sk, off, br, causal, window, sink, &lo,
                       &hi);
      std::printf("C %d %d %d\n", kt, lo, hi);
    }
    std::printf("V ");
    for (int i = 0; i < sq; ++i)
      for (int j = 0; j < sk; ++j) std::putchar(fa::visible(i + off, j, sk, causal, window, sink) ? '1' : '0');
    std::printf("\nB ");
    for (int qt = 0; qt < nq; ++qt)
      for (int kt = 0; kt < nk; ++kt) {
        const int r0 = qt * br + off, r1 = r0 + br - 1, c0 = kt * bc, c1 = c0 + bc - 1;
        const bool e = fa::block_empty(r0, r1, c0, c1, sk, causal, window, sink);
        const bool f = fa::block_full(r0, r1, c0, c1, sk, causal, window, sink);
        std::putchar(e ? (f ? '!' : 'E') : (f ? 'F' : 'P'));
      }
    std::printf("\n");
  }
  return 0;
}
