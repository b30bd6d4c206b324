// Host build of the stored-dS layout (DsMap in launch.h): for each line "Sq Sk causal Hq Hkv B" of
// stdin, prints the region size and, for every (batch x KV head, head in group, query block, key
// block), whether the block is stored and its byte offset.
#include <cstdio>

#include "launch.h"

int main() {
  int Sq, Sk, causal, Hq, Hkv, B;
  while (std::scanf("%d %d %d %d %d %d", &Sq, &Sk, &causal, &Hq, &Hkv, &B) == 6) {
    const fa::DsMap m = fa::ds_map(Hq, Hkv, Sq, Sk, causal);
    std::printf("CFG %d %d %d %d %d %d %lld\n", Sq, Sk, causal, Hq, Hkv, B,
                (long long)B * Hq * m.per_group * 4096);
    for (int bg = 0; bg < B * Hkv; ++bg)
      for (int hg = 0; hg < m.G; ++hg)
        for (int i = 0; i < m.nqb; ++i) {
          std::printf("R %d %d %d %d", bg, hg, i, fa::ds_strip_len(m, i));
          for (int j = 0; j < fa::ds_strip_len(m, i); ++j)
            std::printf(" %zu", fa::ds_block_off(m, bg, hg, i, j));
          std::printf("\n");
        }
  }
  return 0;
}
