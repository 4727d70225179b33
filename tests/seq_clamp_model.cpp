// Host build of the library's packed-sequence index helpers (sage_internal.h):
// reads "nseq max_seqlen total" and nseq+1 offsets per case from stdin and
// prints, per sequence, the token range [start, start + len) the kernels use.
#include <cstdio>
#include <vector>

#include "sage_internal.h"

int main() {
  int nseq, max_seqlen, total;
  while (std::scanf("%d %d %d", &nseq, &max_seqlen, &total) == 3) {
    std::vector<int32_t> cu(nseq + 1);
    for (auto& c : cu) std::scanf("%d", &c);
    for (int s = 0; s < nseq; ++s)
      std::printf("%d %d\n", sage::seq_start(cu.data(), s, total), sage::seq_len(cu.data(), s, max_seqlen, total));
  }
  return 0;
}
