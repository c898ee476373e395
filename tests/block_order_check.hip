// Host check of the kernels' block orders (compiled and run by test_block_order.py; built
// once for the chain kernel and once, with CHECK_GREEDY, for the greedy kernel): the mapping
// from block index to work item is a bijection, and with lazy rows every item of a row group
// of a request follows every item of the request's earlier groups, and its terminal items
// (greedy: its decider) follow all of them -- every wait in the kernels is on a lower block
// index.
#ifdef CHECK_GREEDY
#include "greedy.hip"
#else
#include "chain.hip"
#endif
#include <cstdio>
#include <vector>
#include <algorithm>
int main() {
  using namespace sv;
  long cases = 0;
  for (int B : {1, 2, 3, 7, 64, 100}) for (int R : {1, 2, 3, 6, 9}) for (int LK : {1, 2, 3, 6, 100}) for (int SL : {1, 3, 8})
  for (int S2 : {1, 5, 32}) for (int L : {0, 1, 3, 64, 100}) {
    if (L > B) continue;
#ifdef CHECK_GREEDY
    if (S2 != 1) continue;                 // one decider per request
    GreedyParams p{};
#else
    ChainParams p{};
    p.S2 = S2;
#endif
    p.B = B; p.R = R; p.G = R - 1; p.SL = SL; p.LAG = L;
    p.LK = LK < R ? LK : R; p.J = (R + p.LK - 1) / p.LK;
    const unsigned total = (unsigned)B * (R * SL + S2);
    std::vector<int> seen((size_t)B * (R * SL + S2), 0);
    std::vector<long> grp_last((size_t)B * (p.J + 1), -1), grp_first((size_t)B * (p.J + 1), -1);
    for (unsigned t = 0; t < total; ++t) {
#ifdef CHECK_GREEDY
      const Item it = block_item(p, t);
      const int last = it.decider;
#else
      const Item it = p.J > 1 ? lazy_item(p, t) : block_item(p, t);
      const int last = it.terminal;
#endif
      const int n = last ? S2 : R * SL;
      if (it.b < 0 || it.b >= B || it.idx < 0 || it.idx >= n) { printf("range fail t=%u\n", t); return 1; }
      const size_t key = (size_t)it.b * (R * SL + S2) + (last ? R * SL : 0) + it.idx;
      if (seen[key]++) { printf("dup fail B=%d R=%d LK=%d SL=%d S2=%d L=%d t=%u\n", B, R, LK, SL, S2, L, t); return 1; }
      const int g = last ? p.J : (it.idx / SL) / p.LK;
      const size_t k = (size_t)it.b * (p.J + 1) + g;
      if (grp_first[k] < 0) grp_first[k] = t;
      grp_last[k] = t;
    }
    for (int b = 0; b < B; ++b) for (int g = 1; g <= p.J; ++g)
      if (grp_first[(size_t)b * (p.J + 1) + g] <= grp_last[(size_t)b * (p.J + 1) + g - 1]) {
        printf("order fail B=%d R=%d LK=%d SL=%d S2=%d L=%d b=%d g=%d\n", B, R, LK, SL, S2, L, b, g);
        return 1;
      }
    ++cases;
  }
  printf("block orders ok (%ld cases)\n", cases);
  return 0;
}
