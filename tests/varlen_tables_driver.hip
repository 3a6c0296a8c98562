// Host-only driver for tests/test_host_logic.py: builds the packed-sequence
// chunk and segment tables with the library's own varlen_span / varlen_fill
// (ssd_internal.h), as the table kernel does per sequence, and prints them.
// stdin: T nseq Q L, then nseq + 1 offsets. stdout: nslots nsegslots, then
// one line per chunk slot and one per segment slot (4 integers each).
#include <cstdio>
#include <vector>

#include "ssd_internal.h"

int main() {
  int T, nseq, Q, L;
  if (std::scanf("%d %d %d %d", &T, &nseq, &Q, &L) != 4 || T < 1 || nseq < 1 || Q < 1 || L < 1) return 2;
  std::vector<int> cu(nseq + 1);
  for (int& v : cu)
    if (std::scanf("%d", &v) != 1) return 2;
  const int nslots = ssd::varlen_slots(T, nseq, Q);
  const int nsegslots = ssd::varlen_seg_slots(T, nseq, Q * L);
  std::vector<int4> tab(nslots, int4{0, 0, 0, 0}), stab(nsegslots, int4{0, 0, 0, 0});
  for (int i = 0; i < nseq; ++i) {
    int s0, len;
    ssd::varlen_span(cu.data(), i, T, s0, len);
    ssd::varlen_fill(i, s0, len, Q, L, tab.data(), nslots, stab.data(), nsegslots);
  }
  std::printf("%d %d\n", nslots, nsegslots);
  for (const int4& e : tab) std::printf("%d %d %d %d\n", e.x, e.y, e.z, e.w);
  for (const int4& e : stab) std::printf("%d %d %d %d\n", e.x, e.y, e.z, e.w);
  return 0;
}
