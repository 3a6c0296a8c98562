// Host-only driver for tests/test_host_logic.py, running the library's own
// index helpers (ssd_internal.h) on the host:
//   stdin "T nseq Q" and nseq + 1 offsets: builds the packed-sequence chunk
//   table with varlen_slot_entry, slot by slot as the table kernel does;
//   stdout: nslots, then one line per chunk slot (4 integers);
//   stdin "xcd n": the logical id xcd_swizzle gives each of n work-groups,
//   one per line.
#include <cstdio>
#include <vector>

#include "ssd_internal.h"

int main() {
  char mode[8] = {0};
  if (std::scanf(" %7[a-z]", mode) == 1) {
    int n;
    if (std::scanf("%d", &n) != 1 || n < 1) return 2;
    for (int b = 0; b < n; ++b) std::printf("%d\n", ssd::xcd_swizzle(b, n));
    return 0;
  }
  int T, nseq, Q;
  if (std::scanf("%d %d %d", &T, &nseq, &Q) != 3 || T < 1 || nseq < 1 || Q < 1) return 2;
  std::vector<int> cu(nseq + 1);
  for (int& v : cu)
    if (std::scanf("%d", &v) != 1) return 2;
  const int nslots = ssd::varlen_slots(T, nseq, Q);
  std::vector<int4> tab(nslots);
  for (int c = 0; c < nslots; ++c)
    tab[c] = ssd::varlen_slot_entry(cu.data(), nseq, T, Q, c, [&](int i) {
      return ssd::varlen_first_slot(ssd::clamp_int(cu[i], 0, T), i, Q);
    });
  std::printf("%d\n", nslots);
  for (const int4& e : tab) std::printf("%d %d %d %d\n", e.x, e.y, e.z, e.w);
  return 0;
}
