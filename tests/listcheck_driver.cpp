// Host driver for the block-list check (csrc/listcheck.h), built by
// tests/test_listcheck.py with address and undefined-behaviour sanitizers.
//
// stdin: one case per line, "nk stride cnt e_0 ... e_{stride-1}". Each row is
// copied into a heap array of exactly `stride` ints and the bitmap into one
// of exactly list_seen_words(nk) words, so a read past either is reported
// by the sanitizer. stdout: per case "fault pos fault pos", from the bitmap
// path and from the pairwise path.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "listcheck.h"

int main() {
  long nk, stride, cnt;
  while (std::scanf("%ld %ld %ld", &nk, &stride, &cnt) == 3) {
    std::vector<long> vals((size_t)stride);
    for (long j = 0; j < stride; ++j)
      if (std::scanf("%ld", &vals[(size_t)j]) != 1) return 2;
    int32_t* row = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (size_t)(stride > 0 ? stride : 1)));
    for (long j = 0; j < stride; ++j) row[j] = (int32_t)vals[(size_t)j];
    const int32_t words = bsattn::list_seen_words((int32_t)nk);
    uint32_t* seen = static_cast<uint32_t*>(std::malloc(sizeof(uint32_t) * (size_t)(words > 0 ? words : 1)));
    int32_t pos_a = 0, pos_b = 0;
    const int32_t fa = bsattn::check_list_row(row, (int32_t)cnt, (int32_t)stride, (int32_t)nk,
                                              words > 0 ? seen : nullptr, &pos_a);
    const int32_t fb =
        bsattn::check_list_row(row, (int32_t)cnt, (int32_t)stride, (int32_t)nk, nullptr, &pos_b);
    std::printf("%d %d %d %d\n", fa, pos_a, fb, pos_b);
    std::free(seen);
    std::free(row);
  }
  return 0;
}
