// Validation of one query block's KV-block list, for builds compiled with
// BSATTN_CHECK_LISTS=1. The same function runs in the device check that such
// builds launch before block-sparse attention and in the host test that runs
// it under address and undefined-behaviour sanitizers.
//
// A list is what the selector hands to the attention kernel (vllm-omni PR
// #8335, Purpose: per query head and query block, the selected KV blocks and
// their count): `cnt` entries at the start of a row of `stride` slots, each a
// KV block index in [0, nk), no index twice. The release kernel clamps the
// count, skips entries outside [0, nk) and would count a repeated block twice;
// the checked build reports each of these as a caller error instead.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define BSATTN_HD __host__ __device__
#else
#define BSATTN_HD
#endif

namespace bsattn {

enum ListFault : int32_t {
  kListOk = 0,
  kListCount = 1,      // count outside [0, stride]
  kListRange = 2,      // an entry outside [0, nk)
  kListDuplicate = 3,  // an entry equal to an earlier one
};

// Words of the `seen` bitmap for nk blocks.
BSATTN_HD inline int32_t list_seen_words(int32_t nk) { return nk > 0 ? (nk + 31) / 32 : 0; }

// Checks row[0 .. cnt): reads no slot at or past min(cnt, stride) and no
// bitmap word at or past list_seen_words(nk). With `seen` null, repeats are
// found by comparing each entry with the earlier ones instead (for block
// counts too large for the caller's bitmap). Returns the first fault in list
// order; *pos is the offending slot (-1 for a count fault or no fault).
BSATTN_HD inline int32_t check_list_row(const int32_t* row, int32_t cnt, int32_t stride,
                                        int32_t nk, uint32_t* seen, int32_t* pos) {
  *pos = -1;
  if (cnt < 0 || cnt > stride) return kListCount;
  if (seen != nullptr) {
    const int32_t words = list_seen_words(nk);
    for (int32_t w = 0; w < words; ++w) seen[w] = 0u;
  }
  for (int32_t j = 0; j < cnt; ++j) {
    const int32_t e = row[j];
    if (e < 0 || e >= nk) {
      *pos = j;
      return kListRange;
    }
    bool again = false;
    if (seen != nullptr) {
      const uint32_t bit = 1u << (e & 31);
      again = (seen[e >> 5] & bit) != 0u;
      seen[e >> 5] |= bit;
    } else {
      for (int32_t x = 0; x < j && !again; ++x) again = row[x] == e;
    }
    if (again) {
      *pos = j;
      return kListDuplicate;
    }
  }
  return kListOk;
}

}  // namespace bsattn
