// item_range.h -- token range of one split-KV work item (host and device).
//
// A work item names pages [first_page, first_page + n_pages) of one sequence's
// block-table row.  The range is clipped to the row (max_pages entries) and to
// the sequence's length, in 64-bit arithmetic: first_page * 64 wraps a 32-bit
// int from 2^25 pages on.  A range that starts past the row or past the
// sequence comes out empty, with t_begin = t_end <= seq_len.
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define MLA_HD __host__ __device__
#else
#define MLA_HD
#endif

namespace mla {

struct TokenRange {
  int32_t t_begin, t_end;
};

// first_page, n_pages >= 0 and max_pages >= 0 are the caller's to check.
MLA_HD inline TokenRange item_token_range(int32_t first_page, int32_t n_pages, int32_t max_pages, int32_t seq_len,
                                          int32_t block) {
  const int64_t L = seq_len > 0 ? seq_len : 0;
  const int64_t first = first_page < max_pages ? first_page : max_pages;
  const int64_t end_page = (int64_t)first_page + n_pages;
  const int64_t pmax = end_page < max_pages ? end_page : max_pages;
  const int64_t tb0 = first * block, te0 = pmax * block;
  const int64_t tb = tb0 < L ? tb0 : L;
  const int64_t te = te0 < L ? te0 : L;
  TokenRange r;
  r.t_begin = (int32_t)tb;
  r.t_end = (int32_t)(te > tb ? te : tb);
  return r;
}

}  // namespace mla
