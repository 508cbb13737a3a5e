// plan.cpp -- host-side split-KV planner (pure C++, no HIP calls).
//
// Every sequence's pages are cut into contiguous runs of about `chunk` pages;
// each run is one work item (one work-group).  With chunk_pages <= 0 the chunk
// is chosen so the batch yields at least ~num_cus items, which keeps all
// compute units busy when there are fewer sequences than CUs, while the
// partial results stay small relative to the cache they summarise.  Runs of
// one sequence are as equal as possible.  Items are ordered longest first so
// the dispatcher starts the long ones early (a simple LPT schedule).  Within a
// run of equally long items, the items of one sequence are placed 8 positions
// apart: work-groups are dealt to the chip's 8 XCDs round robin by index, so
// they then share one XCD's L2 and the sequence's query rows are fetched from
// HBM once instead of once per item.
#include <algorithm>
#include <cstdint>
#include <vector>

#include "../../../include/mla.h"

extern "C" mla_status mla_plan_splits(const mla_config* cfg, const int32_t* seq_lens_host, int32_t batch,
                                      int32_t num_cus, int32_t chunk_pages, mla_work_item* items_host,
                                      int32_t max_items, int32_t* n_items, int32_t* split_offsets_host) {
  mla_status s = mla_config_check(cfg);
  if (s != MLA_OK) return s;
  if (batch < 0 || max_items < 0) return MLA_ERR_VALUE;
  if (n_items == nullptr || split_offsets_host == nullptr) return MLA_ERR_NULL;
  if (batch > 0 && seq_lens_host == nullptr) return MLA_ERR_NULL;
  const int64_t block = cfg->block_size;
  int64_t total_pages = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (seq_lens_host[b] < 0) return MLA_ERR_VALUE;
    total_pages += (seq_lens_host[b] + block - 1) / block;
  }
  int64_t chunk = chunk_pages;
  if (chunk <= 0) {
    const int64_t cus = num_cus > 0 ? num_cus : 256;
    chunk = std::max<int64_t>(1, (total_pages + cus - 1) / cus);
  }
  // Count items.
  int64_t count = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t pages = (seq_lens_host[b] + block - 1) / block;
    count += std::max<int64_t>(1, (pages + chunk - 1) / chunk);
  }
  if (count > INT32_MAX) return MLA_ERR_VALUE;
  *n_items = static_cast<int32_t>(count);
  if (count > max_items) return MLA_ERR_WORKSPACE;
  if (count > 0 && items_host == nullptr) return MLA_ERR_NULL;

  std::vector<mla_work_item> v;
  v.reserve(static_cast<size_t>(count));
  int32_t row = 0;
  for (int32_t b = 0; b < batch; ++b) {
    split_offsets_host[b] = row;
    const int64_t pages = (seq_lens_host[b] + block - 1) / block;
    const int64_t n = std::max<int64_t>(1, (pages + chunk - 1) / chunk);
    const int64_t base = pages / n, rem = pages % n;
    int64_t first = 0;
    for (int64_t j = 0; j < n; ++j) {
      const int64_t len = base + (j < rem ? 1 : 0);
      v.push_back(mla_work_item{b, static_cast<int32_t>(first), static_cast<int32_t>(len), row++});
      first += len;
    }
  }
  split_offsets_host[batch] = row;
  std::stable_sort(v.begin(), v.end(),
                   [](const mla_work_item& x, const mla_work_item& y) { return x.n_pages > y.n_pages; });
  constexpr int kXcd = 8;
  std::vector<mla_work_item> out;
  out.reserve(v.size());
  for (size_t r0 = 0; r0 < v.size();) {
    size_t r1 = r0;
    while (r1 < v.size() && v[r1].n_pages == v[r0].n_pages) ++r1;
    // Deal the run's sequences (contiguous after the stable sort) to the queue
    // of the XCD with the fewest items so far, then emit position by position:
    // position p takes the next item of queue p % kXcd (another queue's once
    // that one is empty).
    std::vector<std::vector<mla_work_item>> q(kXcd);
    for (size_t i = r0; i < r1;) {
      size_t e = i;
      while (e < r1 && v[e].seq == v[i].seq) ++e;
      size_t best = 0;
      for (size_t x = 1; x < kXcd; ++x)
        if (q[x].size() < q[best].size()) best = x;
      q[best].insert(q[best].end(), v.begin() + i, v.begin() + e);
      i = e;
    }
    std::vector<size_t> next(kXcd, 0);
    for (size_t k = r0; k < r1; ++k) {
      size_t x = out.size() % kXcd;
      for (size_t tries = 0; tries < kXcd && next[x] >= q[x].size(); ++tries) x = (x + 1) % kXcd;
      out.push_back(q[x][next[x]++]);
    }
    r0 = r1;
  }
  std::copy(out.begin(), out.end(), items_host);
  return MLA_OK;
}
