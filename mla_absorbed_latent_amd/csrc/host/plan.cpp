// plan.cpp -- host-side split-KV planner (pure C++, no HIP calls).
//
// Every sequence's pages are cut into contiguous runs of about `chunk` pages;
// each run is one work item (one work-group).  With chunk_pages <= 0 the chunk
// is chosen between total / (8 num_cus) and total / num_cus by a model of the
// run: the makespan of items dispatched longest first onto the CU that frees
// first (an item costs its pages plus a fixed overhead for its query load and
// partial write, about three pages' time), plus the merge's read of the partials
// (H x 1 KB per item, spread over all CUs).  Uniform batches get one item per
// CU; ragged ones get finer splits where that evens out the CUs' loads.  Runs of
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

#include <functional>
#include <queue>

namespace {

constexpr int64_t kItemOverheadPages = 3;

// Pages of each item when every sequence is cut into runs of about `chunk` pages.
void item_pages(const int32_t* seq_lens, int32_t batch, int64_t block, int64_t chunk, std::vector<int64_t>& out) {
  out.clear();
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t pages = (seq_lens[b] + block - 1) / block;
    const int64_t n = std::max<int64_t>(1, (pages + chunk - 1) / chunk);
    const int64_t base = pages / n, rem = pages % n;
    for (int64_t j = 0; j < n; ++j) out.push_back(base + (j < rem ? 1 : 0));
  }
}

// Modelled completion time: items longest first, each to the CU that frees first.
int64_t modelled_makespan(std::vector<int64_t>& pages, int64_t cus) {
  std::sort(pages.begin(), pages.end(), std::greater<int64_t>());
  std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> free_at;
  for (int64_t i = 0; i < cus; ++i) free_at.push(0);
  int64_t end = 0;
  for (int64_t p : pages) {
    const int64_t t = free_at.top() + p + kItemOverheadPages;
    free_at.pop();
    free_at.push(t);
    end = std::max(end, t);
  }
  return end;
}

}  // namespace

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
    std::vector<int64_t> pages;
    double best = -1.0;
    chunk = 1;
    const int64_t c_hi = std::max<int64_t>(1, (total_pages + cus - 1) / cus);
    const int64_t c_lo = std::max<int64_t>(1, (total_pages + 8 * cus - 1) / (8 * cus));
    for (int64_t c = c_hi; c >= c_lo; --c) {          // ties keep the larger chunk (fewer items)
      item_pages(seq_lens_host, batch, block, c, pages);
      const double t = (double)modelled_makespan(pages, cus) +
                       (double)pages.size() * cfg->num_heads * 2048.0 / ((double)mla_cache_page_bytes(cfg) * cus);
      if (best < 0 || t < best) {
        best = t;
        chunk = c;
      }
    }
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
