// Host-side segment allocator: hands out pool ranges to requests and writes the segment tables
// the attention entry points take. Each request's cache stays in as few contiguous segments of
// the shared pool as the free space allows (Flood README, "Introduction": segmentable blocks
// instead of paged blocks, for the continuity of each request's cache).
//
// Policy. A request owns ranges holding C slots (its capacity); its L <= C keys are the first L
// of them. Growing it by n keys uses spare capacity first; a shortfall of m slots is allocated
// aiming at w = m rounded up to the allocator's granule (w = m when fewer than w slots are
// free), so that one-token growth gets a new range only every granule tokens; reserve() sets
// capacity aside the same way without adding keys. An allocation first extends the last range
// over up to w of the free slots that directly follow it; the rest goes to the smallest free run
// that holds it (lowest start among equals), from the run's start; when no run holds it, the
// largest run (lowest start among equals) gives min(its length, rest) and the remainder is placed
// the same way, until the m needed slots are there. An allocation that does not fit changes
// nothing. Release and truncate free slots (truncate also the spare capacity), merging them with
// neighbouring free runs.
//
// Compaction relocates fragmented requests (two or more ranges), most ranges first, then by
// increasing id, each whole into the smallest free run of the call's start (lowest start among
// equals) that holds its capacity; slots it frees are not reused in the same call, so every
// destination is disjoint from every source and every other destination and the caller may apply
// the moves in any order or all at once (seg_attn_kv_move).
//
// Free runs are kept twice: by start (to find a neighbour and the run after a segment) and by
// (length, start) (best fit and largest run), so every step is logarithmic in the number of
// runs. Requests map to their segment lists.
#include <stdint.h>

#include <algorithm>
#include <iterator>
#include <map>
#include <new>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/seg_attn.h"

struct Request {
  std::vector<seg_attn_segment_t> ranges;  // owned slot ranges, in key order
  int64_t keys = 0;                        // L
  int64_t capacity = 0;                    // C: sum of the ranges' lengths
};

struct seg_attn_allocator {
  int64_t pool_tokens = 0;
  int64_t granule = 1;
  int64_t free_tokens = 0;
  std::map<int64_t, int64_t> by_start;              // free run start -> length
  std::set<std::pair<int64_t, int64_t>> by_length;  // (length, start) of every free run
  std::unordered_map<int64_t, Request> requests;

  void add_run(int64_t start, int64_t len) {
    by_start.emplace(start, len);
    by_length.emplace(len, start);
  }
  void drop_run(std::map<int64_t, int64_t>::iterator it) {
    by_length.erase({it->second, it->first});
    by_start.erase(it);
  }

  // Take n slots from the start of the free run at `it` (n <= its length).
  void take_front(std::map<int64_t, int64_t>::iterator it, int64_t n) {
    const int64_t start = it->first, len = it->second;
    drop_run(it);
    if (len > n) add_run(start + n, len - n);
    free_tokens -= n;
  }

  // Take [start, start + n) out of the free run that holds it.
  void take_range(int64_t start, int64_t n) {
    auto it = std::prev(by_start.upper_bound(start));
    const int64_t rs = it->first, rl = it->second;
    drop_run(it);
    if (start > rs) add_run(rs, start - rs);
    if (start + n < rs + rl) add_run(start + n, rs + rl - (start + n));
    free_tokens -= n;
  }

  // Return [start, start + len) to the free runs, merged with its neighbours.
  void give_back(int64_t start, int64_t len) {
    if (len <= 0) return;
    free_tokens += len;
    auto next = by_start.lower_bound(start);
    if (next != by_start.end() && next->first == start + len) {
      len += next->second;
      auto after = std::next(next);
      drop_run(next);
      next = after;
    }
    if (next != by_start.begin()) {
      auto prev = std::prev(next);
      if (prev->first + prev->second == start) {
        start = prev->first;
        len += prev->second;
        drop_run(prev);
      }
    }
    add_run(start, len);
  }

  // Add at least `need` (aiming at `want`, want >= need) slots to `req`; need <= free_tokens.
  void allocate(Request& req, int64_t need, int64_t want) {
    if (want > free_tokens) want = need;
    std::vector<seg_attn_segment_t>& ranges = req.ranges;
    ranges.reserve(ranges.size() + 4);  // no allocation failure once slots start moving below
    if (!ranges.empty() && want > 0) {  // in place, after the last range
      seg_attn_segment_t& last = ranges.back();
      auto it = by_start.find((int64_t)last.pool_offset + last.length);
      if (it != by_start.end()) {
        const int64_t k = want < it->second ? want : it->second;
        take_front(it, k);
        last.length += (int32_t)k;
        req.capacity += k;
        need -= k;
        want -= k;
      }
    }
    while (need > 0) {
      auto fit = by_length.lower_bound({want, INT64_MIN});
      int64_t start, take;
      if (fit != by_length.end()) {
        start = fit->second;
        take = want;
      } else {  // the largest run, lowest start among equals
        const int64_t longest = by_length.rbegin()->first;
        start = by_length.lower_bound({longest, INT64_MIN})->second;
        take = longest < want ? longest : want;
      }
      if (ranges.size() == ranges.capacity()) ranges.reserve(2 * ranges.size() + 4);
      take_front(by_start.find(start), take);
      ranges.push_back({(int32_t)start, (int32_t)take});
      req.capacity += take;
      need -= take;
      want -= take;
    }
  }
};

extern "C" {

seg_attn_status_t seg_attn_allocator_create(int64_t pool_tokens, int64_t granule,
                                            seg_attn_allocator_t** out) {
  if (out == nullptr) return SEG_ATTN_ERR_INVALID_ARG;
  *out = nullptr;
  if (pool_tokens < 0 || pool_tokens > INT32_MAX || granule < 1 || granule > INT32_MAX)
    return SEG_ATTN_ERR_INVALID_ARG;
  try {
    seg_attn_allocator* a = new seg_attn_allocator();
    a->pool_tokens = pool_tokens;
    a->granule = granule;
    a->free_tokens = 0;
    a->give_back(0, pool_tokens);
    *out = a;
    return SEG_ATTN_OK;
  } catch (...) {
    return SEG_ATTN_ERR_OUT_OF_MEMORY;
  }
}

void seg_attn_allocator_destroy(seg_attn_allocator_t* a) { delete a; }

seg_attn_status_t seg_attn_allocator_grow(seg_attn_allocator_t* a, int64_t request, int64_t n) {
  if (a == nullptr || n < 0) return SEG_ATTN_ERR_INVALID_ARG;
  try {
    auto found = a->requests.find(request);
    const int64_t keys = found == a->requests.end() ? 0 : found->second.keys;
    const int64_t cap = found == a->requests.end() ? 0 : found->second.capacity;
    if (n > INT32_MAX - keys) return SEG_ATTN_ERR_INVALID_ARG;
    const int64_t short_by = keys + n - cap;
    if (short_by > a->free_tokens) return SEG_ATTN_ERR_OUT_OF_MEMORY;
    Request& req = a->requests[request];
    if (short_by > 0) {
      const int64_t want = (short_by + a->granule - 1) / a->granule * a->granule;
      a->allocate(req, short_by, want);
    }
    req.keys += n;
    return SEG_ATTN_OK;
  } catch (...) {
    return SEG_ATTN_ERR_OUT_OF_MEMORY;
  }
}

seg_attn_status_t seg_attn_allocator_grow_batch(seg_attn_allocator_t* a, const int64_t* requests,
                                                const int64_t* n, int32_t count, int32_t* done) {
  if (done) *done = 0;
  if (a == nullptr || count < 0 || (count > 0 && (requests == nullptr || n == nullptr)))
    return SEG_ATTN_ERR_INVALID_ARG;
  for (int32_t i = 0; i < count; ++i) {
    const seg_attn_status_t st = seg_attn_allocator_grow(a, requests[i], n[i]);
    if (st != SEG_ATTN_OK) return st;
    if (done) *done = i + 1;
  }
  return SEG_ATTN_OK;
}

seg_attn_status_t seg_attn_allocator_reserve(seg_attn_allocator_t* a, int64_t request,
                                             int64_t capacity) {
  if (a == nullptr || capacity < 0 || capacity > INT32_MAX) return SEG_ATTN_ERR_INVALID_ARG;
  try {
    auto found = a->requests.find(request);
    const int64_t cap = found == a->requests.end() ? 0 : found->second.capacity;
    const int64_t short_by = capacity - cap;
    if (short_by > a->free_tokens) return SEG_ATTN_ERR_OUT_OF_MEMORY;
    Request& req = a->requests[request];
    if (short_by > 0) a->allocate(req, short_by, short_by);
    return SEG_ATTN_OK;
  } catch (...) {
    return SEG_ATTN_ERR_OUT_OF_MEMORY;
  }
}

seg_attn_status_t seg_attn_allocator_release(seg_attn_allocator_t* a, int64_t request) {
  if (a == nullptr) return SEG_ATTN_ERR_INVALID_ARG;
  try {
    auto it = a->requests.find(request);
    if (it == a->requests.end()) return SEG_ATTN_OK;
    for (const seg_attn_segment_t& s : it->second.ranges) a->give_back(s.pool_offset, s.length);
    a->requests.erase(it);
    return SEG_ATTN_OK;
  } catch (...) {
    return SEG_ATTN_ERR_OUT_OF_MEMORY;
  }
}

seg_attn_status_t seg_attn_allocator_truncate(seg_attn_allocator_t* a, int64_t request,
                                              int64_t new_length) {
  if (a == nullptr || new_length < 0) return SEG_ATTN_ERR_INVALID_ARG;
  try {
    auto it = a->requests.find(request);
    if (it == a->requests.end() || new_length >= it->second.keys) return SEG_ATTN_OK;
    Request& req = it->second;
    int64_t excess = req.capacity - new_length;  // spare capacity goes too
    while (excess > 0 && !req.ranges.empty()) {
      seg_attn_segment_t& last = req.ranges.back();
      const int64_t cut = excess < last.length ? excess : last.length;
      a->give_back((int64_t)last.pool_offset + last.length - cut, cut);
      last.length -= (int32_t)cut;
      if (last.length == 0) req.ranges.pop_back();
      excess -= cut;
      req.capacity -= cut;
    }
    req.keys = new_length;
    return SEG_ATTN_OK;
  } catch (...) {
    return SEG_ATTN_ERR_OUT_OF_MEMORY;
  }
}

seg_attn_status_t seg_attn_allocator_compact(seg_attn_allocator_t* a, seg_attn_move_t* moves,
                                             int64_t capacity, int64_t* n_moves) {
  if (n_moves) *n_moves = 0;
  if (a == nullptr || capacity < 0) return SEG_ATTN_ERR_INVALID_ARG;
  try {
    // Plan on a snapshot of the free runs (by (length, start) for best fit); nothing changes
    // unless the moves fit in the caller's array.
    std::set<std::pair<int64_t, int64_t>> runs;
    for (const auto& r : a->by_start) runs.emplace(r.second, r.first);
    std::vector<std::pair<int64_t, int64_t>> order;  // (-number of ranges, id)
    for (const auto& kv : a->requests)
      if (kv.second.ranges.size() >= 2) order.emplace_back(-(int64_t)kv.second.ranges.size(), kv.first);
    std::sort(order.begin(), order.end());
    std::vector<std::pair<int64_t, int64_t>> plan;  // (id, destination start)
    int64_t count = 0;
    for (const auto& o : order) {
      const Request& req = a->requests.at(o.second);
      auto fit = runs.lower_bound({req.capacity, INT64_MIN});
      if (fit == runs.end()) continue;
      const int64_t start = fit->second, len = fit->first;
      runs.erase(fit);
      if (len > req.capacity) runs.emplace(len - req.capacity, start + req.capacity);
      plan.emplace_back(o.second, start);
      int64_t left = req.keys;
      for (const seg_attn_segment_t& sg : req.ranges) {
        if (left <= 0) break;
        ++count;
        left -= sg.length;
      }
    }
    if (n_moves) *n_moves = count;
    if (count > capacity || (count > 0 && moves == nullptr)) return SEG_ATTN_ERR_WORKSPACE;
    int64_t m = 0, first = 0;
    for (const auto& pl : plan) {
      Request& req = a->requests.at(pl.first);
      const int64_t dst = pl.second;
      a->take_range(dst, req.capacity);
      int64_t left = req.keys, done = 0;
      for (const seg_attn_segment_t& sg : req.ranges) {
        const int64_t n = left < sg.length ? left : sg.length;
        if (n > 0) {
          moves[m++] = {sg.pool_offset, (int32_t)(dst + done), (int32_t)n, (int32_t)first};
          first += n;
        }
        done += n;
        left -= n;
      }
      for (const seg_attn_segment_t& sg : req.ranges) a->give_back(sg.pool_offset, sg.length);
      req.ranges.assign(1, seg_attn_segment_t{(int32_t)dst, (int32_t)req.capacity});
    }
    return SEG_ATTN_OK;
  } catch (...) {
    return SEG_ATTN_ERR_OUT_OF_MEMORY;
  }
}

int64_t seg_attn_allocator_length(const seg_attn_allocator_t* a, int64_t request) {
  if (a == nullptr) return -1;
  auto it = a->requests.find(request);
  return it == a->requests.end() ? 0 : it->second.keys;
}

int64_t seg_attn_allocator_capacity(const seg_attn_allocator_t* a, int64_t request) {
  if (a == nullptr) return -1;
  auto it = a->requests.find(request);
  return it == a->requests.end() ? 0 : it->second.capacity;
}

seg_attn_status_t seg_attn_allocator_tables(const seg_attn_allocator_t* a, const int64_t* requests,
                                            int32_t batch, seg_attn_segment_t* segs,
                                            int64_t segs_capacity, int32_t* seg_indptr,
                                            int32_t* cu_seqlens_k, int64_t* nseg) {
  if (a == nullptr || batch < 0 || segs_capacity < 0 || (batch > 0 && requests == nullptr) ||
      seg_indptr == nullptr || cu_seqlens_k == nullptr)
    return SEG_ATTN_ERR_INVALID_ARG;
  // count first: nothing is written unless everything fits. A request's table lists the ranges
  // that hold its keys, the last one cut at the key count.
  auto ranges_with_keys = [](const Request& r) {
    int64_t n = 0, left = r.keys;
    for (const seg_attn_segment_t& sg : r.ranges) {
      if (left <= 0) break;
      ++n;
      left -= sg.length;
    }
    return n;
  };
  int64_t need = 0, keys = 0;
  for (int32_t b = 0; b < batch; ++b) {
    auto it = a->requests.find(requests[b]);
    if (it == a->requests.end()) continue;
    need += ranges_with_keys(it->second);
    keys += it->second.keys;
  }
  if (nseg) *nseg = need;
  if (need > segs_capacity || (need > 0 && segs == nullptr)) return SEG_ATTN_ERR_WORKSPACE;
  if (need > INT32_MAX || keys > INT32_MAX) return SEG_ATTN_ERR_UNSUPPORTED;
  int64_t s = 0, k = 0;
  seg_indptr[0] = 0;
  cu_seqlens_k[0] = 0;
  for (int32_t b = 0; b < batch; ++b) {
    auto it = a->requests.find(requests[b]);
    if (it != a->requests.end()) {
      int64_t left = it->second.keys;
      for (const seg_attn_segment_t& sg : it->second.ranges) {
        if (left <= 0) break;
        const int32_t len = (int32_t)(left < sg.length ? left : sg.length);
        segs[s++] = {sg.pool_offset, len};
        k += len;
        left -= len;
      }
    }
    seg_indptr[b + 1] = (int32_t)s;
    cu_seqlens_k[b + 1] = (int32_t)k;
  }
  return SEG_ATTN_OK;
}

seg_attn_status_t seg_attn_allocator_stats(const seg_attn_allocator_t* a, int64_t* free_tokens,
                                           int64_t* largest_free_run, int64_t* free_runs,
                                           int64_t* requests) {
  if (a == nullptr) return SEG_ATTN_ERR_INVALID_ARG;
  if (free_tokens) *free_tokens = a->free_tokens;
  if (largest_free_run) *largest_free_run = a->by_length.empty() ? 0 : a->by_length.rbegin()->first;
  if (free_runs) *free_runs = (int64_t)a->by_start.size();
  if (requests) *requests = (int64_t)a->requests.size();
  return SEG_ATTN_OK;
}

seg_attn_status_t seg_attn_allocator_free_runs(const seg_attn_allocator_t* a,
                                               seg_attn_segment_t* runs, int64_t capacity,
                                               int64_t* count) {
  if (a == nullptr || capacity < 0) return SEG_ATTN_ERR_INVALID_ARG;
  const int64_t n = (int64_t)a->by_start.size();
  if (count) *count = n;
  if (n > capacity || (n > 0 && runs == nullptr)) return SEG_ATTN_ERR_WORKSPACE;
  int64_t i = 0;
  for (const auto& r : a->by_start) runs[i++] = {(int32_t)r.first, (int32_t)r.second};
  return SEG_ATTN_OK;
}

}  // extern "C"
