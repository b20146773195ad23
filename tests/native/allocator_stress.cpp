// Randomised stress of the host segment allocator through its C ABI, for a build with the address
// and undefined-behaviour sanitizers (tests/test_allocator_sanitized.py compiles and runs it):
// every allocator operation runs under the sanitizers, and after each one the state reported
// through the ABI is checked for consistency on a bitmap of the pool.
//
//   allocator_stress <seed> <steps> <pool_tokens> <requests> <max_grow> <granule>
//
// Exit status 0 when every check held; a failed check prints it and exits 1.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <cstdint>
#include <random>
#include <vector>

#include "seg_attn.h"

namespace {

int fail(const char* what, long step) {
  fprintf(stderr, "check failed at step %ld: %s\n", step, what);
  exit(1);
}

// The state seen through the ABI: free runs, every request's key segments and capacity. Checks:
// free runs sorted, disjoint, maximal and inside the pool; key segments inside the pool, disjoint
// from each other and from the free runs; each request's segment lengths adding up to its length,
// which is at most its capacity; the capacities and the free slots adding up to the pool.
void check_state(seg_attn_allocator_t* a, int64_t pool, const std::vector<int64_t>& reqs, long step) {
  int64_t free_tokens = -1, largest = -1, nruns = -1, nreq = -1;
  if (seg_attn_allocator_stats(a, &free_tokens, &largest, &nruns, &nreq) != SEG_ATTN_OK) fail("stats", step);
  std::vector<seg_attn_segment_t> runs((size_t)std::max<int64_t>(nruns, 1));
  int64_t cnt = -1;
  if (seg_attn_allocator_free_runs(a, runs.data(), (int64_t)runs.size(), &cnt) != SEG_ATTN_OK) fail("free_runs", step);
  if (cnt != nruns) fail("free run count", step);
  std::vector<uint8_t> owner((size_t)pool, 0);  // 1 free, 2 key slot
  int64_t sum_free = 0, max_run = 0, prev_end = -1;
  for (int64_t i = 0; i < cnt; ++i) {
    const int64_t s = runs[(size_t)i].pool_offset, n = runs[(size_t)i].length;
    if (n <= 0 || s < 0 || s + n > pool) fail("free run outside the pool", step);
    if (s <= prev_end) fail("free runs not sorted, overlapping or not maximal", step);
    prev_end = s + n;
    for (int64_t x = s; x < s + n; ++x) owner[(size_t)x] = 1;
    sum_free += n;
    max_run = std::max(max_run, n);
  }
  if (sum_free != free_tokens || max_run != largest) fail("stats against free runs", step);

  const int32_t batch = (int32_t)reqs.size();
  std::vector<int32_t> ind((size_t)batch + 1), cu((size_t)batch + 1);
  int64_t nseg = -1;
  seg_attn_status_t st = seg_attn_allocator_tables(a, reqs.data(), batch, nullptr, 0, ind.data(), cu.data(), &nseg);
  if (st != SEG_ATTN_OK && st != SEG_ATTN_ERR_WORKSPACE) fail("tables (count)", step);
  std::vector<seg_attn_segment_t> segs((size_t)std::max<int64_t>(nseg, 1));
  if (seg_attn_allocator_tables(a, reqs.data(), batch, segs.data(), (int64_t)segs.size(), ind.data(), cu.data(),
                                &nseg) != SEG_ATTN_OK)
    fail("tables", step);
  int64_t capacity_total = 0;
  for (int32_t b = 0; b < batch; ++b) {
    int64_t len = 0;
    for (int32_t s = ind[(size_t)b]; s < ind[(size_t)b + 1]; ++s) {
      const int64_t o = segs[(size_t)s].pool_offset, n = segs[(size_t)s].length;
      if (n <= 0 || o < 0 || o + n > pool) fail("segment outside the pool", step);
      for (int64_t x = o; x < o + n; ++x) {
        if (owner[(size_t)x] != 0) fail("segment overlaps a free run or another segment", step);
        owner[(size_t)x] = 2;
      }
      len += n;
    }
    if (len != (int64_t)cu[(size_t)b + 1] - cu[(size_t)b]) fail("cu_seqlens against segments", step);
    if (len != seg_attn_allocator_length(a, reqs[(size_t)b])) fail("length against segments", step);
    const int64_t cap = seg_attn_allocator_capacity(a, reqs[(size_t)b]);
    if (cap < len) fail("capacity below length", step);
    capacity_total += cap;
  }
  if (capacity_total + free_tokens != pool) fail("capacities and free slots do not add up to the pool", step);
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 7) {
    fprintf(stderr, "usage: %s seed steps pool_tokens requests max_grow granule\n", argv[0]);
    return 2;
  }
  const unsigned seed = (unsigned)atol(argv[1]);
  const long steps = atol(argv[2]);
  const int64_t pool = atoll(argv[3]);
  const int nreq = atoi(argv[4]);
  const int64_t max_grow = atoll(argv[5]);
  const int64_t granule = atoll(argv[6]);
  std::mt19937_64 rng(seed);
  auto uni = [&](int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); };

  // argument errors first: nothing may be written through a NULL or changed on a bad argument
  seg_attn_allocator_t* a = nullptr;
  if (seg_attn_allocator_create(-1, 1, &a) == SEG_ATTN_OK) fail("create accepted a negative pool", 0);
  if (seg_attn_allocator_create(pool, 0, &a) == SEG_ATTN_OK) fail("create accepted granule 0", 0);
  if (seg_attn_allocator_create(pool, granule, nullptr) == SEG_ATTN_OK) fail("create accepted NULL", 0);
  if (seg_attn_allocator_grow(nullptr, 0, 1) == SEG_ATTN_OK) fail("grow accepted NULL", 0);
  if (seg_attn_allocator_create(pool, granule, &a) != SEG_ATTN_OK || !a) fail("create", 0);
  if (seg_attn_allocator_grow(a, 1, -1) == SEG_ATTN_OK) fail("grow accepted n < 0", 0);

  std::vector<int64_t> reqs;
  for (int i = 0; i < nreq; ++i) reqs.push_back(i % 3 == 2 ? -(int64_t)i * 7919 : (int64_t)i * 1000003);
  std::vector<seg_attn_move_t> moves;
  for (long step = 1; step <= steps; ++step) {
    const int64_t r = reqs[(size_t)uni(0, nreq - 1)];
    const double op = std::uniform_real_distribution<double>(0.0, 1.0)(rng);
    if (op < 0.5) {
      const seg_attn_status_t st = seg_attn_allocator_grow(a, r, uni(0, max_grow));
      if (st != SEG_ATTN_OK && st != SEG_ATTN_ERR_OUT_OF_MEMORY) fail("grow status", step);
    } else if (op < 0.58) {
      const seg_attn_status_t st = seg_attn_allocator_reserve(a, r, uni(0, 3 * max_grow));
      if (st != SEG_ATTN_OK && st != SEG_ATTN_ERR_OUT_OF_MEMORY) fail("reserve status", step);
    } else if (op < 0.66) {
      const int32_t count = (int32_t)uni(1, 8);
      std::vector<int64_t> ids, ns;
      for (int32_t i = 0; i < count; ++i) {
        ids.push_back(reqs[(size_t)uni(0, nreq - 1)]);
        ns.push_back(uni(0, max_grow));
      }
      int32_t done = -1;
      const seg_attn_status_t st = seg_attn_allocator_grow_batch(a, ids.data(), ns.data(), count, &done);
      if (st != SEG_ATTN_OK && st != SEG_ATTN_ERR_OUT_OF_MEMORY) fail("grow_batch status", step);
      if (done < 0 || done > count || (st == SEG_ATTN_OK && done != count)) fail("grow_batch done", step);
    } else if (op < 0.8) {
      if (seg_attn_allocator_release(a, r) != SEG_ATTN_OK) fail("release", step);
    } else if (op < 0.95) {
      const int64_t len = seg_attn_allocator_length(a, r);
      if (seg_attn_allocator_truncate(a, r, uni(0, len + 2)) != SEG_ATTN_OK) fail("truncate", step);
    } else {
      // compaction: count, then plan; sources and destinations pairwise disjoint, `first` the
      // running sum of the lengths, every relocated request left with one segment
      int64_t n = -1;
      seg_attn_status_t st = seg_attn_allocator_compact(a, nullptr, 0, &n);
      if (st != SEG_ATTN_OK && st != SEG_ATTN_ERR_WORKSPACE) fail("compact count status", step);
      if (n > 0) {
        moves.assign((size_t)n, seg_attn_move_t{});
        int64_t m = -1;
        if (seg_attn_allocator_compact(a, moves.data(), n, &m) != SEG_ATTN_OK || m != n) fail("compact", step);
        std::vector<uint8_t> used((size_t)pool, 0);
        int64_t first = 0;
        for (const auto& mv : moves) {
          if (mv.length <= 0 || mv.first != first) fail("compact move record", step);
          first += mv.length;
          for (int64_t x = 0; x < mv.length; ++x) {
            const int64_t s = (int64_t)mv.src_offset + x, d = (int64_t)mv.dst_offset + x;
            if (s < 0 || s >= pool || d < 0 || d >= pool) fail("move outside the pool", step);
            if (used[(size_t)s] || used[(size_t)d]) fail("moves not disjoint", step);
            used[(size_t)s] = used[(size_t)d] = 1;
          }
        }
      }
    }
    if (step % 7 == 0 || step == steps) check_state(a, pool, reqs, step);
  }
  seg_attn_allocator_destroy(a);
  seg_attn_allocator_destroy(nullptr);
  printf("ok %ld steps\n", steps);
  return 0;
}
