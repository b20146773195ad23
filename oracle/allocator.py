"""Plain model of the segment allocator — test infrastructure, never on the product path.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this module. It shares no code with the library's allocator.

Flood keeps each request's KV cache in a few contiguous segments of one shared pool instead of
fixed-size pages, to keep the cache of a request contiguous (Flood README, "Introduction").
The pages say nothing about how those segments are handed out; the policy modelled here (and
implemented by the library) is the plainest one that serves that aim:

- growing a request by n tokens first extends its last segment in place, over the free slots
  that directly follow it;
- the remaining m tokens go into the smallest free run of at least m slots (lowest start among
  equals), taken from the run's start;
- if no free run holds m slots, the largest free run (lowest start among equals) is taken whole
  and the rest is placed the same way, again and again;
- a grow that does not fit in the free slots fails and changes nothing;
- releasing a request frees all its slots; truncating it to L keys frees its keys L, L+1, ...;
- a request's keys are its segments in the order they were added.

The model keeps one boolean per pool slot and finds free runs by scanning it, so that it can be
checked by eye; it is slow and meant for small pools.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np


class AllocatorModel:
    """Bitmap model: used[i] is True when pool slot i belongs to some request."""

    def __init__(self, pool_tokens: int):
        if pool_tokens < 0:
            raise ValueError("pool_tokens must be >= 0")
        self.pool_tokens = int(pool_tokens)
        self.used = np.zeros(self.pool_tokens, dtype=bool)
        self.segs: Dict[int, List[List[int]]] = {}  # request -> [[offset, length], ...]

    # ---------------------------------------------------------------- queries

    def free_runs(self) -> List[Tuple[int, int]]:
        """Maximal runs of free slots as (start, length), in pool order."""
        runs = []
        i = 0
        n = self.pool_tokens
        while i < n:
            if self.used[i]:
                i += 1
                continue
            j = i
            while j < n and not self.used[j]:
                j += 1
            runs.append((i, j - i))
            i = j
        return runs

    def free_tokens(self) -> int:
        return int(self.pool_tokens - self.used.sum())

    def length(self, request: int) -> int:
        return sum(ln for _, ln in self.segs.get(request, []))

    def segments(self, request: int) -> List[Tuple[int, int]]:
        return [(o, ln) for o, ln in self.segs.get(request, [])]

    # ---------------------------------------------------------------- updates

    def _take(self, start: int, n: int):
        assert not self.used[start:start + n].any()
        self.used[start:start + n] = True

    def grow(self, request: int, n: int) -> bool:
        """Add n tokens to the request; False (and no change) if the pool cannot hold them."""
        if n < 0:
            raise ValueError("n must be >= 0")
        if n > self.free_tokens():
            return False
        segs = self.segs.setdefault(request, [])
        left = n
        # 1. in place, after the last segment
        if segs and left > 0:
            end = segs[-1][0] + segs[-1][1]
            k = 0
            while k < left and end + k < self.pool_tokens and not self.used[end + k]:
                k += 1
            if k > 0:
                self._take(end, k)
                segs[-1][1] += k
                left -= k
        # 2./3. best fit, else the largest run whole, repeatedly
        while left > 0:
            runs = self.free_runs()
            fits = [r for r in runs if r[1] >= left]
            if fits:
                start, _ = min(fits, key=lambda r: (r[1], r[0]))
                take = left
            else:
                start, ln = min(runs, key=lambda r: (-r[1], r[0]))
                take = ln
            self._take(start, take)
            segs.append([start, take])
            left -= take
        return True

    def release(self, request: int):
        for off, ln in self.segs.pop(request, []):
            self.used[off:off + ln] = False

    def truncate(self, request: int, new_length: int):
        """Keep the request's first new_length keys and free the rest."""
        if new_length < 0:
            raise ValueError("new_length must be >= 0")
        segs = self.segs.get(request, [])
        excess = self.length(request) - new_length
        while excess > 0 and segs:
            off, ln = segs[-1]
            cut = min(excess, ln)
            self.used[off + ln - cut:off + ln] = False
            segs[-1][1] = ln - cut
            if segs[-1][1] == 0:
                segs.pop()
            excess -= cut

    # ---------------------------------------------------------------- tables

    def tables(self, requests: Sequence[int]):
        """(segs [nseg, 2] int64, seg_indptr [B+1], cu_seqlens_k [B+1]) for the batch, in the
        layout the attention entry points take. Unknown requests have no keys."""
        rows, ind, cu = [], [0], [0]
        for r in requests:
            s = self.segments(int(r))
            rows.extend(s)
            ind.append(ind[-1] + len(s))
            cu.append(cu[-1] + sum(ln for _, ln in s))
        segs = np.array(rows, dtype=np.int64).reshape(-1, 2)
        return segs, np.array(ind, dtype=np.int64), np.array(cu, dtype=np.int64)
