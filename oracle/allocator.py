"""Plain model of the segment allocator — test infrastructure, never on the product path.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this module. It shares no code with the library's allocator.

Flood keeps each request's KV cache in a few contiguous segments of one shared pool instead of
fixed-size pages, to keep the cache of a request contiguous (Flood README, "Introduction").
The pages say nothing about how those segments are handed out; the policy modelled here (and
implemented by the library) is the plainest one that serves that aim:

- a request owns segments, in the order they were added, holding C slots (its capacity); its
  L keys (L <= C) are the first L of those slots, and the tables list only them;
- growing a request by n tokens uses its spare capacity first; a shortfall of m slots is
  allocated as below, aiming at w = m rounded up to the allocator's granule G (w = m if fewer
  than w slots are free), so that a request growing one token at a time gets a new range only
  every G tokens;
- reserving capacity c allocates c - C slots the same way (w = c - C) without adding keys, for
  a caller that knows a request's final length;
- an allocation of w slots (at least m of them needed) first extends the last segment in place,
  over up to w of the free slots that directly follow it; the remaining w' (m') go into the
  smallest free run of at least w' slots (lowest start among equals), taken from its start; if no
  free run holds w', the largest free run (lowest start among equals) gives min(its length, w')
  slots and the rest is placed the same way, until at least m slots were added;
- an allocation that needs more slots than are free fails and changes nothing;
- releasing a request frees all its slots; truncating it to L' < L keys frees every slot after
  its first L' (spare capacity included).

Compaction (the pages name the aim, each request's cache kept contiguous, but no procedure; the
reading modelled here) relocates fragmented requests into single ranges without ever moving data
over data that is still to be moved:

- the free runs at the start of the call are the only destinations (slots freed by the call itself
  are not reused in it), so every destination lies in space that held no live data;
- requests owning two or more ranges are taken in order of decreasing range count, then
  increasing request id; each goes, whole (capacity C), into the smallest of those runs that holds
  C (lowest start among equals), from the run's start, the rest of the run staying available; a
  request that fits nowhere is left as it is;
- a relocated request owns the one range [s, s + C) afterwards, its L keys being its first L
  slots; its old ranges are freed; the moves copy each old range's key slots, in key order, to
  consecutive slots from s.

Every destination is then disjoint from every source and from every other destination, so the
moves may be applied in any order, or all at once.

The model keeps one boolean per pool slot and finds free runs by scanning it, so that it can be
checked by eye; it is slow and meant for small pools.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np


class AllocatorModel:
    """Bitmap model: used[i] is True when pool slot i belongs to some request."""

    def __init__(self, pool_tokens: int, granule: int = 1):
        if pool_tokens < 0 or granule < 1:
            raise ValueError("pool_tokens must be >= 0 and granule >= 1")
        self.pool_tokens = int(pool_tokens)
        self.granule = int(granule)
        self.used = np.zeros(self.pool_tokens, dtype=bool)
        self.segs: Dict[int, List[List[int]]] = {}  # request -> [[offset, slots], ...]
        self.keys: Dict[int, int] = {}               # request -> L

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
        return self.keys.get(request, 0)

    def capacity(self, request: int) -> int:
        return sum(ln for _, ln in self.segs.get(request, []))

    def segments(self, request: int) -> List[Tuple[int, int]]:
        """The segments holding the request's keys: its first L slots, in order."""
        out, left = [], self.length(request)
        for o, ln in self.segs.get(request, []):
            if left <= 0:
                break
            out.append((o, min(ln, left)))
            left -= ln
        return out

    def owned(self, request: int) -> List[Tuple[int, int]]:
        """Every slot range the request owns, spare capacity included."""
        return [(o, ln) for o, ln in self.segs.get(request, [])]

    # ---------------------------------------------------------------- updates

    def _take(self, start: int, n: int):
        assert not self.used[start:start + n].any()
        self.used[start:start + n] = True

    def _allocate(self, request: int, need: int, want: int):
        """Add at least `need` (aiming at `want`) slots to the request; need <= free slots."""
        segs = self.segs.setdefault(request, [])
        if want > self.free_tokens():
            want = need
        # 1. in place, after the last segment
        if segs and want > 0:
            end = segs[-1][0] + segs[-1][1]
            k = 0
            while k < want and end + k < self.pool_tokens and not self.used[end + k]:
                k += 1
            if k > 0:
                self._take(end, k)
                segs[-1][1] += k
                need -= k
                want -= k
        # 2./3. best fit for what is still wanted, else the largest run, until enough
        while need > 0:
            runs = self.free_runs()
            fits = [r for r in runs if r[1] >= want]
            if fits:
                start, _ = min(fits, key=lambda r: (r[1], r[0]))
                take = want
            else:
                start, ln = min(runs, key=lambda r: (-r[1], r[0]))
                take = min(ln, want)
            self._take(start, take)
            segs.append([start, take])
            need -= take
            want -= take

    def _round(self, m: int) -> int:
        return -(-m // self.granule) * self.granule

    def grow(self, request: int, n: int) -> bool:
        """Add n keys to the request; False (and no change) if the pool cannot hold them."""
        if n < 0:
            raise ValueError("n must be >= 0")
        short = self.length(request) + n - self.capacity(request)
        if short > self.free_tokens():
            return False
        self.segs.setdefault(request, [])
        if short > 0:
            self._allocate(request, short, self._round(short))
        self.keys[request] = self.length(request) + n
        return True

    def reserve(self, request: int, capacity: int) -> bool:
        """Make the request's capacity at least `capacity`; False (no change) if it cannot."""
        if capacity < 0:
            raise ValueError("capacity must be >= 0")
        short = capacity - self.capacity(request)
        if short > self.free_tokens():
            return False
        self.segs.setdefault(request, [])
        self.keys.setdefault(request, 0)
        if short > 0:
            self._allocate(request, short, short)
        return True

    def release(self, request: int):
        for off, ln in self.segs.pop(request, []):
            self.used[off:off + ln] = False
        self.keys.pop(request, None)

    def truncate(self, request: int, new_length: int):
        """Keep the request's first new_length keys and free every later slot it owns."""
        if new_length < 0:
            raise ValueError("new_length must be >= 0")
        if request not in self.segs or new_length >= self.length(request):
            return
        segs = self.segs[request]
        excess = self.capacity(request) - new_length
        while excess > 0 and segs:
            off, ln = segs[-1]
            cut = min(excess, ln)
            self.used[off + ln - cut:off + ln] = False
            segs[-1][1] = ln - cut
            if segs[-1][1] == 0:
                segs.pop()
            excess -= cut
        self.keys[request] = new_length

    def compact(self) -> List[Tuple[int, int, int]]:
        """Relocate fragmented requests as described in the module docstring. Returns the moves
        (src_offset, dst_offset, length) the pool data must undergo, in plan order."""
        runs = [list(r) for r in self.free_runs()]  # destinations: the free space at the start
        order = sorted((r for r, sg in self.segs.items() if len(sg) >= 2),
                       key=lambda r: (-len(self.segs[r]), r))
        moves = []
        for r in order:
            cap = self.capacity(r)
            fits = [i for i, (st, ln) in enumerate(runs) if ln >= cap]
            if not fits:
                continue
            i = min(fits, key=lambda i: (runs[i][1], runs[i][0]))
            dst = runs[i][0]
            runs[i][0] += cap
            runs[i][1] -= cap
            left, done = self.length(r), 0
            for off, ln in self.segs[r]:
                n = min(ln, left)
                if n > 0:
                    moves.append((off, dst + done, n))
                done += n
                left -= n
            for off, ln in self.segs[r]:
                self.used[off:off + ln] = False
            self._take(dst, cap)
            self.segs[r] = [[dst, cap]]
        return moves

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


def apply_moves(pool: np.ndarray, moves: Sequence[Tuple[int, int, int]]) -> np.ndarray:
    """A copy of `pool` (first axis = slots) with every move's source slots copied to its
    destination slots, one move after the other."""
    out = np.array(pool, copy=True)
    for src, dst, n in moves:
        out[dst:dst + n] = out[src:src + n]
    return out
