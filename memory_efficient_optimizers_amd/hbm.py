"""Placement of an optimizer step's buffers in the thirds of MI355X HBM.

What is measured on MI355X (288 GiB of HBM3E, all on one GPU):

* Device memory behaves as three 96 GiB thirds of the physical address space.
  The apply pass of an Adafactor step (read G, X and M; write X and M) runs 14-16%
  slower when the parameter X and the first moment M lie in the same third than
  when they lie in different thirds, wherever they sit inside it. For the 7B
  list, that is 23.5-23.8 ms against 20.3-20.6 ms per apply pass.
* What triggers it is two streams of stores into the same third in one pass.
  Leaving out the store of M removes the difference; leaving out a load keeps
  it. One read-modify-write stream alone runs at full speed in any third, and
  so do reads.
* The position of the gradient matters little, about 2% of the pass.

HIP does not expose physical addresses, and a large allocation is made of
power-of-two blocks that the driver places by its own rules. So this module
allocates memory in chunks of 2 GiB, each a single block of the driver's
allocator (2 GiB-aligned, so inside one third). It finds each chunk's third by
timing the library's own apply pass on a probe tensor whose parameter and
first moment sit in a pair of chunks, and then packs each kind of buffer into
chunks of one third:

* parameters in one third;
* first moments in another;
* LAMB's full second moments, and the gradients, in the last.

This way, no pass writes two big streams into one third: Adafactor's apply
writes X and M, and LAMB's moment pass writes M and V.

Used by the benchmark. Callers that place their own state can do the same:
``ChunkPool(...).classify()`` and then ``pack``.
"""
from __future__ import annotations

import math
import statistics
from typing import Callable, Dict, List, Optional, Sequence, Tuple

GiB = 1 << 30
CHUNK = 2 * GiB
ALIGN = 256
# Probe: one (65536, 8192) matrix, its fp32 parameter and first moment filling a
# chunk each, bf16 gradient; its apply pass moves 9.7 GB (1.6-2.0 ms), far past the
# 256 MiB Infinity Cache. Pairs in one third run 12-20% slower than pairs apart;
# within a third the time varies by up to 9% with the chunks' finer placement.
PROBE_SHAPE = (65536, 8192)


def split_two(times: Dict[int, float], min_sep: float = 0.05) -> Optional[Tuple[List[int], List[int]]]:
    """Splits chunk -> time into (slow, fast): first at the threshold that
    maximises the variance between the two groups (Otsu's method), then moved to
    the midpoint between the groups' means until it settles (two-means). None
    unless the means differ by at least ``min_sep`` of the fast group's. Unlike
    the largest gap, this threshold does not follow one outlying time."""
    if len(times) < 2:
        return None
    order = sorted(times, key=times.get)
    vals = [times[c] for c in order]
    n = len(vals)
    total = sum(vals)
    best, cut, left = -1.0, 0, 0.0
    for i in range(1, n):
        left += vals[i - 1]
        m0, m1 = left / i, (total - left) / (n - i)
        between = i * (n - i) * (m1 - m0) ** 2
        if between > best:
            best, cut = between, i
    # refine to the midpoint between the two groups' means (two-means)
    for _ in range(8):
        m0 = sum(vals[:cut]) / cut
        m1 = sum(vals[cut:]) / (n - cut)
        mid = 0.5 * (m0 + m1)
        new_cut = sum(1 for v in vals if v <= mid)
        if new_cut in (0, n) or new_cut == cut:
            break
        cut = new_cut
    m0 = sum(vals[:cut]) / cut
    m1 = sum(vals[cut:]) / (n - cut)
    if m1 - m0 < min_sep * m0:
        return None
    return order[cut:], order[:cut]


def classify(chunks: Sequence[int], probe: Callable[[int, int], float], min_sep: float = 0.05
             ) -> Optional[List[List[int]]]:
    """Groups chunk ids into thirds: chunks whose pair with a reference runs slow
    share its third. ``probe(a, b)`` times the apply pass with the parameter in
    chunk a and the first moment in chunk b. The first reference's times must split
    into a slow and a fast level (split_two); later references sort their chunks
    by the nearer of those two levels. Returns the groups, largest first, or None
    where the times do not split cleanly or make more than three groups."""
    rest = list(chunks)
    groups: List[List[int]] = []
    mid = None  # halfway between the slow and the fast level
    while rest:
        ref, others = rest[0], rest[1:]
        if not others:
            groups.append([ref])
            break
        times = {c: probe(ref, c) for c in others}
        if mid is None:
            split = split_two(times, min_sep)
            if split is None:
                return None
            slow, fast = split
            mid = 0.5 * (statistics.median(times[c] for c in slow) + statistics.median(times[c] for c in fast))
        else:
            slow = [c for c in others if times[c] > mid]
            fast = [c for c in others if times[c] <= mid]
        groups.append([ref] + sorted(slow))
        rest = sorted(fast)
        if len(groups) > 3:
            return None
    return sorted(groups, key=len, reverse=True)


def pack(sizes: Sequence[int], chunk_bytes: int = CHUNK) -> List[Tuple[int, int]]:
    """(chunk index, byte offset) of each buffer, first fit in order, each offset
    256-byte aligned; every size must fit in one chunk."""
    out: List[Tuple[int, int]] = []
    used: List[int] = []
    for n in sizes:
        if n > chunk_bytes:
            raise ValueError(f"a buffer of {n} bytes does not fit in a {chunk_bytes}-byte chunk")
        for i, u in enumerate(used):
            if u + n <= chunk_bytes:
                out.append((i, u))
                used[i] = (u + n + ALIGN - 1) // ALIGN * ALIGN
                break
        else:
            out.append((len(used), 0))
            used.append((n + ALIGN - 1) // ALIGN * ALIGN)
    return out


def chunks_needed(sizes: Sequence[int], chunk_bytes: int = CHUNK) -> int:
    return 1 + max((c for c, _ in pack(sizes, chunk_bytes)), default=-1)


class ChunkPool:
    """2 GiB device chunks (torch uint8 tensors) filling the free memory of the
    current device down to ``keep_free`` bytes, and their thirds."""

    def __init__(self, torch, device="cuda", keep_free: int = 6 * GiB, max_chunks: int = 160):
        self.torch = torch
        self.device = device
        self.chunks = []
        while len(self.chunks) < max_chunks and torch.cuda.mem_get_info()[0] > keep_free + CHUNK:
            self.chunks.append(torch.zeros(CHUNK, dtype=torch.uint8, device=device))
        self.groups: Optional[List[List[int]]] = None

    def probe_fn(self, _lib, repeats: int = 2):
        """The timing probe: the library's Adafactor step (beta1 = 0.9) on one
        PROBE_SHAPE matrix with its parameter in chunk a and its first moment in
        chunk b (gradient and statistics elsewhere); the apply pass's average time
        over ``repeats`` steps after a warm one, from the library's pass events."""
        torch = self.torch
        m, n = PROBE_SHAPE
        grad = torch.zeros(PROBE_SHAPE, dtype=torch.bfloat16, device=self.device)
        grad.normal_(0.0, 1e-3)
        row = torch.zeros(m, dtype=torch.float32, device=self.device)
        col = torch.zeros(n, dtype=torch.float32, device=self.device)
        hp = _lib.adafactor_hparams(beta1=0.9)
        nbytes = m * n * 4
        stream = torch.cuda.current_stream()
        step = [0]

        def view(c):
            return self.chunks[c][:nbytes].view(torch.float32).view(PROBE_SHAPE)

        ws = _lib.workspace(_lib.meo_adafactor_workspace_size([view(0)], [grad]), self.device)

        def probe(a: int, b: int) -> float:
            x, mom = view(a), view(b)
            st = [{"exp_avg": mom, "exp_avg_sq_row": row, "exp_avg_sq_col": col}]
            call = _lib.PreparedStep("adafactor", hp, [x], [grad], st, ws)
            step[0] += 1
            call(step[0], stream)
            torch.cuda.synchronize()
            _lib.meo_profile_enable(True)
            _lib.meo_profile_collect()
            for _ in range(repeats):
                step[0] += 1
                call(step[0], stream)
            torch.cuda.synchronize()
            passes = _lib.meo_profile_collect()
            _lib.meo_profile_enable(False)
            x.zero_()
            mom.zero_()
            rec = passes["adafactor_apply"]
            return rec["ms"] / rec["launches"]

        return probe

    def classify(self, _lib) -> Optional[List[List[int]]]:
        """Groups the chunks by third (largest group first); None if the probe's
        times do not split cleanly (then the chunks keep their allocation order).
        ``self.probe_ms`` records the median probe time of pairs in the same group
        and of pairs in different groups."""
        probe = self.probe_fn(_lib)
        seen: List[Tuple[int, int, float]] = []

        def recorded(a, b):
            t = probe(a, b)
            seen.append((a, b, t))
            return t

        self.groups = classify(range(len(self.chunks)), recorded)
        _lib.meo_release_plans()
        self.probe_ms = None
        if self.groups:
            where = {c: k for k, g in enumerate(self.groups) for c in g}
            same = [t for a, b, t in seen if where[a] == where[b]]
            other = [t for a, b, t in seen if where[a] != where[b]]
            self.probe_ms = {"same_third": statistics.median(same) if same else None,
                             "other_third": statistics.median(other) if other else None,
                             "probes": len(seen)}
        return self.groups

    def views(self, chunk_ids: Sequence[int], shapes: Sequence[tuple], dtypes: Sequence):
        """Tensors of the given shapes and dtypes packed into the given chunks (in
        order, first fit); raises if they do not fit."""
        torch = self.torch
        sizes = [math.prod(s) * torch.empty((), dtype=d).element_size() for s, d in zip(shapes, dtypes)]
        where = pack(sizes)
        if where and max(c for c, _ in where) >= len(chunk_ids):
            raise ValueError(f"{len(chunk_ids)} chunks cannot hold {sum(sizes)} bytes")
        out = []
        for (c, off), n, s, d in zip(where, sizes, shapes, dtypes):
            buf = self.chunks[chunk_ids[c]]
            out.append(buf[off:off + n].view(d).view(s))
        return out

    def release(self, keep: Sequence[int]) -> None:
        """Frees every chunk not in ``keep`` (views keep theirs alive anyway)."""
        keep = set(keep)
        for i in range(len(self.chunks)):
            if i not in keep:
                self.chunks[i] = None
        self.torch.cuda.empty_cache()
