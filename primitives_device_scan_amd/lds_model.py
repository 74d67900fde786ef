"""Bank-conflict model of the 4,096-element LDS tile scans (host-side arithmetic).

The model of "Day 32 -- The CUDA scan algorithm: the tree and the three
kernels" (sections "The stride doubles, and so does the conflict" and
"Results", tile-model table): at level `stride` of the work-efficient tree,
active lane a touches words (2a+1)*stride-1 and (2a+2)*stride-1; lanes are
served in groups, and a group costs as many requests as the most lanes it
puts on one bank. Summed over the groups of every level of both sweeps this
gives the "requests per tile" the page prints (32-lane groups, 32 banks).

On gfx950 a wave64's 4-byte LDS access is served as two 32-lane halves over
32 banks of 4 bytes (measured with a stride probe: stride-s word accesses
cost gcd-style max(1, lanes per bank) cycles per half), so the same model
with 32-lane groups describes one half-wave, and the conflict cycles the
SQ_LDS_BANK_CONFLICT counter reports are the requests beyond one per group,
for every LDS access the kernel makes.
"""
from __future__ import annotations

from collections import Counter


def pad_none(i: int) -> int:
    return i


def pad_one(i: int) -> int:
    return i + (i >> 5)


def pad_two(i: int) -> int:
    return i + (i >> 5) + (i >> 10)


PADS = {"tree": pad_none, "tree_pad1": pad_one, "tree_pad2": pad_two}


def degree(words, banks: int) -> int:
    """Most lanes of one group on a single bank (each lane a distinct word)."""
    return max(Counter(w % banks for w in words).values())


def tree_levels(tile: int = 4096, threads: int = 1024, group: int = 32, banks: int = 32, pad=pad_none):
    """Up-sweep levels: stride, active lanes, groups, and the degree of the
    lo ((2a+1)s-1) and hi ((2a+2)s-1) word patterns of each group. Pairs
    beyond `threads` are taken in further rounds by the same threads."""
    levels = []
    stride = 1
    while stride < tile:
        pairs = tile // (2 * stride)
        groups = []
        for start in range(0, pairs, threads):
            lanes = list(range(start, min(pairs, start + threads)))
            for g in range(0, len(lanes), group):
                ln = lanes[g:g + group]
                lo = [pad((2 * a + 1) * stride - 1) for a in ln]
                hi = [pad((2 * a + 2) * stride - 1) for a in ln]
                groups.append((degree(lo, banks), degree(hi, banks)))
        levels.append({"stride": stride, "lanes": pairs, "groups": len(groups),
                       "degree": max(d for _, d in groups), "groups_detail": groups})
        stride *= 2
    return levels


def tree_requests(pad=pad_none, **kw) -> int:
    """Requests per tile over both sweeps, one access pattern per level (the page's count)."""
    return 2 * sum(sum(d for _, d in lv["groups_detail"]) for lv in tree_levels(pad=pad, **kw))


def hs_requests(tile: int = 4096, group: int = 32) -> int:
    """Hillis-Steele: every word read once per step by adjacent lanes, never in conflict."""
    steps = (tile - 1).bit_length()
    return steps * (tile // group)


def tree_adds(tile: int = 4096) -> int:
    return 2 * (tile - 1)


def hs_adds(tile: int = 4096) -> int:
    d, adds = 1, 0
    while d < tile:
        adds += tile - d
        d *= 2
    return adds


def tree_conflict_cycles(pad=pad_none, **kw) -> int:
    """Conflict cycles per tile for the kernel's own accesses: each up-sweep
    pair reads lo and hi and writes hi; each down-sweep pair reads lo and hi
    and writes both. Load, store and root accesses are conflict-free."""
    total = 0
    for lv in tree_levels(pad=pad, **kw):
        for dlo, dhi in lv["groups_detail"]:
            total += (dlo - 1) + 2 * (dhi - 1)          # up-sweep
            total += 2 * (dlo - 1) + 2 * (dhi - 1)      # down-sweep
    return total
