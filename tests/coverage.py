"""Output rows a sampled parity check compares at shapes too large to check whole.

A seeded random sample alone can miss a class of work unit.  The rows chosen
here are the union of
  * ``n_random`` seeded random rows, the first and last row, and the rows on
    both sides of each edge of the shared-expert range;
  * for every expert of at least 64 tokens (the smallest expert with
    cooperative units: 64 where a wave holds one 32-row fragment, 96 where it
    holds two; the 64-95 token experts of the latter kinds run as wave items
    of two or three row tiles, which the same rows cover), one token in every
    128-row group of its range, at an offset that moves through the group
    from one group to the next (so the four waves and both 32-row fragments
    of a wave are hit across groups), plus the expert's last token (its last,
    usually partial, group);
  * the last token of ``n_small`` seeded experts below that size (the ragged
    tail of a 32-row wave item),
each mapped to the output row it is scattered to.  Every selected row is then
compared on all N columns, with every token routed to it.
"""
from __future__ import annotations

import numpy as np

COOP_MIN_ROWS = 64   # smallest expert given per-group rows (see above)
GROUP_STEP = 128     # rows per cooperative group (256-row groups are two of them)


def coverage_rows(w, row_index: np.ndarray, n_random: int = 16, n_small: int = 16,
                  seed: int = 0) -> np.ndarray:
    counts = np.asarray(w.counts(), np.int64)
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    rng = np.random.default_rng(20_000 + w.seed + seed)
    rows = set(rng.choice(w.batch, size=min(n_random, w.batch), replace=False).tolist())
    rows.update({0, w.batch - 1})
    if w.R > 0:
        for r in (w.shared_offset - 1, w.shared_offset, w.shared_offset + w.R - 1,
                  w.shared_offset + w.R):
            if 0 <= r < w.batch:
                rows.add(r)
    tokens = []
    small = []
    for e, (s, c) in enumerate(zip(starts.tolist(), counts.tolist())):
        if c >= COOP_MIN_ROWS:
            for g0 in range(0, c, GROUP_STEP):
                span = min(GROUP_STEP, c - g0)
                tokens.append(s + g0 + (37 * (g0 // GROUP_STEP) + 11 * e) % span)
            tokens.append(s + c - 1)
        elif c > 0:
            small.append(s + c - 1)
    if small:
        pick = rng.choice(len(small), size=min(n_small, len(small)), replace=False)
        tokens.extend(small[i] for i in pick)
    ri = np.asarray(row_index, np.int64)
    rows.update(int(ri[t]) for t in tokens)
    return np.array(sorted(rows), np.int64)
