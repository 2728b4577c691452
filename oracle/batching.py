"""Oracle of the batch planners (test infrastructure only; see the package
docstring).

Sources: the announcement article's "Serving" section and the README's
"Batching" section (queued requests packed by machine performance, the batch
of highest priority by waiting time, batch size and room to grow at its
padded length runs first, after TurboTransformers' dynamic-programming
scheduler); FIFO packing padded to each batch's longest request is the
baseline of the article's "Performance tests" section.

Readings (the pages give no formula):
  * cost of a batch = t_batch + S(tokens) + t_row * B * P + t_pair * pairs
    with P the longest length in the batch, tokens the summed lengths (rounded
    up to token_quantum), pairs the summed len(len+1)/2; when the forward keeps
    the padding, tokens = B * P and pairs = B * P(P+1)/2; S is linear
    (t_token * tokens) or a table of measured batch times over token counts
    (TurboTransformers' scheduler works from such a table);
  * the plan splits the length-sorted queue (ties by arrival) into runs, the
    least summed cost over all such splits, ties to the longer last batch;
  * run order: longest waiting request first, then more requests, then the
    earliest arrival.
Plain Python loops; sizes here are small.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple


@dataclass(frozen=True)
class Cost:
    t_batch: float = 0.0
    t_token: float = 0.0
    t_row: float = 0.0
    t_pair: float = 0.0
    token_quantum: int = 1
    padded_compute: bool = False
    token_table: Tuple[float, ...] = ()


def token_seconds(tokens: float, c: Cost) -> float:
    """The token term: t_token * tokens, or the measured table -- entry k holds
    a batch of (k + 1) * token_quantum tokens; past the end, the line through
    the last two entries (or through the origin and the only entry)."""
    if not c.token_table:
        return c.t_token * tokens
    q = max(1, c.token_quantum)
    k = int(tokens // q) - 1
    table = c.token_table
    if k < 0:
        return 0.0
    if k < len(table):
        return table[k]
    if len(table) >= 2:
        return table[-1] + (k - (len(table) - 1)) * (table[-1] - table[-2])
    return table[0] * (k + 1)


def batch_cost(batch_lens: Sequence[int], c: Cost) -> float:
    """Seconds to run one batch under the cost model (formula in the module docstring)."""
    B = len(batch_lens)
    P = max(batch_lens)
    if c.padded_compute:
        tokens = float(B * P)
        pairs = float(B) * (float(P) * float(P + 1) / 2.0)
    else:
        tokens = float(sum(batch_lens))
        pairs = float(sum(n * (n + 1) // 2 for n in batch_lens))
    if c.token_quantum > 1:
        tokens = float(math.ceil(tokens / c.token_quantum) * c.token_quantum)
    return c.t_batch + token_seconds(tokens, c) + c.t_row * float(B * P) + c.t_pair * pairs


def fifo_batches(lens: Sequence[int], max_batch: int) -> List[List[int]]:
    """Consecutive groups of max_batch requests in arrival order."""
    return [list(range(i, min(i + max_batch, len(lens)))) for i in range(0, len(lens), max_batch)]


def length_order(lens: Sequence[int]) -> List[int]:
    return sorted(range(len(lens)), key=lambda i: (lens[i], i))


def dp_runs(lens: Sequence[int], max_batch: int, c: Cost, max_tokens: int = 0) -> Tuple[List[Tuple[int, int]], float]:
    """Least-cost split of the length order into runs [lo, hi): returns the runs
    (in order) and the summed cost.  best[i] covers the first i requests."""
    order = length_order(lens)
    n = len(order)
    best = [math.inf] * (n + 1)
    start = [-1] * (n + 1)
    best[0] = 0.0
    for i in range(1, n + 1):
        candidates = []
        for j in range(max(0, i - max_batch), i):
            run = [lens[k] for k in order[j:i]]
            rows = len(run) * max(run) if c.padded_compute else sum(run)
            if best[j] == math.inf or (max_tokens > 0 and rows > max_tokens):
                continue
            candidates.append((best[j] + batch_cost(run, c), j))
        if candidates:
            best[i], start[i] = min(candidates)      # equal cost: the smaller j, i.e. the longer last batch
    if best[n] == math.inf:
        raise ValueError("no feasible plan")
    runs = []
    i = n
    while i > 0:
        runs.append((start[i], i))
        i = start[i]
    return runs[::-1], best[n]


def dynamic_batches(lens: Sequence[int], max_batch: int, c: Cost, max_tokens: int = 0,
                    wait: Optional[Sequence[float]] = None) -> Tuple[List[List[int]], float]:
    """Request indices of each batch in run order, and the plan's summed cost."""
    order = length_order(lens)
    runs, total = dp_runs(lens, max_batch, c, max_tokens)
    batches = [[order[k] for k in range(lo, hi)] for lo, hi in runs]
    w = list(wait) if wait is not None else [0.0] * len(lens)
    batches.sort(key=lambda b: (-max(w[i] for i in b), -len(b), min(b)))
    return [sorted(b) for b in batches], total


def padded_rows(batches: Sequence[Sequence[int]], lens: Sequence[int]) -> int:
    """Rows of the padded layout: sum over batches of B * (longest length)."""
    return sum(len(b) * max(lens[i] for i in b) for b in batches)
