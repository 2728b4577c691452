"""Pins for the batch-planner oracle (CPU only): a hand-worked example,
brute force over every split of the length order (the dynamic programme's
search space) and over every set partition (the claim that runs of the length
order are optimal for costs linear in the tokens), closed forms, and the run
order rules."""
import itertools
import random

import pytest

import oracle
from oracle import Cost


def test_hand_worked_example():
    # lengths 5, 3, 9, 1, 2 (arrival order), at most 2 per batch, cost 1 s per batch,
    # 10 ms per token, 1 ms per padded row.  Sorted: 1 2 3 5 9.  Candidate splits
    # (by hand): {1,2}{3,5}{9}: 1.034 + 1.090 + 1.099 = 3.223;
    # {1}{2,3}{5,9}: 1.011 + 1.056 + 1.158 = 3.225;  three batches is the least
    # possible count with 5 requests at 2 per batch, and the first is cheapest.
    c = Cost(t_batch=1.0, t_token=0.01, t_row=0.001)
    batches, total = oracle.dynamic_batches([5, 3, 9, 1, 2], 2, c)
    assert total == pytest.approx(3.223, rel=1e-12)
    assert batches == [[0, 1], [3, 4], [2]]        # two full batches first (earliest arrival first), then {9}
    assert oracle.batch_cost([1, 2], c) == pytest.approx(1.034, rel=1e-12)
    assert oracle.batch_cost([5, 9], c) == pytest.approx(1.158, rel=1e-12)


def _compositions(n, cap):
    """All splits of range(n) into consecutive runs of length <= cap."""
    for cuts in itertools.product([0, 1], repeat=max(0, n - 1)):
        runs, lo = [], 0
        for i, c in enumerate(cuts, start=1):
            if c:
                runs.append((lo, i))
                lo = i
        runs.append((lo, n))
        if all(hi - lo <= cap for lo, hi in runs):
            yield runs


def _set_partitions(items):
    if not items:
        yield []
        return
    first, rest = items[0], items[1:]
    for part in _set_partitions(rest):
        for k in range(len(part)):
            yield part[:k] + [[first] + part[k]] + part[k + 1:]
        yield [[first]] + part


COSTS = [
    Cost(t_batch=1.0, t_token=0.01, t_row=0.002, t_pair=1e-5),
    Cost(t_batch=0.3, t_token=0.02, t_row=0.0, t_pair=0.0, token_quantum=8),
    Cost(t_batch=0.5, t_token=0.01, t_row=0.001, t_pair=1e-4, padded_compute=True),
    Cost(t_batch=0.0, t_token=1.0, t_row=0.5, t_pair=0.0),
]


@pytest.mark.parametrize("ci", range(len(COSTS)))
def test_dp_is_the_least_cost_split_of_the_length_order(ci):
    rng = random.Random(100 + ci)
    c = COSTS[ci]
    for _ in range(40):
        n = rng.randint(1, 9)
        lens = [rng.randint(1, 20) for _ in range(n)]
        cap = rng.randint(1, 4)
        max_tokens = rng.choice([0, 0, 40])
        order = oracle.length_order(lens)
        best = None
        for runs in _compositions(n, cap):
            groups = [[lens[k] for k in order[lo:hi]] for lo, hi in runs]
            rows = [len(g) * max(g) if c.padded_compute else sum(g) for g in groups]
            if max_tokens and max(rows) > max_tokens:
                continue
            tot = sum(oracle.batch_cost(g, c) for g in groups)
            best = tot if best is None else min(best, tot)
        runs, total = oracle.dp_runs(lens, cap, c, max_tokens)
        assert total == pytest.approx(best, rel=1e-12, abs=1e-12)
        assert sum(oracle.batch_cost([lens[k] for k in order[lo:hi]], c) for lo, hi in runs) == \
            pytest.approx(total, rel=1e-12)


@pytest.mark.parametrize("ci", [0, 2, 3])
def test_runs_of_the_length_order_are_optimal_for_linear_costs(ci):
    """Over every set partition (token_quantum = 1): no grouping beats the best
    split of the length order -- the reason the planner may search runs only."""
    rng = random.Random(7 + ci)
    c = COSTS[ci]
    for _ in range(12):
        n = rng.randint(1, 7)
        lens = [rng.randint(1, 30) for _ in range(n)]
        cap = rng.randint(1, 3)
        best = min(sum(oracle.batch_cost([lens[i] for i in blk], c) for blk in part)
                   for part in _set_partitions(list(range(n))) if all(len(b) <= cap for b in part))
        assert oracle.dp_runs(lens, cap, c)[1] == pytest.approx(best, rel=1e-12, abs=1e-12)


def test_equal_lengths_closed_form():
    L, cap, k = 37, 8, 5
    c = Cost(t_batch=2.0, t_token=0.1, t_row=0.01, t_pair=1e-4)
    batches, total = oracle.dynamic_batches([L] * (cap * k), cap, c)
    assert [len(b) for b in batches] == [cap] * k
    one = 2.0 + 0.1 * cap * L + 0.01 * cap * L + 1e-4 * cap * L * (L + 1) / 2
    assert total == pytest.approx(k * one, rel=1e-12)
    assert oracle.padded_rows(batches, [L] * (cap * k)) == cap * k * L


def test_token_table_closed_forms():
    # entry k: (k+1) * 100 tokens; inside the table the entry itself, past it the
    # line through the last two entries, below one quantum nothing
    c = Cost(token_quantum=100, token_table=(1.0, 1.5, 1.8))
    assert oracle.token_seconds(100, c) == 1.0 and oracle.token_seconds(300, c) == 1.8
    assert oracle.token_seconds(500, c) == pytest.approx(1.8 + 2 * 0.3)
    assert oracle.batch_cost([150, 40], c) == 1.5                 # 190 tokens round up to 200
    one = Cost(token_quantum=10, token_table=(2.0,))
    assert oracle.token_seconds(30, one) == 6.0
    # a table that is exactly linear reproduces the linear model
    lin = Cost(t_row=0.01, token_quantum=64, token_table=tuple(0.002 * 64 * (k + 1) for k in range(8)))
    ref = Cost(t_row=0.01, t_token=0.002, token_quantum=64)
    for lens in ([5, 60, 200], [64] * 8, [1]):
        assert oracle.batch_cost(lens, lin) == pytest.approx(oracle.batch_cost(lens, ref), rel=1e-12)


def test_dp_with_a_table_is_the_least_cost_split():
    rng = random.Random(3)
    c = Cost(t_row=0.001, token_quantum=16, token_table=(1.0, 1.2, 1.3, 1.35, 1.4))
    for _ in range(30):
        n = rng.randint(1, 8)
        lens = [rng.randint(1, 40) for _ in range(n)]
        cap = rng.randint(1, 4)
        order = oracle.length_order(lens)
        best = min(sum(oracle.batch_cost([lens[k] for k in order[lo:hi]], c) for lo, hi in runs)
                   for runs in _compositions(n, cap))
        assert oracle.dp_runs(lens, cap, c)[1] == pytest.approx(best, rel=1e-12)


def test_fifo_and_padded_rows():
    lens = [3, 10, 2, 2, 7]
    b = oracle.fifo_batches(lens, 2)
    assert b == [[0, 1], [2, 3], [4]]
    assert oracle.padded_rows(b, lens) == 2 * 10 + 2 * 2 + 7


def test_run_order_rules():
    lens = [4, 4, 9, 9, 9, 1]
    # 1 s per batch, 1 s per padded row: {1}{4,4}{9,9,9} costs 3 + 1 + 8 + 27 = 39,
    # {1,4,4}{9,9,9} costs 2 + 12 + 27 = 41, so one batch per distinct length
    c = Cost(t_batch=1.0, t_token=0.0, t_row=1.0)
    # no waiting: larger batches first ({9,9,9} then {4,4} then {1}); earliest arrival breaks ties
    batches, _ = oracle.dynamic_batches(lens, 3, c)
    assert sorted(map(tuple, batches)) == [(0, 1), (2, 3, 4), (5,)]
    assert batches[0] == [2, 3, 4]
    # the request of length 1 has waited longest: its batch runs first
    batches_w, _ = oracle.dynamic_batches(lens, 3, c, wait=[0, 0, 0, 0, 0, 5.0])
    assert batches_w[0] == [5]
    # padded compute: a batch is padded to its longest request
    c_pad = Cost(t_batch=0.0, t_token=1.0, padded_compute=True)
    assert oracle.batch_cost([1, 9], c_pad) == 18.0 and oracle.batch_cost([4, 4], c_pad) == 8.0


def test_token_limit_and_errors():
    c = Cost(t_batch=1.0, t_token=0.01)
    batches, _ = oracle.dynamic_batches([10, 10, 10, 10], 4, c, max_tokens=20)
    assert all(sum([10] * len(b)) <= 20 for b in batches) and len(batches) == 2
    with pytest.raises(ValueError):
        oracle.dp_runs([50], 4, c, max_tokens=20)
