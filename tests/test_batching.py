"""The native batch planners of libee (host code, no GPU) against the oracle:
the same plan and the same summed cost, bit for bit (both evaluate the cost
formula in the same order in IEEE double, without fused multiply-adds), on
random queues and on the 1024-request stream of the 48-layer workload."""
import random

import pytest

import oracle
import variable_length_padding_amd as ee
import workloads
from oracle import Cost


def _native_cost(c: Cost) -> ee.BatchCost:
    n = ee.BatchCost(c.t_batch, c.t_token, c.t_row, c.t_pair, c.token_quantum, 1 if c.padded_compute else 0)
    if c.token_table:
        n.set_table(c.token_table)
    return n


# a concave measured-looking table: seconds for 1..16 K tokens
_TABLE = tuple(0.03 + 0.00012 * 1024 * (k + 1) * (1.0 + 0.3 / (k + 1)) for k in range(16))


COSTS = [
    Cost(t_batch=0.05, t_token=1.3e-4, t_row=1.2e-8, t_pair=2.0e-10, token_quantum=256),
    Cost(t_batch=0.05, t_token=1.3e-4, t_row=1.2e-8, t_pair=2.0e-10, padded_compute=True),
    Cost(t_batch=1.0, t_token=0.01, t_row=0.001),
    Cost(t_batch=0.0, t_token=1.0, t_row=0.25, t_pair=1e-3, token_quantum=7),
    Cost(t_row=5e-9, token_quantum=1024, token_table=_TABLE),
    Cost(token_quantum=1024, padded_compute=True, token_table=_TABLE[:3]),
    Cost(t_batch=0.01, token_quantum=64, token_table=(0.5,)),
]


@pytest.mark.parametrize("ci", range(len(COSTS)))
def test_dynamic_plan_matches_oracle(ci):
    rng = random.Random(31 + ci)
    c = COSTS[ci]
    for trial in range(25):
        n = rng.randint(1, 300)
        lens = [rng.randint(1, 256) for _ in range(n)]
        cap = rng.choice([1, 4, 16, 64])
        max_tokens = rng.choice([0, 0, 4096]) if not c.padded_compute else rng.choice([0, 16384])
        wait = [rng.choice([0.0, 0.5, 1.0]) for _ in range(n)] if trial % 3 == 0 else None
        plan, total = ee.ee_plan_dynamic(lens, cap, _native_cost(c), max_tokens, wait)
        ref, ref_total = oracle.dynamic_batches(lens, cap, c, max_tokens, wait)
        assert ee.batches_of(plan) == ref
        assert total == ref_total


def test_stream_workload_plans():
    w = workloads.get("gpt3-48l-stream")
    lens = [n for g in workloads.request_stream(w, 1234) for n in g]
    assert len(lens) == 1024
    for c in COSTS[:2]:
        plan, total = ee.ee_plan_dynamic(lens, w.batch, _native_cost(c))
        ref, ref_total = oracle.dynamic_batches(lens, w.batch, c)
        assert ee.batches_of(plan) == ref and total == ref_total
    fifo = ee.batches_of(ee.ee_plan_fifo(lens, w.batch))
    assert fifo == oracle.fifo_batches(lens, w.batch)
    assert [[lens[i] for i in b] for b in fifo] == workloads.request_stream(w, 1234)
    # padding kept: sorting by length removes most of FIFO's padded rows
    dyn = ee.batches_of(ee.ee_plan_dynamic(lens, w.batch, _native_cost(COSTS[1]))[0])
    assert oracle.padded_rows(dyn, lens) < 0.6 * oracle.padded_rows(fifo, lens)


def test_cost_eval_matches_oracle():
    rng = random.Random(5)
    for c in COSTS:
        for _ in range(20):
            lens = [rng.randint(1, 256) for _ in range(rng.randint(1, 64))]
            assert ee.ee_batch_cost_eval(lens, _native_cost(c)) == oracle.batch_cost(lens, c)


def test_planner_errors():
    c = _native_cost(COSTS[2])
    with pytest.raises(ee.EEError):
        ee.ee_plan_dynamic([3, 0, 2], 4, c)                   # a length < 1
    with pytest.raises(ee.EEError):
        ee.ee_plan_dynamic([3, 2], 0, c)                      # max_batch < 1
    with pytest.raises(ee.EEError):
        ee.ee_plan_dynamic([300, 2], 4, c, max_tokens=256)    # longer than the token limit
    with pytest.raises(ee.EEError):
        ee.ee_plan_dynamic([3, 2], 4, ee.BatchCost(-1.0, 0, 0, 0, 1, 0))
    with pytest.raises(ee.EEError):
        ee.ee_plan_dynamic([3, 2], 4, ee.BatchCost(0, 0, 0, 0, 1, 0).set_table([0.1, -0.2]))
    assert ee.ee_plan_dynamic([], 4, c) == ([], 0.0)
    assert ee.ee_plan_fifo([], 4) == []
