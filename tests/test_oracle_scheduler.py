"""Pins for the reference continuous-batching scheduler (CPU only).

The scheduler oracle is checked against step-by-step traces worked out by
hand (tests/golden/scheduler_traces.json) and, on random traces, against
invariants the policy fixes whatever the details: the step budget and the
running cap hold, chunks are bounded, every request ends with exactly its
prompt plus output tokens cached, slots are distinct and agree with the
block tables, a finished request's blocks are free at once, and the
reservation model never preempts.
"""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from conftest import GOLDEN
from oracle.scheduler import RefScheduler


def _traces():
    with open(os.path.join(GOLDEN, "scheduler_traces.json")) as f:
        return json.load(f)["traces"]


def _build(cfg, requests):
    s = RefScheduler(cfg["num_blocks"], cfg["block_size"], cfg["max_num_seqs"],
                     cfg["max_num_batched_tokens"], cfg["chunk_size"], cfg["reserve_tokens"],
                     host_blocks=cfg["host_blocks"])
    for name, p, o in requests:
        s.add_request(name, p, o)
    return s


@pytest.mark.parametrize("trace", _traces(), ids=lambda t: t["name"])
def test_hand_worked_traces(trace):
    s = _build(trace["config"], trace["requests"])
    for k, want in enumerate(trace["steps"]):
        got = s.step()
        rows = [[r[0], r[1], r[2], r[3]] for r in got["rows"]]
        assert rows == want["rows"], (k, want["why"])
        assert got["num_decode"] == want["num_decode"], k
        assert got["slots"] == want["slots"], (k, want["why"])
        assert got["finished"] == want["finished"], k
        assert got["preempted"] == want["preempted"], k
        if "swap_in" in want:
            assert [list(p) for p in got["swap_in"]] == want["swap_in"], (k, want["why"])
            assert [list(p) for p in got["swap_out"]] == want["swap_out"], (k, want["why"])
        # the counters behind the reported slot utilisation (cached tokens
        # over allocated or reserved slots), worked by hand per step
        assert s.stats() == want["stats"], (k, want["why"])
    assert s.stats()["finished"] == len(trace["requests"])
    assert s.alloc.num_free() == trace["config"]["num_blocks"]


def run_to_end(s, requests, max_steps=100000):
    """Drive a scheduler until every request finished; check the invariants
    of every step; return the list of step results."""
    cfg_bs = s.block_size
    total = {rid: p + o for rid, p, o in requests}
    tokens = {rid: 0 for rid, _, _ in requests}
    out = []
    for _ in range(max_steps):
        st_ = s.step()
        out.append(st_)
        rows = st_["rows"]
        assert sum(r[1] for r in rows) == len(st_["slots"]) <= s.budget
        assert len(rows) <= s.max_num_seqs
        assert len(s.running) <= s.max_num_seqs
        assert len(set(r[0] for r in rows)) == len(rows)            # one row per request
        assert all(r[1] == 1 for r in rows[:st_["num_decode"]])
        assert all(1 <= r[1] <= s.chunk for r in rows[st_["num_decode"]:])
        assert len(set(st_["slots"])) == len(st_["slots"])          # distinct slots
        for rid in st_["preempted"]:
            if rid not in s.alloc.swapped:
                tokens[rid] = 0                                     # recomputed later
        k = 0
        for rid, q, ctx, table in rows:
            new = st_["slots"][k:k + q]
            k += q
            for i, slot in enumerate(new):                          # slot formula
                pos = ctx - q + i
                assert slot == table[pos // cfg_bs] * cfg_bs + pos % cfg_bs
            assert len(table) == -(-ctx // cfg_bs)
            tokens[rid] = ctx
        for rid in st_["finished"]:
            assert tokens[rid] == total[rid]                        # all its tokens
            assert rid not in s.alloc.tables                        # freed at once
        held = sum(len(t) for q, t in s.alloc.tables.items() if q not in s.alloc.swapped)
        assert held + s.alloc.num_free() == s.num_blocks
        in_host = sum(len(s.alloc.tables[q]) for q in s.alloc.swapped)
        assert in_host + s.alloc.num_free_host() == s.alloc.num_host_blocks
        if not s.running and not s.waiting:
            return out
    raise AssertionError("trace did not drain")


traces = st.lists(st.tuples(st.integers(1, 40), st.integers(1, 30)), min_size=1, max_size=12)


@settings(max_examples=80, deadline=None)
@given(reqs=traces, bs=st.sampled_from([1, 2, 4, 8]), seqs=st.integers(1, 5),
       budget=st.integers(1, 24), chunk=st.integers(1, 16), spare=st.integers(0, 12),
       host=st.sampled_from([0, 0, 4, 16, 64]), data=st.data())
def test_random_traces_keep_the_invariants(reqs, bs, seqs, budget, chunk, spare, host, data):
    need = max(-(-(p + o) // bs) for p, o in reqs)
    nb = need + spare
    order = data.draw(st.permutations(list(range(nb))))
    s = RefScheduler(nb, bs, seqs, budget, chunk, 0, order, host_blocks=host)
    requests = [(i, p, o) for i, (p, o) in enumerate(reqs)]
    for rid, p, o in requests:
        s.add_request(rid, p, o)
    run_to_end(s, requests)
    assert s.total_finished == len(requests)


@settings(max_examples=30, deadline=None)
@given(reqs=traces, bs=st.sampled_from([2, 4]), seqs=st.integers(1, 6),
       budget=st.integers(4, 24), chunk=st.integers(1, 16), extra=st.integers(0, 40))
def test_reservation_model_never_preempts(reqs, bs, seqs, budget, chunk, extra):
    reserve = max(p + o for p, o in reqs)
    nb = -(-reserve // bs) * 2 + extra
    s = RefScheduler(nb, bs, seqs, budget, chunk, reserve)
    requests = [(i, p, o) for i, (p, o) in enumerate(reqs)]
    for rid, p, o in requests:
        s.add_request(rid, p, o)
    steps = run_to_end(s, requests)
    assert s.total_preempted == 0
    per = -(-reserve // bs)
    # the reservation caps the running set at num_blocks // blocks per reservation
    assert max(len(x["rows"]) for x in steps) <= min(seqs, nb // per)


def test_finished_blocks_serve_the_next_request_in_the_same_step():
    # one block pool of 2 slots: B can only start when A's block is back
    s = RefScheduler(1, 2, 2, 4, 2)
    s.add_request("A", 1, 1)
    s.add_request("B", 1, 1)
    a = s.step()
    assert [r[0] for r in a["rows"]] == ["A"]
    b = s.step()
    assert [r[0] for r in b["rows"]] == ["A"] and b["num_decode"] == 1
    c = s.step()
    assert c["finished"] == ["A"] and [r[0] for r in c["rows"]] == ["B"]


def test_rejects_requests_that_never_fit():
    s = RefScheduler(4, 4, 2, 8, 4, reserve_tokens=10)
    with pytest.raises(ValueError):
        s.add_request(0, 8, 3)          # 11 tokens > reservation of 10
    t = RefScheduler(2, 4, 2, 8, 4)
    with pytest.raises(ValueError):
        t.add_request(0, 6, 3)          # 3 blocks > pool of 2
    with pytest.raises(ValueError):
        t.add_request(1, 0, 3)
