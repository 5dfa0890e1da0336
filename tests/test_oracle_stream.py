"""Pins for the layer-stream schedule simulator: the read counts the pages print,
a hand-worked log, and the happens-before invariant for every ring size."""
import json
import os

import pytest

from oracle import stream_sim as ss

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")


def test_read_counts_match_pages():
    g = json.load(open(GOLDEN))
    for L in (1, 3, 24, 32):
        sft = ss.copies(ss.simulate(ss.sft_schedule(L), 2))
        dpo = ss.copies(ss.simulate(ss.dpo_schedule(L), 2))
        assert len(sft) == g["sft_reads_per_layer"]["value"] * L
        assert len(dpo) == 3 * L
        # the pages' 1.52x also counts reads outside the layer stack; the stack alone is 1.5x
        assert abs(len(dpo) / len(sft) - g["dpo_over_sft_stack_reads"]["value"]) <= 0.021


def test_hand_worked_log_l3_nbuf2():
    # schedule [0, 1, 2, 2, 1, 0]; two buffers; copies run one call ahead
    log = ss.simulate(ss.sft_schedule(3), 2)
    C, S = ss.COPY, ss.STEP
    assert log == [
        (C, 0, 0, 0, 0, -1), (C, 0, 1, 1, 1, -1), (S, 0, 0, 0, 0, 0),
        (C, 1, 2, 2, 0, 0), (S, 1, 1, 1, 1, 1),
        (C, 2, 3, 2, 1, 1), (S, 2, 2, 2, 0, 2),
        (C, 3, 4, 1, 0, 2), (S, 3, 3, 2, 1, 3),
        (C, 4, 5, 0, 1, 3), (S, 4, 4, 1, 0, 4),
        (S, 5, 5, 0, 1, 5),
    ]


@pytest.mark.parametrize("nbuf", range(2, 9))
@pytest.mark.parametrize("L", [1, 2, 5, 32])
def test_happens_before(nbuf, L):
    for sched in (ss.sft_schedule(L), ss.dpo_schedule(L)):
        log = ss.simulate(sched, nbuf)
        ss.check_happens_before(log, sched, nbuf)
        # the copy stream never runs more than nbuf - 1 layers ahead of compute
        for kind, call, j, *_ in log:
            if kind == ss.COPY:
                assert j <= call + nbuf - 1


def test_happens_before_catches_a_missing_wait():
    log = ss.simulate(ss.sft_schedule(4), 2)
    bad = [e if not (e[0] == ss.COPY and e[2] == 3) else (e[0], e[1], e[2], e[3], e[4], -1) for e in log]
    with pytest.raises(AssertionError):
        ss.check_happens_before(bad, ss.sft_schedule(4), 2)


def test_resident_copies_each_shard_once():
    sched = ss.sft_schedule(6)
    log = ss.simulate(sched, 6, n_shards=6, resident=True)
    cps = ss.copies(log)
    assert sorted(e[3] for e in cps) == list(range(6))
    steps = [e for e in log if e[0] == ss.STEP]
    assert [e[3] for e in steps] == sched and all(e[4] == e[3] for e in steps)


# ------------------------------------------------------------------ reuse variant
def test_reuse_hand_worked_logs_l3_nbuf2():
    # schedule [0, 1, 2, 2, 1, 0], two buffers, two passes.  Pass 0: shards 2 and 1 are
    # still in their buffers at the turn; shard 0 then goes into the least recently used
    # buffer (b0, last used at call 3), issued at call 4.  Pass 1 starts with shards 0
    # and 1 in place.
    C, S = ss.COPY, ss.STEP
    p0, p1 = ss.simulate_reuse(ss.sft_schedule(3), 2, passes=2)
    assert p0 == [
        (C, 0, 0, 0, 0, -1), (C, 0, 1, 1, 1, -1), (S, 0, 0, 0, 0, 0),
        (C, 1, 2, 2, 0, 0), (S, 1, 1, 1, 1, 1),
        (S, 2, 2, 2, 0, 2),
        (S, 3, 2, 2, 0, 2),
        (C, 4, 5, 0, 0, 3), (S, 4, 1, 1, 1, 1),
        (S, 5, 5, 0, 0, 5),
    ]
    assert p1 == [
        (S, 0, -1, 0, 0, -1),
        (C, 1, 2, 2, 0, 0), (S, 1, -1, 1, 1, -1),
        (S, 2, 2, 2, 0, 2),
        (S, 3, 2, 2, 0, 2),
        (C, 4, 5, 0, 0, 3), (S, 4, -1, 1, 1, -1),
        (S, 5, 5, 0, 0, 5),
    ]


@pytest.mark.parametrize("nbuf", [2, 3, 8])
@pytest.mark.parametrize("L", [1, 2, 5, 32])
def test_reuse_copy_counts(nbuf, L):
    """Closed forms: with L > nbuf an SFT pass copies 2L - nbuf layers first (the last
    nbuf forward layers serve the first backward calls), then 2L - 2 nbuf (the first
    nbuf layers are still in place from the previous backward); DPO adds L to each (its
    policy forward restarts at layer 0, long evicted).  With L <= nbuf every shard stays
    resident after the first pass."""
    for sched, extra in ((ss.sft_schedule(L), 0), (ss.dpo_schedule(L), L)):
        counts = [len(ss.copies(log)) for log in ss.simulate_reuse(sched, nbuf, passes=3)]
        if L > nbuf:
            assert counts == [2 * L - nbuf + extra, 2 * L - 2 * nbuf + extra, 2 * L - 2 * nbuf + extra]
        else:
            assert counts == [L, 0, 0]


@pytest.mark.parametrize("nbuf", range(2, 9))
@pytest.mark.parametrize("L", [1, 2, 5, 32])
def test_reuse_happens_before(nbuf, L):
    for sched in (ss.sft_schedule(L), ss.dpo_schedule(L)):
        ss.check_reuse_log(ss.simulate_reuse(sched, nbuf, passes=3), sched, nbuf)


def test_reuse_check_catches_a_missing_wait_and_a_wrong_buffer():
    sched = ss.sft_schedule(5)
    logs = ss.simulate_reuse(sched, 2, passes=2)
    first_copy_with_wait = next(i for i, e in enumerate(logs[0]) if e[0] == ss.COPY and e[5] >= 0)
    bad = list(logs[0])
    e = bad[first_copy_with_wait]
    bad[first_copy_with_wait] = (e[0], e[1], e[2], e[3], e[4], -1)
    with pytest.raises(AssertionError):
        ss.check_reuse_log([bad], sched, 2)
    step = next(i for i, e in enumerate(logs[1]) if e[0] == ss.STEP and e[2] == -1)
    bad = list(logs[1])
    e = bad[step]
    bad[step] = (e[0], e[1], e[2], e[3], 1 - e[4], e[5])
    with pytest.raises(AssertionError):
        ss.check_reuse_log([logs[0], bad], sched, 2)


# ------------------------------------------------------------------ head slot of a stack step
@pytest.mark.parametrize("L,nbuf", [(3, 2), (5, 3), (4, 8)])
@pytest.mark.parametrize("dpo", [False, True])
@pytest.mark.parametrize("efh", [False, True])
def test_stack_step_log_ring_part_is_the_ring_simulator(L, nbuf, dpo, efh):
    lg = ss.stack_step_log(L, nbuf, dpo, efh)
    sched = ss.dpo_schedule(L) if dpo else ss.sft_schedule(L)
    assert [e for e in lg if e[0] in (ss.COPY, ss.STEP)] == ss.simulate(sched, nbuf)
    calls = [e[1] for e in lg]
    assert calls == sorted(calls)   # events come in call order


@pytest.mark.parametrize("L", [2, 3, 6])
@pytest.mark.parametrize("dpo", [False, True])
def test_slot_holds_embedding_at_start_and_lm_head_at_each_turn(L, dpo):
    """Embed_tokens and the untied lm_head share one slot (the deep dive, "How layer
    streaming works"): replayed over three steps, the slot holds the embedding at each
    step's start and lm_head at each forward/backward turn (twice for DPO: reference and
    policy heads)."""
    n = 0
    start = None
    for step in range(3):
        lg = ss.stack_step_log(L, 2, dpo, first=(step == 0), loads_before=n)
        ss.check_slot_log(lg, L, dpo, start=start)
        n += 3 if step == 0 else 2      # (first: the whole embedding,) lm_head, the next embedding
        start = L


@pytest.mark.parametrize("dpo", [False, True])
def test_slot_reads_per_step(dpo):
    """Per step the shared slot reads one embedding and one lm_head (the embedding of the
    first step whole, later ones in L parts of the backward); reading the embedding rows
    from the host table leaves only one lm_head load, in the first step."""
    L = 4
    for first in (True, False):
        lg = ss.stack_step_log(L, 2, dpo, first=first)
        loads = [e for e in lg if e[0] == ss.SLOT_COPY]
        emb_parts = [e for e in loads if e[3] == L]
        lm = [e for e in loads if e[3] == L + 1]
        assert len(lm) == 1 and lm[0][4] == -1
        # the embedding: whole before the first step, and L parts (one per backward call)
        # for the next step
        assert [e[4] for e in emb_parts] == ([-1] if first else []) + [-1 - p for p in range(L)]
        assert [e[1] for e in emb_parts[-L:]] == [k + 1 for k in range((2 * L if dpo else L), (3 if dpo else 2) * L)]
        efh = ss.stack_step_log(L, 2, dpo, embed_from_host=True, first=first)
        assert [e[3] for e in efh if e[0] == ss.SLOT_COPY] == ([L + 1] if first else [])
        assert sum(1 for e in efh if e[0] == ss.SLOT_WAIT) == (2 if dpo else 1)


def test_slot_check_catches_a_late_lm_head_and_an_early_embedding_part():
    L = 3
    good = ss.stack_step_log(L, 2, first=False, loads_before=2)
    ss.check_slot_log(good, L, start=L)
    # lm_head loaded after the turn's wait: the head would read the embedding
    i = next(i for i, e in enumerate(good) if e[0] == ss.SLOT_COPY and e[3] == L + 1)
    w = next(i for i, e in enumerate(good) if e[0] == ss.SLOT_WAIT and e[1] > 0)
    late = good[:i] + good[i + 1:w] + [good[w], good[i]] + good[w + 1:]
    with pytest.raises(AssertionError):
        ss.check_slot_log(late, L, start=L)
    # part 0 of the next embedding moved before the turn's wait
    p0 = next(i for i, e in enumerate(good) if e[0] == ss.SLOT_COPY and e[3] == L and e[4] == -1)
    early = good[:w] + [good[p0]] + good[w:p0] + good[p0 + 1:]
    with pytest.raises(AssertionError):
        ss.check_slot_log(early, L, start=L)


@pytest.mark.parametrize("L", [2, 3, 5, 8])
@pytest.mark.parametrize("dpo", [False, True])
@pytest.mark.parametrize("lead", [1, 2, 3])
def test_early_lm_head_and_lead_parts_keep_the_slot_valid(L, dpo, lead):
    """lm_head loaded one forward call before the last and several embedding parts issued at
    the first backward call: over three steps the slot still holds the embedding at each
    step's start and lm_head at each turn, every part is issued once and in order, and the
    layer ring's events are unchanged."""
    lead = min(lead, L)
    n, start = 0, None
    sched = ss.dpo_schedule(L) if dpo else ss.sft_schedule(L)
    for step in range(3):
        lg = ss.stack_step_log(L, 2, dpo, first=(step == 0), loads_before=n, lm_head_call=max(L - 2, 0),
                               lead_parts=lead)
        ss.check_slot_log(lg, L, dpo, start=start)
        assert [e for e in lg if e[0] in (ss.COPY, ss.STEP)] == ss.simulate(sched, 2)
        parts = [e for e in lg if e[0] == ss.SLOT_COPY and e[3] == L and e[4] <= -1 and not (step == 0 and e[1] == 0)]
        assert [-1 - e[4] for e in parts] == list(range(L))
        n_fwd = 2 * L if dpo else L
        assert [e[1] for e in parts[:lead]] == [n_fwd + 1] * lead
        assert [e[1] for e in parts[lead:]] == [n_fwd + 1 + i for i in range(1, L - lead + 1)]
        lm = [e for e in lg if e[0] == ss.SLOT_COPY and e[3] == L + 1]
        assert len(lm) == 1 and lm[0][1] == max(L - 2, 0) + 1
        n += 3 if step == 0 else 2
        start = L


def test_slot_check_catches_lm_head_before_the_embedding_is_used():
    """A negative control for the early lm_head: loaded before the first call's wait, it
    would overwrite the embedding the step starts from."""
    L = 4
    lg = ss.stack_step_log(L, 2, first=False, loads_before=2, lm_head_call=L - 2)
    i = next(i for i, e in enumerate(lg) if e[0] == ss.SLOT_COPY and e[3] == L + 1)
    w0 = next(i for i, e in enumerate(lg) if e[0] == ss.SLOT_WAIT and e[1] == 0)
    bad = [lg[i]] + lg[:i] + lg[i + 1:]
    assert bad.index(lg[i]) < w0 + 1
    with pytest.raises(AssertionError):
        ss.check_slot_log(bad, L, start=L)
