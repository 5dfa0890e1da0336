"""Layer-stream schedule and the event log a correct engine must produce.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What the pages fix (the Soup deep dive, "How layer streaming works", and the
4 GB-laptop article, "Layer streaming: technical implementation"):
* the frozen base is cut into per-layer shards kept in (page-locked) host RAM;
* a few preallocated device layer buffers -- 2 by default, 2 to 8 through
  ``stream_buffers`` ("Streaming config keys") -- are filled by a separate
  stream with the next layer while the current one computes;
* every decoder layer is read twice per SFT step: once for the forward and once
  for the checkpoint recompute in backward;
* DPO reads the layer stack more often per step than SFT (1.52x on the 4 GB
  article, "Computational trade-off"): its reference pass is the same streamed
  base with the adapters off.

Readings (the pages give no schedule rule): call k of a step uses buffer
k mod nbuf; at call k the copy stream is kept nbuf-1 layers ahead, i.e. every
copy j <= k + nbuf - 1 not yet issued is issued; copy j goes to buffer
j mod nbuf and must wait until the compute of call j - nbuf (the buffer's
previous user) has finished; call k's compute waits for copy k.  In resident
mode every shard has its own buffer, all shards are copied once on the first
call, and call k waits for the copy of its own shard.

Reuse variant (a reading beyond the pages' ring, which copies every read): each
pass is planned from what the buffers hold.  A position whose shard sits intact in
some buffer uses it without a copy; otherwise its shard goes into the least
recently used buffer (lowest index on ties), after the release of that buffer's
last user u in the pass, issued at call max(j - nbuf + 1, u + 1).  For a STEP of
this variant, ``j`` is the position whose copy filled the buffer (-1: a previous
pass).

The event log is a list of tuples (kind, call, j, layer, buffer, wait):
  COPY  issued during call ``call``: schedule position j, shard ``layer``,
        into ``buffer``, after the release of call ``wait`` (-1: no wait)
  STEP  call ``call`` computes shard ``layer`` from ``buffer`` once copy ``j``
        is done (``wait`` == j)
"""
from __future__ import annotations

COPY = 0
STEP = 1


def sft_schedule(n_layers: int) -> list[int]:
    """Forward 0..L-1, then backward (recompute + gradient) L-1..0: two reads per layer."""
    return list(range(n_layers)) + list(range(n_layers - 1, -1, -1))


def dpo_schedule(n_layers: int) -> list[int]:
    """Adapter-off reference forward, then the SFT schedule: three reads per layer."""
    return list(range(n_layers)) + sft_schedule(n_layers)


def simulate(schedule, n_bufs: int, n_shards: int | None = None, resident: bool = False):
    """Return the event log of one pass over ``schedule`` (see the module header)."""
    sched = list(schedule)
    n = len(sched)
    log = []
    if resident:
        shards = n_shards if n_shards is not None else (max(sched) + 1 if sched else 0)
        for k in range(n):
            if k == 0:
                for s in range(shards):
                    log.append((COPY, 0, s, s, s, -1))
            s = sched[k]
            log.append((STEP, k, s, s, s, s))
        return log
    issued = 0
    for k in range(n):
        while issued < n and issued <= k + n_bufs - 1:
            j = issued
            log.append((COPY, k, j, sched[j], j % n_bufs, j - n_bufs if j >= n_bufs else -1))
            issued += 1
        log.append((STEP, k, k, sched[k], k % n_bufs, k))
    return log


def copies(log) -> list[tuple]:
    return [e for e in log if e[0] == COPY]


def check_happens_before(log, schedule, n_bufs: int) -> None:
    """Replay the ring and assert that no buffer is overwritten while a call may still use it.

    A copy into buffer b for position j may start only after the compute of call
    j - nbuf (the previous user of b) has been released, and that release must
    come from a call that has already been made when the copy is issued.  Every
    step must find its own shard in its buffer.
    """
    content = {}
    made = -1
    for kind, call, j, layer, buf, wait in log:
        if kind == COPY:
            prev_user = j - n_bufs
            if prev_user >= 0:
                assert wait == prev_user, (j, wait)
                assert prev_user < call, "release not yet recorded when the copy is issued"
            else:
                assert wait == -1
            content[buf] = (j, layer)
        else:
            assert call == made + 1, "calls out of order"
            made = call
            assert content.get(buf) == (j, layer), (call, buf, content.get(buf))
            assert layer == schedule[call]


def simulate_reuse(schedule, n_bufs: int, passes: int = 1):
    """Event logs of ``passes`` consecutive passes of the reuse variant (module header)."""
    sched = list(schedule)
    n = len(sched)
    holder = [None] * n_bufs          # shard in each buffer
    last_seen = [-1] * n_bufs         # when each buffer was last used (a clock over passes)
    clock = 0
    logs = []
    for _ in range(passes):
        # plan: buffer per position, and for copies the last user in this pass and the call
        plan = []
        last_user = [-1] * n_bufs
        filled_by = [-1] * n_bufs
        for j, shard in enumerate(sched):
            held = [b for b in range(n_bufs) if holder[b] == shard]
            if held:
                b = held[-1]
                plan.append((b, None))
            else:
                b = min(range(n_bufs), key=lambda q: (last_seen[q], q))
                issue_at = max(j - n_bufs + 1, last_user[b] + 1, 0)
                plan.append((b, (last_user[b], issue_at)))
                holder[b] = shard
                filled_by[b] = j
            last_user[b] = j
            last_seen[b] = clock + j
            plan[-1] = plan[-1] + (filled_by[b],)
        # events, in the order the calls produce them
        log = []
        nxt = 0
        for k in range(n):
            while nxt < n and (plan[nxt][1] is None or plan[nxt][1][1] <= k):
                b, cp, _ = plan[nxt]
                if cp is not None:
                    log.append((COPY, k, nxt, sched[nxt], b, cp[0]))
                nxt += 1
            b, _, src = plan[k]
            log.append((STEP, k, src, sched[k], b, src))
        logs.append(log)
        clock += n
    return logs


def check_reuse_log(logs, schedule, n_bufs: int) -> None:
    """Replay passes of the reuse variant: every step finds its shard in its buffer, and
    a copy overwrites a buffer only after the release of its last user, a call already
    made when the copy is issued (or a call of an earlier pass)."""
    content = {}
    for log in logs:
        last_user = {}
        made = -1
        for kind, call, j, layer, buf, wait in log:
            if kind == COPY:
                assert wait == last_user.get(buf, -1), (j, buf, wait, last_user.get(buf))
                assert wait < call or wait == -1, "release not yet recorded when the copy is issued"
                assert j <= call + n_bufs - 1, "copy issued more than nbuf - 1 calls ahead"
                content[buf] = layer
            else:
                assert call == made + 1, "calls out of order"
                made = call
                assert layer == schedule[call]
                assert content.get(buf) == layer, (call, buf, content.get(buf), layer)
                last_user[buf] = call


# ------------------------------------------------------------------ the head slot of a stack step
SLOT_COPY = 2
SLOT_WAIT = 3


def stack_step_log(n_layers: int, n_bufs: int, dpo: bool = False, embed_from_host: bool = False,
                   first: bool = True, loads_before: int = 0, lm_head_call: int | None = None,
                   lead_parts: int = 1):
    """Event log of one step of the streamed stack with its head slot (layer ring as in
    ``simulate``).  The slot holds embed_tokens at the start of the step and the untied
    lm_head at the forward/backward turn (the Soup deep dive, "How layer streaming works":
    embed_tokens and lm_head share one device slot).  Slot schedule of the stack (a reading:
    the pages only say that they share it):

    * the embedding is loaded whole before the first step; in every backward call one of L
      parts of the next step's embedding follows that call's layer copies (part 0 waits
      for the head, the slot's last user);
    * lm_head is loaded after forward call ``lm_head_call`` of the (first) forward pass (by
      default the last one, L - 1) and waited for right after the stream step of the first
      call past each forward pass (DPO: the reference pass and the policy pass), where the
      head runs;
    * the first backward call issues ``lead_parts`` parts of the next embedding (part 0
      first, waiting for the head), every later backward call one more, until all L are
      issued;
    * ``embed_from_host``: the embedding rows are read from the host table, so the slot
      only ever holds lm_head, loaded once at the start of the first step.

    A SLOT_COPY event is (SLOT_COPY, call, load index, shard, -1 whole or -1 - part,
    previous load index for a whole load or part 0, else -1); a SLOT_WAIT event is
    (SLOT_WAIT, call, last complete load, -1, -1, last complete load).  The shard ids of
    the slot are ``n_layers`` (embed_tokens) and ``n_layers + 1`` (lm_head); ``loads_before``
    counts the slot loads completed in earlier steps."""
    L = n_layers
    E, LM = L, L + 1
    sched = dpo_schedule(L) if dpo else sft_schedule(L)
    ring = simulate(sched, n_bufs)
    n_fwd = 2 * L if dpo else L
    lm_at = L - 1 if lm_head_call is None else lm_head_call
    assert 0 <= lm_at < L and 1 <= lead_parts <= L
    n = loads_before
    log = []

    def whole(call, shard):
        nonlocal n
        log.append((SLOT_COPY, call, n, shard, -1, n - 1))
        n += 1

    def wait(call):
        log.append((SLOT_WAIT, call, n - 1, -1, -1, n - 1))

    if embed_from_host:
        if first:
            whole(0, LM)
    else:
        if first:
            whole(0, E)
        wait(0)
    for k in range(len(sched)):
        log.extend(e for e in ring if e[1] == k)
        if k == L or k == n_fwd:
            wait(k + 1)
        if k < n_fwd:
            if k == lm_at and not embed_from_host:
                whole(k + 1, LM)
        elif not embed_from_host:
            i = k - n_fwd
            first_p = 0 if i == 0 else lead_parts + i - 1
            last_p = lead_parts - 1 if i == 0 else first_p
            for p in range(first_p, min(last_p, L - 1) + 1):
                log.append((SLOT_COPY, k + 1, n, E, -1 - p, n - 1 if p == 0 else -1))
                if p == L - 1:
                    n += 1
    return log


def check_slot_log(log, n_layers: int, dpo: bool = False, start=None) -> None:
    """Replay the slot events of one stack step: at the wait before call 0 the slot holds
    embed_tokens, at each wait of the turn it holds lm_head, and no load into the slot is
    issued between the lm_head load and the last wait for it (the head's use).  A load is
    logged as consecutive parts 0, 1, ... of one shard (buffer -1 - part; a whole load is
    its own part 0), and a wait can only follow a complete load, so at a wait the slot
    holds the shard of the last load.  ``start``: what the slot holds when the step begins
    (None before the first step)."""
    L = n_layers
    E, LM = L, L + 1
    content, loading, lm_waits_left = start, None, (2 if dpo else 1)
    for kind, call, j, shard, buf, wait in log:
        if kind == SLOT_COPY:
            part = -1 - buf
            if part == 0:
                assert content != LM or lm_waits_left == 0 or call == 0, \
                    "slot overwritten while the head still needs lm_head"
                content, loading = None, (shard, 0)
            else:
                assert loading == (shard, part - 1), "parts out of order"
                loading = (shard, part)
        elif kind == SLOT_WAIT:
            if loading is not None:
                content, loading = loading[0], None
            if call == 0:
                assert content == E, "embedding not in the slot at the start of the step"
            else:
                assert content == LM, "lm_head not in the slot at the turn"
                lm_waits_left -= 1
    assert lm_waits_left == 0
