"""GPU checks of the layer stream and of a streamed stack step.

* the engine's event log equals the oracle's schedule simulator (ring sizes 2..8, SFT and
  DPO schedules, resident mode) and every step's buffer holds its layer's shard bytes;
* a streamed pass gives bitwise the same outputs and gradients as a resident pass
  (the pages hold the streamed-vs-resident logit difference at 0.0);
* a small streamed stack step matches the oracle layer step for every layer, and its
  output side (embedding rows, token log-probs, the lm_head input gradient, the DPO loss
  and coefficients) matches the oracle's head on the same shards, ids and labels;
* the loss computed a chunk of tokens at a time equals the loss computed in one piece.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import synthgen  # noqa: E402
from lora_fine_tuning_nf4_amd import lnf4  # noqa: E402
from lora_fine_tuning_nf4_amd.stack import StreamedStack  # noqa: E402
from oracle import head as ohead  # noqa: E402
from oracle import layer as olayer  # noqa: E402
from oracle import lora as olora  # noqa: E402
from oracle import nf4 as onf4  # noqa: E402
from oracle import stream_sim as ss  # noqa: E402
from helpers import bf16_f64, check_tol  # noqa: E402


def _pinned_shards(n, nbytes, seed=0):
    rs = np.random.default_rng(seed)
    out = []
    for i in range(n):
        h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        h.copy_(torch.from_numpy(rs.integers(0, 256, nbytes, dtype=np.uint8)))
        out.append(h)
    return out


@pytest.mark.parametrize("nbuf", [2, 3, 8])
@pytest.mark.parametrize("mode", ["sft", "dpo"])
def test_stream_log_and_buffers_match_simulator(nbuf, mode):
    L, nbytes = 5, 4096 + 512
    shards = _pinned_shards(L, nbytes, seed=nbuf)
    bufs = [torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    sched = ss.sft_schedule(L) if mode == "sft" else ss.dpo_schedule(L)
    copy = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    st = lnf4.stream_create(shards, [nbytes] * L, bufs, nbytes + 256, sched, 0, copy)
    try:
        for step in range(2):  # two passes: the second starts behind the first pass's releases
            for k in range(len(sched)):
                p = lnf4.stream_layer_step(st, k, comp)
                j = [i for i, b in enumerate(bufs) if b.data_ptr() == p]
                assert j == [k % nbuf]
                got = bufs[j[0]][:nbytes].cpu()   # reads on the compute stream, after the wait
                assert torch.equal(got, shards[sched[k]]), (step, k)
            assert lnf4.stream_log(st) == ss.simulate(sched, nbuf)
            lnf4.stream_reset(st, comp)
        with pytest.raises(lnf4.LNF4Error):
            lnf4.stream_layer_step(st, 1, comp)   # out of order
    finally:
        torch.cuda.synchronize()
        lnf4.stream_destroy(st)


@pytest.mark.parametrize("nbuf", [2, 3, 8])
@pytest.mark.parametrize("mode", ["sft", "dpo"])
def test_reuse_log_and_buffers_match_simulator(nbuf, mode):
    """Reuse mode over three passes: the engine's log equals the oracle simulator's, and
    every call finds its shard's bytes in the buffer it is given."""
    L, nbytes = 5, 4096 + 512
    shards = _pinned_shards(L, nbytes, seed=20 + nbuf)
    bufs = [torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    sched = ss.sft_schedule(L) if mode == "sft" else ss.dpo_schedule(L)
    comp = torch.cuda.current_stream()
    st = lnf4.stream_create(shards, [nbytes] * L, bufs, nbytes + 256, sched, lnf4.STREAM_REUSE, torch.cuda.Stream())
    want = ss.simulate_reuse(sched, nbuf, passes=3)
    try:
        b0 = lnf4.stream_bytes_copied(st)
        for step in range(3):
            for k in range(len(sched)):
                p = lnf4.stream_layer_step(st, k, comp)
                j = [i for i, b in enumerate(bufs) if b.data_ptr() == p]
                assert len(j) == 1
                assert torch.equal(bufs[j[0]][:nbytes].cpu(), shards[sched[k]]), (step, k)
            assert lnf4.stream_log(st) == want[step], step
            lnf4.stream_reset(st, comp)
        n_copies = sum(len(ss.copies(lg)) for lg in want)
        assert lnf4.stream_bytes_copied(st) - b0 == n_copies * nbytes
    finally:
        torch.cuda.synchronize()
        lnf4.stream_destroy(st)


@pytest.mark.parametrize("nbuf,n_stage,drop", [(2, 1, False), (2, 2, True), (3, 8, False), (8, 3, True)])
def test_disk_tier_log_and_buffers_match_simulator(nbuf, n_stage, drop, tmp_path):
    """Layer shards read from a file through n_stage pinned staging buffers: over three
    passes the engine's log equals the ring's simulator log (the disk tier only delays
    copies), every call finds its shard's bytes, and the reader has read every position."""
    import os
    L, nbytes = 5, 4096 + 512
    shards = _pinned_shards(L, nbytes, seed=40 + nbuf)
    stride = 8192
    path = tmp_path / "shards.bin"
    with open(path, "wb") as f:
        for h in shards:
            f.write(h.numpy().tobytes() + bytes(stride - nbytes))
    stage = [torch.empty(stride + 4096, dtype=torch.uint8, pin_memory=True) for _ in range(n_stage)]
    addrs = [(t.data_ptr() + 4095) // 4096 * 4096 for t in stage]
    bufs = [torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    sched = ss.sft_schedule(L)
    comp = torch.cuda.current_stream()
    st = lnf4.stream_create_disk(str(path), [i * stride for i in range(L)], addrs, stride, [nbytes] * L, bufs,
                                 nbytes + 256, sched, torch.cuda.Stream(), drop_cache=drop)
    try:
        for step in range(3):
            for k in range(len(sched)):
                p = lnf4.stream_layer_step(st, k, comp)
                j = [i for i, b in enumerate(bufs) if b.data_ptr() == p]
                assert j == [k % nbuf]
                assert torch.equal(bufs[j[0]][:nbytes].cpu(), shards[sched[k]]), (step, k)
            assert lnf4.stream_log(st) == ss.simulate(sched, nbuf)
            lnf4.stream_reset(st, comp)
        torch.cuda.synchronize()
        got, secs = lnf4.stream_disk_stats(st)
        assert got >= 3 * len(sched) * nbytes and secs >= 0.0
        with pytest.raises(lnf4.LNF4Error):
            lnf4.stream_slot_load(st, 0, comp)   # no slot, and no host copy of the shard
    finally:
        torch.cuda.synchronize()
        lnf4.stream_destroy(st)
    os.remove(path)


def test_resident_log_matches_simulator():
    L, nbytes = 4, 2048
    shards = _pinned_shards(L, nbytes, seed=7)
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(L)]
    sched = ss.sft_schedule(L)
    comp = torch.cuda.current_stream()
    st = lnf4.stream_create(shards, [nbytes] * L, bufs, nbytes, sched, lnf4.STREAM_RESIDENT, torch.cuda.Stream())
    try:
        for k in range(len(sched)):
            p = lnf4.stream_layer_step(st, k, comp)
            assert p == bufs[sched[k]].data_ptr()
        assert lnf4.stream_log(st) == ss.simulate(sched, L, n_shards=L, resident=True)
        assert lnf4.stream_bytes_copied(st) == L * nbytes
    finally:
        torch.cuda.synchronize()
        lnf4.stream_destroy(st)


def test_rejects_unpinned_host_memory():
    h = torch.empty(1024, dtype=torch.uint8)  # pageable
    b = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(lnf4.LNF4Error) as ei:
        lnf4.stream_create([h, h], [1024, 1024], [b, b], 1024, [0, 1], 0, torch.cuda.Stream())
    assert ei.value.code == lnf4.LNF4_EINVAL


def _small_workload(fmt="nf4", adapted=("q", "v"), rank=8):
    shapes = synthgen._decoder_shapes(256, 4, 2, 64, 512)  # q 256x256, k/v 128x256, gate/up 512x256, down 256x512
    return synthgen.Workload(f"small_{fmt}", 200, shapes, rank, 2.0 * rank, adapted, layers=3, fmt=fmt,
                             vocab=320, hidden=256)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).copy()


HEAD_OUT = ("h0", "logp", "dh", "ref_logp", "ref_sums", "pol_sums", "loss", "coef")


def _snapshot(stack):
    torch.cuda.synchronize()
    out = {"y": {p: t.view(torch.int16).cpu().numpy().copy() for p, t in stack.y.items()},
           "dx": [t.view(torch.int16).cpu().numpy().copy() for t in stack.dx], "grads": [], "head": {}}
    for ls in stack.layers:
        out["grads"].append({p: (ls.dA[p].cpu().numpy().copy(), ls.dB[p].cpu().numpy().copy()) for p in ls.dA})
    for name in HEAD_OUT:
        t = getattr(stack, name, None)
        if t is not None:
            out["head"][name] = t.cpu().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy().copy()
    return out


def _same(a, b):
    for p in a["y"]:
        assert np.array_equal(a["y"][p], b["y"][p]), p
    for g in range(len(a["dx"])):
        assert np.array_equal(a["dx"][g], b["dx"][g]), g
    for l, gr in enumerate(a["grads"]):
        for p in gr:
            assert np.array_equal(gr[p][0], b["grads"][l][p][0])
            assert np.array_equal(gr[p][1], b["grads"][l][p][1])
    assert a["head"].keys() == b["head"].keys()
    for k in a["head"]:
        assert np.array_equal(a["head"][k], b["head"][k]), k


@pytest.mark.parametrize("dpo", [False, True])
def test_resident_graph_replays_equal_eager(dpo):
    """The resident step captured as a HIP graph: every replay gives the eager resident
    step's outputs bitwise, with eager work between the replays (the outputs overwritten,
    then a streamed step, which writes the same outputs)."""
    wl = _small_workload("nf4")
    stack = StreamedStack(wl, n_bufs=2, seed=3, dpo=dpo)
    try:
        stack.step(resident=True)
        ref = _snapshot(stack)
        for rep in range(3):
            for t in list(stack.y.values()) + list(stack.dx) + [stack.dh, stack.logp]:
                t.fill_(7)
            for ls in stack.layers:
                for p in ls.dA:
                    ls.dA[p].fill_(-1.0)
                    ls.dB[p].fill_(-1.0)
            stack.step_graph()
            _same(ref, _snapshot(stack))
            stack.step()
            _same(ref, _snapshot(stack))
    finally:
        stack.close()


def test_resident_graph_on_a_fresh_stack():
    """The graph captured on a stack that has run no resident step: the eager steps ahead
    of the capture copy the layers in and see every copy complete, so the capture issues
    no stream work, and the replay gives the eager resident step's outputs."""
    stack = StreamedStack(_small_workload("nf4"), n_bufs=2, seed=3)
    try:
        stack.step_graph()
        got = _snapshot(stack)
        stack.step(resident=True)
        _same(_snapshot(stack), got)
    finally:
        stack.close()


def test_copy_stream_one_per_device_and_not_the_compute_stream():
    """The library's copy stream: one per device, the same handle on every call, distinct from
    the compute stream; the stacks issue their layer copies on it."""
    import ctypes
    c1, c2, k = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
    assert lnf4.lib().stream_copy_stream(0, ctypes.byref(c1)) == 0
    assert lnf4.lib().stream_copy_stream(0, ctypes.byref(c2)) == 0
    assert lnf4.lib().stream_compute_stream(0, ctypes.byref(k)) == 0
    assert c1.value and c1.value == c2.value and c1.value != k.value
    assert lnf4.stream_copy_stream(0).cuda_stream == c1.value
    for bad in (-1, torch.cuda.device_count()):
        with pytest.raises(lnf4.LNF4Error, match="EINVAL|device"):
            lnf4.stream_copy_stream(bad)
    stack = StreamedStack(_small_workload("nf4"), n_bufs=2, seed=3)
    try:
        assert stack.copy.cuda_stream == c1.value
    finally:
        stack.close()


def test_compute_stream_one_per_device():
    """The library hands out one compute stream per device (the same handle on every call)
    and rejects a device that does not exist; the stacks run their kernels on it."""
    import ctypes
    h1, h2 = ctypes.c_void_p(), ctypes.c_void_p()
    assert lnf4.lib().stream_compute_stream(0, ctypes.byref(h1)) == 0
    assert lnf4.lib().stream_compute_stream(0, ctypes.byref(h2)) == 0
    assert h1.value and h1.value == h2.value
    assert lnf4.stream_compute_stream(0).cuda_stream == h1.value
    for bad in (-1, torch.cuda.device_count()):
        with pytest.raises(lnf4.LNF4Error, match="EINVAL|device"):
            lnf4.stream_compute_stream(bad)
    stack = StreamedStack(_small_workload("nf4"), n_bufs=2, seed=3)
    try:
        assert stack.compute.cuda_stream == h1.value
        assert stack.copy.cuda_stream != h1.value
    finally:
        stack.close()


@pytest.mark.parametrize("caller", ["null", "side"])
def test_step_is_ordered_with_the_callers_stream(caller):
    """A step called with the null stream or a side stream current runs after that stream's
    earlier work (a few milliseconds of products, then fills of every output) and that
    stream's later work (clones of the outputs) runs after the step: the clones and the
    outputs equal a plain step's, bitwise.  The null stream is ordered with the compute
    stream by the default-flag stream rules, a side stream by explicit event waits."""
    stack = StreamedStack(_small_workload("nf4"), n_bufs=2, seed=3)
    try:
        stack.step()
        ref = _snapshot(stack)
        outs = list(stack.y.values()) + list(stack.dx) + [stack.dh, stack.logp]
        grads = [t for ls in stack.layers for p in ls.dA for t in (ls.dA[p], ls.dB[p])]
        side = torch.cuda.Stream() if caller == "side" else torch.cuda.default_stream()
        assert (side.cuda_stream == 0) == (caller == "null")
        m = torch.randn(4096, 4096, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            for _ in range(30):
                m = (m @ m) * 1e-3
            for t in outs:
                t.fill_(7)
            for t in grads:
                t.fill_(-1.0)
            stack.step()
            clones = [t.clone() for t in outs + grads]
        torch.cuda.synchronize()
        _same(ref, _snapshot(stack))
        for t, c in zip(outs + grads, clones):
            assert torch.equal(t, c)
    finally:
        stack.close()


@pytest.mark.parametrize("fmt,dpo,reuse,efh", [("nf4", False, False, False), ("bf16", False, False, False),
                                               ("nf4", True, False, False), ("nf4", False, True, False),
                                               ("nf4", True, True, False), ("nf4", False, False, True),
                                               ("nf4", True, False, True)])
def test_streamed_equals_resident_bitwise(fmt, dpo, reuse, efh):
    """efh: the embedding rows read from the page-locked host table (the slot keeps lm_head)."""
    wl = _small_workload(fmt)
    stack = StreamedStack(wl, n_bufs=2, seed=3, dpo=dpo, reuse=reuse, embed_from_host=efh)
    try:
        stack.step()
        a = _snapshot(stack)
        stack.step(resident=True)
        b = _snapshot(stack)
        stack.step()
        c = _snapshot(stack)
    finally:
        stack.close()
    assert "dh" in a["head"]
    for snap in (b, c):
        _same(a, snap)


def test_disk_tier_read_error_is_reported(tmp_path):
    """A shard that can no longer be read (the file shrank after the context was created)
    fails the stream_layer_step call that needs it, with the errno text; the reader thread
    stops cleanly at destroy."""
    L, nbytes = 3, 4096
    shards = _pinned_shards(L, nbytes, seed=7)
    path = tmp_path / "shards.bin"
    with open(path, "wb") as f:
        for h in shards:
            f.write(h.numpy().tobytes())
    stage = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    sched = ss.sft_schedule(L)
    comp = torch.cuda.current_stream()
    os_truncate = __import__("os").truncate
    st = lnf4.stream_create_disk(str(path), [i * nbytes for i in range(L)], stage, nbytes, [nbytes] * L, bufs,
                                 nbytes, sched, torch.cuda.Stream())
    try:
        os_truncate(path, nbytes)   # shards 1 and 2 are gone (the reader may hold shard 1 already)
        with pytest.raises(lnf4.LNF4Error) as ei:
            for k in range(len(sched)):   # position 2 (shard 2) is read only after call 0
                lnf4.stream_layer_step(st, k, comp)
        assert "failed" in str(ei.value)
    finally:
        torch.cuda.synchronize()
        lnf4.stream_destroy(st)


@pytest.mark.parametrize("dpo,drop", [(False, True), (True, False)])
def test_disk_tier_step_equals_resident_bitwise(dpo, drop, tmp_path):
    """A stack step whose layers stream from a file (head slot from pinned RAM) gives
    bitwise the same outputs and gradients as the resident step."""
    stack = StreamedStack(_small_workload("nf4"), n_bufs=2, seed=5, dpo=dpo)
    try:
        stack.step(resident=True)
        a = _snapshot(stack)
        stack.use_disk(str(tmp_path / "layers.bin"), read_ahead=2, drop_cache=drop)
        stack.step()
        b = _snapshot(stack)
        stack.step()
        c = _snapshot(stack)
        got, _ = stack.disk_stats()
        assert got >= 2 * len(stack.schedule) * stack.shard_bytes
    finally:
        stack.close()
    for snap in (b, c):
        _same(a, snap)


@pytest.mark.parametrize("dpo,chunk", [(False, 64), (False, 7), (True, 100)])
def test_chunked_loss_equals_one_piece(dpo, chunk):
    """The head and its loss over chunks of tokens (the last one ragged) give bitwise the
    outputs of one piece: every row's logits, log-prob and gradient are the same sums."""
    wl = _small_workload("nf4")
    snaps = []
    for lc in (None, chunk):
        stack = StreamedStack(wl, n_bufs=2, seed=4, dpo=dpo, loss_chunk=lc)
        try:
            assert stack.chunk == (stack.T if lc is None else chunk)
            stack.step()
            snaps.append(_snapshot(stack))
        finally:
            stack.close()
    _same(snaps[0], snaps[1])


def _host_weights(stack, layer):
    """Decoded weights of one layer, read back from its pinned host shard with the oracle."""
    wl = stack.wl
    blob = stack.host[layer].numpy()
    W = {}
    for pi, p in enumerate(synthgen.PROJ_ORDER):
        o, i = wl.shapes[p]
        d0, a0 = stack.offsets[2 * pi], stack.offsets[2 * pi + 1]
        if stack.fmt == lnf4.FMT_NF4:
            codes = blob[d0:d0 + o * i // 2].reshape(o, i // 2)
            absmax = blob[a0:a0 + o * i // 16].view(np.float32)
            W[p] = onf4.decode_f64(codes, absmax)
        else:
            W[p] = bf16_f64(blob[d0:d0 + o * i * 2].view(np.uint16).reshape(o, i))
    return W


def _logp_bound(l, lab):
    """|logp_gpu - logp| per token, l being the oracle's bf16-rounded logits: a GPU logit
    (bf16 of an fp32 sum) can sit one bf16 step (relative 2^-8) away from the oracle's
    where the fp32 and fp64 sums straddle a rounding boundary, so the bound is
    2^-8 (|l_lab| + sum_j p_j |l_j|), plus 1e-4 for the fp32 accumulation and
    log-sum-exp."""
    lp, _ = ohead.log_softmax_rows(l)
    rows = np.arange(l.shape[0])
    return 2.0 ** -8 * (np.abs(l[rows, lab]) + (np.exp(lp) * np.abs(l)).sum(axis=1)) + 1e-4


def _check_head(stack, dpo):
    wl = stack.wl
    V, H, T = wl.vocab, wl.hidden, stack.T
    emb = stack.all_shards[stack.head_ids[0]].numpy().view(np.uint16).reshape(V, H)
    lm = bf16_f64(stack.all_shards[stack.head_ids[1]].numpy().view(np.uint16).reshape(V, H))
    ids, lab = stack.ids.cpu().numpy(), stack.labels.cpu().numpy()
    assert np.array_equal(_bits(stack.h0), ohead.embed_gather(emb, ids))
    h = bf16_f64(_bits(stack.h_last))
    # the logits and their gradient are bf16 tensors by definition of the head's calls
    # (lora_linear_fwd writes bf16(y), lnf4_cross_entropy writes bf16(dlogits)): the
    # oracle rounds them where the definition does
    def bf16(a):
        return bf16_f64(onf4.bf16_rne_bits(a))

    l = bf16(olora.linear_fwd(h, lm)[0])
    bound = _logp_bound(l, lab)
    logp = stack.logp.cpu().numpy()
    if not dpo:
        logp_o, _, d = ohead.cross_entropy(l, lab)
        assert np.all(np.abs(logp - logp_o) <= bound)
    else:
        S, beta = stack.seq_len, stack.beta
        l_ref = bf16(olora.linear_fwd(bf16_f64(_bits(stack.h_last_ref)), lm)[0])
        bound_ref = _logp_bound(l_ref, lab)
        logp_ref_o = ohead.cross_entropy(l_ref, lab)[0]
        logp_o = ohead.cross_entropy(l, lab)[0]
        assert np.all(np.abs(stack.ref_logp.cpu().numpy() - logp_ref_o) <= bound_ref)
        assert np.all(np.abs(logp - logp_o) <= bound)
        sums_ref_o, sums_o = ohead.sequence_sums(logp_ref_o, S), ohead.sequence_sums(logp_o, S)
        bs_ref, bs = ohead.sequence_sums(bound_ref, S), ohead.sequence_sums(bound, S)
        assert np.all(np.abs(stack.ref_sums.cpu().numpy() - sums_ref_o) <= bs_ref)
        assert np.all(np.abs(stack.pol_sums.cpu().numpy() - sums_o) <= bs)
        loss_o, coef_o = ohead.dpo_loss(sums_o, sums_ref_o, beta)
        dm = beta * (bs + bs_ref).reshape(-1, 2).sum(axis=1)          # margin error bound per pair
        P = len(dm)
        assert abs(float(stack.loss.cpu()[0]) - loss_o) <= dm.mean() + 1e-6
        assert np.all(np.abs(stack.coef.cpu().numpy() - coef_o) <= np.repeat(beta / P * dm / 4, 2) + 1e-6)
        _, _, d = ohead.cross_entropy(l, lab, grad_scale=ohead.dpo_token_scale(coef_o, S))
    dh_o = olora.linear_bwd(h, bf16(d), lm)[0]
    check_tol(bf16_f64(_bits(stack.dh)), dh_o, "dh (lm_head input gradient)")


@pytest.mark.parametrize("dpo,efh", [(False, False), (True, False), (False, True)])
def test_stack_step_matches_oracle(dpo, efh):
    wl = _small_workload("nf4", adapted=("q", "k", "v", "o", "gate", "up", "down"), rank=4)
    stack = StreamedStack(wl, n_bufs=2, seed=5, dpo=dpo, embed_from_host=efh)
    try:
        stack.step()
        torch.cuda.synchronize()
        # the shared output buffers hold the last layer processed: layer 0 (backward ends there)
        for layer in range(stack.L):
            ls = stack.layers[layer]
            W = _host_weights(stack, layer)
            ad = {p: (bf16_f64(ls.A[p].view(torch.int16).cpu().numpy().view(np.uint16)),
                      bf16_f64(ls.B[p].view(torch.int16).cpu().numpy().view(np.uint16)), wl.scale) for p in ls.A}
            xs = {gi: bf16_f64(x.view(torch.int16).cpu().numpy().view(np.uint16)) for gi, x in enumerate(ls.x)}
            dys = {p: bf16_f64(d.view(torch.int16).cpu().numpy().view(np.uint16)) for p, d in ls.dy.items()}
            ref = olayer.layer_step(W, ad, xs, dys, dpo=dpo)
            for p in ls.A:
                check_tol(ls.dA[p].cpu().numpy(), ref["grads"][p][0], f"L{layer} dA {p}")
                check_tol(ls.dB[p].cpu().numpy(), ref["grads"][p][1], f"L{layer} dB {p}")
            if layer == 0:
                for p, t in stack.y.items():
                    check_tol(bf16_f64(t.view(torch.int16).cpu().numpy().view(np.uint16)), ref["recompute"][p],
                              f"y {p}")
                for gi, t in enumerate(stack.dx):
                    check_tol(bf16_f64(t.view(torch.int16).cpu().numpy().view(np.uint16)), ref["dx"][gi],
                              f"dx group {gi}")
        _check_head(stack, dpo)
    finally:
        stack.close()


@pytest.mark.parametrize("n_parts", [1, 3, 7])
def test_slot_load_in_parts(n_parts):
    L, nbytes, slot_bytes = 3, 4096, 3 * 4096 + 100
    shards = _pinned_shards(L, nbytes, seed=11)
    head = _pinned_shards(1, slot_bytes - 100, seed=12)[0]
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    slot = torch.zeros(slot_bytes, dtype=torch.uint8, device="cuda")
    comp = torch.cuda.current_stream()
    st = lnf4.stream_create(shards + [head], [nbytes] * L + [head.numel()], bufs, nbytes, [0, 1, 2], 0,
                            torch.cuda.Stream(), slot, slot_bytes)
    try:
        b0 = lnf4.stream_bytes_copied(st)
        for part in range(n_parts):
            if part > 0:
                with pytest.raises(lnf4.LNF4Error) as ei:   # the load is not complete yet
                    lnf4.stream_slot_wait(st, comp)
                assert ei.value.code == lnf4.LNF4_ESTATE
            with pytest.raises(lnf4.LNF4Error):              # parts go in order
                lnf4.stream_slot_load_part(st, L, part + 1, n_parts, comp)
            lnf4.stream_slot_load_part(st, L, part, n_parts, comp)
        p = lnf4.stream_slot_wait(st, comp)
        assert p == slot.data_ptr()
        assert torch.equal(slot[:head.numel()].cpu(), head)
        assert lnf4.stream_bytes_copied(st) - b0 == head.numel()
        ev = [e for e in lnf4.stream_log(st) if e[0] == lnf4.EV_SLOT_COPY]
        assert [e[4] for e in ev] == [-1 - q for q in range(n_parts)]
    finally:
        torch.cuda.synchronize()
        lnf4.stream_destroy(st)


def test_no_recompute_gives_the_same_gradients():
    """Skipping the backward's forward re-run (the saved u stands in for the recomputed
    one, which is bitwise the same) changes no gradient."""
    wl = _small_workload("nf4", adapted=("q", "k", "v", "o", "gate", "up", "down"), rank=4)
    snaps = []
    for rc in (True, False):
        stack = StreamedStack(wl, n_bufs=2, seed=6, recompute=rc)
        try:
            stack.step()
            snaps.append(_snapshot(stack))
        finally:
            stack.close()
    a, b = snaps
    for g in range(len(a["dx"])):
        assert np.array_equal(a["dx"][g], b["dx"][g]), g
    for l, gr in enumerate(a["grads"]):
        for p in gr:
            assert np.array_equal(gr[p][0], b["grads"][l][p][0])
            assert np.array_equal(gr[p][1], b["grads"][l][p][1])
    assert np.array_equal(a["head"]["dh"], b["head"]["dh"])


def _estate(fn, *a):
    with pytest.raises(lnf4.LNF4Error) as ei:
        fn(*a)
    assert ei.value.code == lnf4.LNF4_ESTATE, str(ei.value)


@pytest.mark.parametrize("disk", [False, True])
def test_destroy_is_idempotent_and_a_destroyed_context_gives_estate(disk, tmp_path):
    """stream_destroy twice returns OK both times; every stream call on the destroyed
    handle returns ESTATE without touching it; a context created afterwards gets another
    address and works, and the old handle still gives ESTATE."""
    L, nbytes = 3, 4096
    shards = _pinned_shards(L, nbytes, seed=11)
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    slot = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sched = ss.sft_schedule(L)
    comp = torch.cuda.current_stream()
    if disk:
        path = tmp_path / "shards.bin"
        with open(path, "wb") as f:
            for h in shards:
                f.write(h.numpy().tobytes())
        stage = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(2)]

        def make():
            return lnf4.stream_create_disk(str(path), [i * nbytes for i in range(L)], stage, nbytes, [nbytes] * L,
                                           bufs, nbytes, sched, torch.cuda.Stream(), host_shards=shards,
                                           slot_buf=slot, slot_bytes=nbytes)
    else:
        def make():
            return lnf4.stream_create(shards, [nbytes] * L, bufs, nbytes, sched, 0, torch.cuda.Stream(),
                                      slot_buf=slot, slot_bytes=nbytes)
    st = make()
    lnf4.stream_layer_step(st, 0, comp)
    lnf4.stream_slot_load(st, 0, comp)
    lib = lnf4.lib()
    assert lib.stream_destroy(st) == lnf4.LNF4_OK
    assert lib.stream_destroy(st) == lnf4.LNF4_OK
    for fn, a in ((lnf4.stream_layer_step, (st, 1, comp)), (lnf4.stream_log, (st,)),
                  (lnf4.stream_reset, (st, comp)), (lnf4.stream_slot_load, (st, 0, comp)),
                  (lnf4.stream_slot_load_part, (st, 0, 0, 2, comp)), (lnf4.stream_slot_wait, (st, comp)),
                  (lnf4.stream_bytes_copied, (st,)), (lnf4.stream_disk_stats, (st,))):
        _estate(fn, *a)
    st2 = make()
    try:
        assert st2 != st
        for k in range(len(sched)):
            p = lnf4.stream_layer_step(st2, k, comp)
            j = [i for i, b in enumerate(bufs) if b.data_ptr() == p]
            assert torch.equal(bufs[j[0]].cpu(), shards[sched[k]]), k
        assert lnf4.stream_log(st2) == ss.simulate(sched, 2)
        _estate(lnf4.stream_log, st)
    finally:
        torch.cuda.synchronize()
        lnf4.stream_destroy(st2)
    _estate(lnf4.stream_layer_step, st2, 0, comp)


@pytest.mark.parametrize("n_stage", [1, 2, 3])
def test_disk_tier_reset_in_the_middle_of_a_pass(n_stage, tmp_path):
    """A disk-tier pass abandoned after 3 calls and reset: the reader restarts at the next
    pass, and a whole pass then runs with the log of the ring simulator and every buffer
    holding its shard; a second reset after a finished pass keeps working."""
    L, nbytes, nbuf = 4, 4096, 2
    shards = _pinned_shards(L, nbytes, seed=60 + n_stage)
    path = tmp_path / "shards.bin"
    with open(path, "wb") as f:
        for h in shards:
            f.write(h.numpy().tobytes())
    stage = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(n_stage)]
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    sched = ss.sft_schedule(L)
    comp = torch.cuda.current_stream()
    st = lnf4.stream_create_disk(str(path), [i * nbytes for i in range(L)], stage, nbytes, [nbytes] * L, bufs,
                                 nbytes, sched, torch.cuda.Stream())
    try:
        for k in range(3):
            lnf4.stream_layer_step(st, k, comp)
        lnf4.stream_reset(st, comp)
        for rep in range(2):
            for k in range(len(sched)):
                p = lnf4.stream_layer_step(st, k, comp)
                j = [i for i, b in enumerate(bufs) if b.data_ptr() == p]
                assert j == [k % nbuf]
                assert torch.equal(bufs[j[0]].cpu(), shards[sched[k]]), (rep, k)
            assert lnf4.stream_log(st) == ss.simulate(sched, nbuf)
            lnf4.stream_reset(st, comp)
    finally:
        torch.cuda.synchronize()
        lnf4.stream_destroy(st)


@pytest.mark.parametrize("dpo", [False, True])
@pytest.mark.parametrize("efh", [False, True])
@pytest.mark.parametrize("nbuf", [2, 3])
def test_stack_log_matches_the_slot_simulator(dpo, efh, nbuf):
    """Three steps of a stack with its head slot: each step's event log (layer ring and
    slot loads and waits) equals the oracle's stack-step simulator, and the bytes copied
    per step are the layer copies plus the slot loads it lists."""
    wl = _small_workload()
    stack = StreamedStack(wl, n_bufs=nbuf, seed=9, dpo=dpo, embed_from_host=efh)
    stack.keep_log = True
    L = stack.L
    try:
        n = 0
        for step in range(3):
            b0 = stack.bytes_copied()
            stack.step()
            want = ss.stack_step_log(L, nbuf, dpo, efh, first=(step == 0), loads_before=n,
                                     lm_head_call=stack.lm_head_call, lead_parts=stack.lead_parts)
            assert stack.last_log == want, step
            ss.check_slot_log(want, L, dpo, start=None if step == 0 else (L + 1 if efh else L))
            n += (1 if step == 0 else 0) if efh else (3 if step == 0 else 2)
            layer_bytes = stack.shard_bytes * len(stack.schedule)
            slot = (stack.all_shards[L + 1].numel() if step == 0 else 0) if efh else \
                stack.all_shards[L].numel() * (2 if step == 0 else 1) + stack.all_shards[L + 1].numel()
            assert stack.bytes_copied() - b0 == layer_bytes + slot, step
    finally:
        stack.close()
