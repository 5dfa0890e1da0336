"""A layer-streamed stack of frozen NF4 (or bf16) decoder-layer projections with LoRA,
driven through the lnf4 C ABI.

One step follows the layer-streaming schedule (Soup deep dive, "Core feature: how layer
streaming works"): every layer is read once for the forward and once more for the
backward, where its forward is recomputed from the checkpointed inputs and the input
gradients and adapter gradients are formed; a DPO step first runs the same streamed base
with the adapters off (4 GB-laptop Soup article, "Memory-free reference model").  The
vocab-sized embed_tokens and untied lm_head share one device slot.

The output side runs where the slot schedule puts it: the embedding lookup of the step's
token ids at the start (embed_tokens in the slot), and at the forward/backward turn the
untied lm_head (a bf16 [vocab, hidden] GEMM), the token cross-entropy and the lm_head's
input gradient, optionally a chunk of tokens at a time (the ``stream_loss_chunk`` key of
the Soup deep dive, "Streaming config keys").  A DPO step takes log-prob sums over each
sequence in the reference pass and the policy pass and turns the sigmoid preference loss
into per-sequence gradient scales of the policy's cross-entropy.

The attention core, norms and activations between the projections are not on this path,
so every projection group reads its own synthetic checkpointed input, every projection
its own synthetic output gradient, and the lm_head a synthetic final hidden state (one
for the policy pass, one for the reference pass).  All work is enqueued by C ABI calls;
this module only lays out memory and orders the calls.
"""
from __future__ import annotations

import contextlib
import os
from dataclasses import dataclass

import torch

import synthgen
from . import lnf4

GROUPS = synthgen.GROUPS
PROJ_ORDER = synthgen.PROJ_ORDER


def sft_schedule(L: int):
    return list(range(L)) + list(range(L - 1, -1, -1))


def dpo_schedule(L: int):
    return list(range(L)) + sft_schedule(L)


@dataclass
class LayerState:
    x: list            # per group: checkpointed input [T, in]
    dy: dict           # per projection: output gradient [T, out]
    u: dict            # adapted projection -> saved u [T, r] fp32
    A: dict
    B: dict
    dA: dict
    dB: dict


@contextlib.contextmanager
def on_stream(stream):
    """Run the block with `stream` (the library's compute stream, or a stream being captured)
    current, after the caller's stream's earlier work, and order the caller's stream's later
    work after the block.  Nothing to join when they are one stream.  Nothing either when
    the caller is on the null stream: the compute stream already orders itself with the
    null stream (default-flag stream rules), and an explicit wait left pending on the null
    stream would make every launch of the block wait behind a check against it (measured:
    the 8B step 8-10% slower)."""
    cur = torch.cuda.current_stream(stream.device)
    if cur == stream:
        yield
        return
    if cur.cuda_stream == 0:
        with torch.cuda.stream(stream):
            yield
        return
    stream.wait_stream(cur)
    with torch.cuda.stream(stream):
        yield
    cur.wait_stream(stream)


class StepPacer:
    """Keeps the host about one streamed step ahead of the GPU: once a step has enqueued its
    first layer call (and with it the copies of its first layers, which wait only for the
    buffers' last users), the host sleeps on a blocking-sync event recorded at the end of
    the previous step before it enqueues the rest.  Left to run ahead, the host fills HIP's
    command queue and then sits blocked inside kernel launches, and in that state the layer
    copies of the Llama-8B-shaped stack ran at 49.5 instead of 56.2 GB/s (197 against
    180.5 ms per step; the link was idle for the same 3.5-4 ms of each step either way)."""

    def __init__(self):
        self.ev = None

    def wait(self):
        if self.ev is not None:
            self.ev.synchronize()
            self.ev = None

    def mark(self, stream):
        ev = torch.cuda.Event(blocking=True)
        ev.record(stream)
        self.ev = ev


class StreamedStack:
    def __init__(self, wl: synthgen.Workload, n_bufs: int = 2, seed: int = 0,
                 layers: int | None = None, tokens: int | None = None, head_slot: bool = True,
                 dpo: bool | None = None, loss_chunk: int | None = None, reuse: bool = False,
                 recompute: bool = True, embed_from_host: bool = False, device: str = "cuda"):
        self.wl = wl
        self.L = layers if layers is not None else wl.layers
        self.T = tokens if tokens is not None else wl.tokens
        self.fmt = lnf4.FMT_NF4 if wl.fmt == "nf4" else lnf4.FMT_BF16
        self.dpo = ("ref" in wl.passes) if dpo is None else dpo
        self.n_bufs = n_bufs
        self.seed = seed
        self.reuse = reuse          # buffers that still hold a needed layer are used without a copy
        self.recompute = recompute  # False: the backward uses the forward's saved u and skips the re-run
        # True: the embedding lookup reads its T rows straight from the page-locked host table
        # and the slot keeps the untied lm_head from one step to the next (no per-step slot copies)
        self.embed_from_host = embed_from_host
        dev = torch.device(device)
        self.dev = dev
        T = self.T
        outs = [wl.shapes[p][0] for p in PROJ_ORDER]
        ins = [wl.shapes[p][1] for p in PROJ_ORDER]
        self.offsets, self.shard_bytes = lnf4.lnf4_shard_layout(outs, ins, self.fmt)
        # the kernels run on the library's compute stream, which has a hardware queue of its
        # own: a copy stream that shared the compute stream's queue would serialise with it
        self.compute = lnf4.stream_compute_stream(dev)
        self.copy = lnf4.stream_copy_stream(dev)   # a hardware queue of its own

        # ---- pinned host shards (one contiguous blob per layer), built on the device
        self.host = []
        stage = torch.empty(self.shard_bytes, dtype=torch.uint8, device=dev)
        for layer in range(self.L):
            self._fill_shard(stage, layer)
            h = torch.empty(self.shard_bytes, dtype=torch.uint8, pin_memory=True)
            h.copy_(stage)
            self.host.append(h)
        del stage
        self.bufs = [torch.empty(self.shard_bytes, dtype=torch.uint8, device=dev) for _ in range(self.n_bufs)]

        # ---- head slot: bf16 embed_tokens and untied lm_head [vocab, hidden]
        self.slot = None
        self.head_ids = []
        shards = list(self.host)
        sizes = [self.shard_bytes] * self.L
        if head_slot and wl.vocab > 0:
            nbytes = wl.vocab * wl.hidden * 2
            for name in ("embed", "lm_head"):
                t = synthgen.device_normal((wl.vocab, wl.hidden), 0.02, seed, "head", name, dtype=torch.bfloat16)
                h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
                h.copy_(t.view(torch.uint8).reshape(-1))
                del t
                self.head_ids.append(len(shards))
                shards.append(h)
                sizes.append(nbytes)
            self.slot = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.all_shards = shards
        self._init_output_side(loss_chunk)

        # ---- per-layer adapters, checkpointed inputs, output gradients, gradients
        r = wl.rank
        self.layers = []
        for layer in range(self.L):
            xs = [synthgen.device_normal((T, wl.shapes[g[0]][1]), 1.0, seed, "x", layer, gi, dtype=torch.bfloat16)
                  for gi, g in enumerate(GROUPS)]
            dys = {p: synthgen.device_normal((T, wl.shapes[p][0]), 1.0, seed, "dy", layer, p, dtype=torch.bfloat16)
                   for p in PROJ_ORDER}
            A, B, dA, dB, u = {}, {}, {}, {}, {}
            for p in wl.adapted:
                o, i = wl.shapes[p]
                A[p] = synthgen.device_uniform((r, i), 1.0 / i ** 0.5, seed, "A", layer, p, dtype=torch.bfloat16)
                B[p] = synthgen.device_normal((o, r), 0.01, seed, "B", layer, p, dtype=torch.bfloat16)
                dA[p] = torch.zeros((r, i), dtype=torch.float32, device=dev)
                dB[p] = torch.zeros((o, r), dtype=torch.float32, device=dev)
                u[p] = torch.zeros((T, r), dtype=torch.float32, device=dev)
            self.layers.append(LayerState(xs, dys, u, A, B, dA, dB))
        self.y = {p: torch.empty((T, wl.shapes[p][0]), dtype=torch.bfloat16, device=dev) for p in PROJ_ORDER}
        self.dx = [torch.empty((T, wl.shapes[g[0]][1]), dtype=torch.bfloat16, device=dev) for g in GROUPS]
        ws = 0
        for gi, g in enumerate(GROUPS):
            ws = max(ws, lnf4.lora_group_bwd_workspace(self._projs(0, gi, 256, bwd=True), T),
                     lnf4.lora_group_fwd_workspace(self._projs(0, gi, 256), T))
        self.ws_bytes = max(ws, 256)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)

        sched = dpo_schedule(self.L) if self.dpo else sft_schedule(self.L)
        self.schedule = sched
        torch.cuda.synchronize(dev)
        slot_bytes = self.slot.numel() if self.slot is not None else 0
        mode = lnf4.STREAM_REUSE if reuse else lnf4.STREAM_RING
        self.st = lnf4.stream_create(shards, sizes, self.bufs, self.shard_bytes, sched, mode, self.copy, self.slot,
                                     slot_bytes)
        self.timers = None
        # when a list: (event before, event after) on the compute stream around every call that
        # makes compute wait for a copy (layer steps and slot waits); between the two events
        # the stream runs no kernel, so their distance is the time compute was blocked
        self.wait_events = None
        # when a list: per stream call that may issue copies, (tag, call, event on the compute
        # stream just before it, event on the copy stream just after it, bytes the call
        # issued); the call's copies wait for nothing later than the first event, and are
        # done when the copy stream reaches the second
        self.copy_marks = None
        # streamed steps wait for the previous streamed step before they are enqueued
        self.pacer = StepPacer()
        # head-slot schedule: lm_head is loaded after forward call lm_head_call, so that it is
        # in the slot when the forward ends and the head runs while the first backward layers
        # copy; the first backward call issues lead_parts parts of the next embedding (the
        # link would otherwise wait for the first backward layer's compute there), every
        # later one a single part
        self.lm_head_call = self.L - 2 if self.L >= 2 else self.L - 1
        self.lead_parts = min(3, self.L)
        self.keep_log = False        # True: step() keeps the pass's event log in last_log
        self.last_log = None
        self._embed_in_slot = False   # the next step's embed_tokens was loaded during the last backward
        self._lm_head_in_slot = False  # embed_from_host: the lm_head was loaded into the slot
        self.st_res = None
        self._graph = None            # the resident step captured as a HIP graph (resident_graph)
        self.res_bufs = None

    def _init_output_side(self, loss_chunk):
        """Token ids, labels, the synthetic final hidden states, and the head's logits,
        log-prob and gradient buffers (nothing when the workload has no head slot)."""
        self.head = self.slot is not None
        if not self.head:
            return
        wl, T, dev, seed = self.wl, self.T, self.dev, self.seed
        V, H = wl.vocab, wl.hidden
        bf16, f32 = torch.bfloat16, torch.float32
        self.ids = synthgen.device_token_ids(T, V, seed, "ids")
        self.labels = synthgen.device_token_ids(T, V, seed, "labels")
        self.h0 = torch.empty((T, H), dtype=bf16, device=dev)                  # embedding rows
        self.h_last = synthgen.device_normal((T, H), 1.0, seed, "h_last", dtype=bf16)
        self.logp = torch.empty(T, dtype=f32, device=dev)
        self.dh = torch.empty((T, H), dtype=bf16, device=dev)                  # gradient into h_last
        chunk = T if not loss_chunk else min(int(loss_chunk), T)
        if self.dpo:
            self.seq_len = int(wl.extra.get("seq_len", T // 4))
            self.beta = float(wl.extra.get("beta", 0.1))
            if T % (2 * self.seq_len):
                raise ValueError(f"T={T} is not a whole number of (chosen, rejected) pairs of {self.seq_len}")
            self.n_seq = T // self.seq_len
            # a chunk covers whole sequences, so its rows find their sequence's scale
            chunk = max(self.seq_len, chunk // self.seq_len * self.seq_len)
            self.h_last_ref = synthgen.device_normal((T, H), 1.0, seed, "h_last_ref", dtype=bf16)
            self.ref_logp = torch.empty(T, dtype=f32, device=dev)
            self.ref_sums = torch.empty(self.n_seq, dtype=f32, device=dev)
            self.pol_sums = torch.empty(self.n_seq, dtype=f32, device=dev)
            self.loss = torch.empty(1, dtype=f32, device=dev)
            self.coef = torch.empty(self.n_seq, dtype=f32, device=dev)
        self.chunk = chunk
        self.logits = torch.empty((chunk, V), dtype=bf16, device=dev)       # dlogits overwrite it in place
        self.head_ws_bytes = max(256, lnf4.lora_linear_bwd_workspace(chunk, V, H, 0))
        self.head_ws = torch.empty(self.head_ws_bytes, dtype=torch.uint8, device=dev)
        self.res_head = None

    def enable_resident(self):
        """A second context over the same host shards with one device buffer per layer:
        every layer is copied once, then steps run with no host-to-device traffic (the same
        kernels, the same addresses pattern): the H2D-removed reference run."""
        if self.st_res is None:
            self.res_bufs = [torch.empty(self.shard_bytes, dtype=torch.uint8, device=self.dev) for _ in range(self.L)]
            self.st_res = lnf4.stream_create(self.host, [self.shard_bytes] * self.L, self.res_bufs, self.shard_bytes,
                                             self.schedule, lnf4.STREAM_RESIDENT, self.copy)
            if self.head:
                # embed_tokens and lm_head each resident in a buffer of their own
                self.res_head = []
                for sid in self.head_ids:
                    h = self.all_shards[sid]
                    d = torch.empty(h.numel(), dtype=torch.uint8, device=self.dev)
                    d.copy_(h)
                    self.res_head.append(d)
                torch.cuda.synchronize(self.dev)
        return self.st_res

    # ------------------------------------------------------------------ set-up helpers
    def _fill_shard(self, stage, layer):
        wl = self.wl
        for pi, p in enumerate(PROJ_ORDER):
            o, i = wl.shapes[p]
            w = synthgen.device_normal((o, i), 0.02, self.seed, "W", layer, p)
            d0, a0 = self.offsets[2 * pi], self.offsets[2 * pi + 1]
            if self.fmt == lnf4.FMT_NF4:
                codes = stage[d0:d0 + o * i // 2]
                absmax = stage[a0:a0 + (o * i // 64) * 4].view(torch.float32)
                lnf4.nf4_quantize(w, o * i, 64, codes, absmax)
            else:
                stage[d0:d0 + o * i * 2].view(torch.bfloat16).copy_(w.to(torch.bfloat16).reshape(-1))
            del w
        torch.cuda.synchronize(self.dev)

    def _weight(self, base: int, pi: int):
        o, i = self.wl.shapes[PROJ_ORDER[pi]]
        d0, a0 = self.offsets[2 * pi], self.offsets[2 * pi + 1]
        return lnf4.make_weight(self.fmt, base + d0, (base + a0) if self.fmt == lnf4.FMT_NF4 else None, o, i, 64)

    def _projs(self, layer: int, gi: int, base: int, bwd: bool = False, adapters: bool = True):
        wl, st = self.wl, self.layers[layer]
        out = []
        for p in GROUPS[gi]:
            pi = PROJ_ORDER.index(p)
            W = self._weight(base, pi)
            on = adapters and p in wl.adapted
            out.append(lnf4.make_proj(
                W, A=st.A[p] if on else None, B=st.B[p] if on else None, r=wl.rank if on else 0,
                scale=wl.scale if on else 0.0, y=self.y[p], u=st.u[p] if on else None,
                dy=st.dy[p] if bwd else None, dA=st.dA[p] if (bwd and on) else None,
                dB=st.dB[p] if (bwd and on) else None))
        return out

    # ------------------------------------------------------------------ one step
    def _mark(self, key, end: int):
        tm = self.timers
        if tm is not None and key in tm:
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(self.compute)
            tm[key][end].append(ev)

    def _waited(self, fn):
        """Run a stream call that enqueues a wait on the compute stream, bracketed by timing
        events when wait_events is set."""
        we = self.wait_events
        if we is None:
            return fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.compute)
        out = fn()
        e1.record(self.compute)
        we.append((e0, e1))
        return out

    def _copying(self, st, tag, k, fn):
        """Run a stream call of context st that may issue copies, bracketed by copy_marks
        events when set."""
        cm = self.copy_marks
        if cm is None:
            return fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0 = lnf4.stream_bytes_copied(st)
        e0.record(self.compute)
        out = fn()
        e1.record(self.copy)
        cm.append((tag, k, e0, e1, lnf4.stream_bytes_copied(st) - b0))
        return out

    def _lm_head(self, ptr):
        return lnf4.make_weight(lnf4.FMT_BF16, ptr, None, self.wl.vocab, self.wl.hidden, 64)

    def _chunks(self):
        return [(c0, min(self.chunk, self.T - c0)) for c0 in range(0, self.T, self.chunk)]

    def _logits(self, W, h, c0, n):
        lnf4.lora_linear_fwd(W, h[c0:c0 + n], n, None, None, 0, 0.0, self.logits, None, self.compute)

    def _head_dx(self, W, c0, n):
        # dh = dlogits W (the lm_head is frozen: no weight gradient)
        lnf4.lora_linear_bwd(W, self.h_last[c0:c0 + n], self.logits, n, None, None, 0, 0.0, None,
                             self.dh[c0:c0 + n], None, None, 0, self.head_ws, self.head_ws_bytes, self.compute)

    def _embed(self, table_ptr):
        lnf4.lnf4_embed_gather(table_ptr, self.wl.vocab, self.wl.hidden, self.ids, self.T, self.h0, self.compute)

    def _head_sft(self, ptr):
        """Mean token cross-entropy: logits, log-probs and dlogits (in place), dh."""
        self._mark(("head", "sft"), 0)
        W, V = self._lm_head(ptr), self.wl.vocab
        for c0, n in self._chunks():
            self._logits(W, self.h_last, c0, n)
            lnf4.lnf4_cross_entropy(self.logits, n, V, self.labels[c0:], 1.0 / self.T, None, 1, self.logp[c0:],
                                    self.logits, self.compute)
            self._head_dx(W, c0, n)
        self._mark(("head", "sft"), 1)

    def _head_ref(self, ptr):
        """Reference pass (adapters off): token log-probs and their per-sequence sums."""
        self._mark(("head", "ref"), 0)
        W, V = self._lm_head(ptr), self.wl.vocab
        for c0, n in self._chunks():
            self._logits(W, self.h_last_ref, c0, n)
            lnf4.lnf4_cross_entropy(self.logits, n, V, self.labels[c0:], 1.0, None, 1, self.ref_logp[c0:], None,
                                    self.compute)
        lnf4.lnf4_sequence_sums(self.ref_logp, self.n_seq, self.seq_len, self.ref_sums, self.compute)
        self._mark(("head", "ref"), 1)

    def _head_dpo(self, ptr):
        """Policy pass: log-prob sums, the sigmoid preference loss and its coefficients,
        then dlogits = -coef_seq * (softmax - onehot) and dh.  With one chunk the logits
        are still in place for the gradient; with several they are computed again."""
        self._mark(("head", "pol"), 0)
        W, V, S = self._lm_head(ptr), self.wl.vocab, self.seq_len
        chunks = self._chunks()
        for c0, n in chunks:
            self._logits(W, self.h_last, c0, n)
            lnf4.lnf4_cross_entropy(self.logits, n, V, self.labels[c0:], 1.0, None, 1, self.logp[c0:], None,
                                    self.compute)
        lnf4.lnf4_sequence_sums(self.logp, self.n_seq, S, self.pol_sums, self.compute)
        lnf4.lnf4_dpo_loss(self.pol_sums, self.ref_sums, self.n_seq // 2, self.beta, self.loss, self.coef,
                           self.compute)
        for c0, n in chunks:
            if len(chunks) > 1:
                self._logits(W, self.h_last, c0, n)
            lnf4.lnf4_cross_entropy(self.logits, n, V, self.labels[c0:], -1.0, self.coef[c0 // S:], S, None,
                                    self.logits, self.compute)
            self._head_dx(W, c0, n)
        self._mark(("head", "pol"), 1)

    def _group_fwd(self, layer, gi, base, adapters, u_saved=False):
        """u_saved: the recompute, whose u = x A^T the forward of the same layer already wrote
        (same checkpointed x, same adapters), so the call reads it instead of recomputing it."""
        key = ("fwd", gi, adapters)
        self._mark(key, 0)
        on = (2 if u_saved else 1) if adapters else 0
        lnf4.lora_group_fwd_ws(self._projs(layer, gi, base, adapters=adapters), self.layers[layer].x[gi], self.T,
                               on, self.ws, self.ws_bytes, self.compute)
        self._mark(key, 1)

    def _group_bwd(self, layer, gi, base):
        key = ("bwd", gi, True)
        self._mark(key, 0)
        lnf4.lora_group_bwd(self._projs(layer, gi, base, bwd=True), self.layers[layer].x[gi], self.T, self.dx[gi],
                            0, self.ws, self.ws_bytes, self.compute)
        self._mark(key, 1)

    def step(self, resident: bool = False, compute: bool = True):
        """One training step over the whole stack (all calls asynchronous on the compute stream,
        ordered after the caller's stream's earlier work; the caller's later work waits for
        it).  resident=True runs the same step from the resident context (no layer copies;
        the head matrices sit in buffers of their own).  compute=False issues the same
        stream calls (copies, waits, slot loads) without the kernels: the time of the
        stream schedule alone.  A streamed step waits on the host, after its first layer
        call, for the previous streamed step to finish (StepPacer); a resident step, which
        copies nothing, does not."""
        pace = not resident and self.pacer is not None
        with on_stream(self.compute):
            self._step(resident, compute, pace)
            if pace:
                self.pacer.mark(self.compute)

    def _step(self, resident: bool, compute: bool, pace: bool = False):
        L = self.L
        st = self.enable_resident() if resident else self.st
        slot = self.slot is not None and not resident
        head = self.head and compute
        if slot and self.embed_from_host:
            if not self._lm_head_in_slot:   # loaded once; the embedding never enters the slot
                self._copying(st, "slot", -1, lambda: lnf4.stream_slot_load(st, self.head_ids[1], self.compute))
                self._lm_head_in_slot = True
            if head:
                self._embed(self.all_shards[self.head_ids[0]])   # T rows over the host link
        elif slot:
            if not self._embed_in_slot:   # first step: nothing trickled in yet
                self._copying(st, "slot", -1, lambda: lnf4.stream_slot_load(st, self.head_ids[0], self.compute))
            ptr = self._waited(lambda: lnf4.stream_slot_wait(st, self.compute))
            self._embed_in_slot = False
            if head:
                self._embed(ptr)
        elif head:
            self._embed(self.res_head[0])
        n_fwd = 2 * L if self.dpo else L
        for k, layer in enumerate(self.schedule):
            base = self._waited(lambda: self._copying(st, "layer", k, lambda: lnf4.stream_layer_step(st, k, self.compute)))
            if pace and k == 0:
                self.pacer.wait()
            if k == L or k == n_fwd:
                # the output head of the forward pass that just ended.  It runs after this
                # call's stream step, which released the last forward layer's buffer, so the
                # next layer copy overlaps the head instead of waiting behind it.
                if slot:
                    ptr = self._waited(lambda: lnf4.stream_slot_wait(st, self.compute))
                elif head:
                    ptr = self.res_head[1]
                if head:
                    if not self.dpo:
                        self._head_sft(ptr)
                    elif k == L:
                        self._head_ref(ptr)
                    else:
                        self._head_dpo(ptr)
            if k < n_fwd:
                ref_pass = self.dpo and k < L
                for gi in range(len(GROUPS) if compute else 0):
                    self._group_fwd(layer, gi, base, adapters=not ref_pass)
                if slot and k == self.lm_head_call and not self.embed_from_host:
                    # the untied lm_head takes the slot before the end of the first forward
                    # pass and stays there for the second (DPO)
                    self._copying(st, "slot", k, lambda: lnf4.stream_slot_load(st, self.head_ids[1], self.compute))
            else:
                if slot and not self.embed_from_host:
                    # the next step's embed_tokens trickles into the slot in L parts between
                    # the layer copies: lead_parts at the first backward call, then one per call
                    i = k - n_fwd
                    p0 = 0 if i == 0 else self.lead_parts + i - 1
                    p1 = self.lead_parts - 1 if i == 0 else p0
                    for p in range(p0, min(p1, L - 1) + 1):
                        self._copying(st, "part", k, lambda: lnf4.stream_slot_load_part(st, self.head_ids[0], p, L,
                                                                                     self.compute))
                for gi in range(len(GROUPS) if compute and self.recompute else 0):
                    self._group_fwd(layer, gi, base, adapters=True, u_saved=True)   # recompute from the checkpoints
                for gi in reversed(range(len(GROUPS) if compute else 0)):
                    self._group_bwd(layer, gi, base)
        if self.keep_log:
            self.last_log = lnf4.stream_log(st)
        lnf4.stream_reset(st, self.compute)
        if slot and not self.embed_from_host:
            self._embed_in_slot = True

    def rebuffer(self, n_bufs: int):
        """Replace the ring context with one over n_bufs device buffers (same host shards,
        schedule, slot and mode)."""
        torch.cuda.synchronize(self.dev)
        lnf4.stream_destroy(self.st)
        self.st = None
        self.n_bufs = n_bufs
        self.bufs = [torch.empty(self.shard_bytes, dtype=torch.uint8, device=self.dev) for _ in range(n_bufs)]
        sizes = [self.shard_bytes] * self.L + [h.numel() for h in self.all_shards[self.L:]]
        slot_bytes = self.slot.numel() if self.slot is not None else 0
        mode = lnf4.STREAM_REUSE if self.reuse else lnf4.STREAM_RING
        self.st = lnf4.stream_create(self.all_shards, sizes, self.bufs, self.shard_bytes, self.schedule, mode,
                                     self.copy, self.slot, slot_bytes)
        self._embed_in_slot = False
        self._lm_head_in_slot = False

    def log(self):
        return lnf4.stream_log(self.st)

    def use_disk(self, path: str, read_ahead: int = 2, drop_cache: bool = True):
        """Disk tier: write the layer shards to `path` (each at a 4 KiB-aligned offset) and
        stream them from there through `read_ahead` pinned staging buffers; the head
        shards stay in pinned RAM.  With drop_cache the file's pages leave the page cache
        once written and after every read, so each pass reads the device.  Replaces the
        ring context (same schedule and buffers)."""
        torch.cuda.synchronize(self.dev)
        align = 4096
        stride = (self.shard_bytes + align - 1) // align * align
        pad = bytes(stride - self.shard_bytes)
        with open(path, "wb") as f:
            for h in self.host:
                f.write(memoryview(h.numpy()))
                f.write(pad)
            if drop_cache:
                f.flush()
                os.fsync(f.fileno())
                os.posix_fadvise(f.fileno(), 0, 0, os.POSIX_FADV_DONTNEED)
        n = len(self.all_shards)
        offsets = [i * stride for i in range(self.L)] + [0] * (n - self.L)
        self.stage = []
        addrs = []
        for _ in range(read_ahead):
            t = torch.empty(stride + align, dtype=torch.uint8, pin_memory=True)
            self.stage.append(t)
            addrs.append((t.data_ptr() + align - 1) // align * align)
        host = [None] * self.L + list(self.all_shards[self.L:])
        sizes = [self.shard_bytes] * self.L + [h.numel() for h in self.all_shards[self.L:]]
        slot_bytes = self.slot.numel() if self.slot is not None else 0
        st = lnf4.stream_create_disk(path, offsets, addrs, stride, sizes, self.bufs, self.shard_bytes, self.schedule,
                                     self.copy, host_shards=host, drop_cache=drop_cache, slot_buf=self.slot,
                                     slot_bytes=slot_bytes)
        lnf4.stream_destroy(self.st)
        self.st = st
        self.disk_path = path
        self._embed_in_slot = False
        self._lm_head_in_slot = False

    def disk_stats(self):
        """(bytes read from the disk file, seconds in reads) of a disk-tier context."""
        return lnf4.stream_disk_stats(self.st)

    def bytes_copied(self) -> int:
        return lnf4.stream_bytes_copied(self.st)

    def resident_graph(self):
        """The resident step captured as one HIP graph: the same kernel launches, in the same
        order and on the same buffers, recorded once on a capture stream, so a replay costs
        one launch from the host instead of about 40 per layer.  Built on first use, after
        eager resident steps: the resident stream calls issue no stream work once a call
        has seen its layer's one copy complete (see stream_layer_step), so the first eager
        step copies every layer in, and the second, after a device synchronisation, sees
        every copy complete.  A step reads its inputs and writes its outputs in place, so
        every replay gives the eager step's results."""
        if self._graph is None:
            if self.timers is not None or self.wait_events is not None:
                raise RuntimeError("resident_graph: timing instrumentation is on")
            for _ in range(2):
                self.step(resident=True)
                torch.cuda.synchronize(self.dev)
            graph = torch.cuda.CUDAGraph()
            prev = self.compute
            try:
                with torch.cuda.graph(graph, stream=torch.cuda.Stream(self.dev)):
                    self.compute = torch.cuda.current_stream(self.dev)
                    self.step(resident=True)
            finally:
                self.compute = prev
            self._graph = graph
        return self._graph

    def step_graph(self):
        """One resident step by replaying the captured graph on the compute stream."""
        g = self.resident_graph()
        with on_stream(self.compute):
            g.replay()

    def close(self):
        self._graph = None
        if self.st is not None or self.st_res is not None:
            torch.cuda.synchronize(self.dev)
        if self.st is not None:
            lnf4.stream_destroy(self.st)
            self.st = None
        if self.st_res is not None:
            lnf4.stream_destroy(self.st_res)
            self.st_res = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
