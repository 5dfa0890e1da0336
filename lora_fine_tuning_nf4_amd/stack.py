"""A layer-streamed stack of frozen NF4 (or bf16) decoder-layer projections with LoRA,
driven through the lnf4 C ABI.

One step follows the layer-streaming schedule (Soup deep dive, "Core feature: how layer
streaming works"): every layer is read once for the forward and once more for the
backward, where its forward is recomputed from the checkpointed inputs and the input
gradients and adapter gradients are formed; a DPO step first runs the same streamed base
with the adapters off (4 GB-laptop Soup article, "Memory-free reference model").  The
vocab-sized embed_tokens and untied lm_head share one device slot.

Only the linear projections are on this path: the attention core, norms, activations and
the loss head between them are not, so every projection group reads its own synthetic
checkpointed input and every projection its own synthetic output gradient.  All work is
enqueued by C ABI calls; this module only lays out memory and orders the calls.
"""
from __future__ import annotations

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


class StreamedStack:
    def __init__(self, wl: synthgen.Workload, n_bufs: int = 2, seed: int = 0,
                 layers: int | None = None, tokens: int | None = None, head_slot: bool = True,
                 dpo: bool | None = None, device: str = "cuda"):
        self.wl = wl
        self.L = layers if layers is not None else wl.layers
        self.T = tokens if tokens is not None else wl.tokens
        self.fmt = lnf4.FMT_NF4 if wl.fmt == "nf4" else lnf4.FMT_BF16
        self.dpo = ("ref" in wl.passes) if dpo is None else dpo
        self.n_bufs = n_bufs
        self.seed = seed
        dev = torch.device(device)
        self.dev = dev
        T = self.T
        outs = [wl.shapes[p][0] for p in PROJ_ORDER]
        ins = [wl.shapes[p][1] for p in PROJ_ORDER]
        self.offsets, self.shard_bytes = lnf4.lnf4_shard_layout(outs, ins, self.fmt)
        self.compute = torch.cuda.current_stream(dev)
        self.copy = torch.cuda.Stream(dev)

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
            ws = max(ws, lnf4.lora_group_bwd_workspace(self._projs(0, gi, 256, bwd=True), T))
        self.ws_bytes = max(ws, 256)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)

        sched = dpo_schedule(self.L) if self.dpo else sft_schedule(self.L)
        self.schedule = sched
        torch.cuda.synchronize(dev)
        slot_bytes = self.slot.numel() if self.slot is not None else 0
        self.st = lnf4.stream_create(shards, sizes, self.bufs, self.shard_bytes, sched, 0, self.copy, self.slot,
                                     slot_bytes)
        self.timers = None
        self._embed_in_slot = False   # the next step's embed_tokens was loaded during the last backward
        self.st_res = None
        self.res_bufs = None

    def enable_resident(self):
        """A second context over the same host shards with one device buffer per layer:
        every layer is copied once, then steps run with no host-to-device traffic (the same
        kernels, the same addresses pattern): the H2D-removed reference run."""
        if self.st_res is None:
            self.res_bufs = [torch.empty(self.shard_bytes, dtype=torch.uint8, device=self.dev) for _ in range(self.L)]
            self.st_res = lnf4.stream_create(self.host, [self.shard_bytes] * self.L, self.res_bufs, self.shard_bytes,
                                             self.schedule, 1, self.copy)
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
    def _group_fwd(self, layer, gi, base, adapters):
        tm = self.timers
        key = ("fwd", gi, adapters)
        if tm is not None and key in tm:
            tm[key][0].append(torch.cuda.Event(enable_timing=True))
            tm[key][0][-1].record(self.compute)
        lnf4.lora_group_fwd(self._projs(layer, gi, base, adapters=adapters), self.layers[layer].x[gi], self.T,
                            1 if adapters else 0, self.compute)
        if tm is not None and key in tm:
            tm[key][1].append(torch.cuda.Event(enable_timing=True))
            tm[key][1][-1].record(self.compute)

    def _group_bwd(self, layer, gi, base):
        tm = self.timers
        key = ("bwd", gi, True)
        if tm is not None and key in tm:
            tm[key][0].append(torch.cuda.Event(enable_timing=True))
            tm[key][0][-1].record(self.compute)
        lnf4.lora_group_bwd(self._projs(layer, gi, base, bwd=True), self.layers[layer].x[gi], self.T, self.dx[gi],
                            0, self.ws, self.ws_bytes, self.compute)
        if tm is not None and key in tm:
            tm[key][1].append(torch.cuda.Event(enable_timing=True))
            tm[key][1][-1].record(self.compute)

    def step(self, resident: bool = False, compute: bool = True):
        """One training step over the whole stack (all calls asynchronous on the compute stream).
        resident=True runs the same step from the resident context (no layer copies).
        compute=False issues the same stream calls (copies, waits, slot loads) without the
        GEMM calls: the time of the stream schedule alone."""
        L = self.L
        st = self.enable_resident() if resident else self.st
        slot = self.slot is not None and not resident
        if slot:
            if not self._embed_in_slot:   # first step: nothing trickled in yet
                lnf4.stream_slot_load(st, self.head_ids[0], self.compute)   # embed_tokens
            lnf4.stream_slot_wait(st, self.compute)
            self._embed_in_slot = False
        n_fwd = 2 * L if self.dpo else L
        for k, layer in enumerate(self.schedule):
            base = lnf4.stream_layer_step(st, k, self.compute)
            if k < n_fwd:
                ref_pass = self.dpo and k < L
                for gi in range(len(GROUPS) if compute else 0):
                    self._group_fwd(layer, gi, base, adapters=not ref_pass)
                if k == n_fwd - 1 and slot:
                    # the untied lm_head takes the slot for the loss at the forward/backward turn
                    lnf4.stream_slot_load(st, self.head_ids[1], self.compute)
                    lnf4.stream_slot_wait(st, self.compute)
            else:
                if slot:
                    # the backward is compute-bound: the next step's embed_tokens trickles into
                    # the slot in one piece per layer, between the layer copies
                    lnf4.stream_slot_load_part(st, self.head_ids[0], k - n_fwd, L, self.compute)
                for gi in range(len(GROUPS) if compute else 0):   # recompute from the checkpointed inputs
                    self._group_fwd(layer, gi, base, adapters=True)
                for gi in reversed(range(len(GROUPS) if compute else 0)):
                    self._group_bwd(layer, gi, base)
        lnf4.stream_reset(st, self.compute)
        if slot:
            self._embed_in_slot = True

    def log(self):
        return lnf4.stream_log(self.st)

    def bytes_copied(self) -> int:
        return lnf4.stream_bytes_copied(self.st)

    def close(self):
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
