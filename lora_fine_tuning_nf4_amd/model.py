"""A whole layer-streamed decoder model trained with LoRA: embedding, L decoder layers
(RMSNorm, q/k/v with RoPE, causal GQA attention, o, residual, RMSNorm, gate/up, SwiGLU,
down, residual), final RMSNorm, untied lm_head and the token loss, forward and backward,
all through the lnf4 C ABI.

The frozen layer weights stream from pinned host shards through the layer buffers (the
Soup deep dive, "Core feature: how layer streaming works"): each layer is read for the
forward and again in backward, where its forward is recomputed from the checkpointed
layer input (only the layer inputs are kept between the passes) before its gradients are
formed.  A shard holds the seven NF4 (or bf16) projections and the layer's two RMSNorm
weights.  embed_tokens and the lm_head share the head slot; the final norm weight stays
resident.  A DPO step first runs the whole model with the adapters off (the reference
log-prob sums), then the policy forward, the preference loss and the backward.

All arithmetic runs in the library's kernels; this module lays out memory and orders calls.
"""
from __future__ import annotations

import torch

import synthgen
from . import lnf4
from .stack import PROJ_ORDER, StepPacer, dpo_schedule, on_stream, sft_schedule

QKV, O, GU, DOWN = ("q", "k", "v"), ("o",), ("gate", "up"), ("down",)


def _round256(n: int) -> int:
    return (n + 255) // 256 * 256


class StreamedDecoder:
    def __init__(self, wl: synthgen.Workload, n_bufs: int = 2, seed: int = 0, layers: int | None = None,
                 tokens: int | None = None, dpo: bool | None = None, loss_chunk: int | None = None,
                 reuse: bool = False, device: str = "cuda"):
        arch = wl.extra.get("arch")
        if arch is None or wl.vocab <= 0:
            raise ValueError(f"workload {wl.name} has no decoder architecture or vocabulary")
        self.wl, self.arch = wl, arch
        self.L = layers if layers is not None else wl.layers
        self.T = T = tokens if tokens is not None else wl.tokens
        self.H = H = wl.hidden
        self.nh, self.nkv, self.D = arch["n_heads"], arch["n_kv"], arch["head_dim"]
        self.S = arch["seq_len"]
        self.eps = float(arch["eps"])
        self.fmt = lnf4.FMT_NF4 if wl.fmt == "nf4" else lnf4.FMT_BF16
        self.dpo = ("ref" in wl.passes) if dpo is None else dpo
        self.seed, self.n_bufs = seed, n_bufs
        dev = self.dev = torch.device(device)
        self.compute = lnf4.stream_compute_stream(dev)   # a hardware queue of its own
        self.pacer = StepPacer()   # streamed steps wait for the previous streamed step
        # head-slot schedule, as in StreamedStack: lm_head loaded after forward call
        # lm_head_call, lead_parts embedding parts at the first backward call
        self.lm_head_call = self.L - 2 if self.L >= 2 else self.L - 1
        self.lead_parts = min(3, self.L)
        self.copy = lnf4.stream_copy_stream(dev)   # a hardware queue of its own
        bf16, f32 = torch.bfloat16, torch.float32
        if T % self.S:
            raise ValueError(f"T={T} is not a whole number of sequences of {self.S}")

        # ---- shard layout: the projections, then the two norm weights
        outs = [wl.shapes[p][0] for p in PROJ_ORDER]
        ins = [wl.shapes[p][1] for p in PROJ_ORDER]
        self.offsets, proj_bytes = lnf4.lnf4_shard_layout(outs, ins, self.fmt)
        self.g1_off = _round256(proj_bytes)
        self.g2_off = self.g1_off + _round256(2 * H)
        self.shard_bytes = self.g2_off + _round256(2 * H)
        self.host = []
        stage = torch.zeros(self.shard_bytes, dtype=torch.uint8, device=dev)
        for layer in range(self.L):
            self._fill_shard(stage, layer)
            h = torch.empty(self.shard_bytes, dtype=torch.uint8, pin_memory=True)
            h.copy_(stage)
            self.host.append(h)
        del stage
        self.bufs = [torch.empty(self.shard_bytes, dtype=torch.uint8, device=dev) for _ in range(n_bufs)]

        # ---- head slot, resident final norm, token ids and labels
        V = wl.vocab
        nbytes = V * H * 2
        shards, sizes = list(self.host), [self.shard_bytes] * self.L
        self.head_ids = []
        for name in ("embed", "lm_head"):
            t = synthgen.device_normal((V, H), 0.02, seed, "head", name, dtype=bf16)
            hb = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
            hb.copy_(t.view(torch.uint8).reshape(-1))
            del t
            self.head_ids.append(len(shards))
            shards.append(hb)
            sizes.append(nbytes)
        self.all_shards = shards
        self.slot = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.g_final = (synthgen.device_normal((H,), 0.1, seed, "norm_f") + 1.0).to(bf16)
        self.ids = synthgen.device_token_ids(T, V, seed, "ids")
        self.labels = synthgen.device_token_ids(T, V, seed, "labels")
        self.rope = torch.empty(self.S * self.D, dtype=f32, device=dev)
        lnf4.lnf4_rope_table(self.S, self.D, float(arch["rope_base"]), self.rope, self.compute)

        # ---- adapters and their gradients (per layer), saved rank-r activations
        r = wl.rank
        self.A, self.B, self.dA, self.dB, self.u = [], [], [], [], []
        for layer in range(self.L):
            A, B, dA, dB, u = {}, {}, {}, {}, {}
            for p in wl.adapted:
                o_, i_ = wl.shapes[p]
                A[p] = synthgen.device_uniform((r, i_), 1.0 / i_ ** 0.5, seed, "A", layer, p, dtype=bf16)
                B[p] = synthgen.device_normal((o_, r), 0.01, seed, "B", layer, p, dtype=bf16)
                dA[p] = torch.zeros((r, i_), dtype=f32, device=dev)
                dB[p] = torch.zeros((o_, r), dtype=f32, device=dev)
                u[p] = torch.zeros((T, r), dtype=f32, device=dev)
            for lst, val in ((self.A, A), (self.B, B), (self.dA, dA), (self.dB, dB), (self.u, u)):
                lst.append(val)

        # ---- activations: layer-input checkpoints and one layer's working set
        E = lambda *shape: torch.empty(shape, dtype=bf16, device=dev)
        nq, nk, I = self.nh * self.D, self.nkv * self.D, wl.shapes["gate"][0]
        self.xs = [E(T, H) for _ in range(self.L + 1)]
        self.a, self.q, self.k, self.v, self.o = E(T, H), E(T, nq), E(T, nk), E(T, nk), E(T, nq)
        self.po, self.h, self.m, self.dn = E(T, H), E(T, H), E(T, H), E(T, H)
        self.g, self.up, self.s = E(T, I), E(T, I), E(T, I)
        self.lse = torch.empty(self.nh * T, dtype=f32, device=dev)
        self.rstd1, self.rstd2, self.rstd_f = (torch.empty(T, dtype=f32, device=dev) for _ in range(3))
        self.ds, self.dg, self.dup = E(T, I), E(T, I), E(T, I)
        self.dm, self.dh, self.da, self.do = E(T, H), E(T, H), E(T, H), E(T, nq)
        self.dq, self.dk, self.dv = E(T, nq), E(T, nk), E(T, nk)
        self.dx = [E(T, H), E(T, H)]
        self.attn_ws_bytes = lnf4.lnf4_attn_bwd_workspace(T, self.nh, self.nkv, self.D)
        self.attn_ws = torch.empty(self.attn_ws_bytes, dtype=torch.uint8, device=dev)
        self.hN, self.dhN = E(T, H), E(T, H)
        self.logp = torch.empty(T, dtype=f32, device=dev)
        chunk = T if not loss_chunk else min(int(loss_chunk), T)
        if self.dpo:
            self.seq_len = int(wl.extra.get("seq_len", T // 4))
            self.beta = float(wl.extra.get("beta", 0.1))
            self.n_seq = T // self.seq_len
            chunk = max(self.seq_len, chunk // self.seq_len * self.seq_len)
            self.ref_logp = torch.empty(T, dtype=f32, device=dev)
            self.ref_sums, self.pol_sums, self.coef = (torch.empty(self.n_seq, dtype=f32, device=dev)
                                                       for _ in range(3))
            self.loss = torch.empty(1, dtype=f32, device=dev)
        self.chunk = chunk
        self.logits = E(chunk, V)
        self.head_ws_bytes = max(256, lnf4.lora_linear_bwd_workspace(chunk, V, H, 0))
        self.head_ws = torch.empty(self.head_ws_bytes, dtype=torch.uint8, device=dev)
        ws = 256
        for grp in (QKV, O, GU, DOWN):
            ws = max(ws, lnf4.lora_group_bwd_workspace(self._projs(0, grp, 256, bwd=True), T),
                     lnf4.lora_group_fwd_workspace(self._projs(0, grp, 256), T))
        self.ws_bytes = ws
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev)

        self.schedule = dpo_schedule(self.L) if self.dpo else sft_schedule(self.L)
        torch.cuda.synchronize(dev)
        self.st = lnf4.stream_create(shards, sizes, self.bufs, self.shard_bytes, self.schedule,
                                     lnf4.STREAM_REUSE if reuse else lnf4.STREAM_RING, self.copy, self.slot, nbytes)
        self.st_res = None
        self.res_bufs = None
        self.res_head = None
        self._embed_in_slot = False

    # ------------------------------------------------------------------ set-up
    def _fill_shard(self, stage, layer):
        wl = self.wl
        for pi, p in enumerate(PROJ_ORDER):
            o_, i_ = wl.shapes[p]
            w = synthgen.device_normal((o_, i_), 0.02, self.seed, "W", layer, p)
            d0, a0 = self.offsets[2 * pi], self.offsets[2 * pi + 1]
            if self.fmt == lnf4.FMT_NF4:
                lnf4.nf4_quantize(w, o_ * i_, 64, stage[d0:d0 + o_ * i_ // 2],
                                  stage[a0:a0 + (o_ * i_ // 64) * 4].view(torch.float32))
            else:
                stage[d0:d0 + o_ * i_ * 2].view(torch.bfloat16).copy_(w.to(torch.bfloat16).reshape(-1))
            del w
        for off, name in ((self.g1_off, "norm1"), (self.g2_off, "norm2")):
            g = (synthgen.device_normal((self.H,), 0.1, self.seed, name, layer) + 1.0).to(torch.bfloat16)
            stage[off:off + 2 * self.H].view(torch.bfloat16).copy_(g)
        torch.cuda.synchronize(self.dev)

    def enable_resident(self):
        """A resident context over the same shards (every layer in a buffer of its own,
        copied once) and the head matrices in buffers of their own: the H2D-removed run."""
        if self.st_res is None:
            self.res_bufs = [torch.empty(self.shard_bytes, dtype=torch.uint8, device=self.dev) for _ in range(self.L)]
            self.st_res = lnf4.stream_create(self.host, [self.shard_bytes] * self.L, self.res_bufs, self.shard_bytes,
                                             self.schedule, lnf4.STREAM_RESIDENT, self.copy)
            self.res_head = []
            for sid in self.head_ids:
                h = self.all_shards[sid]
                d = torch.empty(h.numel(), dtype=torch.uint8, device=self.dev)
                d.copy_(h)
                self.res_head.append(d)
            torch.cuda.synchronize(self.dev)
        return self.st_res

    def _weight(self, base: int, p: str):
        pi = PROJ_ORDER.index(p)
        o_, i_ = self.wl.shapes[p]
        d0, a0 = self.offsets[2 * pi], self.offsets[2 * pi + 1]
        return lnf4.make_weight(self.fmt, base + d0, (base + a0) if self.fmt == lnf4.FMT_NF4 else None, o_, i_, 64)

    def _projs(self, layer, group, base, adapters=True, bwd=False, ys=None, dys=None):
        wl = self.wl
        out = []
        for j, p in enumerate(group):
            on = adapters and p in wl.adapted
            out.append(lnf4.make_proj(
                self._weight(base, p), A=self.A[layer][p] if on else None, B=self.B[layer][p] if on else None,
                r=wl.rank if on else 0, scale=wl.scale if on else 0.0, y=ys[j] if ys else None,
                u=self.u[layer][p] if on else None, dy=dys[j] if dys else None,
                dA=self.dA[layer][p] if (bwd and on) else None, dB=self.dB[layer][p] if (bwd and on) else None))
        return out

    # ------------------------------------------------------------------ one layer
    def _layer_fwd(self, layer, base, x_in, x_out, adapters=True, u_saved=False):
        """u_saved: the recompute of a layer whose forward already wrote every u = x A^T from
        the same checkpointed input (the calls read them instead of recomputing them)."""
        T, H, cs = self.T, self.H, self.compute
        on = (2 if u_saved else 1) if adapters else 0
        lnf4.lnf4_rmsnorm_fwd(x_in, T, H, base + self.g1_off, self.eps, self.a, self.rstd1, cs)
        lnf4.lora_group_fwd_ws(self._projs(layer, QKV, base, adapters, ys=(self.q, self.k, self.v)), self.a, T, on,
                               self.ws, self.ws_bytes, cs)
        lnf4.lnf4_rope(self.q, T, self.nh, self.D, self.S, self.rope, 0, cs)
        lnf4.lnf4_rope(self.k, T, self.nkv, self.D, self.S, self.rope, 0, cs)
        lnf4.lnf4_attn_fwd(self.q, self.k, self.v, T, self.nh, self.nkv, self.D, self.S, self.o, self.lse, cs)
        lnf4.lora_group_fwd_ws(self._projs(layer, O, base, adapters, ys=(self.po,)), self.o, T, on,
                               self.ws, self.ws_bytes, cs)
        lnf4.lnf4_add(x_in, self.po, T * H, self.h, cs)
        lnf4.lnf4_rmsnorm_fwd(self.h, T, H, base + self.g2_off, self.eps, self.m, self.rstd2, cs)
        lnf4.lora_group_fwd_ws(self._projs(layer, GU, base, adapters, ys=(self.g, self.up)), self.m, T, on,
                               self.ws, self.ws_bytes, cs)
        lnf4.lnf4_swiglu_fwd(self.g, self.up, self.g.numel(), self.s, cs)
        lnf4.lora_group_fwd_ws(self._projs(layer, DOWN, base, adapters, ys=(self.dn,)), self.s, T, on,
                               self.ws, self.ws_bytes, cs)
        if x_out is not None:
            lnf4.lnf4_add(self.h, self.dn, T * H, x_out, cs)

    def _layer_bwd(self, layer, base, x_in, dout, dx_out):
        """Recompute the layer from its checkpointed input, then its backward."""
        T, H, cs = self.T, self.H, self.compute
        self._layer_fwd(layer, base, x_in, None, True, u_saved=True)
        gb = lambda grp, x, dys, dx: lnf4.lora_group_bwd(self._projs(layer, grp, base, True, True, dys=dys), x, T, dx,
                                                          0, self.ws, self.ws_bytes, cs)
        gb(DOWN, self.s, (dout,), self.ds)
        lnf4.lnf4_swiglu_bwd(self.g, self.up, self.ds, self.g.numel(), self.dg, self.dup, cs)
        gb(GU, self.m, (self.dg, self.dup), self.dm)
        lnf4.lnf4_rmsnorm_bwd(self.h, T, H, base + self.g2_off, self.rstd2, self.dm, dout, self.dh, cs)
        gb(O, self.o, (self.dh,), self.do)
        lnf4.lnf4_attn_bwd(self.q, self.k, self.v, self.o, self.lse, self.do, T, self.nh, self.nkv, self.D, self.S,
                           self.dq, self.dk, self.dv, self.attn_ws, self.attn_ws_bytes, cs)
        lnf4.lnf4_rope(self.dq, T, self.nh, self.D, self.S, self.rope, 1, cs)
        lnf4.lnf4_rope(self.dk, T, self.nkv, self.D, self.S, self.rope, 1, cs)
        gb(QKV, self.a, (self.dq, self.dk, self.dv), self.da)
        lnf4.lnf4_rmsnorm_bwd(x_in, T, H, base + self.g1_off, self.rstd1, self.da, self.dh, dx_out, cs)

    # ------------------------------------------------------------------ output side
    def _lm(self, ptr):
        return lnf4.make_weight(lnf4.FMT_BF16, ptr, None, self.wl.vocab, self.H, 64)

    def _chunks(self):
        return [(c0, min(self.chunk, self.T - c0)) for c0 in range(0, self.T, self.chunk)]

    def _final_norm(self, x_last):
        lnf4.lnf4_rmsnorm_fwd(x_last, self.T, self.H, self.g_final, self.eps, self.hN, self.rstd_f, self.compute)

    def _logits(self, W, c0, n):
        lnf4.lora_linear_fwd(W, self.hN[c0:c0 + n], n, None, None, 0, 0.0, self.logits, None, self.compute)

    def _head_dx(self, W, c0, n):
        lnf4.lora_linear_bwd(W, self.hN[c0:c0 + n], self.logits, n, None, None, 0, 0.0, None, self.dhN[c0:c0 + n],
                             None, None, 0, self.head_ws, self.head_ws_bytes, self.compute)

    def _head_sft(self, ptr):
        W, V, cs = self._lm(ptr), self.wl.vocab, self.compute
        for c0, n in self._chunks():
            self._logits(W, c0, n)
            lnf4.lnf4_cross_entropy(self.logits, n, V, self.labels[c0:], 1.0 / self.T, None, 1, self.logp[c0:],
                                    self.logits, cs)
            self._head_dx(W, c0, n)

    def _head_ref(self, ptr):
        W, V, cs = self._lm(ptr), self.wl.vocab, self.compute
        for c0, n in self._chunks():
            self._logits(W, c0, n)
            lnf4.lnf4_cross_entropy(self.logits, n, V, self.labels[c0:], 1.0, None, 1, self.ref_logp[c0:], None, cs)
        lnf4.lnf4_sequence_sums(self.ref_logp, self.n_seq, self.seq_len, self.ref_sums, cs)

    def _head_dpo(self, ptr):
        W, V, S, cs = self._lm(ptr), self.wl.vocab, self.seq_len, self.compute
        chunks = self._chunks()
        for c0, n in chunks:
            self._logits(W, c0, n)
            lnf4.lnf4_cross_entropy(self.logits, n, V, self.labels[c0:], 1.0, None, 1, self.logp[c0:], None, cs)
        lnf4.lnf4_sequence_sums(self.logp, self.n_seq, S, self.pol_sums, cs)
        lnf4.lnf4_dpo_loss(self.pol_sums, self.ref_sums, self.n_seq // 2, self.beta, self.loss, self.coef, cs)
        for c0, n in chunks:
            if len(chunks) > 1:
                self._logits(W, c0, n)
            lnf4.lnf4_cross_entropy(self.logits, n, V, self.labels[c0:], -1.0, self.coef[c0 // S:], S, None,
                                    self.logits, cs)
            self._head_dx(W, c0, n)

    # ------------------------------------------------------------------ one step
    def step(self, resident: bool = False):
        """One training step of the decoder (asynchronous on the compute stream, ordered after
        the caller's stream's earlier work; the caller's later work waits for it).  A streamed
        step waits on the host, after its first layer call, for the previous streamed step to
        finish (StepPacer)."""
        pace = not resident and self.pacer is not None
        with on_stream(self.compute):
            self._step(resident, pace)
            if pace:
                self.pacer.mark(self.compute)

    def _step(self, resident: bool, pace: bool = False):
        L, cs = self.L, self.compute
        st = self.enable_resident() if resident else self.st
        if not resident:
            if not self._embed_in_slot:
                lnf4.stream_slot_load(st, self.head_ids[0], cs)
            emb = lnf4.stream_slot_wait(st, cs)
            self._embed_in_slot = False
        else:
            emb = self.res_head[0]
        lnf4.lnf4_embed_gather(emb, self.wl.vocab, self.H, self.ids, self.T, self.xs[0], cs)
        n_fwd = 2 * L if self.dpo else L
        ref_x = [self.dx[0], self.dx[1]]  # the reference pass keeps no checkpoints
        dout_i = 0
        for k, layer in enumerate(self.schedule):
            base = lnf4.stream_layer_step(st, k, cs)
            if pace and k == 0:
                self.pacer.wait()
            if k == L or k == n_fwd:
                # the output head of the forward pass that just ended (after this call's
                # stream step, so the next layer copy overlaps it)
                ptr = lnf4.stream_slot_wait(st, cs) if not resident else self.res_head[1]
                if self.dpo and k == L:
                    self._final_norm(ref_x[(L - 1) % 2])
                    self._head_ref(ptr)
                else:
                    self._final_norm(self.xs[L])
                    self._head_dpo(ptr) if self.dpo else self._head_sft(ptr)
                    lnf4.lnf4_rmsnorm_bwd(self.xs[L], self.T, self.H, self.g_final, self.rstd_f, self.dhN, None,
                                          self.dx[0], cs)
                    dout_i = 0
            if k < n_fwd:
                if self.dpo and k < L:   # reference pass, adapters off
                    x_in = self.xs[0] if layer == 0 else ref_x[(layer - 1) % 2]
                    self._layer_fwd(layer, base, x_in, ref_x[layer % 2], adapters=False)
                else:
                    self._layer_fwd(layer, base, self.xs[layer], self.xs[layer + 1], adapters=True)
                if k == self.lm_head_call and not resident:
                    lnf4.stream_slot_load(st, self.head_ids[1], cs)   # lm_head takes the slot
            else:
                if not resident:
                    i = k - n_fwd
                    p0 = 0 if i == 0 else self.lead_parts + i - 1
                    p1 = self.lead_parts - 1 if i == 0 else p0
                    for p in range(p0, min(p1, L - 1) + 1):
                        lnf4.stream_slot_load_part(st, self.head_ids[0], p, L, cs)
                self._layer_bwd(layer, base, self.xs[layer], self.dx[dout_i], self.dx[1 - dout_i])
                dout_i = 1 - dout_i
        lnf4.stream_reset(st, cs)
        if not resident:
            self._embed_in_slot = True
        self.dx0 = self.dx[dout_i]   # gradient at the embedding output

    def bytes_copied(self) -> int:
        return lnf4.stream_bytes_copied(self.st)

    def close(self):
        torch.cuda.synchronize(self.dev)
        for st in (self.st, self.st_res):
            if st is not None:
                lnf4.stream_destroy(st)
        self.st = self.st_res = None

    def __del__(self):
        try:
            if self.st is not None or self.st_res is not None:
                self.close()
        except Exception:
            pass
