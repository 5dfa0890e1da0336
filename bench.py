#!/usr/bin/env python3
"""Train tokens/s of the layer-streamed NF4 + LoRA stack on one MI355X.

One step = one pass of the whole hot path over one batch: the embed slot copy and the
embedding lookup, the forward of every layer (fused NF4 decode + MFMA GEMMs + rank-r
LoRA terms, streamed from pinned host shards through 2 device layer buffers), the
lm_head slot copy, the untied lm_head GEMM, token cross-entropy and lm_head input
gradient, and the backward of every layer in reverse (second read of the layer, forward
recompute, input gradients, adapter gradients).  Default workload: the Llama-3.1-8B-shaped stack (32
layers of q, k, v, o, gate, up, down NF4 projections, LoRA r=8 alpha=32 on q and v,
batch 1 x seq 2048), synthetic seeded weights and activations already resident in device
memory / pinned host memory when the timed region starts.

Prints one JSON line.  Everything else goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0
CSRC = os.path.join(ROOT, "lora_fine_tuning_nf4_amd", "csrc")
# sources the forward GEMM kernel is compiled from: a counter summary taken on other sources
# no longer describes the kernel that runs
FWD_KERNEL_SOURCES = ("gemm.hip", "common.hpp", "kernels.hpp", "nf4_table.hpp")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "k_fwd_nf4_gate_up_llama8b_T2048.traffic.txt")
CAL_ELEMS = 64 << 20        # float32 elements of the calibration copy (256 MiB read + 256 MiB written)
# the dominant launch (gate|up forward at the 8B shape, T = 2048) and the input-gradient
# launch of the same group, as rocprofv3 names them: kernel symbol and grid in threads
DOM_KERNEL = "k_fwd_nf4<256, 4>"
DOM_GRID = (768 + 256) * 256        # 768 tiles of 256 x 256 and 256 tiles of 128 x 256
DX_KERNEL = "k_dxq<256>"
DX_GRID = 128 * 2 * 256             # 128 tiles of 256 x 256, K in 2 splits


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_flops(wl, group, kind):
    """Algorithmic flops of one grouped GEMM launch (2 M N K)."""
    T = wl.tokens
    outs = [wl.shapes[p][0] for p in group]
    in_f = wl.shapes[group[0]][1]
    return 2.0 * T * sum(outs) * in_f


def fwd_bytes(wl, group):
    """Algorithmic HBM bytes of one grouped NF4 forward launch: x read once, codes and absmax
    read once, y written once (bf16), plus the adapters' B and u when adapted."""
    T = wl.tokens
    in_f = wl.shapes[group[0]][1]
    b = 2 * T * in_f
    for p in group:
        o = wl.shapes[p][0]
        b += o * in_f // 2 + 4 * (o * in_f // 64) + 2 * T * o
        if p in wl.adapted:
            b += 2 * o * wl.rank + 4 * T * wl.rank
    return b


def dx_bytes(wl, group):
    """Algorithmic HBM bytes of one grouped NF4 input-gradient launch: each projection's dy
    and codes + absmax read once, dx written once (bf16), plus v and A when adapted."""
    T = wl.tokens
    in_f = wl.shapes[group[0]][1]
    b = 2 * T * in_f
    for p in group:
        o = wl.shapes[p][0]
        b += 2 * T * o + o * in_f // 2 + 4 * (o * in_f // 64)
        if p in wl.adapted:
            b += 2 * wl.rank * in_f + 4 * T * wl.rank
    return b


def workload(name):
    import synthgen
    return synthgen.WORKLOADS[name]


def head_summary(wl, stack, head_ms):
    """Time of the output side at the forward/backward turn (lm_head GEMMs + cross-entropy
    [+ sequence sums and DPO loss]) and the rate of its two GEMMs."""
    if not stack.head:
        return None
    T, V, H = stack.T, wl.vocab, wl.hidden
    n_chunks = -(-T // stack.chunk)
    out = {"loss_chunk_tokens": stack.chunk, "chunks": n_chunks}
    for part, ms in head_ms.items():
        gemms = 2 if part in ("sft", "pol") else 1                # logits, and dh where there is a gradient
        if part == "pol" and n_chunks > 1:
            gemms += 1                                            # logits again for the gradient pass
        flops = gemms * 2.0 * T * V * H
        out[f"{part}_ms"] = round(ms, 4)
        out[f"{part}_gemm_tflops_incl_loss"] = round(flops / (ms / 1000.0) / 1e12, 2)
    return out


def library_bf16_same_shape(M: int, N: int, K: int, reps: int = 20):
    """Context for the dominant kernel's fraction of peak: torch's bf16 GEMM (hipBLASLt) on
    plain bf16 weights of the same shape, y = x W^T, timed with events on this GPU.  It does
    no NF4 decode and no LoRA term; it is reported beside the roofline, not used by the path."""
    import torch
    import torch.nn.functional as F
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    for _ in range(3):
        F.linear(x, w)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        F.linear(x, w)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tflops = 2.0 * M * N * K / (ms / 1000.0) / 1e12
    del x, w
    return {"what": "torch.nn.functional.linear in bf16 (hipBLASLt), plain bf16 weights, no decode, no LoRA",
            "M": M, "N": N, "K": K, "ms": round(ms, 4), "tflops": round(tflops, 2),
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in FWD_KERNEL_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the gate|up forward kernel, from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary; None when that summary is missing or was taken on
    other kernel sources."""
    try:
        kv = {}
        with open(TRAFFIC_PROFILE) as fh:
            for line in fh:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None, "stale (kernel sources changed since the counters were taken)"
        return int(float(kv["traffic_bytes_per_launch"])), os.path.relpath(TRAFFIC_PROFILE, ROOT)
    except (OSError, KeyError, ValueError):
        return None, "no counter summary"


def _oracle_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def _oracle_layer_time(wl, seed: int):
    """The oracle, as it stands, on one layer-step of a workload: NF4 decode of the seven
    projections once per read of the layer (2 reads for SFT, 3 with the DPO reference pass;
    none for bf16 weights), then the layer step (fwd, recompute, bwd [+ adapter-off fwd])
    at the workload's T.  Returns (seconds, detail)."""
    import synthgen
    from oracle import layer as olayer
    from oracle import nf4 as onf4

    T = wl.tokens
    dpo = "ref" in wl.passes
    codes, absmax, wbf = {}, {}, {}
    for p in synthgen.PROJ_ORDER:
        o, i = wl.shapes[p]
        w = synthgen.weight_f32(o, i, seed, "cpu", p)
        if wl.fmt == "nf4":
            codes[p], absmax[p] = onf4.quantize(w)
        else:
            wbf[p] = onf4.bf16_bits_to_f64(synthgen.to_bf16_bits(w))
    xs = {gi: onf4.bf16_bits_to_f64(synthgen.act_bits(T, wl.shapes[g[0]][1], seed, "cpu-x", gi))
          for gi, g in enumerate(synthgen.GROUPS)}
    dys = {p: onf4.bf16_bits_to_f64(synthgen.act_bits(T, wl.shapes[p][0], seed, "cpu-dy", p))
           for p in synthgen.PROJ_ORDER}
    ad = {}
    for p in wl.adapted:
        o, i = wl.shapes[p]
        ad[p] = (onf4.bf16_bits_to_f64(synthgen.adapter_a_bits(wl.rank, i, seed, "cpu", p)),
                 onf4.bf16_bits_to_f64(synthgen.adapter_b_bits(o, wl.rank, seed, "cpu", p)), wl.scale)
    reads = 3 if dpo else 2
    t0 = time.perf_counter()
    Wd = ({p: onf4.decode_f64(codes[p], absmax[p]) for p in synthgen.PROJ_ORDER} if wl.fmt == "nf4" else wbf)
    t1 = time.perf_counter()
    olayer.layer_step(Wd, ad, xs, dys, dpo=dpo)
    t2 = time.perf_counter()
    dec = (t1 - t0) if wl.fmt == "nf4" else 0.0
    secs = reads * dec + (t2 - t1)
    return secs, {"decode_s": round(dec, 3), "decodes_per_layer_step": reads if wl.fmt == "nf4" else 0,
                  "layer_step_s": round(t2 - t1, 3)}


def _oracle_linear_time(wl, seed: int):
    """The oracle on the single-linear workload in full: one NF4 decode, forward, backward."""
    import synthgen
    from oracle import lora as olora
    from oracle import nf4 as onf4

    (o, i), = wl.shapes.values()
    T = wl.tokens
    codes, absmax = onf4.quantize(synthgen.weight_f32(o, i, seed, "cpu-lin"))
    x = onf4.bf16_bits_to_f64(synthgen.act_bits(T, i, seed, "cpu-lin", "x"))
    dy = onf4.bf16_bits_to_f64(synthgen.act_bits(T, o, seed, "cpu-lin", "dy"))
    A = onf4.bf16_bits_to_f64(synthgen.adapter_a_bits(wl.rank, i, seed, "cpu-lin"))
    B = onf4.bf16_bits_to_f64(synthgen.adapter_b_bits(o, wl.rank, seed, "cpu-lin"))
    t0 = time.perf_counter()
    Wd = onf4.decode_f64(codes, absmax)
    olora.linear_fwd(x, Wd, A, B, wl.scale)
    olora.linear_bwd(x, dy, Wd, A, B, wl.scale)
    return time.perf_counter() - t0


def cpu_baseline(wl, seed: int, layers: int):
    """The oracle, as it stands (fp64 numpy, never tuned for speed), timed on the host cores.

    The reported value is the benchmark's own workload: one layer-step at its T, scaled
    to the stack (tokens per second of a step of `layers` layer-steps; the output side is
    not included).  Beside it, per configuration: the single linear in full (fwd + bwd) on
    one thread and on all threads, one Qwen2.5-0.5B layer-step on one thread and on all
    threads, and one layer-step of the Qwen2.5-3B bf16 and the 8B DPO workloads on all
    threads, each at its real T."""
    import synthgen
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    cores = _oracle_threads()
    per = {}

    def one_thread(fn):
        if threadpool_limits is None:
            return None
        with threadpool_limits(limits=1):
            return fn()

    lin = synthgen.WORKLOADS["linear896"]
    t_all = _oracle_linear_time(lin, seed)
    t_one = one_thread(lambda: _oracle_linear_time(lin, seed))
    per["linear896"] = {"what": "one NF4 decode + fwd + bwd of the 896x896 linear, T=256",
                        "seconds": {"all_threads": round(t_all, 4), "one_thread": None if t_one is None else round(t_one, 4)},
                        "tokens_per_s": {"all_threads": round(lin.tokens / t_all, 1),
                                         "one_thread": None if t_one is None else round(lin.tokens / t_one, 1)}}
    for name, single in (("qwen05b", True), (wl.name, False), ("qwen3b_bf16", False), ("llama8b_dpo", False)):
        if name in per:
            continue
        w = synthgen.WORKLOADS[name]
        s_all, det = _oracle_layer_time(w, seed)
        rec = {"what": f"one {name} layer-step at T={w.tokens}", "seconds": {"all_threads": round(s_all, 3)},
               "tokens_per_s_layer": {"all_threads": round(w.tokens / s_all, 2)},
               "tokens_per_s_stack": {"all_threads": round(w.tokens / (w.layers * s_all), 3)}, **det}
        if single:
            s_one, _ = one_thread(lambda: _oracle_layer_time(w, seed)) or (None, None)
            rec["seconds"]["one_thread"] = None if s_one is None else round(s_one, 3)
            rec["tokens_per_s_layer"]["one_thread"] = None if s_one is None else round(w.tokens / s_one, 2)
        per[name] = rec
        log(f"cpu baseline {name}: {rec}")
    main = per[wl.name] if wl.name in per else None
    if main is None:   # the single linear as the benchmark workload
        value = per["linear896"]["tokens_per_s"]["all_threads"]
        sample = per["linear896"]["what"]
        secs = per["linear896"]["seconds"]["all_threads"]
    else:
        secs = main["seconds"]["all_threads"]
        value = wl.tokens / (layers * secs)
        sample = (f"one {wl.name} layer at T={wl.tokens}: NF4 decode of the 7 projections once per read of the "
                  f"layer + oracle layer step fwd/recompute/bwd; stack step = {layers} x layer (output side not "
                  f"included)")
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle", "sample": sample,
            "seconds_per_layer_step": secs, "per_config": per}


def dequant_share(wl, seed: int, reps: int = 10):
    """Fused NF4 GEMMs against the unfused path (nf4_dequant of the layer to bf16, then the
    same GEMMs on bf16 weights) for one resident layer step (forward + recompute + backward)."""
    import torch
    import synthgen
    from lora_fine_tuning_nf4_amd import lnf4
    from lora_fine_tuning_nf4_amd.stack import GROUPS

    T = wl.tokens
    dev = "cuda"
    groups = []
    for g in GROUPS:
        in_f = wl.shapes[g[0]][1]
        x = synthgen.device_normal((T, in_f), 1.0, seed, "ds-x", *g, dtype=torch.bfloat16)
        ent = {"x": x, "dx": torch.empty(T, in_f, dtype=torch.bfloat16, device=dev), "p": []}
        for p in g:
            o, i = wl.shapes[p]
            w = synthgen.device_normal((o, i), 0.02, seed, "ds-w", p)
            codes = torch.empty(o * i // 2, dtype=torch.uint8, device=dev)
            am = torch.empty(o * i // 64, dtype=torch.float32, device=dev)
            lnf4.nf4_quantize(w, o * i, 64, codes, am)
            del w
            on = p in wl.adapted
            d = {"codes": codes, "am": am, "o": o, "i": i, "on": on,
                 "wbf": torch.empty(o * i, dtype=torch.bfloat16, device=dev),
                 "y": torch.empty(T, o, dtype=torch.bfloat16, device=dev),
                 "dy": synthgen.device_normal((T, o), 1.0, seed, "ds-dy", p, dtype=torch.bfloat16)}
            if on:
                d["A"] = synthgen.device_uniform((wl.rank, i), 1.0 / i ** 0.5, seed, "ds-A", p, dtype=torch.bfloat16)
                d["B"] = synthgen.device_normal((o, wl.rank), 0.01, seed, "ds-B", p, dtype=torch.bfloat16)
                d["u"] = torch.empty(T, wl.rank, device=dev)
                d["dA"] = torch.empty(wl.rank, i, device=dev)
                d["dB"] = torch.empty(o, wl.rank, device=dev)
            ent["p"].append(d)
        groups.append(ent)

    def projs(ent, fmt):
        out = []
        for d in ent["p"]:
            W = (lnf4.make_weight(lnf4.FMT_NF4, d["codes"], d["am"], d["o"], d["i"]) if fmt == lnf4.FMT_NF4
                 else lnf4.make_weight(lnf4.FMT_BF16, d["wbf"], None, d["o"], d["i"]))
            on = d["on"]
            out.append(lnf4.make_proj(W, A=d.get("A"), B=d.get("B"), r=wl.rank if on else 0,
                                      scale=wl.scale if on else 0.0, y=d["y"], u=d.get("u"), dy=d["dy"],
                                      dA=d.get("dA"), dB=d.get("dB")))
        return out

    ws_bytes = max(lnf4.lora_group_bwd_workspace(projs(e, lnf4.FMT_NF4), T) for e in groups)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def gemms(fmt):
        for e in groups:                      # forward
            lnf4.lora_group_fwd(projs(e, fmt), e["x"], T, 1)
        for e in groups:                      # recompute
            lnf4.lora_group_fwd(projs(e, fmt), e["x"], T, 1)
        for e in reversed(groups):            # backward
            lnf4.lora_group_bwd(projs(e, fmt), e["x"], T, e["dx"], 0, ws, ws_bytes)

    def dequant():
        for e in groups:
            for d in e["p"]:
                lnf4.nf4_dequant(d["codes"], d["am"], d["o"] * d["i"], 64, d["wbf"])

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    fused = timed(lambda: gemms(lnf4.FMT_NF4))
    dq = timed(dequant)
    bf = timed(lambda: gemms(lnf4.FMT_BF16))
    # the unfused path decodes the layer once per read: twice per layer step
    unfused = 2 * dq + bf
    return {"layer_step_fused_ms": round(fused, 4), "dequant_layer_ms": round(dq, 4),
            "layer_step_bf16_gemms_ms": round(bf, 4), "layer_step_unfused_ms": round(unfused, 4),
            "dequant_share_of_unfused": round(2 * dq / unfused, 4),
            "fused_speedup_over_unfused": round(unfused / fused, 3),
            "dequant_GBps": round(sum(d["o"] * d["i"] for e in groups for d in e["p"]) * 2.5625 / (dq / 1000) / 1e9, 1)}


def t_sweep(wl, seed: int, nbuf: int, steps: int, tokens=(2048, 4096, 8192)):
    """Streamed and resident stack step at several batch sizes (where copy stops dominating)."""
    import torch
    from lora_fine_tuning_nf4_amd.stack import StreamedStack

    out = []
    for T in tokens:
        stack = StreamedStack(wl, n_bufs=nbuf, seed=seed, tokens=T)
        try:
            res = {}
            for mode in ("streamed", "resident"):
                for _ in range(2):
                    stack.step(resident=(mode == "resident"))
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(steps):
                    stack.step(resident=(mode == "resident"))
                torch.cuda.synchronize()
                ms = (time.perf_counter() - t0) * 1000.0 / steps
                res[mode] = {"ms_per_step": round(ms, 2), "tokens_per_s": round(T / (ms / 1000.0), 1)}
        finally:
            stack.close()
            del stack
            _release_memory()
        out.append({"tokens": T, **res, "exposed_copy_ms": round(res["streamed"]["ms_per_step"] -
                                                                  res["resident"]["ms_per_step"], 2)})
        log(f"T={T}: {out[-1]}")
    return out


def stream_variants(wl, args, L):
    """The same streamed step with the stream variants: buffer reuse (a layer still in a
    buffer is not copied again: at the forward/backward turn and at the next step's
    start), no recompute (the backward uses the forward's saved rank-r activations
    and skips the forward re-run; the layer is still read twice, for dx), and the
    embedding rows read from the page-locked host table (the slot then keeps lm_head
    from step to step: no per-step slot copies)."""
    import torch
    from lora_fine_tuning_nf4_amd.stack import StreamedStack

    out = {}
    for name, kw in (("reuse", {"reuse": True}), ("no_recompute", {"recompute": False}),
                     ("reuse_no_recompute", {"reuse": True, "recompute": False}),
                     ("embed_from_host", {"embed_from_host": True}),
                     ("embed_from_host_reuse", {"embed_from_host": True, "reuse": True})):
        stack = StreamedStack(wl, n_bufs=args.nbuf, seed=args.seed, layers=L, loss_chunk=args.loss_chunk, **kw)
        try:
            for _ in range(max(2, args.warmup)):
                stack.step()
            torch.cuda.synchronize()
            b0 = stack.bytes_copied()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                stack.step()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1000.0 / args.steps
            h2d = (stack.bytes_copied() - b0) // args.steps
            gbps = _copy_only_gbps(stack)
            out[name] = {"ms_per_step": round(ms, 3), "tokens_per_s": round(stack.T / (ms / 1000.0), 2),
                         "h2d_bytes_per_step": h2d,
                         "compute_blocked_on_copies_ms": round(_blocked_on_copies(stack), 3),
                         "copy_only_GBps": round(gbps, 2), "link_floor_ms_per_step": round(h2d / (gbps * 1e6), 3)}
        finally:
            stack.close()
            del stack
            _release_memory()
        log(f"variant {name}: {out[name]}")
    return out


def disk_run(wl, args, L):
    """The disk variant, reported with the stream variants; run after every other
    streamed measurement so that its file and page-cache traffic precede none of them."""
    try:
        rec = disk_variant(wl, args, L)
    except (OSError, RuntimeError) as e:  # e.g. no room for the 3.9 GB shard file: report, do not fail the bench
        rec = {"error": f"{type(e).__name__}: {e}"}
    log(f"variant disk: {rec}")
    return rec


def disk_variant(wl, args, L):
    """The disk tier: the layer shards are written to a file and every step reads them back
    from the device (their pages are dropped from the page cache after each read) through
    two pinned staging buffers (the pages' default read-ahead), then copies them through
    the same ring; the head slot stays in pinned RAM.  One warm-up step and at most two
    timed steps: the step is bound by the disk."""
    import shutil
    import tempfile
    import torch
    from lora_fine_tuning_nf4_amd.stack import StreamedStack

    d = tempfile.mkdtemp(prefix="lnf4_disk_", dir=os.environ.get("TMPDIR", "/tmp"))
    stack = StreamedStack(wl, n_bufs=args.nbuf, seed=args.seed, layers=L, loss_chunk=args.loss_chunk)
    try:
        stack.use_disk(os.path.join(d, "layers.bin"), read_ahead=2, drop_cache=True)
        stack.step()
        torch.cuda.synchronize()
        r0, s0 = stack.disk_stats()
        b0 = stack.bytes_copied()
        n = max(1, min(2, args.steps))
        t0 = time.perf_counter()
        for _ in range(n):
            stack.step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1000.0 / n
        r1, s1 = stack.disk_stats()
        return {"ms_per_step": round(ms, 3), "tokens_per_s": round(stack.T / (ms / 1000.0), 2),
                "read_ahead": 2, "disk_bytes_per_step": (r1 - r0) // n,
                "disk_read_GBps": round((r1 - r0) / max(s1 - s0, 1e-9) / 1e9, 2),
                "h2d_bytes_per_step": (stack.bytes_copied() - b0) // n, "steps_timed": n}
    finally:
        stack.close()
        del stack
        _release_memory()
        shutil.rmtree(d, ignore_errors=True)


def _release_memory():
    """Give cached device memory and cached page-locked host memory back: a later run's
    pinned shards are then allocated afresh instead of landing beside a previous run's
    cached blocks (later runs on a host full of cached pinned blocks streamed slower)."""
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if hasattr(torch._C, "_host_emptyCache"):
        torch._C._host_emptyCache()


def _timed_steps(stack, steps: int, warmup: int, resident: bool = False):
    import torch
    for _ in range(warmup):
        stack.step(resident=resident)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        stack.step(resident=resident)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1000.0 / steps


def _timed_graph(stack, steps: int, warmup: int):
    """ms per resident step replayed from its captured HIP graph (capture not timed)."""
    import torch
    stack.resident_graph()
    for _ in range(warmup):
        stack.step_graph()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        stack.step_graph()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1000.0 / steps


def _gemm_rate(stack, wl, resident: bool = False):
    """TFLOP/s of the grouped GEMM calls (skinny LoRA kernels included) over one step, HIP
    events around every call."""
    import torch
    from lora_fine_tuning_nf4_amd.stack import GROUPS
    keys = [("fwd", gi, True) for gi in range(len(GROUPS))] + [("bwd", gi, True) for gi in range(len(GROUPS))]
    if stack.dpo:
        keys += [("fwd", gi, False) for gi in range(len(GROUPS))]
    stack.timers = {k: ([], []) for k in keys}
    stack.step(resident=resident)
    torch.cuda.synchronize()
    tm, stack.timers = stack.timers, None
    ms = flops = 0.0
    for (kind, gi, _on), (st, en) in tm.items():
        ms += sum(a.elapsed_time(b) for a, b in zip(st, en))
        flops += gemm_flops(wl, GROUPS[gi], kind) * len(st)
    return {"gemm_ms_per_step": round(ms, 3), "gemm_tflops": round(flops / (ms / 1000.0) / 1e12, 2),
            "gemm_frac_of_peak": round(flops / (ms / 1000.0) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def _copy_only_gbps(stack, reps: int = 4) -> float:
    """The link's copy-only rate right now: the stack's first shard copied into its first
    device buffer `reps` times on the copy stream, nothing else running.  Taken beside each
    streamed measurement, so a slow stretch of the host link shows in the record."""
    import torch
    hb, db, cs = stack.host[0], stack.bufs[0], stack.copy
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(cs):
        e0.record(cs)
        for _ in range(reps):
            db[:hb.numel()].copy_(hb, non_blocking=True)
        e1.record(cs)
    torch.cuda.synchronize()
    return reps * hb.numel() / (e0.elapsed_time(e1) / 1000.0) / 1e9


def _copy_rate_under_load(stack, reps: int = 8):
    """The link's rate while the compute stream is busy: the stack's first shard copied into
    its first device buffer `reps` times on the copy stream while the compute stream runs,
    back to back, (a) nothing, (b) the gate|up forward GEMM of the layer held in the second
    buffer, (c) a bf16 8192^3 library GEMM (matrix cores, little HBM traffic), (d) a 1 GiB
    device-to-device copy (HBM traffic, no matrix work).  The load is enqueued first and
    outlasts the copies."""
    import torch
    hb, db, cs, comp = stack.host[0], stack.bufs[0], stack.copy, stack.compute
    projs = stack._projs(0, 2, stack.bufs[1].data_ptr(), adapters=False)
    x = stack.layers[0].x[2]
    a = torch.randn(8192, 8192, device=stack.dev).to(torch.bfloat16)
    b = torch.randn(8192, 8192, device=stack.dev).to(torch.bfloat16)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=stack.dev)
    dst = torch.empty_like(src)
    copy_ms = reps * hb.numel() / 50e9 * 1000.0

    def load(kind):
        if kind == "nf4_gate_up_fwd":
            for _ in range(int(copy_ms / 0.4) + 10):
                lnf4.lora_group_fwd(projs, x, stack.T, 0, comp)
        elif kind == "bf16_gemm_8192":
            with torch.cuda.stream(comp):
                for _ in range(int(copy_ms / 0.6) + 10):
                    torch.matmul(a, b)
        elif kind == "hbm_copy_1GiB":
            with torch.cuda.stream(comp):
                for _ in range(int(copy_ms / 0.25) + 10):
                    dst.copy_(src)

    from lora_fine_tuning_nf4_amd import lnf4
    out = {}
    for kind in ("none", "nf4_gate_up_fwd", "bf16_gemm_8192", "hbm_copy_1GiB", "none"):
        torch.cuda.synchronize()
        load(kind)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(cs):
            e0.record(cs)
            for _ in range(reps):
                db[:hb.numel()].copy_(hb, non_blocking=True)
            e1.record(cs)
        torch.cuda.synchronize()
        key = kind if kind not in out else kind + "_again"
        out[key] = round(reps * hb.numel() / (e0.elapsed_time(e1) / 1000.0) / 1e9, 2)
    del a, b, src, dst
    return out


def _blocked_on_copies(stack, steps: int = 1):
    """Compute-stream time per step blocked on copies (layer copies and slot loads): HIP
    events on the compute stream right before and after every call that enqueues such a
    wait; no kernel runs between the two, so their distance is the blocked time."""
    import torch
    stack.wait_events = []
    for _ in range(steps):
        stack.step()
    torch.cuda.synchronize()
    we, stack.wait_events = stack.wait_events, None
    return sum(a.elapsed_time(b) for a, b in we) / steps


def _copy_timeline(stack):
    """Where the link's time goes in one streamed step.  Every stream call that may issue
    copies is bracketed by an event on the compute stream just before it (where the call
    records the release that its copies wait for) and one on the copy stream just after it
    (reached when its copies are done).  A call's copies start at the later of the copy
    stream's previous mark and that release (the first call of a pass and the later parts
    of a slot load wait for nothing recorded at the call), so the link is idle before them
    for the difference, and busy for the rest of the interval."""
    import torch
    torch.cuda.synchronize()
    ref_c = torch.cuda.Event(enable_timing=True)
    ref_x = torch.cuda.Event(enable_timing=True)
    ref_c.record(stack.compute)
    ref_x.record(stack.copy)
    stack.copy_marks = []
    stack.step()
    end = torch.cuda.Event(enable_timing=True)
    end.record(stack.compute)
    torch.cuda.synchronize()
    marks, stack.copy_marks = stack.copy_marks, None
    t = lambda ev: ref_c.elapsed_time(ev)
    prev = t(ref_x)
    L = stack.L
    n_fwd = 2 * L if stack.dpo else L
    first_part = next((i for i, m in enumerate(marks) if m[0] == "part"), None)  # part 0 waits for the head
    groups = {"fwd_layer": [], "bwd_layer": [], "slot": []}
    idle = {"forward": 0.0, "backward": 0.0}
    busy_total = idle_total = 0.0
    bytes_total = 0
    for mi, (tag, k, e0, e1, nbytes) in enumerate(marks):
        t1 = t(e1)
        if nbytes <= 0:
            prev = max(prev, t1)
            continue
        waits = (tag == "layer" and k > 0) or tag == "slot" or (tag == "part" and mi == first_part)
        start = max(prev, t(e0)) if waits else prev
        gap, busy = start - prev, max(t1 - start, 1e-6)
        phase = "forward" if (0 <= k < n_fwd) else "backward"
        if tag == "slot" and k < 0:
            phase = "forward"
        idle[phase] += gap
        idle_total += gap
        busy_total += busy
        bytes_total += nbytes
        key = "slot" if tag in ("slot", "part") else ("fwd_layer" if k < n_fwd else "bwd_layer")
        groups[key].append((busy, nbytes))
        prev = t1

    def summary(v):
        if not v:
            return None
        ms = [b for b, _ in v]
        return {"n": len(v), "mean_ms": round(sum(ms) / len(ms), 3), "min_ms": round(min(ms), 3),
                "max_ms": round(max(ms), 3), "GBps": round(sum(n for _, n in v) / (sum(ms) / 1000.0) / 1e9, 2)}

    return {"step_ms": round(t(end), 3), "link_busy_ms": round(busy_total, 3), "link_idle_ms": round(idle_total, 3),
            "link_idle_ms_by_pass": {k: round(v, 3) for k, v in idle.items()},
            "GBps_while_busy": round(bytes_total / (busy_total / 1000.0) / 1e9, 2),
            "copy_stream_done_ms": round(prev, 3), "bytes": bytes_total,
            "forward_layer_copies": summary(groups["fwd_layer"]), "backward_layer_copies": summary(groups["bwd_layer"]),
            "slot_copies": summary(groups["slot"])}


def other_configs(args):
    """The other workloads of the path, two or more timed steps each: the Qwen2.5-0.5B-shaped
    NF4 stack streamed and resident, the Qwen2.5-3B-shaped bf16 stack at 2, 4 and 8 device
    buffers (and resident), and the DPO step on the 8B stack streamed and resident."""
    import torch
    import synthgen
    from lora_fine_tuning_nf4_amd.stack import StreamedStack

    out = {}
    for name, nbufs, steps, warm in (("qwen05b", (2,), 5, 2), ("qwen3b_bf16", (2, 4, 8), 2, 1),
                                     ("llama8b_dpo", (2,), 2, 1)):
        wl = synthgen.WORKLOADS[name]
        t0 = time.perf_counter()
        stack = StreamedStack(wl, n_bufs=nbufs[0], seed=args.seed)
        rec = {"layers": stack.L, "tokens_per_step": stack.T, "weights": wl.fmt,
               "lora": {"r": wl.rank, "alpha": wl.alpha, "targets": list(wl.adapted)},
               "setup_s": round(time.perf_counter() - t0, 1)}
        try:
            for nb in nbufs:
                if nb != stack.n_bufs:
                    stack.rebuffer(nb)
                b0 = stack.bytes_copied()
                ms = _timed_steps(stack, steps, warm)
                h2d = (stack.bytes_copied() - b0) // (steps + warm)
                gbps = _copy_only_gbps(stack)
                rec[f"streamed_nbuf{nb}"] = {"ms_per_step": round(ms, 3),
                                             "tokens_per_s": round(stack.T / (ms / 1000.0), 1),
                                             "h2d_bytes_per_step": h2d,
                                             "compute_blocked_on_copies_ms": round(_blocked_on_copies(stack), 3),
                                             "copy_only_GBps": round(gbps, 2),
                                             "link_floor_ms_per_step": round(h2d / (gbps * 1e6), 3)}
            ms = _timed_steps(stack, steps, warm, resident=True)
            rec["resident"] = {"ms_per_step": round(ms, 3), "tokens_per_s": round(stack.T / (ms / 1000.0), 1),
                               **_gemm_rate(stack, wl, resident=True)}
            gms = _timed_graph(stack, max(steps, 5), warm)
            rec["resident_graph"] = {"ms_per_step": round(gms, 3), "tokens_per_s": round(stack.T / (gms / 1000.0), 1)}
        finally:
            stack.close()
            del stack
            _release_memory()
        out[name] = rec
        log(f"config {name}: {rec}")
    return out


def decoder_model_run(args):
    """The whole decoder model on the 8B stack (embedding, 32 real decoder layers with
    RMSNorm, RoPE, causal GQA attention, SwiGLU and residuals, final norm, lm_head and
    loss, forward + recompute + backward), streamed and resident, and the attention
    kernels alone at that shape (HIP events, 20 launches each)."""
    import torch
    import synthgen
    from lora_fine_tuning_nf4_amd import lnf4
    from lora_fine_tuning_nf4_amd.model import StreamedDecoder

    wl = synthgen.WORKLOADS[args.workload]
    if wl.extra.get("arch") is None or wl.vocab <= 0:
        return None
    out = {}
    m = StreamedDecoder(wl, n_bufs=args.nbuf, seed=args.seed, loss_chunk=args.loss_chunk)
    try:
        for mode in ("streamed", "resident"):
            res = mode == "resident"
            for _ in range(max(1, args.warmup)):
                m.step(resident=res)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                m.step(resident=res)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1000.0 / args.steps
            out[f"{mode}_ms_per_step"] = round(ms, 3)
            out[f"{mode}_tokens_per_s"] = round(m.T / (ms / 1000.0), 2)
            if not res:
                out["streamed_copy_only_GBps"] = round(_copy_only_gbps(m), 2)
        # attention alone, on the model's own buffers (the last layer's q, k, v, o)
        T, nh, nkv, D, S = m.T, m.nh, m.nkv, m.D, m.S
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fwd_flops = 2.0 * 2.0 * nh * D * (S * (S + 1) / 2.0) * (T // S)   # causal (query, key) pairs
        bwd_flops = 2.5 * fwd_flops
        for name, fn, fl in (
                ("fwd", lambda: lnf4.lnf4_attn_fwd(m.q, m.k, m.v, T, nh, nkv, D, S, m.o, m.lse), fwd_flops),
                ("bwd", lambda: lnf4.lnf4_attn_bwd(m.q, m.k, m.v, m.o, m.lse, m.do, T, nh, nkv, D, S, m.dq, m.dk,
                                                   m.dv, m.attn_ws, m.attn_ws_bytes), bwd_flops)):
            fn()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(20):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 20
            out[f"attention_{name}_ms"] = round(ms, 4)
            out[f"attention_{name}_tflops"] = round(fl / (ms / 1000.0) / 1e12, 1)
        out["attention_flops_note"] = ("algorithmic: fwd 2 products x 2 flops per causal (query, key) pair and head "
                                       "dim; bwd 2.5x fwd (score recompute, dV, dP, dQ, dK)")
    finally:
        m.close()
        del m
        _release_memory()
    log(f"decoder model: {out}")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--nbuf", type=int, default=2)
    ap.add_argument("--layers", type=int, default=None, help="override the layer count (testing)")
    ap.add_argument("--no-resident", action="store_true", help="skip the H2D-removed reference run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-model", action="store_true",
                    help="skip the whole-decoder-model run (attention, norms, SwiGLU between the projections)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the stream-variant runs (buffer reuse, no recompute, disk tier)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (Qwen2.5-0.5B NF4, Qwen2.5-3B bf16 at 2/4/8 buffers, 8B DPO)")
    ap.add_argument("--loss-chunk", type=int, default=None,
                    help="tokens per chunk of the output head and its loss (default: all tokens at once)")
    ap.add_argument("--study", action="store_true",
                    help="also measure the dequant share (fused vs dequant + bf16 GEMMs) and a T sweep")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("bench.py measures one GPU only: the streamed NF4+LoRA path runs on a single MI355X "
               f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}); multi-GPU data parallelism is not built")
        log(msg)
        print(json.dumps({"error": msg, "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import synthgen
    from lora_fine_tuning_nf4_amd import lnf4
    from lora_fine_tuning_nf4_amd.stack import GROUPS, StreamedStack

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    lnf4.lib()  # fail loudly if the HIP library is missing
    wl = synthgen.WORKLOADS[args.workload]
    L = args.layers if args.layers is not None else wl.layers
    torch.cuda.set_device(0)

    t_setup = time.perf_counter()
    stack = StreamedStack(wl, n_bufs=args.nbuf, seed=args.seed, layers=L, loss_chunk=args.loss_chunk)
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f} s: {L} layers x {stack.shard_bytes / 1e6:.1f} MB shards, "
        f"nbuf={args.nbuf}, T={stack.T}")

    for _ in range(args.warmup):
        stack.step()
    torch.cuda.synchronize()

    # ---- timed region: K streamed steps; HIP events on the compute stream (where the
    # kernels run) around every launch of the dominant kernel only, so the events cost the
    # step next to nothing
    dom_key = ("fwd", 2, True)
    stack.timers = {dom_key: ([], [])}
    b0 = stack.bytes_copied()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        stack.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    b1 = stack.bytes_copied()
    dom_timer = stack.timers[dom_key]
    stack.timers = None
    ms_per_step = (t1 - t0) * 1000.0 / args.steps
    tokens = stack.T
    value = tokens / (ms_per_step / 1000.0)

    # per-call GEMM times (ms) for the breakdown: extra steps after the timed region with
    # events around every grouped call
    keys = [("fwd", gi, True) for gi in range(len(GROUPS))] + [("bwd", gi, True) for gi in range(len(GROUPS))]
    if stack.dpo:
        keys += [("fwd", gi, False) for gi in range(len(GROUPS))]
    head_keys = ([("head", "ref"), ("head", "pol")] if stack.dpo else [("head", "sft")]) if stack.head else []
    keys += head_keys
    n_bd = max(1, min(2, args.steps))
    stack.timers = {k: ([], []) for k in keys}
    for _ in range(n_bd):
        stack.step()
    torch.cuda.synchronize()
    timers = stack.timers
    stack.timers = None
    call_ms, head_ms = {}, {}
    for k, (st, en) in timers.items():
        ms = [a.elapsed_time(b) for a, b in zip(st, en)]
        if k[0] == "head":
            head_ms[k[1]] = sum(ms) / max(1, len(ms))
        else:
            call_ms[k] = ms
    blocked_ms = _blocked_on_copies(stack, n_bd)
    timeline = _copy_timeline(stack)
    log(f"[bench] copy timeline of one streamed step: {timeline}")
    gemm_time_ms = sum(sum(v) for v in call_ms.values()) / n_bd
    gemm_flops_step = 0.0
    for (kind, gi, _on), ts in call_ms.items():
        gemm_flops_step += gemm_flops(wl, GROUPS[gi], kind) * len(ts) / n_bd
    # dominant kernel: the gate|up forward GEMM (the largest single launch of the step),
    # timed inside the timed region
    dom = [a.elapsed_time(b) for a, b in zip(*dom_timer)]
    dom_ms = sum(dom) / len(dom)
    dom_flops = gemm_flops(wl, GROUPS[2], "fwd")
    achieved = dom_flops / (dom_ms / 1000.0) / 1e12
    dx_dom = call_ms[("bwd", 2, True)]
    dx_ms = sum(dx_dom) / len(dx_dom)

    traffic, traffic_src = measured_traffic()
    if (wl.name, stack.T, L) != ("llama8b", 2048, 32):
        traffic, traffic_src = None, "counters were taken on the llama8b T=2048 gate|up launch only"
    breakdown = {f"{k[0]}_{'+'.join(GROUPS[k[1]])}{'' if k[2] else '_adapters_off'}_ms":
                 round(sum(v) / len(v), 4) for k, v in call_ms.items() if v}

    result = {
        "metric": "train tokens/s, 8B-shape NF4+LoRA layer fwd+bwd (streamed stack step)",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights quantized to NF4 on the device, N(0,1) bf16 activations)",
        "config": {"workload": wl.name, "layers": L, "tokens_per_step": tokens, "global_batch": 1,
                   "seq_len": tokens, "lora": {"r": wl.rank, "alpha": wl.alpha, "targets": list(wl.adapted)},
                   "weights": wl.fmt, "stream_buffers": args.nbuf,
                   "head_slot": bool(stack.slot is not None), "loss_chunk": stack.chunk if stack.head else None,
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic, "traffic_source": traffic_src,
            "algorithmic_bytes_per_launch": fwd_bytes(wl, GROUPS[2]),
            "kernel": (f"k_fwd_nf4<BM=256,4 waves> gate|up forward: M={stack.T} N={sum(wl.shapes[p][0] for p in GROUPS[2])} "
                       f"K={wl.shapes[GROUPS[2][0]][1]} (fused NF4 decode), one launch (256x256 tiles; a last "
                       f"round that would leave compute units idle runs as 128x256 tiles in the same launch)"),
            "flops_per_launch": dom_flops, "avg_launch_ms": round(dom_ms, 4),
            "launches_timed": len(dom),
        },
        "gemm": {
            "tflops_all_grouped_gemms": round(gemm_flops_step / (gemm_time_ms / 1000.0) / 1e12, 2),
            "frac_of_peak_all_gemms": round(gemm_flops_step / (gemm_time_ms / 1000.0) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "gemm_ms_per_step": round(gemm_time_ms, 3),
            "dx_gate_up_ms": round(dx_ms, 4),
            "dx_gate_up_tflops": round(gemm_flops(wl, GROUPS[2], "bwd") / (dx_ms / 1000) / 1e12, 2),
            "per_call_avg_ms": breakdown,
        },
        "head": head_summary(wl, stack, head_ms),
        "h2d": {
            "bytes_per_step": (b1 - b0) // args.steps,
            "avg_GBps_over_step": round((b1 - b0) / args.steps / (ms_per_step / 1000.0) / 1e9, 2),
            "compute_blocked_on_copies_ms_per_step": round(blocked_ms, 3),
            "compute_blocked_share_of_step": round(blocked_ms / ms_per_step, 4),
            "copy_timeline": timeline,
        },
    }

    # the library's bf16 GEMM at the dominant launch's shape, as context for its fraction of peak
    result["roofline"]["library_bf16_same_shape"] = library_bf16_same_shape(
        stack.T, sum(wl.shapes[p][0] for p in GROUPS[2]), wl.shapes[GROUPS[2][0]][1])
    log(f"[bench] library bf16 GEMM at the dominant shape: {result['roofline']['library_bf16_same_shape']}")

    if not args.no_resident:
        for _ in range(max(1, args.warmup)):
            stack.step(resident=True)
        torch.cuda.synchronize()
        r0 = time.perf_counter()
        for _ in range(args.steps):
            stack.step(resident=True)
        torch.cuda.synchronize()
        r_ms = (time.perf_counter() - r0) * 1000.0 / args.steps
        result["resident_h2d_removed"] = {
            "ms_per_step": round(r_ms, 3), "tokens_per_s": round(tokens / (r_ms / 1000.0), 2),
            "exposed_copy_ms_per_step": round(ms_per_step - r_ms, 3),
        }
        g_ms = _timed_graph(stack, args.steps, max(1, args.warmup))
        result["resident_h2d_removed"]["graph_replay_ms_per_step"] = round(g_ms, 3)
        result["resident_h2d_removed"]["graph_replay_tokens_per_s"] = round(tokens / (g_ms / 1000.0), 2)

    # the same stream calls (layer copies, slot loads, event waits) without any kernel: the
    # time the copy schedule of the ring takes by itself
    for _ in range(max(1, args.warmup)):
        stack.step(compute=False)
    torch.cuda.synchronize()
    s0 = time.perf_counter()
    n_sched = max(2, min(args.steps, 5))
    for _ in range(n_sched):
        stack.step(compute=False)
    torch.cuda.synchronize()
    result["h2d"]["schedule_only_ms_per_step"] = round((time.perf_counter() - s0) * 1000.0 / n_sched, 3)

    # copy-only rate of the link (the same copies, no compute)
    hb = stack.host[0]
    db = stack.bufs[0]
    cs = stack.copy
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(cs):
        e0.record(cs)
        for _ in range(8):
            db.copy_(hb, non_blocking=True)
        e1.record(cs)
    torch.cuda.synchronize()
    result["h2d"]["copy_only_GBps"] = round(8 * hb.numel() / (e0.elapsed_time(e1) / 1000.0) / 1e9, 2)
    # the step's bytes at that rate: the floor of any schedule on this link
    result["h2d"]["link_floor_ms_per_step"] = round(result["h2d"]["bytes_per_step"] / (result["h2d"]["copy_only_GBps"] * 1e6), 3)
    result["h2d"]["copy_GBps_under_load"] = _copy_rate_under_load(stack)
    log(f"[bench] link rate under compute load: {result['h2d']['copy_GBps_under_load']}")
    # every shard once (host placement can differ between shards)
    rates = []
    for h in stack.host:
        with torch.cuda.stream(cs):
            e0.record(cs)
            db[:h.numel()].copy_(h, non_blocking=True)
            e1.record(cs)
        torch.cuda.synchronize()
        rates.append(h.numel() / (e0.elapsed_time(e1) / 1000.0) / 1e9)
    result["h2d"]["per_shard_GBps"] = {"min": round(min(rates), 2), "mean": round(sum(rates) / len(rates), 2),
                                       "max": round(max(rates), 2)}
    if stack.slot is not None:
        head = {}
        for name, sid in zip(("embed", "lm_head"), stack.head_ids):
            h = stack.all_shards[sid]
            with torch.cuda.stream(cs):
                e0.record(cs)
                stack.slot[:h.numel()].copy_(h, non_blocking=True)
                e1.record(cs)
            torch.cuda.synchronize()
            head[name + "_GBps"] = round(h.numel() / (e0.elapsed_time(e1) / 1000.0) / 1e9, 2)
        h = stack.all_shards[stack.head_ids[0]]
        part = (h.numel() + L - 1) // L
        with torch.cuda.stream(cs):
            e0.record(cs)
            for q in range(L):
                stack.slot[q * part:min((q + 1) * part, h.numel())].copy_(h[q * part:min((q + 1) * part, h.numel())],
                                                                           non_blocking=True)
            e1.record(cs)
        torch.cuda.synchronize()
        head[f"embed_in_{L}_parts_GBps"] = round(h.numel() / (e0.elapsed_time(e1) / 1000.0) / 1e9, 2)
        result["h2d"]["head_slot"] = head
    # a plain device copy of known size, the reference point that scales rocprofv3's
    # FETCH_SIZE / WRITE_SIZE counters to bytes in a counter run of this same command
    ca = torch.ones(CAL_ELEMS, dtype=torch.float32, device="cuda")
    cb = torch.empty_like(ca)
    torch.neg(ca, out=cb)
    torch.cuda.synchronize()
    result["pmc_calibration"] = {"kernel": "torch neg, float32 elementwise", "bytes_read": 4 * CAL_ELEMS,
                                 "bytes_written": 4 * CAL_ELEMS}
    del ca, cb

    stack.close()
    del stack
    _release_memory()

    if not args.no_variants:
        result["stream_variants"] = stream_variants(wl, args, L)
        _release_memory()
    if not args.no_model and L == wl.layers:
        result["decoder_model"] = decoder_model_run(args)
        _release_memory()
    if not args.no_configs and wl.name == "llama8b" and L == wl.layers:
        result["other_configs"] = other_configs(args)
    if not args.no_variants:
        result["stream_variants"]["disk"] = disk_run(wl, args, L)
        _release_memory()

    if args.study:
        log("study: dequant share ...")
        result["study"] = {"dequant_share": dequant_share(wl, args.seed)}
        _release_memory()
        log("study: T sweep ...")
        result["study"]["t_sweep"] = t_sweep(wl, args.seed, args.nbuf, max(2, args.steps // 2))

    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on one layer ...")
        result["cpu_baseline"] = cpu_baseline(wl, args.seed, L)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
