"""Parity at the full layer shapes of the benchmark configurations, in the launch
configuration the benchmark times (grouped q|k|v, gate|up and down calls at the
configuration's T, the forward through the workspace form the stack calls, so the Qwen2.5-0.5B
and Llama-8B down projections run their K-split launches), on sampled outputs the oracle computes one by one: whole rows of y and
dx, whole columns of dA, whole rows of dB.  Llama-3.1-8B NF4 (every group at T = 2048, and
the DPO step's T = 4096), Qwen2.5-0.5B NF4 with rank 16 on every projection, Qwen2.5-3B bf16
weights."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import synthgen  # noqa: E402
from lora_fine_tuning_nf4_amd import lnf4  # noqa: E402
from oracle import nf4 as onf4  # noqa: E402
from helpers import bf16_f64, check_tol, dev_f32, dev_u16, dev_u8, host_f32, host_u16  # noqa: E402

CASES = [("llama8b", ("q", "k", "v")), ("llama8b", ("o",)), ("llama8b", ("gate", "up")), ("llama8b", ("down",)),
         ("llama8b_dpo", ("gate", "up")),
         ("qwen05b", ("q", "k", "v")), ("qwen05b", ("gate", "up")), ("qwen05b", ("down",)),
         ("qwen3b_bf16", ("q", "k", "v")), ("qwen3b_bf16", ("gate", "up"))]


def _group(WL, names, seed=0):
    T = WL.tokens
    in_f = WL.shapes[names[0]][1]
    x = synthgen.act_bits(T, in_f, seed, "full-x", *names)
    P = {}
    for p in names:
        o, i = WL.shapes[p]
        w = synthgen.weight_f32(o, i, seed, "full", p)
        on = p in WL.adapted
        d = dict(on=on, o=o, A=synthgen.adapter_a_bits(WL.rank, i, seed, "full", p) if on else None,
                 B=synthgen.adapter_b_bits(o, WL.rank, seed, "full", p) if on else None,
                 dy=synthgen.act_bits(T, o, seed, "full-dy", p))
        if WL.fmt == "nf4":
            d["codes"], d["absmax"] = onf4.quantize(w)
        else:
            d["wbits"] = synthgen.to_bf16_bits(w)
        P[p] = d
    return x, P


def _dev(WL, names, x, P):
    T = WL.tokens
    dev = {"x": dev_u16(x)}
    projs = []
    for p in names:
        d = P[p]
        o, i = WL.shapes[p]
        d["y"] = torch.empty((T, o), dtype=torch.int16, device="cuda")
        d["ddy"] = dev_u16(d["dy"])
        if d["on"]:
            d["dA_in"], d["dB_in"] = dev_u16(d["A"]), dev_u16(d["B"])
            d["u"] = torch.empty((T, WL.rank), dtype=torch.float32, device="cuda")
            d["dA"] = torch.empty((WL.rank, i), dtype=torch.float32, device="cuda")
            d["dB"] = torch.empty((o, WL.rank), dtype=torch.float32, device="cuda")
        if WL.fmt == "nf4":
            d["dcodes"], d["dabsmax"] = dev_u8(d["codes"]), dev_f32(d["absmax"])
            W = lnf4.make_weight(lnf4.FMT_NF4, d["dcodes"], d["dabsmax"], o, i, 64)
        else:
            d["dw"] = dev_u16(d["wbits"])
            W = lnf4.make_weight(lnf4.FMT_BF16, d["dw"], None, o, i, 64)
        projs.append(lnf4.make_proj(W, A=d.get("dA_in"), B=d.get("dB_in"), r=WL.rank if d["on"] else 0,
                                    scale=WL.scale if d["on"] else 0.0, y=d["y"], u=d.get("u"), dy=d["ddy"],
                                    dA=d.get("dA"), dB=d.get("dB")))
    return dev, projs


@pytest.mark.parametrize("wl_name,names", CASES, ids=[f"{w}-{'_'.join(n)}" for w, n in CASES])
def test_full_size_group_sampled(wl_name, names):
    WL = synthgen.WORKLOADS[wl_name]
    T = WL.tokens
    # sampled rows: both ends, one in each 256-row tile of the first half, a few inside tiles
    ROWS = sorted(set([0, 1, 255, 256, 511, 777, T // 2 + 3, T - 129, T - 1]))
    x, P = _group(WL, names)
    dev, projs = _dev(WL, names, x, P)
    in_f = WL.shapes[names[0]][1]
    dx = torch.empty((T, in_f), dtype=torch.int16, device="cuda")
    # one workspace for both directions, as the stack sizes it: the forward takes its K-split
    # launch where it has one (the Qwen2.5-0.5B down projection)
    fwd_ws = lnf4.lora_group_fwd_workspace(projs, T)
    assert (fwd_ws > 0) == (names == ("down",) and wl_name in ("qwen05b", "llama8b")), "which launches take K splits"
    ws_bytes = max(lnf4.lora_group_bwd_workspace(projs, T), fwd_ws)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    lnf4.lora_group_fwd_ws(projs, dev["x"], T, 1, ws, ws_bytes)
    lnf4.lora_group_bwd(projs, dev["x"], T, dx, 0, ws, ws_bytes)
    torch.cuda.synchronize()

    xs = bf16_f64(x[ROWS])
    dx_ref = np.zeros((len(ROWS), in_f))
    xf = None
    for p in names:
        d = P[p]
        Wd = onf4.decode_f64(d["codes"], d["absmax"]) if WL.fmt == "nf4" else bf16_f64(d["wbits"])
        y_ref = xs @ Wd.T
        dyr = bf16_f64(d["dy"][ROWS])
        dx_ref += dyr @ Wd
        if d["on"]:
            A, B = bf16_f64(d["A"]), bf16_f64(d["B"])
            y_ref += WL.scale * (xs @ A.T) @ B.T
            dx_ref += WL.scale * (dyr @ B) @ A
            # adapter gradients need the whole batch: sampled columns of dA, rows of dB
            if xf is None:
                xf = bf16_f64(x)
            dyf = bf16_f64(d["dy"])
            v = dyf @ B
            u = xf @ A.T
            cols = [0, 5, in_f // 2, in_f - 1]
            check_tol(host_f32(d["dA"])[:, cols], WL.scale * v.T @ xf[:, cols], f"dA {p}")
            orow = [0, 3, d["o"] // 2, d["o"] - 1]
            check_tol(host_f32(d["dB"])[orow], WL.scale * dyf[:, orow].T @ u, f"dB {p}")
            check_tol(host_f32(d["u"])[ROWS], xs @ A.T, f"u {p}")
        check_tol(bf16_f64(host_u16(d["y"])[ROWS]), y_ref, f"y {p}")
        del Wd
    check_tol(bf16_f64(host_u16(dx)[ROWS]), dx_ref, "dx")


@pytest.mark.parametrize("T", [2048, 4096])
def test_lm_head_gemms_full_size_sampled_rows(T):
    """The untied lm_head of the 8B head at the loss turn (T = 2048 SFT, 4096 DPO), in one
    launch each: logits = h W^T (K = 4096, N = 128256) and dh = dlogits W (K = 128256 in
    256-row tiles with 32-row K-blocks: two splits at T = 2048, none at 4096), adapter
    off; sampled rows of both against the fp64 oracle, summed over vocabulary chunks of W."""
    V, H = 128256, 4096
    W = synthgen.device_normal((V, H), 0.02, 12, "lm_head_full", dtype=torch.bfloat16)
    h = synthgen.device_normal((T, H), 1.0, 12, "h_full", dtype=torch.bfloat16)
    dl = synthgen.device_normal((T, V), 1e-3, 12, "dlogits_full", dtype=torch.bfloat16)
    Wd = lnf4.make_weight(lnf4.FMT_BF16, W, None, V, H, 64)
    logits = torch.empty((T, V), dtype=torch.bfloat16, device="cuda")
    dh = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws_bytes = lnf4.lora_linear_bwd_workspace(T, V, H, 0)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    lnf4.lora_linear_fwd(Wd, h, T, None, None, 0, 0.0, logits, None)
    lnf4.lora_linear_bwd(Wd, h, dl, T, None, None, 0, 0.0, None, dh, None, None, 0, ws, ws_bytes)
    torch.cuda.synchronize()
    ROWS = [0, 1, 255, 256, 777, T // 2 + 3, T - 129, T - 1]
    ridx = torch.tensor(ROWS, dtype=torch.int64, device="cuda")
    hs = bf16_f64(host_u16(h.index_select(0, ridx).view(torch.int16)))
    dls = bf16_f64(host_u16(dl.index_select(0, ridx).view(torch.int16)))
    logits_ref = np.zeros((len(ROWS), V))
    dh_ref = np.zeros((len(ROWS), H))
    step = 16384
    for v0 in range(0, V, step):
        v1 = min(V, v0 + step)
        Wc = bf16_f64(host_u16(W[v0:v1].view(torch.int16)))
        logits_ref[:, v0:v1] = hs @ Wc.T
        dh_ref += dls[:, v0:v1] @ Wc
        del Wc
    check_tol(bf16_f64(host_u16(logits.index_select(0, ridx).view(torch.int16))), logits_ref, "logits")
    check_tol(bf16_f64(host_u16(dh.index_select(0, ridx).view(torch.int16))), dh_ref, "dh")
