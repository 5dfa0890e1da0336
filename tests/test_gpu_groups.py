"""Grouped calls with uneven adapter ranks.  The projections of a group share x, so their
ranks are concatenated in one skinny launch (u = x A^T in the forward, dA against x in the
backward) and each projection's rank columns must land in its own u, dA and dB; v = dy B
of each projection stages B [out][r] rows (16-byte pieces when r % 8 == 0, single
elements otherwise).  Checked against the fp64 oracle per projection (y, u, dA, dB) and for
the group's summed dx, at ragged T (T = 1 included), ranks that straddle the 16-rank tiles,
the 64-rank limit, r = 1, and out_f = 8."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import synthgen  # noqa: E402
from lora_fine_tuning_nf4_amd import lnf4  # noqa: E402
from oracle import lora as olora  # noqa: E402
from oracle import nf4 as onf4  # noqa: E402
from helpers import bf16_f64, check_tol, dev_f32, dev_u16, dev_u8, host_f32, host_u16  # noqa: E402

# T, in_f, [(out_f, r), ...], weight format (0 NF4, 1 bf16)
CASES = [
    (77, 192, [(200, 3), (64, 13), (136, 24)], 0),   # R = 40: three rank tiles, odd ranks across tile edges
    (1, 128, [(96, 20), (64, 20), (32, 24)], 0),     # one token; R = 64, the limit with dx
    (130, 256, [(256, 8), (72, 5), (512, 16)], 1),   # bf16 weights
    (300, 320, [(264, 64)], 0),                       # one projection at the rank limit
    (45, 64, [(8, 7), (16, 1)], 0),                   # out_f = 8 (one K group of v = dy B), r = 1
    # bf16, 2 x 64 tiles of 256 x 256 (the last column tile ragged) in 2 splits of 66 of the
    # 131 K-blocks: the dx GEMM's 5-stage ring of 32-row K-blocks, each split crossing from
    # one projection into the next; the first projection's last 32-row block holds 8 rows,
    # the other two's are wholly past out_f
    (300, 16320, [(4136, 8), (2064, 4), (2072, 4)], 1),
    # bf16, 2 x 258 tiles of 256 x 256: the forward's 5-stage ring of 32-wide K-blocks (the
    # second projection's last column tile ragged)
    (300, 320, [(32808, 8), (32800, 4)], 1),
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}_in{c[1]}_r{'-'.join(str(r) for _, r in c[2])}_f{c[3]}"
                                               for c in CASES])
def test_group_uneven_ranks(case):
    T, in_f, projs_spec, fmt = case
    seed = 21
    x = synthgen.act_bits(T, in_f, seed, "group-x", in_f)
    xd = dev_u16(x)
    host, projs, keep = [], [], []
    for p, (o, r) in enumerate(projs_spec):
        w = synthgen.weight_f32(o, in_f, seed, "group-w", p)
        A = synthgen.adapter_a_bits(r, in_f, seed, "group", p)
        B = synthgen.adapter_b_bits(o, r, seed, "group", p, std=0.05)
        dy = synthgen.act_bits(T, o, seed, "group-dy", p)
        scale = 16.0 / r
        if fmt == 0:
            codes, absmax = onf4.quantize(w)
            Wd = onf4.decode_f64(codes, absmax)
            dc, da = dev_u8(codes), dev_f32(absmax)
            W = lnf4.make_weight(lnf4.FMT_NF4, dc, da, o, in_f, 64)
            keep += [dc, da]
        else:
            wb = synthgen.to_bf16_bits(w)
            Wd = bf16_f64(wb)
            dw = dev_u16(wb)
            W = lnf4.make_weight(lnf4.FMT_BF16, dw, None, o, in_f, 64)
            keep.append(dw)
        d = dict(A=dev_u16(A), B=dev_u16(B), dy=dev_u16(dy),
                 y=torch.empty((T, o), dtype=torch.int16, device="cuda"),
                 u=torch.empty((T, r), dtype=torch.float32, device="cuda"),
                 dA=torch.empty((r, in_f), dtype=torch.float32, device="cuda"),
                 dB=torch.empty((o, r), dtype=torch.float32, device="cuda"))
        keep.append(d)
        projs.append(lnf4.make_proj(W, A=d["A"], B=d["B"], r=r, scale=scale, y=d["y"], u=d["u"], dy=d["dy"],
                                    dA=d["dA"], dB=d["dB"]))
        host.append(dict(Wd=Wd, A=bf16_f64(A), B=bf16_f64(B), dy=bf16_f64(dy), scale=scale, d=d))

    lnf4.lora_group_fwd(projs, xd, T, 1)
    dx = torch.empty((T, in_f), dtype=torch.int16, device="cuda")
    ws_bytes = lnf4.lora_group_bwd_workspace(projs, T)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    lnf4.lora_group_bwd(projs, xd, T, dx, 0, ws, ws_bytes)
    torch.cuda.synchronize()

    xf = bf16_f64(x)
    dx_ref = np.zeros((T, in_f))
    for p, h in enumerate(host):
        y_ref, u_ref = olora.linear_fwd(xf, h["Wd"], h["A"], h["B"], h["scale"])
        dxp, dA_ref, dB_ref = olora.linear_bwd(xf, h["dy"], h["Wd"], h["A"], h["B"], h["scale"])
        dx_ref += dxp
        check_tol(bf16_f64(host_u16(h["d"]["y"])), y_ref, f"y {p}")
        check_tol(host_f32(h["d"]["u"]), u_ref, f"u {p}")
        check_tol(host_f32(h["d"]["dA"]), dA_ref, f"dA {p}")
        check_tol(host_f32(h["d"]["dB"]), dB_ref, f"dB {p}")
    check_tol(bf16_f64(host_u16(dx)), dx_ref, "dx")


def test_group_u_independent_of_rank_neighbours():
    """u of a projection is bitwise the same whether its ranks are alone in the skinny launch
    or concatenated after another projection's (the K split and the per-element sums depend
    on K alone)."""
    T, in_f, seed = 96, 256, 5
    x = dev_u16(synthgen.act_bits(T, in_f, seed, "nb-x"))
    outs = []
    specs = [(128, 16), (64, 24)]
    mats = []
    for p, (o, r) in enumerate(specs):
        codes, absmax = onf4.quantize(synthgen.weight_f32(o, in_f, seed, "nb-w", p))
        mats.append((dev_u8(codes), dev_f32(absmax), dev_u16(synthgen.adapter_a_bits(r, in_f, seed, "nb", p)),
                     dev_u16(synthgen.adapter_b_bits(o, r, seed, "nb", p))))
    for members in ((0, 1), (1,)):
        projs, us = [], []
        for p in members:
            o, r = specs[p]
            dc, da, A, B = mats[p]
            y = torch.empty((T, o), dtype=torch.int16, device="cuda")
            u = torch.empty((T, r), dtype=torch.float32, device="cuda")
            projs.append(lnf4.make_proj(lnf4.make_weight(lnf4.FMT_NF4, dc, da, o, in_f, 64), A=A, B=B, r=r,
                                        scale=1.0, y=y, u=u))
            us.append((p, u, y))
        lnf4.lora_group_fwd(projs, x, T, 1)
        torch.cuda.synchronize()
        outs.append({p: host_f32(u) for p, u, _ in us})
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))


def test_forward_with_u_given_reads_u():
    """adapters_enabled = 2 (the checkpoint recompute): the call reads u instead of computing
    it. With the u of an earlier call on the same x, y is bitwise that call's y; with u
    changed, y changes (so u was read, not recomputed), and u itself is left as given."""
    T, in_f, seed = 200, 320, 8
    x = dev_u16(synthgen.act_bits(T, in_f, seed, "ug-x"))
    projs, outs = [], []
    for p, (o, r) in enumerate([(264, 8), (136, 16)]):
        codes, absmax = onf4.quantize(synthgen.weight_f32(o, in_f, seed, "ug-w", p))
        dc, da = dev_u8(codes), dev_f32(absmax)
        A = dev_u16(synthgen.adapter_a_bits(r, in_f, seed, "ug", p))
        B = dev_u16(synthgen.adapter_b_bits(o, r, seed, "ug", p, std=0.05))
        y = torch.empty((T, o), dtype=torch.int16, device="cuda")
        u = torch.empty((T, r), dtype=torch.float32, device="cuda")
        projs.append(lnf4.make_proj(lnf4.make_weight(lnf4.FMT_NF4, dc, da, o, in_f, 64), A=A, B=B, r=r,
                                    scale=16.0 / r, y=y, u=u))
        outs.append((y, u, dc, da, A, B))
    lnf4.lora_group_fwd(projs, x, T, 1)
    torch.cuda.synchronize()
    first = [(host_u16(y).copy(), host_f32(u).copy()) for y, u, *_ in outs]
    for y, *_ in outs:
        y.zero_()
    lnf4.lora_group_fwd(projs, x, T, 2)
    torch.cuda.synchronize()
    for (y, u, *_), (y1, u1) in zip(outs, first):
        assert np.array_equal(host_u16(y), y1)
        assert np.array_equal(host_f32(u).view(np.uint32), u1.view(np.uint32))
    outs[0][1].mul_(2.0)
    lnf4.lora_group_fwd(projs, x, T, 2)
    torch.cuda.synchronize()
    assert not np.array_equal(host_u16(outs[0][0]), first[0][0])
    assert np.array_equal(host_f32(outs[0][1]).view(np.uint32), (2.0 * first[0][1]).view(np.uint32))
    assert np.array_equal(host_u16(outs[1][0]), first[1][0])
