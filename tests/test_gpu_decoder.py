"""GPU parity of the decoder-layer glue (RMSNorm, RoPE, SwiGLU, residual add) and of
causal GQA attention against oracle/decoder.py, through the C ABI.

Bounds (the oracle runs in fp64 on the same bf16 inputs; ``q16`` is its bf16 storage):
  elementwise and row outputs   |got - ref| <= 2^-7 |ref| + a: a kernel value is the
      bf16 rounding of an fp32 result, the reference the bf16 rounding of the fp64 one;
      the two differ by at most one bf16 step (<= 2^-7 of the value) when the fp32
      error straddles a rounding boundary; ``a`` bounds that fp32 error where a
      difference of large terms can cancel (RMSNorm backward, RoPE)
  attention o                   |got - ref| <= 2^-8 (2^-7 sum_j p_j |v_j| + |ref|) + 1e-6:
      the probabilities enter the value product as a bf16 hi + lo pair (relative error
      <= 2^-16 each; the 2^-7 factor leaves room for the fp32 exponentials), plus the
      output's rounding
  lse                           |got - ref| <= 1e-5 (1 + |ref|)   (fp32 sums)
  attention dq, dk, dv          (the backward run on the oracle's o and lse)
                                |err| <= 2e-2 rms(ref) + 2^-8 |ref| per element: the GEMM
      bar plus the bf16 rounding of the element itself (these gradients are heavy-
      tailed, max/rms > 10 for the first tokens of a sequence, where half a bf16 step
      of the largest element alone exceeds 2e-2 rms)
  residual add                  bitwise (the sum of two bf16 values is exact in fp32)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

from lora_fine_tuning_nf4_amd import lnf4  # noqa: E402
from oracle import decoder as od  # noqa: E402
import synthgen  # noqa: E402
from helpers import bf16_f64, dev_f32, dev_u16, host_f32, host_u16  # noqa: E402

EPS32 = 2.0 ** -23


def sync():
    torch.cuda.synchronize()


def bits(shape, seed, *keys, std=1.0, mean=0.0):
    return synthgen.to_bf16_bits(synthgen.normal_f32(shape, std, seed, *keys) + np.float32(mean))


def empty16(*shape):
    return torch.empty(shape, dtype=torch.int16, device="cuda")


def within(got, ref, extra=0.0, name=""):
    bound = 2.0 ** -7 * np.abs(ref) + extra
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{name}: {int(bad.sum())} beyond the bound, first {np.argwhere(bad)[0]}"


# ------------------------------------------------------------------ RMSNorm
@pytest.mark.parametrize("T,H", [(37, 264), (5, 4096), (1, 8)])
def test_rmsnorm_forward(T, H):
    x, g = bits((T, H), 1, "x", T, H, std=2.0), bits((H,), 1, "g", H, std=0.1, mean=1.0)
    y, r = empty16(T, H), torch.empty(T, dtype=torch.float32, device="cuda")
    lnf4.lnf4_rmsnorm_fwd(dev_u16(x), T, H, dev_u16(g), 1e-5, y, r)
    sync()
    ref, rref = od.rmsnorm(bf16_f64(x), bf16_f64(g), 1e-5)
    within(bf16_f64(host_u16(y)), od.q16(ref), name="y")
    assert np.all(np.abs(host_f32(r) - rref) <= 1e-6 * rref)


@pytest.mark.parametrize("T,H,res", [(19, 256, True), (3, 4096, False)])
def test_rmsnorm_backward(T, H, res):
    x, g = bits((T, H), 2, "x", std=2.0), bits((H,), 2, "g", std=0.1, mean=1.0)
    dy, dr = bits((T, H), 2, "dy"), bits((T, H), 2, "dres")
    xd, gd = dev_u16(x), dev_u16(g)
    r = torch.empty(T, dtype=torch.float32, device="cuda")
    lnf4.lnf4_rmsnorm_fwd(xd, T, H, gd, 1e-5, empty16(T, H), r)
    dx = empty16(T, H)
    lnf4.lnf4_rmsnorm_bwd(xd, T, H, gd, r, dev_u16(dy), dev_u16(dr) if res else None, dx)
    sync()
    x64, g64, dy64 = bf16_f64(x), bf16_f64(g), bf16_f64(dy)
    _, rr = od.rmsnorm(x64, g64, 1e-5)
    t1 = rr[:, None] * g64[None, :] * dy64
    t2 = x64 * (rr ** 3)[:, None] * np.mean(x64 * g64[None, :] * dy64, axis=1, keepdims=True)
    ref = od.rmsnorm_bwd(x64, g64, rr, dy64) + (bf16_f64(dr) if res else 0.0)
    extra = 64 * EPS32 * (np.abs(t1) + np.abs(t2) + (np.abs(bf16_f64(dr)) if res else 0.0))
    within(bf16_f64(host_u16(dx)), od.q16(ref), extra, "dx")


# ------------------------------------------------------------------ RoPE
@pytest.mark.parametrize("S,D,base", [(64, 64, 1e6), (2048, 128, 500000.0)])
def test_rope_table(S, D, base):
    tab = torch.empty(S * D, dtype=torch.float32, device="cuda")
    lnf4.lnf4_rope_table(S, D, base, tab)
    sync()
    c, s = od.rope_angles(S, S, D, base)
    got = host_f32(tab).reshape(S, D // 2, 2)
    assert np.all(np.abs(got[:, :, 0] - c) <= 2 * EPS32 / 2) and np.all(np.abs(got[:, :, 1] - s) <= 2 * EPS32 / 2)


@pytest.mark.parametrize("T,S,nh,D", [(130, 64, 3, 64), (256, 128, 8, 128)])
def test_rope_forward_and_inverse(T, S, nh, D):
    x = bits((T, nh * D), 3, "x", T, nh, D)
    base = 500000.0
    tab = torch.empty(S * D, dtype=torch.float32, device="cuda")
    lnf4.lnf4_rope_table(S, D, base, tab)
    xd = dev_u16(x)
    lnf4.lnf4_rope(xd, T, nh, D, S, tab, 0)
    sync()
    got = bf16_f64(host_u16(xd))
    c, s = od.rope_angles(T, S, D, base)
    x64 = bf16_f64(x)
    ref = od.rope(x64, c, s, nh, D)
    xh = np.abs(x64).reshape(T, nh, 2, D // 2)
    mag = np.broadcast_to((xh[:, :, 0] + xh[:, :, 1])[:, :, None, :], (T, nh, 2, D // 2)).reshape(T, nh * D)
    within(got, od.q16(ref), 8 * EPS32 * mag, "rope")
    lnf4.lnf4_rope(xd, T, nh, D, S, tab, 1)
    sync()
    back = bf16_f64(host_u16(xd))
    assert np.max(np.abs(back - x64)) <= 2.0 ** -6 * np.max(np.abs(x64))


# ------------------------------------------------------------------ SwiGLU, add
def test_swiglu_forward_backward_and_add():
    n = 8 * 1003
    g, u, ds = bits((n,), 4, "g", std=3.0), bits((n,), 4, "u"), bits((n,), 4, "ds")
    gd, ud, dsd = dev_u16(g), dev_u16(u), dev_u16(ds)
    s, dg, du, sm = empty16(n), empty16(n), empty16(n), empty16(n)
    lnf4.lnf4_swiglu_fwd(gd, ud, n, s)
    lnf4.lnf4_swiglu_bwd(gd, ud, dsd, n, dg, du)
    lnf4.lnf4_add(gd, ud, n, sm)
    sync()
    g64, u64, ds64 = bf16_f64(g), bf16_f64(u), bf16_f64(ds)
    rdg, rdu = od.swiglu_bwd(g64, u64, ds64)
    mag = np.abs(ds64 * u64) * (1 + np.abs(g64))
    within(bf16_f64(host_u16(s)), od.q16(od.swiglu(g64, u64)), 8 * EPS32 * np.abs(g64 * u64), "s")
    within(bf16_f64(host_u16(dg)), od.q16(rdg), 16 * EPS32 * mag, "dg")
    within(bf16_f64(host_u16(du)), od.q16(rdu), 8 * EPS32 * np.abs(ds64 * g64), "du")
    assert np.array_equal(host_u16(sm), od.nf4.bf16_rne_bits(g64 + u64))


# ------------------------------------------------------------------ attention
def _attn_case(T, S, nh, nkv, D, seed):
    q = bits((T, nh * D), seed, "q", T, nh, D)
    k = bits((T, nkv * D), seed, "k", T, nkv, D)
    v = bits((T, nkv * D), seed, "v", T, nkv, D)
    do = bits((T, nh * D), seed, "do", T, nh, D, std=0.1)
    return q, k, v, do


def _run_attention(q, k, v, do, T, S, nh, nkv, D, o_in, lse_in):
    """GPU forward, and GPU backward from the given o, lse (the oracle's, so that the
    backward is checked on its own inputs; the forward's own o differs from them within
    the forward's bound)."""
    qd, kd, vd, dod = dev_u16(q), dev_u16(k), dev_u16(v), dev_u16(do)
    o, lse = empty16(T, nh * D), torch.empty(nh * T, dtype=torch.float32, device="cuda")
    lnf4.lnf4_attn_fwd(qd, kd, vd, T, nh, nkv, D, S, o, lse)
    dq, dk, dv = empty16(T, nh * D), empty16(T, nkv * D), empty16(T, nkv * D)
    wsb = lnf4.lnf4_attn_bwd_workspace(T, nh, nkv, D)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    lnf4.lnf4_attn_bwd(qd, kd, vd, dev_u16(o_in), dev_f32(lse_in), dod, T, nh, nkv, D, S, dq, dk, dv, ws, wsb)
    sync()
    return (bf16_f64(host_u16(o)), host_f32(lse).reshape(nh, T), bf16_f64(host_u16(dq)), bf16_f64(host_u16(dk)),
            bf16_f64(host_u16(dv)))


def _attention(q, k, v, do, T, S, nh, nkv, D, sel_q=slice(None), sel_k=slice(None), nh_c=None, nkv_c=None):
    """Run the GPU kernels on the whole problem; check the selected heads against the oracle."""
    nh_c, nkv_c = nh_c or nh, nkv_c or nkv
    q64, k64, v64, do64 = bf16_f64(q[:, sel_q]), bf16_f64(k[:, sel_k]), bf16_f64(v[:, sel_k]), bf16_f64(do[:, sel_q])
    o_ref, lse_ref = od.attention(q64, k64, v64, nh_c, nkv_c, D, S)
    o16 = od.nf4.bf16_rne_bits(o_ref)
    # the backward's o and lse inputs: the oracle's for the checked heads (zero elsewhere)
    o_in = np.zeros((T, nh * D), np.uint16)
    o_in[:, sel_q] = o16
    lse_in = np.zeros((nh, T), np.float32)
    lse_in[: nh_c] = lse_ref
    o, lse, dq, dk, dv = _run_attention(q, k, v, do, T, S, nh, nkv, D, o_in, lse_in)
    o, lse, dq, dk, dv = o[:, sel_q], lse[:nh_c], dq[:, sel_q], dk[:, sel_k], dv[:, sel_k]
    pv, _ = od.attention(q64, k64, np.abs(v64), nh_c, nkv_c, D, S)
    bound = 2.0 ** -8 * (2.0 ** -7 * pv + np.abs(o_ref)) + 1e-6
    assert np.all(np.abs(o - o_ref) <= bound), np.max(np.abs(o - o_ref) - bound)
    assert np.all(np.abs(lse - lse_ref) <= 1e-5 * (1 + np.abs(lse_ref)))
    dq_r, dk_r, dv_r = od.attention_bwd(q64, k64, v64, bf16_f64(o16), lse_in[:nh_c].astype(np.float64), do64,
                                        nh_c, nkv_c, D, S)
    for name, g, r in (("dq", dq, dq_r), ("dk", dk, dk_r), ("dv", dv, dv_r)):
        check_grad(g, r, name)
    return o, lse, dq, dk, dv


def check_grad(got, ref, name):
    assert np.all(np.isfinite(got)), name
    rms = float(np.sqrt(np.mean(ref * ref)))
    excess = np.abs(got - ref) - (2e-2 * rms + 2.0 ** -8 * np.abs(ref))
    assert excess.max() <= 0, f"{name}: exceeds the bound by {excess.max():.3e} (rms {rms:.3e}) at {np.argmax(excess)}"


@pytest.mark.parametrize("T,S,nh,nkv,D", [(128, 64, 4, 2, 64), (256, 128, 8, 2, 128), (384, 128, 14, 2, 64),
                                          (192, 192, 4, 4, 128)])
def test_attention_matches_oracle(T, S, nh, nkv, D):
    print(f"attention T={T} S={S} heads={nh}/{nkv} D={D}", flush=True)
    q, k, v, do = _attn_case(T, S, nh, nkv, D, 5)
    _attention(q, k, v, do, T, S, nh, nkv, D)


def test_attention_8b_shape_one_kv_group():
    """The Llama-8B layer's attention (T = 2048, 32 query / 8 kv heads, D = 128) on the
    GPU; the oracle checks kv head 0 and its 4 query heads (the others are the same
    kernels on other columns)."""
    T, S, nh, nkv, D = 2048, 2048, 32, 8, 128
    q, k, v, do = _attn_case(T, S, nh, nkv, D, 6)
    _attention(q, k, v, do, T, S, nh, nkv, D, sel_q=slice(0, 4 * D), sel_k=slice(0, D), nh_c=4, nkv_c=1)


def test_attention_is_reproducible():
    T, S, nh, nkv, D = 256, 128, 4, 2, 128
    q, k, v, do = _attn_case(T, S, nh, nkv, D, 7)
    o_in = np.zeros((T, nh * D), np.uint16)
    lse_in = np.zeros((nh, T), np.float32)
    a = _run_attention(q, k, v, do, T, S, nh, nkv, D, o_in, lse_in)
    b = _run_attention(q, k, v, do, T, S, nh, nkv, D, o_in, lse_in)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
