"""Shared helpers for the parity tests: host <-> device transfer of bf16 bit patterns,
synthetic cases built with ``synthgen`` and quantized by the oracle, and the tolerance
check (max |err| <= 2e-2 * rms(ref) per output tensor, the ref being the fp64 oracle)."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

import synthgen
from oracle import lora as olora
from oracle import nf4 as onf4

TOL = 2e-2


def dev_u16(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16).copy()).cuda()


def dev_u8(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8).copy()).cuda()


def dev_f32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).copy()).cuda()


def host_u16(t) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16).copy()


def host_f32(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32)


def bf16_f64(bits) -> np.ndarray:
    return onf4.bf16_bits_to_f64(bits)


def check_tol(got: np.ndarray, ref: np.ndarray, name: str, tol: float = TOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    assert err <= tol * rms + 1e-30, f"{name}: max|err|={err:.3e} > {tol}*rms(ref)={tol * rms:.3e}"
    return err, rms


@dataclass
class LinearCase:
    """One projection: host arrays (oracle side) and their device copies (GPU side)."""
    T: int
    out_f: int
    in_f: int
    r: int
    scale: float
    fmt: int               # 0 NF4, 1 bf16
    w32: np.ndarray        # fp32 [out, in]
    codes: np.ndarray      # NF4 packed [out, in/2] (fmt 0)
    absmax: np.ndarray     # NF4 [out*in/64] (fmt 0)
    wbits: np.ndarray      # bf16 bits [out, in] (fmt 1)
    Wd: np.ndarray         # fp64 decoded / bf16 weight as the GEMM sees it
    A: np.ndarray          # bf16 bits [r, in]
    B: np.ndarray          # bf16 bits [out, r]
    x: np.ndarray          # bf16 bits [T, in]
    dy: np.ndarray         # bf16 bits [T, out]


def make_case(seed, T, out_f, in_f, r, alpha, fmt=0, tag="case", x=None) -> LinearCase:
    w32 = synthgen.weight_f32(out_f, in_f, seed, tag)
    if fmt == 0:
        codes, absmax = onf4.quantize(w32)
        Wd = onf4.decode_f64(codes, absmax)
        wbits = np.zeros((0,), np.uint16)
    else:
        codes, absmax = np.zeros((0,), np.uint8), np.zeros((0,), np.float32)
        wbits = synthgen.to_bf16_bits(w32)
        Wd = bf16_f64(wbits)
    A = synthgen.adapter_a_bits(r, in_f, seed, tag) if r > 0 else np.zeros((0, in_f), np.uint16)
    B = synthgen.adapter_b_bits(out_f, r, seed, tag) if r > 0 else np.zeros((out_f, 0), np.uint16)
    if x is None:
        x = synthgen.act_bits(T, in_f, seed, tag, "x")
    dy = synthgen.act_bits(T, out_f, seed, tag, "dy")
    scale = (alpha / r) if r > 0 else 0.0
    return LinearCase(T, out_f, in_f, r, scale, fmt, w32, codes, absmax, wbits, Wd, A, B, x, dy)


def oracle_fwd(c: LinearCase, adapters=True):
    if adapters and c.r > 0:
        return olora.linear_fwd(bf16_f64(c.x), c.Wd, bf16_f64(c.A), bf16_f64(c.B), c.scale)
    return olora.linear_fwd(bf16_f64(c.x), c.Wd)


def oracle_bwd(c: LinearCase, adapters=True):
    if adapters and c.r > 0:
        return olora.linear_bwd(bf16_f64(c.x), bf16_f64(c.dy), c.Wd, bf16_f64(c.A), bf16_f64(c.B), c.scale)
    return olora.linear_bwd(bf16_f64(c.x), bf16_f64(c.dy), c.Wd)


class DevCase:
    """Device copies of a LinearCase plus the lnf4 weight descriptor."""

    def __init__(self, c: LinearCase):
        import torch
        from lora_fine_tuning_nf4_amd import lnf4
        self.c = c
        if c.fmt == 0:
            self.wdata = dev_u8(c.codes)
            self.absmax = dev_f32(c.absmax)
        else:
            self.wdata = dev_u16(c.wbits)
            self.absmax = None
        self.W = lnf4.make_weight(c.fmt, self.wdata, self.absmax, c.out_f, c.in_f, 64)
        self.A = dev_u16(c.A) if c.r > 0 else None
        self.B = dev_u16(c.B) if c.r > 0 else None
        self.x = dev_u16(c.x)
        self.dy = dev_u16(c.dy)
        dev = torch.device("cuda")
        self.y = torch.empty((c.T, c.out_f), dtype=torch.int16, device=dev)
        self.u = torch.empty((max(c.T, 1), max(c.r, 1)), dtype=torch.float32, device=dev)
        self.dx = torch.empty((c.T, c.in_f), dtype=torch.int16, device=dev)
        self.dA = torch.empty((max(c.r, 1), c.in_f), dtype=torch.float32, device=dev)
        self.dB = torch.empty((c.out_f, max(c.r, 1)), dtype=torch.float32, device=dev)
