"""Seeded synthetic inputs, shared by the oracle tests and the GPU path.

This module only draws random numbers and describes workload shapes; it holds
none of the method's arithmetic (no code table, no quantization, no GEMM).
Conversion of random fp32 draws to bf16 goes through torch's own conversion.

Distributions (the pages train on real checkpoints and datasets, which are not
used here; these synthetic stand-ins have the checkpoints' layer shapes):
  frozen weight W   ~ N(0, 0.02)            fp32, later quantized to NF4
  adapter A         ~ U(-1/sqrt(in), +1/sqrt(in))   bf16 (PyTorch Linear default init)
  adapter B         ~ N(0, 0.01)            bf16
  activations x     ~ N(0, 1)               bf16
  output grads dy   ~ N(0, 1)               bf16
  token ids         ~ U{0, ..., vocab-1}    int32 (inputs and labels)
Every tensor has its own stream, keyed by (seed, workload, layer, name).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

# ------------------------------------------------------------------ workloads
PROJ_ORDER = ("q", "k", "v", "o", "gate", "up", "down")


def _decoder_shapes(hidden: int, q_heads: int, kv_heads: int, head_dim: int, inter: int):
    q = q_heads * head_dim
    kv = kv_heads * head_dim
    return {
        "q": (q, hidden), "k": (kv, hidden), "v": (kv, hidden), "o": (hidden, q),
        "gate": (inter, hidden), "up": (inter, hidden), "down": (hidden, inter),
    }


@dataclass(frozen=True)
class Workload:
    name: str
    tokens: int                  # T = batch x seq per step
    shapes: dict                 # projection -> (out, in)
    rank: int
    alpha: float
    adapted: tuple               # projections carrying adapters
    layers: int = 1
    fmt: str = "nf4"             # "nf4" or "bf16" frozen weights
    vocab: int = 0               # embed / lm_head rows for the head slot (0: no slot)
    hidden: int = 0
    passes: tuple = ("fwd", "recompute", "bwd")
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return self.alpha / self.rank


def _arch(n_heads: int, n_kv: int, head_dim: int, seq_len: int, eps: float, rope_base: float):
    """What a whole decoder layer needs beyond the projection shapes (the configs give the
    head counts and dims; eps and the RoPE base are the models' published values)."""
    return {"arch": {"n_heads": n_heads, "n_kv": n_kv, "head_dim": head_dim, "seq_len": seq_len, "eps": eps,
                     "rope_base": rope_base}}


WORKLOADS = {
    # single 896x896 linear, r8 alpha16, 256 tokens
    "linear896": Workload("linear896", 256, {"w": (896, 896)}, 8, 16.0, ("w",)),
    # Qwen2.5-0.5B-shaped layer x24, batch 4 x seq 512, r16 on all seven
    "qwen05b": Workload("qwen05b", 4 * 512, _decoder_shapes(896, 14, 2, 64, 4864), 16, 32.0,
                        PROJ_ORDER, layers=24, hidden=896, extra=_arch(14, 2, 64, 512, 1e-6, 1e6)),
    # Llama-3.1-8B-shaped stack x32 + head slot, batch 1 x seq 2048, r8 alpha32 on q, v
    "llama8b": Workload("llama8b", 2048, _decoder_shapes(4096, 32, 8, 128, 14336), 8, 32.0,
                        ("q", "v"), layers=32, vocab=128256, hidden=4096,
                        extra=_arch(32, 8, 128, 2048, 1e-5, 500000.0)),
    # Qwen2.5-3B-shaped bf16 stack x36, batch 2 x seq 1024, r16 on all seven
    "qwen3b_bf16": Workload("qwen3b_bf16", 2 * 1024, _decoder_shapes(2048, 16, 2, 128, 11008), 16, 32.0,
                            PROJ_ORDER, layers=36, fmt="bf16", hidden=2048,
                            extra=_arch(16, 2, 128, 1024, 1e-6, 1e6)),
    # DPO step on the llama8b stack: 2 pairs x (chosen, rejected) x 1024 tokens
    # (beta: the preference loss's temperature; the pages give none, 0.1 is the common default)
    "llama8b_dpo": Workload("llama8b_dpo", 2 * 2 * 1024, _decoder_shapes(4096, 32, 8, 128, 14336), 8, 32.0,
                            ("q", "v"), layers=32, vocab=128256, hidden=4096,
                            passes=("ref", "fwd", "recompute", "bwd"),
                            extra={"seq_len": 1024, "beta": 0.1, **_arch(32, 8, 128, 1024, 1e-5, 500000.0)}),
}

# q, k, v share the attention input; gate, up share the MLP input
GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


# ------------------------------------------------------------------ host draws
def rng(seed: int, *keys) -> np.random.Generator:
    """A numpy Generator whose stream is fixed by (seed, keys)."""
    h = hashlib.sha256(repr((int(seed),) + tuple(str(k) for k in keys)).encode()).digest()
    return np.random.Generator(np.random.PCG64(int.from_bytes(h[:16], "little")))


def normal_f32(shape, std: float, seed: int, *keys) -> np.ndarray:
    return (rng(seed, *keys).standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def uniform_f32(shape, bound: float, seed: int, *keys) -> np.ndarray:
    return rng(seed, *keys).uniform(-bound, bound, size=shape).astype(np.float32)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp32 values, via torch's conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def weight_f32(out_f: int, in_f: int, seed: int, *keys) -> np.ndarray:
    return normal_f32((out_f, in_f), 0.02, seed, "W", *keys)


def adapter_a_bits(r: int, in_f: int, seed: int, *keys) -> np.ndarray:
    return to_bf16_bits(uniform_f32((r, in_f), 1.0 / np.sqrt(in_f), seed, "A", *keys))


def adapter_b_bits(out_f: int, r: int, seed: int, *keys, std: float = 0.01) -> np.ndarray:
    return to_bf16_bits(normal_f32((out_f, r), std, seed, "B", *keys))


def act_bits(rows: int, cols: int, seed: int, *keys) -> np.ndarray:
    return to_bf16_bits(normal_f32((rows, cols), 1.0, seed, "act", *keys))


def token_ids(n: int, vocab: int, seed: int, *keys) -> np.ndarray:
    """n uniform random token ids in [0, vocab), int32."""
    return rng(seed, "ids", *keys).integers(0, vocab, size=n).astype(np.int32)


# ------------------------------------------------------------------ device draws
def device_normal(shape, std: float, seed: int, *keys, dtype=None, device="cuda"):
    """torch normal draws made on the device (large workloads), keyed like the host draws."""
    import torch
    h = hashlib.sha256(repr((int(seed),) + tuple(str(k) for k in keys)).encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
    return t if dtype is None else t.to(dtype)


def device_uniform(shape, bound: float, seed: int, *keys, dtype=None, device="cuda"):
    import torch
    h = hashlib.sha256(repr((int(seed),) + tuple(str(k) for k in keys)).encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    t = (torch.rand(shape, generator=g, device=device, dtype=torch.float32) * 2.0 - 1.0) * bound
    return t if dtype is None else t.to(dtype)


def device_token_ids(n: int, vocab: int, seed: int, *keys, device="cuda"):
    """n uniform random token ids in [0, vocab) drawn on the device, int32."""
    import torch
    h = hashlib.sha256(repr((int(seed),) + tuple(str(k) for k in keys)).encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    return torch.randint(0, vocab, (n,), generator=g, device=device, dtype=torch.int64).to(torch.int32)
