"""NF4 blockwise 4-bit weight format: code table, bf16 rounding, quantize, decode.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source.  The pages name the format and nothing more: the 4 GB-laptop Soup
article (section "Configuration and training") stores the frozen base with
``quantization: 4bit`` as NF4, and the Soup deep dive (section "What the
published numbers say and don't say") quotes its Llama-3.1-8B runs as "NF4
LoRA".  Everything below the name is a reading, stated once here:

* Code table.  16 levels built from standard-normal quantiles, with exactly
  -1, 0 and +1 among them: 8 positive levels at the quantiles of the
  probabilities 1/2 + j*(delta-1/2)/8, j = 1..8, 7 negative levels at minus
  the quantiles of 1/2 + j*(delta-1/2)/7, j = 1..7, and 0; all divided by the
  largest (the quantile of delta), so the ends are exactly -1 and +1.  delta is
  the mean of 1 - 1/30 and 1 - 1/32.  Computed in fp64, rounded once to fp32,
  sorted ascending: index 0 is -1, index 7 is 0, index 15 is +1.
* Blocks.  The [out, in] weight is flattened row-major and cut into blocks of
  64 consecutive elements (``in`` must be a multiple of 64, so a block never
  straddles a row).  Each block has one fp32 absmax = max |w| over the block.
* Quantize.  v = w / absmax in fp32 (IEEE division), code = the index i that
  minimises |v - T[i]| in fp32, the lowest index on a tie.  An all-zero block
  gets code 7 (the 0 level) everywhere.
* Packing.  Two codes per byte; byte j of a row holds element 2j in its high
  nibble and element 2j+1 in its low nibble.
* Decode.  w' = bf16_rne(fp32(T[code] * absmax)): one fp32 product, one
  round-to-nearest-even to bf16, no fused operation with anything else.
"""
from __future__ import annotations

import numpy as np
from scipy.special import ndtri  # inverse standard-normal CDF (library primitive)

BLOCKSIZE = 64
# outermost probability: the mean of 1 - 1/30 and 1 - 1/32
DELTA = 1.0 - (1.0 / 30.0 + 1.0 / 32.0) / 2.0


def nf4_levels_f64() -> np.ndarray:
    """The 16 NF4 levels in fp64, ascending (construction in the module header)."""
    pos = [ndtri(0.5 + j * (DELTA - 0.5) / 8.0) for j in range(1, 9)]
    neg = [-ndtri(0.5 + j * (DELTA - 0.5) / 7.0) for j in range(1, 8)]
    levels = np.array(sorted(neg + [0.0] + pos), dtype=np.float64)
    return levels / ndtri(DELTA)


def nf4_table() -> np.ndarray:
    """The code table T[0..15] as fp32 (the fp64 levels rounded once)."""
    return nf4_levels_f64().astype(np.float32)


# ---------------------------------------------------------------- bf16 rounding
def bf16_rne_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 with round-to-nearest-even; return the 16-bit patterns.

    bf16 keeps the top 16 bits of an fp32.  Round to nearest: add half an ulp
    of the kept part (0x7FFF) plus the kept part's lowest bit (so an exact tie
    goes to the even neighbour), then truncate.  A carry out of the mantissa
    moves into the exponent, which is the correct rounding (up to infinity on
    overflow).  NaNs map to a quiet NaN of the same sign.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    nan = np.isnan(f)
    if nan.any():
        r[nan] = ((u[nan] >> 16) & 0x8000) | 0x7FC0
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns to fp64 (exact)."""
    return bf16_bits_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------- quantize
def _nearest_codes(v: np.ndarray, table: np.ndarray) -> np.ndarray:
    """argmin_i |v - T[i]| in fp32 with ties to the lowest i (numpy argmin keeps the first)."""
    d = np.abs(v[:, None] - table[None, :])  # fp32 - fp32 -> fp32
    return np.argmin(d, axis=1).astype(np.uint8)


def quantize_codes(w, blocksize: int = BLOCKSIZE):
    """Quantize an fp32 [out, in] weight to unpacked codes [out, in] and absmax [out*in/blocksize]."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % blocksize != 0:
        raise ValueError("weight must be [out, in] with in a multiple of the blocksize")
    table = nf4_table()
    blocks = w.reshape(-1, blocksize)
    absmax = np.max(np.abs(blocks), axis=1).astype(np.float32)
    codes = np.full(blocks.shape, 7, dtype=np.uint8)
    step = max(1, (1 << 20) // blocksize)  # bound the [n, 16] temporaries
    for b0 in range(0, blocks.shape[0], step):
        sl = slice(b0, b0 + step)
        am = absmax[sl]
        nz = am > 0
        if not nz.any():
            continue
        v = (blocks[sl][nz] / am[nz, None]).astype(np.float32)  # fp32 IEEE division
        sub = codes[sl]
        sub[nz] = _nearest_codes(v.reshape(-1), table).reshape(v.shape)
        codes[sl] = sub
    return codes.reshape(w.shape), absmax


def pack_codes(codes) -> np.ndarray:
    """[out, in] codes (0..15) -> [out, in/2] bytes; element 2j in the high nibble."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    return ((c[:, 0::2] << 4) | c[:, 1::2]).astype(np.uint8)


def unpack_codes(packed) -> np.ndarray:
    """[out, in/2] bytes -> [out, in] codes (inverse of pack_codes)."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p >> 4
    out[:, 1::2] = p & 0x0F
    return out


def quantize(w, blocksize: int = BLOCKSIZE):
    """Quantize fp32 [out, in] -> (packed codes uint8 [out, in/2], absmax fp32 [out*in/blocksize])."""
    codes, absmax = quantize_codes(w, blocksize)
    return pack_codes(codes), absmax


# ---------------------------------------------------------------- decode
def decode_f32(packed, absmax, blocksize: int = BLOCKSIZE) -> np.ndarray:
    """fp32 products T[code] * absmax, shape [out, in] (before the bf16 rounding)."""
    codes = unpack_codes(packed)
    table = nf4_table()
    vals = table[codes].reshape(-1, blocksize)
    am = np.ascontiguousarray(absmax, dtype=np.float32).reshape(-1, 1)
    return (vals * am).astype(np.float32).reshape(codes.shape)  # one fp32 product


def decode_bf16_bits(packed, absmax, blocksize: int = BLOCKSIZE) -> np.ndarray:
    """Decoded weight W' as bf16 bit patterns [out, in]."""
    return bf16_rne_bits(decode_f32(packed, absmax, blocksize))


def decode_f64(packed, absmax, blocksize: int = BLOCKSIZE) -> np.ndarray:
    """Decoded weight W' (bf16 values) widened to fp64, for the GEMM definitions."""
    return bf16_bits_to_f64(decode_bf16_bits(packed, absmax, blocksize))
