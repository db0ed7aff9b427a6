"""Seeded synthetic inputs for the three block formats.

This module only draws random numbers and packs them into the byte layouts;
it holds no dequantisation or dot-product arithmetic.  It is the one module
that both the HIP path's tests/bench and the CPU checker read their inputs
from.

Distributions follow the Llama-8B-shaped decode workloads the pages measure:

* Q4_K ("Writing a high performant GEMV + dequant for Metal", section "What is
  a weight block?"): 144-byte super-blocks of 256 weights.  fp16 ``d`` and
  ``dmin`` ~ U(1e-3, 1e-2) rounded to nearest-even, the 12 packed scale/min
  bytes uniform (every 6-bit scale and min then uniform on 0..63), the 128
  nibble bytes uniform.
* NVFP4 W4A16 (Mojo ``fp4_gemv`` module page): nibble bytes uniform (all 16
  E2M1 codes), one E4M3 scale per 16 weights drawn as |N(0, 0.05)| and
  rounded to the nearest E4M3 value by torch's ``float8_e4m3fn`` cast.
* TQ1_0 ("metal: TQ1_0 kernel performance", section 1): 54-byte blocks of
  ``qs[48] | qh[4] | d``.  Trits iid uniform over {-1, 0, +1}, which is the
  same as drawing each qs byte uniformly from the 243 five-trit codes and
  each qh byte uniformly from the 81 four-trit codes (fifth trit zero).
  ``d`` ~ U(1e-2, 5e-2) in fp16.

* Dense fp16 / bf16 (the Mojo page's bf16 comparison GEMV): weights
  N(0, 0.02) rounded to nearest-even in the element type, [n][k] row-major.

Activations are fp16 (Q4_K, TQ1_0, dense fp16) or bf16 (NVFP4, dense bf16)
draws of N(0, 1); the epilogue's c vector is N(0, 1) in its element type.

All draws use numpy's PCG64 so a seed names one input exactly.
"""
from __future__ import annotations

import numpy as np

Q4K_BLOCK_BYTES = 144
TQ1_BLOCK_BYTES = 54
QK = 256  # weights per Q4_K / TQ1_0 block
NVFP4_SF = 16  # weights per E4M3 scale

# Seeds used by the tests and the bench: weight seed = 1000 + case,
# activation seed = 2000 + case.
W_SEED = 1000
X_SEED = 2000


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def tq1_codes(ntrits: int) -> np.ndarray:
    """Byte codes of all base-3 tuples of ``ntrits`` trits (most significant
    first), padded with zero trits to five.  Code of value v = ceil(256 v / 243),
    the smallest byte whose digits read back as v (an encoder, not a decoder)."""
    vals = np.arange(3 ** ntrits, dtype=np.int64) * 3 ** (5 - ntrits)
    return ((256 * vals + 242) // 243).astype(np.uint8)


def x_f16(k: int, seed: int) -> np.ndarray:
    """fp16 activations ~N(0,1) (round to nearest even), as uint16 bits."""
    return _rng(seed).standard_normal(k).astype(np.float16).view(np.uint16)


def x_bf16(k: int, seed: int) -> np.ndarray:
    """bf16 activations ~N(0,1) (round to nearest even), as uint16 bits."""
    import torch

    v = torch.from_numpy(_rng(seed).standard_normal(k).astype(np.float32))
    return v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def q4k_weights(n: int, k: int, seed: int) -> np.ndarray:
    """Q4_K matrix [n, k/256 * 144] uint8, row-major, K contiguous."""
    assert k % QK == 0
    nb = k // QK
    rng = _rng(seed)
    blk = rng.integers(0, 256, size=(n, nb, Q4K_BLOCK_BYTES), dtype=np.uint8)
    d = rng.uniform(1e-3, 1e-2, size=(n, nb)).astype(np.float16)
    dmin = rng.uniform(1e-3, 1e-2, size=(n, nb)).astype(np.float16)
    blk[:, :, 0:2] = d.view(np.uint8).reshape(n, nb, 2)
    blk[:, :, 2:4] = dmin.view(np.uint8).reshape(n, nb, 2)
    return blk.reshape(n, nb * Q4K_BLOCK_BYTES)


def nvfp4_weights(n: int, k: int, seed: int, sigma: float = 0.05) -> np.ndarray:
    """NVFP4 matrix as ONE buffer: n*k/2 nibble bytes ([n][k/2], even element
    in the low nibble) followed by n*k/16 E4M3 scale bytes ([n][k/16])."""
    import torch

    assert k % 32 == 0
    rng = _rng(seed)
    nib = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    s = np.abs(rng.standard_normal((n, k // NVFP4_SF)) * sigma).astype(np.float32)
    sc = torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.concatenate([nib.reshape(-1), sc.reshape(-1)])


def tq1_weights(n: int, k: int, seed: int) -> np.ndarray:
    """TQ1_0 matrix [n, k/256 * 54] uint8: per block qs[48] | qh[4] | fp16 d."""
    assert k % QK == 0
    nb = k // QK
    rng = _rng(seed)
    c5 = tq1_codes(5)
    c4 = tq1_codes(4)
    blk = np.empty((n, nb, TQ1_BLOCK_BYTES), dtype=np.uint8)
    blk[:, :, 0:48] = c5[rng.integers(0, c5.size, size=(n, nb, 48))]
    blk[:, :, 48:52] = c4[rng.integers(0, c4.size, size=(n, nb, 4))]
    d = rng.uniform(1e-2, 5e-2, size=(n, nb)).astype(np.float16)
    blk[:, :, 52:54] = d.view(np.uint8).reshape(n, nb, 2)
    return blk.reshape(n, nb * TQ1_BLOCK_BYTES)


def f16_weights(n: int, k: int, seed: int, sigma: float = 0.02) -> np.ndarray:
    """Dense fp16 matrix [n][k] as n*k*2 little-endian bytes."""
    v = (_rng(seed).standard_normal((n, k)) * sigma).astype(np.float16)
    return v.view(np.uint8).reshape(n, 2 * k)


def bf16_weights(n: int, k: int, seed: int, sigma: float = 0.02) -> np.ndarray:
    """Dense bf16 matrix [n][k] as n*k*2 little-endian bytes."""
    import torch

    v = torch.from_numpy((_rng(seed).standard_normal((n, k)) * sigma).astype(np.float32))
    bits = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return bits.view(np.uint8).reshape(n, 2 * k).copy()


# ---- exact-arithmetic inputs ------------------------------------------------
# Weights and activations whose every product and every partial sum is exact
# in fp32, in any summation order (as long as sum_i |x_i| |w_i| stays below
# 2^24 units of the finest product): the GEMV then has exactly one correct
# fp32 result per row.  Scale factors are powers of two, activations are -1,
# 0 or +1.  Only byte patterns are drawn here.

F16_POW2 = {-2: 0x3400, -1: 0x3800, 0: 0x3C00, 1: 0x4000}  # fp16 codes of 2^e
E4M3_POW2 = (0x28, 0x30, 0x38, 0x40, 0x48)  # OCP E4M3 codes of 2^-2 .. 2^2


def x_ternary(fmt: str, k: int, seed: int) -> np.ndarray:
    """Activations -1, 0 or +1 (equally likely) as fp16 or bf16 codes."""
    one = 0x3F80 if x_dtype(fmt) == "bf16" else 0x3C00
    t = _rng(seed).integers(-1, 2, size=k)
    return np.where(t == 0, 0, np.where(t > 0, one, one | 0x8000)).astype(np.uint16)


def q4k_weights_exact(n: int, k: int, seed: int, small: bool = False) -> np.ndarray:
    """Q4_K matrix with d = dmin = 1.0; scale bytes and nibbles uniform, or
    (small) every 6-bit scale and min below 16 (bytes 0-7 masked to their low
    nibble, whose top two bits feed groups 4-7)."""
    blk = q4k_weights(n, k, seed).reshape(n, k // QK, Q4K_BLOCK_BYTES)
    blk[:, :, 0:4] = np.frombuffer(np.uint16(F16_POW2[0]).tobytes() * 2, dtype=np.uint8)
    if small:
        blk[:, :, 4:12] &= 0x0F
    return blk.reshape(n, -1)


def nvfp4_weights_exact(n: int, k: int, seed: int) -> np.ndarray:
    """NVFP4 matrix with nibbles uniform and every scale a power of two in
    [1/4, 4], its sign bit random (the format ignores it)."""
    rng = _rng(seed)
    nib = rng.integers(0, 256, size=n * k // 2, dtype=np.uint8)
    sc = np.array(E4M3_POW2, dtype=np.uint8)[rng.integers(0, len(E4M3_POW2), size=n * k // NVFP4_SF)]
    sc |= (rng.integers(0, 2, size=sc.size) << 7).astype(np.uint8)
    return np.concatenate([nib, sc])


def tq1_weights_exact(n: int, k: int, seed: int) -> np.ndarray:
    """TQ1_0 matrix with trits uniform and d = +-2^e, e in -2..1."""
    blk = tq1_weights(n, k, seed).reshape(n, k // QK, TQ1_BLOCK_BYTES)
    rng = _rng(seed + 1)
    codes = np.array(list(F16_POW2.values()), dtype=np.uint16)[rng.integers(0, len(F16_POW2), size=blk.shape[:2])]
    codes |= (rng.integers(0, 2, size=codes.shape) << 15).astype(np.uint16)
    blk[:, :, 52:54] = codes.view(np.uint8).reshape(n, k // QK, 2)
    return blk.reshape(n, -1)


def dense_weights_exact(fmt: str, n: int, k: int, seed: int) -> np.ndarray:
    """Dense fp16 / bf16 matrix of integers -8..8 (exact in both types)."""
    v = _rng(seed).integers(-8, 9, size=(n, k)).astype(np.float32)
    if fmt == "f16":
        return v.astype(np.float16).view(np.uint8).reshape(n, 2 * k)
    return (v.view(np.uint32) >> 16).astype(np.uint16).view(np.uint8).reshape(n, 2 * k)


def weights_exact(fmt: str, n: int, k: int, seed: int, small: bool = False) -> np.ndarray:
    if fmt == "q4k":
        return q4k_weights_exact(n, k, seed, small)
    if fmt == "nvfp4":
        return nvfp4_weights_exact(n, k, seed)
    if fmt == "tq1":
        return tq1_weights_exact(n, k, seed)
    return dense_weights_exact(fmt, n, k, seed)


def weights(fmt: str, n: int, k: int, seed: int) -> np.ndarray:
    return {"q4k": q4k_weights, "nvfp4": nvfp4_weights, "tq1": tq1_weights,
            "f16": f16_weights, "bf16": bf16_weights}[fmt](n, k, seed)


def x_dtype(fmt: str) -> str:
    """Element type of the activations of a weight format."""
    return "bf16" if fmt in ("nvfp4", "bf16") else "f16"


def activations(fmt: str, k: int, seed: int) -> np.ndarray:
    return x_bf16(k, seed) if x_dtype(fmt) == "bf16" else x_f16(k, seed)


def vector(n: int, dtype: str, seed: int) -> np.ndarray:
    """N(0, 1) vector of n elements: float32 for "f32", else fp16 / bf16 codes."""
    if dtype == "f32":
        return _rng(seed).standard_normal(n).astype(np.float32)
    return x_bf16(n, seed) if dtype == "bf16" else x_f16(n, seed)


def weight_bytes(fmt: str, n: int, k: int) -> int:
    """Bytes of the packed weight buffer."""
    if fmt == "q4k":
        return n * (k // QK) * Q4K_BLOCK_BYTES
    if fmt == "tq1":
        return n * (k // QK) * TQ1_BLOCK_BYTES
    if fmt == "nvfp4":
        return n * k // 2 + n * k // NVFP4_SF
    if fmt in ("f16", "bf16"):
        return 2 * n * k
    raise ValueError(fmt)
