"""Seeded synthetic inputs for the KV-cache codec.

This module only draws numbers: it holds none of the codec's arithmetic and
is shared, unchanged, by the CPU oracle tests, the GPU parity tests and the
benchmark.  Every tensor it returns is bf16 (raw 16-bit patterns are what the
library consumes) except the sign vector, which is int8 +-1.

Recipes (one per workload; K and V use independent streams):

* ``roundtrip``: K, V ~ N(0, 1); per (layer, kv-head) four distinct channels
  are multiplied by 20 (outlier channels).
* ``decode_append``: K, V ~ N(0, 1) times a per-(layer, kv-head, channel)
  sigma ~ LogNormal(0, 0.5) shared by every sequence.
* ``prefill``: K, V ~ N(0, 1) with 1% of the entries (iid Bernoulli(0.01))
  replaced by Student-t with 3 degrees of freedom.
* ``normal``: K, V ~ N(0, 1).

Shapes are ``[layers, tokens, kv_heads, head_dim]``; a decode step's
``tokens`` axis is the sequence axis (one new token per sequence).

The value-path sign vector is one +-1 entry per head-dim element, shared by
every head and layer.  The pages draw it from a seeded RNG (seed 42) whose
stream is not reproducible here, so it is drawn from splitmix64 seeded with
42: entry j is +1 when the top bit of the (j+1)-th output is set, else -1.
"""
from __future__ import annotations

import numpy as np
import torch

_MASK64 = (1 << 64) - 1


def splitmix64_stream(seed: int, n: int) -> list[int]:
    """First ``n`` outputs of splitmix64 (Steele, Lea, Flood 2014)."""
    out = []
    state = seed & _MASK64
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        z = z ^ (z >> 31)
        out.append(z)
    return out


def sign_vector(head_dim: int, seed: int = 42) -> np.ndarray:
    """+-1 int8 vector of length ``head_dim`` (top bit of splitmix64 outputs)."""
    z = splitmix64_stream(seed, head_dim)
    return np.array([1 if (v >> 63) else -1 for v in z], dtype=np.int8)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _one_tensor(recipe: str, shape, seed: int, device) -> torch.Tensor:
    """Draw one bf16 tensor of ``shape`` = [L, T, H, d] layer by layer."""
    L, T, H, d = shape
    g = _gen(seed, device)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    if recipe == "decode_append":
        sigma = torch.exp(0.5 * _normal((L, 1, H, d), g, device))
    if recipe == "roundtrip":
        boost = torch.ones((L, 1, H, d), dtype=torch.float32, device=device)
        for layer in range(L):
            for h in range(H):
                ch = torch.randperm(d, generator=g, device=device)[:4]
                boost[layer, 0, h, ch] = 20.0
    for layer in range(L):
        x = _normal((T, H, d), g, device)
        if recipe == "roundtrip":
            x = x * boost[layer]
        elif recipe == "decode_append":
            x = x * sigma[layer]
        elif recipe == "prefill":
            pick = torch.rand((T, H, d), generator=g, device=device) < 0.01
            n = int(pick.sum().item())
            z = _normal((n,), g, device)
            chi2 = (_normal((n, 3), g, device) ** 2).sum(dim=1)
            x[pick] = z / torch.sqrt(chi2 / 3.0)
        elif recipe != "normal":
            raise ValueError(f"unknown recipe {recipe!r}")
        out[layer] = x.to(torch.bfloat16)
    return out


def kv_inputs(recipe: str, layers: int, tokens: int, kv_heads: int,
              head_dim: int, seed: int, device="cpu"):
    """(K, V) bf16 tensors of shape [layers, tokens, kv_heads, head_dim]."""
    shape = (layers, tokens, kv_heads, head_dim)
    k = _one_tensor(recipe, shape, 2 * seed, device)
    v = _one_tensor(recipe, shape, 2 * seed + 1, device)
    return k, v


def queries(batch: int, q_heads: int, head_dim: int, seed: int, device="cpu"):
    """bf16 decode queries [batch, q_heads, head_dim] ~ N(0, 1)."""
    g = _gen(seed, device)
    return _normal((batch, q_heads, head_dim), g, device).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a bf16 tensor as its raw uint16 patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


# Named workloads: (recipe, layers, tokens, kv_heads, head_dim, k_bits, v_bits, seed)
WORKLOADS = {
    "roundtrip_k8v3_d128": ("roundtrip", 1, 256, 8, 128, 8, 3, 1001),
    "decode_append_k8v3_d128": ("decode_append", 64, 32, 8, 128, 8, 3, 1002),
    "prefill_k8v3_d128": ("prefill", 64, 8192, 8, 128, 8, 3, 1003),
    "wide_k4v4_d256": ("normal", 48, 4096, 4, 256, 4, 4, 1004),
    "wide_k5v2_d512": ("normal", 48, 1024, 4, 512, 5, 2, 1005),
}

# Fused decode attention workload: batch, q_heads, kv_heads, head_dim, context
DECODE_ATTN = {"batch": 16, "q_heads": 32, "kv_heads": 8, "head_dim": 128,
               "context": 32768, "k_bits": 8, "v_bits": 3, "seed": 1006}


# ------------------------------------------------- paper-variant parameters
# The paper variant of the codec draws two d x d matrices once: a random
# rotation and, for its optional residual stage, a Gaussian projection.  They
# are random draws, so they are inputs here, given in bf16 like the cache rows.

def _bf16_of_f64(a: np.ndarray) -> np.ndarray:
    return bf16_bits(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(torch.bfloat16))


def dense_rotation(head_dim: int, seed: int = 43) -> np.ndarray:
    """Haar-random orthogonal [d, d] matrix as bf16 patterns: the Q factor of
    the QR decomposition of a standard normal matrix (numpy PCG64, ``seed``),
    its columns multiplied by the signs of R's diagonal so that the draw is
    uniform over the orthogonal group, then rounded to bf16."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((head_dim, head_dim))
    q, r = np.linalg.qr(g)
    q = q * np.where(np.diag(r) < 0, -1.0, 1.0)[None, :]
    return _bf16_of_f64(q)


def qjl_projection(head_dim: int, seed: int = 44) -> np.ndarray:
    """[d, d] matrix of iid N(0, 1) entries (numpy PCG64, ``seed``) as bf16 patterns."""
    rng = np.random.default_rng(seed)
    return _bf16_of_f64(rng.standard_normal((head_dim, head_dim)))


# ------------------------------------------------- arbitrary plane contents
# Decoders must accept any bytes a plane can hold, not only what the quantizer
# writes: the TurboQuant page's decoder edge suites cover zero, signed zero,
# fp16 subnormals and large scales, and a follow-up adds NaNs, infinities and
# arbitrary zero-point fractions ("Packed-value decode fusion investigation").

# fp16 patterns of those cases: +-0, the smallest and largest subnormals, the
# smallest normal, +-65504, +-Inf, NaNs of several payloads and signs, 1, -1,
# a fraction (0x3555 ~ 0.333) and 2^-5.
FP16_SPECIAL = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x83FF, 0x0400, 0x7BFF, 0xFBFF,
                         0x7C00, 0xFC00, 0x7E00, 0x7C01, 0xFE00, 0xFFFF, 0x3C00, 0xBC00, 0x3555,
                         0x1400], dtype=np.uint16)
FP16_SPECIAL_FINITE = FP16_SPECIAL[(FP16_SPECIAL & 0x7C00) != 0x7C00]


def _fp16_any(rng, shape, special):
    """Half uniformly random 16-bit patterns, a quarter drawn from `special`,
    a quarter finite with a random fraction and exponent field 1..30."""
    out = rng.integers(0, 1 << 16, size=shape, dtype=np.uint64).astype(np.uint16)
    pick = rng.random(shape)
    sp = pick < 0.25
    out[sp] = special[rng.integers(0, len(special), size=int(sp.sum()))]
    fin = (pick >= 0.25) & (pick < 0.5)
    n = int(fin.sum())
    out[fin] = ((rng.integers(0, 2, n) << 15) | (rng.integers(1, 31, n) << 10)
                | rng.integers(0, 1024, n)).astype(np.uint16)
    return out


def arbitrary_planes(lead, row_bytes: dict, seed: int, bounded: bool = False) -> dict:
    """Random contents for the five planes, shaped lead + [row bytes]
    (k_q, v_q as uint8; k_scale, k_zero, v_scale as uint16 fp16 patterns).

    Index bytes are uniform.  With bounded=False every fp16 element is
    arbitrary (any pattern, NaN and infinities included).  With bounded=True
    they are finite: zero points arbitrary (fractions, subnormals, signed
    zeros, up to +-65504), each key scale a random fp16 whose magnitude keeps
    (|zero| + 128) * |scale| below 4, subnormal or zero now and then, so that
    attention scores stay in a range where softmax is not one-hot; value
    scales any finite fp16."""
    rng = np.random.default_rng(seed)
    lead = tuple(lead)
    out = {}
    for n in ("k_q", "v_q"):
        out[n] = rng.integers(0, 256, size=lead + (row_bytes[n],), dtype=np.uint64).astype(np.uint8)
    gshape = lead + (row_bytes["k_scale"] // 2,)
    if not bounded:
        for n in ("k_scale", "k_zero", "v_scale"):
            out[n] = _fp16_any(rng, gshape, FP16_SPECIAL)
        return out
    zero = _fp16_any(rng, gshape, FP16_SPECIAL_FINITE)
    bad = (zero & 0x7C00) == 0x7C00
    zero[bad] &= 0x83FF                      # a non-finite draw becomes a subnormal
    zmag = np.abs(zero.view(np.float16).astype(np.float64))
    e = np.ceil(np.log2(zmag + 128.0)).astype(np.int64)      # |zero| + 128 <= 2^e
    field = 16 - e - rng.integers(0, 7, size=gshape)        # 2^(field - 15) * (1 + f) < 2^(2 - e)
    field[rng.random(gshape) < 0.1] = 0                     # subnormal or zero scales
    field = np.clip(field, 0, 30)
    scale = ((rng.integers(0, 2, size=gshape) << 15) | (field << 10)
             | rng.integers(0, 1024, size=gshape)).astype(np.uint16)
    vs = _fp16_any(rng, gshape, FP16_SPECIAL_FINITE)
    bad = (vs & 0x7C00) == 0x7C00
    vs[bad] &= 0x83FF
    out["k_scale"], out["k_zero"], out["v_scale"] = scale, zero, vs
    return out
