"""Seeded synthetic activation tensors for the PlaneZip codec.

This module only makes inputs: it holds none of the codec's arithmetic, and
both the CPU oracle's tests and the HIP path's tests and benchmark read their
inputs from here, so that the two sides see the same bytes.

The PlaneZip paper's activations were recorded while five networks trained
on real datasets (§IV "Tensor capture"); those captures are not available, so
these generators stand in for them with the same shapes and the structure
that matters to the codec: ReLU and causal-mask zeros, exponent bits shared
between neighbours, dense near-incompressible normalised outputs, and
BF16 tensors obtained from FP32 by round-to-nearest-even, as the paper does
for its BF16 numbers (§IV).

Every tensor is returned as a ``Tensor`` holding its raw little-endian bytes
(uint8), the element-type code (0 = BF16, 1 = FP32, 2 = other) and the symbol
width the codec should use.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

BF16, FP32, OTHER = 0, 1, 2


@dataclass
class Tensor:
    name: str
    data: np.ndarray          # uint8, the tensor's bytes
    dtype: int                # 0 BF16, 1 FP32, 2 other
    elem_bits: int            # symbol width passed to the codec
    shape: tuple = field(default_factory=tuple)

    @property
    def nbytes(self) -> int:
        return int(self.data.size)

    def sha256(self) -> str:
        return hashlib.sha256(self.data.tobytes()).hexdigest()


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """FP32 -> BF16 bit patterns (uint16) by round-to-nearest-even; NaNs stay
    quiet NaNs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = ((u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), rounded)
    return rounded


def _bf16_tensor(name: str, x: np.ndarray) -> Tensor:
    return Tensor(name, bf16_rne(x).reshape(-1).view(np.uint8), BF16, 16, tuple(x.shape))


def _fp32_tensor(name: str, x: np.ndarray) -> Tensor:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return Tensor(name, x.reshape(-1).view(np.uint8), FP32, 32, tuple(x.shape))


def _gelu(x: np.ndarray) -> np.ndarray:
    from scipy.special import erf

    x = x.astype(np.float32)
    return (np.float32(0.5) * x * (np.float32(1.0) + erf(x / np.float32(np.sqrt(2.0))))).astype(np.float32)


def _causal_softmax(rng: np.random.Generator, batch: int, heads: int, seq: int) -> np.ndarray:
    """Softmax of N(0,1) logits over j <= i, exact zeros above the diagonal,
    in float32 with max-subtraction; returned as BF16 bit patterns."""
    out = np.empty((batch, heads, seq, seq), dtype=np.uint16)
    upper = np.triu(np.ones((seq, seq), dtype=bool), k=1)
    for b in range(batch):
        for h in range(heads):
            z = rng.standard_normal((seq, seq), dtype=np.float32)
            z[upper] = -np.inf
            z -= z.max(axis=1, keepdims=True)
            e = np.exp(z)
            e /= e.sum(axis=1, keepdims=True)
            e[upper] = 0.0
            out[b, h] = bf16_rne(e)
    return out


def _u16_block(values) -> np.ndarray:
    return np.asarray(values, dtype=np.uint64).astype("<u2")


def corner_blocks(seed: int = 100) -> np.ndarray:
    """64 BF16 corner-case blocks (64 symbols each), returned as uint16 (64, 64):
    (A) 12 zero blocks, (B) 13 constant blocks, (C) 13 Inf/NaN blocks,
    (D) 13 uniform random-bit blocks, (E) 13 alternating-sign blocks."""
    rng = np.random.default_rng(seed)
    blocks = []
    const = lambda v: np.full(64, v, dtype=np.uint16)

    def finite_bits(k):
        out = []
        while len(out) < k:
            v = int(rng.integers(0, 1 << 16))
            if (v & 0x7F80) != 0x7F80:
                out.append(v)
        return out

    # (A) all-zero: +0.0 and -0.0.
    blocks += [const(0x0000)] * 10 + [const(0x8000)] * 2
    # (B) constants: 1.0, -1.0, smallest subnormal, smallest normal, largest
    # finite, ~3.14, and 7 random finite constants.
    for v in [0x3F80, 0xBF80, 0x0001, 0x0080, 0x7F7F, 0x4049] + finite_bits(7):
        blocks.append(const(v))
    # (C) Inf / NaN patterns.
    for v in [0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0xFFFF]:
        blocks.append(const(v))
    blocks.append(np.array([0x7F80, 0xFF80] * 32, dtype=np.uint16))
    blocks.append(np.array([0x7F80, 0x7FC0] * 32, dtype=np.uint16))
    specials = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81], dtype=np.uint16)
    for _ in range(2):
        blocks.append(specials[rng.integers(0, specials.size, 64)])
    for _ in range(2):
        payload = rng.integers(1, 0x80, 64).astype(np.uint16)
        sign = rng.integers(0, 2, 64).astype(np.uint16) << 15
        blocks.append((sign | 0x7F80 | payload).astype(np.uint16))
    relu = bf16_rne(np.maximum(rng.standard_normal(64).astype(np.float32), 0))
    relu[::8] = 0x7F80
    blocks.append(relu)
    # (D) uniform random bits.
    for _ in range(13):
        blocks.append(rng.integers(0, 1 << 16, 64).astype(np.uint16))
    # (E) alternating sign.
    alt = lambda v: np.array([v, v | 0x8000] * 32, dtype=np.uint16)
    blocks.append(alt(0x3F80))
    for v in finite_bits(4):
        blocks.append(alt(v & 0x7FFF))
    for _ in range(4):
        mag = bf16_rne(np.abs(rng.standard_normal(64).astype(np.float32)))
        mag[1::2] |= 0x8000
        blocks.append(mag)
    for _ in range(2):
        r = bf16_rne(np.maximum(rng.standard_normal(64).astype(np.float32), 0))
        nz = r != 0
        flip = np.zeros(64, bool)
        flip[1::2] = True
        r[flip & nz] |= 0x8000
        blocks.append(r)
    blocks.append(np.array([0x0000, 0x8000] * 32, dtype=np.uint16))
    blocks.append(alt(0x0001))
    out = np.stack(blocks).astype(np.uint16)
    assert out.shape == (64, 64), out.shape
    return out


def relu_smoke() -> list[Tensor]:
    """Codec smoke test (BF16): ReLU(N(0,1)), 524,288 values from seed 0,
    followed by the 64 corner-case blocks (chunks 256 and 257)."""
    rng = np.random.default_rng(0)
    x = np.maximum(rng.standard_normal(524288, dtype=np.float32), np.float32(0))
    body = bf16_rne(x)
    full = np.concatenate([body, corner_blocks(100).reshape(-1)])
    return [Tensor("smoke_relu_corners", full.view(np.uint8), BF16, 16, (full.size,))]


def _box3x3(z: np.ndarray) -> np.ndarray:
    """3x3 box filter per (n, c) plane, zero padding, always divided by 9;
    the nine shifted views are summed in (dy, dx) row-major order in float32."""
    n, c, h, w = z.shape
    pad = np.zeros((n, c, h + 2, w + 2), dtype=np.float32)
    pad[:, :, 1:-1, 1:-1] = z
    acc = np.zeros_like(z)
    for dy in range(3):
        for dx in range(3):
            acc += pad[:, :, dy:dy + h, dx:dx + w]
    return acc / np.float32(9.0)


def cnn_feature_maps_fp32() -> list[Tensor]:
    """FP32 CNN feature maps: NCHW 32x64x56x56, ReLU(0.5 * box3x3(N(0,1)))
    from seed 1; about half the values are exact zeros and neighbours share
    exponent bits."""
    rng = np.random.default_rng(1)
    z = rng.standard_normal((32, 64, 56, 56), dtype=np.float32)
    y = np.maximum(_box3x3(z) * np.float32(0.5), np.float32(0))
    return [_fp32_tensor("cnn_relu_fp32", y)]


def gpt2_small_activations() -> list[Tensor]:
    """GPT-2 (124M) saved activations at batch 8, sequence 1024 (BF16), seed 2:
    MLP GELU output 8x1024x3072 and causal attention probabilities
    8x12x1024x1024 (exact zeros above the diagonal)."""
    rng = np.random.default_rng(2)
    g = _gelu(rng.standard_normal((8, 1024, 3072), dtype=np.float32))
    gelu = _bf16_tensor("gpt2_mlp_gelu", g)
    del g
    probs = _causal_softmax(rng, 8, 12, 1024)
    attn = Tensor("gpt2_attn_probs", probs.reshape(-1).view(np.uint8), BF16, 16, probs.shape)
    return [gelu, attn]


def vit_layernorm() -> list[Tensor]:
    """ViT-B/16 LayerNorm output 64x197x768, x*g + b with x ~ N(0,1),
    g ~ U(0.5, 1.5) and b ~ N(0, 0.1) per channel (0.1 read as the standard
    deviation), seed 3; as BF16 (RNE) and as FP32. Dense and nearly
    incompressible."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 197, 768), dtype=np.float32)
    g = rng.uniform(0.5, 1.5, 768).astype(np.float32)
    b = (rng.standard_normal(768) * 0.1).astype(np.float32)
    y = (x * g + b).astype(np.float32)
    return [_bf16_tensor("vit_layernorm_bf16", y), _fp32_tensor("vit_layernorm_fp32", y)]


def gpt2xl_activations() -> list[Tensor]:
    """GPT-2-XL saved activations at batch 8, sequence 1024, hidden 1600
    (BF16), seed 4: MLP GELU output 8x1024x6400, causal softmax scores
    8x25x1024x1024 and the residual stream 8x1024x1600 ~ N(0,1); about
    0.55 GB in total, coded as three separate tensors."""
    rng = np.random.default_rng(4)
    g = _gelu(rng.standard_normal((8, 1024, 6400), dtype=np.float32))
    gelu = _bf16_tensor("gpt2xl_mlp_gelu", g)
    del g
    probs = _causal_softmax(rng, 8, 25, 1024)
    attn = Tensor("gpt2xl_attn_probs", probs.reshape(-1).view(np.uint8), BF16, 16, probs.shape)
    del probs
    resid = _bf16_tensor("gpt2xl_residual", rng.standard_normal((8, 1024, 1600), dtype=np.float32))
    return [gelu, attn, resid]


# The workloads by name: generator and description.
WORKLOADS = {
    "relu-smoke": (relu_smoke, "codec smoke test: BF16 ReLU(N(0,1)) 1 MiB + 64 corner blocks"),
    "cnn-fp32": (cnn_feature_maps_fp32, "FP32 CNN feature maps NCHW 32x64x56x56, ReLU(0.5*box3x3(N(0,1)))"),
    "gpt2-small": (gpt2_small_activations, "GPT-2 124M BF16 activations, batch 8 seq 1024: GELU 8x1024x3072 "
                   "+ causal attention 8x12x1024x1024"),
    "vit-layernorm": (vit_layernorm, "ViT-B/16 LayerNorm output 64x197x768, BF16 and FP32"),
    "gpt2-xl": (gpt2xl_activations, "GPT-2-XL BF16 activations, batch 8 seq 1024: GELU 8x1024x6400 "
                "+ causal softmax 8x25x1024x1024 + residual 8x1024x1600"),
}


def workload(name: str) -> list[Tensor]:
    return WORKLOADS[name][0]()


def sample_blocks(t: Tensor, count: int, seed: int = 0) -> np.ndarray:
    """`count` whole 128-byte blocks of a tensor, chosen uniformly without
    replacement (the tensor must hold whole blocks)."""
    nb = t.nbytes // 128
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.choice(nb, size=min(count, nb), replace=False))
    return t.data[: nb * 128].reshape(nb, 128)[idx]


def edge_tensors(seed: int = 5) -> list[Tensor]:
    """Tensors outside the workloads: ragged tails, whole raw chunks, all-zero
    data, and random/ReLU data of awkward lengths, for both widths."""
    rng = np.random.default_rng(seed)
    out = []
    relu = bf16_rne(np.maximum(rng.standard_normal(1 << 16, dtype=np.float32), 0)).view(np.uint8)
    for n in [1, 2, 3, 5, 64, 127, 128, 129, 255, 256, 300, 4095, 4096, 4097, 8191, 8192, 8193]:
        out.append(Tensor(f"relu_bf16_{n}B", relu[:n].copy(), BF16, 16, (n,)))
    out.append(Tensor("random_64KiB", rng.integers(0, 256, 1 << 16, dtype=np.uint8), BF16, 16, (1 << 16,)))
    out.append(Tensor("zeros_64KiB", np.zeros(1 << 16, np.uint8), BF16, 16, (1 << 16,)))
    out.append(Tensor("zeros_64KiB_w32", np.zeros(1 << 16, np.uint8), FP32, 32, (1 << 16,)))
    f32 = np.maximum(rng.standard_normal(40000, dtype=np.float32), 0).view(np.uint8)
    for n in [4, 100, 4100, 40000 * 4 - 12]:
        out.append(Tensor(f"relu_fp32_{n}B", f32[:n].copy(), FP32, 32, (n,)))
    out.append(Tensor("relu_bf16_as_w32", relu[:20000].copy(), BF16, 32, (20000,)))
    return out


def dropout_mask(nbytes: int, keep: float = 0.9, seed: int = 6) -> Tensor:
    """One-byte 0/1 dropout masks, P(1) = keep; an 'other' type coded with
    32-bit symbols (§III-A)."""
    rng = np.random.default_rng(seed)
    m = (rng.random(nbytes) < keep).astype(np.uint8)
    return Tensor(f"dropout_mask_p{keep}", m, OTHER, 32, (nbytes,))


def int64_indices(count: int) -> Tensor:
    """int64 indices 1..count (all below 2**31, no zero low words), an 'other'
    type coded with 32-bit symbols."""
    a = np.arange(1, count + 1, dtype="<i8")
    return Tensor("int64_indices", a.view(np.uint8), OTHER, 32, (count,))


def mixed_large(nbytes: int, seed: int = 12) -> Tensor:
    """A BF16 tensor of any length (here: several GiB, so that its stream
    passes 4 GiB) built from 32 KB tiles in runs of sixteen: twelve tiles of
    uniform random bytes (chunks kept raw), one whose 128-byte blocks
    alternate random and all-zero, one repeating a ReLU(N(0,1)) tile, one
    all-zero and one zero in its first half. About 0.84 of the bytes stay
    raw."""
    rng = np.random.default_rng(seed)
    data = rng.integers(0, 256, nbytes, dtype=np.uint8)
    tile = 32768
    rows = data[: (nbytes // tile) * tile].reshape(-1, tile)
    relu = bf16_rne(np.maximum(rng.standard_normal(tile // 2, dtype=np.float32), np.float32(0)))
    rows[12::16].reshape(-1, tile // 256, 256)[:, :, 128:] = 0
    rows[13::16] = relu.view(np.uint8)
    rows[14::16] = 0
    rows[15::16, : tile // 2] = 0
    return Tensor(f"mixed_{nbytes}B", data, BF16, 16, (nbytes,))
