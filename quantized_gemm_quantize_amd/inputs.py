"""Seeded synthetic inputs for the W8A8 linear layer.

This module holds none of the layer's arithmetic: it draws random numbers,
rounds the activations to bf16 with PyTorch's own float32 -> bfloat16 cast,
and rearranges a dense int8 weight into block-sparse arrays (pure indexing).
Quantization, products and scaling are done by the code under test and by the
oracle, each on its own.

Workloads (shapes of the pages' examples):
  tiny              X [16,256],   W [128,256]
  decode            X [16,4096],  W [4096,4096]          (M-small, memory bound)
  prefill_outliers  X [2048,4096] with 1% of input channels x20, W [4096,4096]
  large_m           X [38400,1024], W [4096,1024]        (the A100 int8 vs fp16
                                                          shape in triton issue #634)
  bsr               X [16448,1280] (64 images x 257 tokens), W [5120,1280] as
                    64x64 blocks with 90% of the blocks zero (ViT-H MLP fc1 shape
                    from the bsr_dense_addmm warning in pytorch/ao PR #821)
  bsr_fc2           X [16448,5120], W [1280,5120] as 64x64 blocks with 80% of the
                    blocks zero (the ViT-H MLP fc2 shape of the same warning, at
                    the 0.8 linear sparsity of that benchmark command)
  sparse24          the prefill_outliers layer with a 2:4 weight: in every group
                    of 4 consecutive weights along K two are zero (the
                    semi-structured pattern of the pages' cuSPARSELt route)
  sparse24_decode   the decode layer with a 2:4 weight

Draw order from numpy.random.default_rng(seed) (PCG64): X ~ N(0,1) float32,
then the outlier channels, then W = 0.02 * N(0,1) float32, then the block mask,
then the 2:4 pattern (one of the 6 pairs of kept positions per group of 4,
uniform).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

CONFIGS = {
    "tiny": dict(M=16, K=256, N=128),
    "decode": dict(M=16, K=4096, N=4096),
    "prefill_outliers": dict(M=2048, K=4096, N=4096, outlier_frac=0.01, outlier_scale=20.0),
    "large_m": dict(M=38400, K=1024, N=4096),
    "bsr": dict(M=16448, K=1280, N=5120, bs=64, zero_frac=0.9),
    "bsr_fc2": dict(M=16448, K=5120, N=1280, bs=64, zero_frac=0.8),
    "sparse24": dict(M=2048, K=4096, N=4096, outlier_frac=0.01, outlier_scale=20.0,
                     sparse24=True),
    "sparse24_decode": dict(M=16, K=4096, N=4096, sparse24=True),
}

# Order of the configurations as the workload list states them.
CONFIG_ORDER = ["tiny", "decode", "prefill_outliers", "large_m", "bsr", "bsr_fc2", "sparse24",
                "sparse24_decode"]

# The 6 ways to keep 2 of 4 positions, as (p0, p1) with p0 < p1.
PAIRS_24 = [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]


@dataclass
class LinearInputs:
    """One synthetic linear layer: X as bf16 bit patterns, W as float32."""
    name: str
    x_bits: np.ndarray            # uint16 [M,K], bf16 bit patterns
    w: np.ndarray                 # float32 [N,K] (zero outside kept blocks for BSR)
    block_mask: np.ndarray | None = None   # bool [N/bs, K/bs] for BSR
    bs: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def M(self) -> int:
        return self.x_bits.shape[0]

    @property
    def K(self) -> int:
        return self.x_bits.shape[1]

    @property
    def N(self) -> int:
        return self.w.shape[0]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 with PyTorch's cast (nearest-even); return uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_inputs(name: str, seed: int = 0, M: int | None = None) -> LinearInputs:
    """Draw the named workload; M overrides the row count (same draw recipe)."""
    cfg = dict(CONFIGS[name])
    if M is not None:
        cfg["M"] = M
    return make_linear(cfg["M"], cfg["N"], cfg["K"], seed=seed,
                       outlier_frac=cfg.get("outlier_frac", 0.0),
                       outlier_scale=cfg.get("outlier_scale", 1.0),
                       bs=cfg.get("bs", 0), zero_frac=cfg.get("zero_frac", 0.0),
                       sparse24=cfg.get("sparse24", False), name=name)


def make_linear(M: int, N: int, K: int, seed: int = 0, outlier_frac: float = 0.0,
                outlier_scale: float = 1.0, bs: int = 0, zero_frac: float = 0.0,
                sparse24: bool = False, name: str = "random") -> LinearInputs:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    meta = {"seed": seed, "numpy": np.__version__}
    if outlier_frac > 0.0:
        n_out = int(round(outlier_frac * K))
        chans = rng.choice(K, n_out, replace=False)
        x[:, chans] *= np.float32(outlier_scale)
        meta["outlier_channels"] = np.sort(chans)
    w = np.float32(0.02) * rng.standard_normal((N, K), dtype=np.float32)
    mask = None
    if bs:
        nbr, nbc = N // bs, K // bs
        total = nbr * nbc
        n_keep = total - int(round(zero_frac * total))
        keep = rng.permutation(total)[:n_keep]
        mask = np.zeros(total, dtype=bool)
        mask[keep] = True
        mask = mask.reshape(nbr, nbc)
        dense_mask = np.repeat(np.repeat(mask, bs, axis=0), bs, axis=1)
        w = np.where(dense_mask, w, np.float32(0.0)).astype(np.float32)
        meta["nnzb"] = int(n_keep)
    if sparse24:
        assert K % 4 == 0
        pattern = rng.integers(0, len(PAIRS_24), size=(N, K // 4))
        keep = np.zeros((len(PAIRS_24), 4), dtype=bool)
        for i, (p0, p1) in enumerate(PAIRS_24):
            keep[i, [p0, p1]] = True
        w = np.where(keep[pattern].reshape(N, K), w, np.float32(0.0)).astype(np.float32)
        meta["sparse24"] = True
    return LinearInputs(name=name, x_bits=f32_to_bf16_bits(x), w=w, block_mask=mask, bs=bs,
                        meta=meta)


# W4A16 layers (pytorch/ao PR #153 benchmark shapes: M = 16 .. 1024 at N = K = 4096,
# group size 128, bf16 activations, scales and zeros).
W4A16_CONFIGS = {
    "w4a16_decode": dict(M=16, K=4096, N=4096, G=128),
    "w4a16": dict(M=1024, K=4096, N=4096, G=128),
}
W4A16_M = [16, 32, 128, 256, 512, 1024]


@dataclass
class W4A16Inputs:
    """One synthetic W4A16 layer: bf16 (or binary16) X, packed 4-bit weights, group scales and
    zeros in the same 16-bit format."""
    x_bits: np.ndarray       # uint16 [M,K], bf16 (half: binary16) bit patterns
    wq4: np.ndarray          # uint8 [N,K/2]: q[n,2j] in the low nibble of byte j, q[n,2j+1] high
    scales: np.ndarray       # uint16 [N,K/G], same format
    zeros: np.ndarray        # uint16 [N,K/G], same format
    G: int
    half: bool = False


def pack_u4(q: np.ndarray) -> np.ndarray:
    """u4 codes [N,K] -> bytes [N,K/2], even columns in the low nibble (bit placement only)."""
    q = np.asarray(q, np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def make_w4a16(M: int, N: int, K: int, G: int = 128, seed: int = 0,
               signed: bool = False, half: bool = False) -> W4A16Inputs:
    """X ~ N(0,1), codes uniform on 0..15, scales uniform on [0.004, 0.012) and zero points
    uniform on [6, 9) for unsigned codes (u4), on [-1.5, 1.5) for signed ones (s4, the codes
    read as -8..7), X, scales and zeros rounded to bf16 (half: to IEEE binary16): the
    magnitudes of a 4-bit group quantization of N(0, 0.02) weights. Draw order: X, codes,
    scales, zeros."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    scales = rng.uniform(0.004, 0.012, size=(N, K // G)).astype(np.float32)
    lo, hi = (-1.5, 1.5) if signed else (6.0, 9.0)
    zeros = rng.uniform(lo, hi, size=(N, K // G)).astype(np.float32)
    to16 = (lambda a: a.astype(np.float16).view(np.uint16)) if half else f32_to_bf16_bits
    return W4A16Inputs(x_bits=to16(x), wq4=pack_u4(q), scales=to16(scales), zeros=to16(zeros),
                       G=G, half=half)


def make_w4a16_inputs(name: str, seed: int = 0, M: int | None = None) -> W4A16Inputs:
    cfg = W4A16_CONFIGS[name]
    return make_w4a16(M if M is not None else cfg["M"], cfg["N"], cfg["K"], cfg["G"], seed)


def bsr_from_dense(w_dense: np.ndarray, block_mask: np.ndarray, bs: int):
    """Gather the kept bs x bs blocks of a dense [N,K] array into BSR arrays.

    crow int32 [N/bs+1], col int32 [nnzb] ascending within a block row, values
    [nnzb,bs,bs] with values[j][i][c] = w[r*bs+i, col[j]*bs+c] (each block row
    stays K-contiguous, like the dense [N,K] weight). Pure indexing.
    """
    N, K = w_dense.shape
    nbr, nbc = N // bs, K // bs
    assert block_mask.shape == (nbr, nbc)
    crow = np.zeros(nbr + 1, np.int32)
    crow[1:] = np.cumsum(block_mask.sum(axis=1))
    rows, cols = np.nonzero(block_mask)          # row-major order: ascending col per row
    blocks = w_dense.reshape(nbr, bs, nbc, bs).transpose(0, 2, 1, 3)
    values = np.ascontiguousarray(blocks[rows, cols])
    return crow, cols.astype(np.int32), values


def dense_from_bsr(crow: np.ndarray, col: np.ndarray, values: np.ndarray, N: int, K: int):
    """Scatter BSR arrays back to a dense [N,K] array (absent blocks are zero)."""
    bs = values.shape[1]
    out = np.zeros((N, K), dtype=values.dtype)
    for r in range(N // bs):
        for j in range(int(crow[r]), int(crow[r + 1])):
            c = int(col[j])
            out[r * bs:(r + 1) * bs, c * bs:(c + 1) * bs] = values[j]
    return out
