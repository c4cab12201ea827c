"""Seeded synthetic inputs for the GPTQ layer solver.

This module only draws random numbers and lays them out; it holds none of the
solver's arithmetic (no Hessian, no factorization, no quantizer).  Both the
fp64 oracle and the GPU path consume the exact bytes produced here.

Workloads (shapes follow the GPTQ wiki page, "minimal implementation" and
"results" sections, and the nanoGPT blog post, "results" section):

  1  one 512x512 layer, fp32, correlated AR(1) inputs (rho = 0.9), 2048 rows;
     4-bit per-row grid.  The wiki page's minimal-implementation section reports
     GPTQ against RTN on exactly this kind of input (512-dim, 2048 samples).
  2  nanoGPT-like stack: 6 blocks x {qkv 1152x384, attn-proj 384x384,
     fc 1536x384, fc-proj 384x1536}, fp32, 10 x 64 x 256 = 163840 calibration
     rows per layer, LayerNorm-like rows with 2% Student-t(3) outlier channels.
  3  4096x4096 attention projection, fp16, 262144 calibration rows with a
     rank-64 covariance and 1% outlier channels at 20x; 4-bit, group 128.
  4  MLP pair W_up 11008x4096 / W_down 4096x11008, fp16; X_down is a SiLU-gated
     product of two Gaussian streams; 3-bit per row.
  5  175B-class FFN shapes 49152x12288 / 12288x49152, fp16, X with a k^-1
     eigenvalue spectrum built from an exactly orthogonal Hadamard mix,
     streamed in 16384-row chunks; 3-bit, group 128.

Seeds: workload 1 uses ``default_rng(0)`` drawing W first, then Z.  All others
use ``default_rng(SeedSequence([0, workload, layer, tensor, chunk]))`` so that a
chunk can be regenerated on its own.  Values are drawn in float64 and cast by
round-to-nearest to the stated dtype.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterator, List, Optional

import numpy as np

CHUNK_ROWS = 16384

# tensor ids inside a workload's seed sequence
T_W, T_X, T_XPARAM = 0, 1, 2


def _rng(workload: int, layer: int, tensor: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([0, workload, layer, tensor, chunk]))


@dataclasses.dataclass
class LayerSpec:
    """One linear layer of a workload: W [d_row x d_col], X [n_rows x d_col]."""
    workload: int
    layer: int
    name: str
    d_row: int
    d_col: int
    n_rows: int
    w_dtype: str          # "f32" | "f16"
    x_dtype: str          # "f32" | "f16"
    w_std: float
    bits: int
    group_size: int       # 0 = one grid per row
    block_size: int = 128
    percdamp: float = 0.01
    x_kind: str = "ar1"   # ar1 | lnorm | lowrank | silu | powerlaw

    @property
    def np_w_dtype(self):
        return np.float16 if self.w_dtype == "f16" else np.float32

    @property
    def np_x_dtype(self):
        return np.float16 if self.x_dtype == "f16" else np.float32

    def scaled(self, d_row: Optional[int] = None, d_col: Optional[int] = None,
               n_rows: Optional[int] = None) -> "LayerSpec":
        """Same recipe at a smaller size (used for parity at oracle-friendly sizes)."""
        return dataclasses.replace(self, d_row=d_row or self.d_row,
                                   d_col=d_col or self.d_col,
                                   n_rows=n_rows or self.n_rows)


def workload_layers(workload: int) -> List[LayerSpec]:
    """The layers of one workload, at full size."""
    if workload == 1:
        return [LayerSpec(1, 0, "ar1_512", 512, 512, 2048, "f32", "f32", 0.02, 4, 0,
                          x_kind="ar1")]
    if workload == 2:
        out = []
        shapes = [("qkv", 1152, 384), ("attn_proj", 384, 384), ("fc", 1536, 384),
                  ("fc_proj", 384, 1536)]
        for blk in range(6):
            for k, (nm, dr, dc) in enumerate(shapes):
                out.append(LayerSpec(2, blk * 4 + k, f"h{blk}.{nm}", dr, dc, 10 * 64 * 256,
                                     "f32", "f32", 0.02, 4, 0, x_kind="lnorm"))
        return out
    if workload == 3:
        return [LayerSpec(3, 0, "attn_4096", 4096, 4096, 128 * 2048, "f16", "f16", 0.015,
                          4, 128, x_kind="lowrank")]
    if workload == 4:
        return [LayerSpec(4, 0, "w_up", 11008, 4096, 128 * 2048, "f16", "f16", 0.015, 3, 0,
                          x_kind="lowrank"),
                LayerSpec(4, 1, "w_down", 4096, 11008, 128 * 2048, "f16", "f16", 0.015, 3, 0,
                          x_kind="silu")]
    if workload == 5:
        return [LayerSpec(5, 0, "w_fc", 49152, 12288, 128 * 2048, "f16", "f16", 0.01, 3, 128,
                          x_kind="powerlaw"),
                LayerSpec(5, 1, "w_proj", 12288, 49152, 128 * 2048, "f16", "f16", 0.01, 3, 128,
                          x_kind="powerlaw")]
    raise ValueError(f"unknown workload {workload}")


# ---------------------------------------------------------------------------
# weights
# ---------------------------------------------------------------------------

def make_weight(spec: LayerSpec) -> np.ndarray:
    """W [d_row x d_col] = w_std * N(0, 1), cast to the layer's dtype."""
    if spec.workload == 1:
        rng = np.random.default_rng(0)
        w = spec.w_std * rng.standard_normal((spec.d_row, spec.d_col))
        return w.astype(spec.np_w_dtype)
    rng = _rng(spec.workload, spec.layer, T_W)
    w = spec.w_std * rng.standard_normal((spec.d_row, spec.d_col))
    return w.astype(spec.np_w_dtype)


# ---------------------------------------------------------------------------
# calibration inputs
# ---------------------------------------------------------------------------

def ar1_lower_factor(d: int, rho: float) -> np.ndarray:
    """Closed-form lower factor L of the AR(1) covariance S_ij = rho^|i-j|.

    L[k, 0] = rho^k and L[k, j] = sqrt(1 - rho^2) * rho^(k - j) for 1 <= j <= k.
    """
    k = np.arange(d)
    diff = k[:, None] - k[None, :]
    L = np.where(diff >= 0, np.power(rho, np.maximum(diff, 0).astype(np.float64)), 0.0)
    L[:, 1:] *= math.sqrt(1.0 - rho * rho)
    return L


def _ar1_rows(z: np.ndarray, rho: float) -> np.ndarray:
    """X = Z L^T with L the closed-form AR(1) factor, as a matrix product."""
    return z @ ar1_lower_factor(z.shape[1], rho).T


def _lowrank_params(spec: LayerSpec, rank: int = 64):
    rng = _rng(spec.workload, spec.layer, T_XPARAM)
    a = rng.standard_normal((rank, spec.d_col)) / math.sqrt(rank)
    n_out = max(1, int(round(0.01 * spec.d_col)))
    ch = np.sort(rng.choice(spec.d_col, size=n_out, replace=False))
    return a, ch


def _lnorm_params(spec: LayerSpec):
    rng = _rng(spec.workload, spec.layer, T_XPARAM)
    n_out = max(1, int(round(0.02 * spec.d_col)))
    return np.sort(rng.choice(spec.d_col, size=n_out, replace=False))


def _powerlaw_params(spec: LayerSpec):
    d = spec.d_col
    m = int(round(math.log2(d // 3)))
    if 3 * (1 << m) != d:
        raise ValueError("power-law recipe needs d_col = 3 * 2^m")
    rng = _rng(spec.workload, spec.layer, T_XPARAM)
    k = np.arange(1, d + 1, dtype=np.float64)
    hd = np.sum(1.0 / k)
    s = np.sqrt(d / (k * hd))                      # s_k^2 = d k^-1 / H_d: mean eigenvalue 1
    signs = rng.choice(np.array([-1.0, 1.0]), size=d)
    q3, r3 = np.linalg.qr(rng.standard_normal((3, 3)))
    q3 = q3 * np.sign(np.diag(r3))[None, :]
    perm = rng.permutation(d)
    return m, s, signs, q3, perm


def _fwht_rows(y: np.ndarray) -> np.ndarray:
    """Unnormalized Walsh-Hadamard transform along the last axis (length 2^m)."""
    y = y.copy()
    n = y.shape[-1]
    h = 1
    while h < n:
        v = y.reshape(*y.shape[:-1], n // (2 * h), 2, h)
        a = v[..., 0, :].copy()
        b = v[..., 1, :]
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        h *= 2
    return y


def make_x_chunk(spec: LayerSpec, chunk: int, rows: Optional[int] = None) -> np.ndarray:
    """Rows [chunk*CHUNK_ROWS, ...) of X, row-major [rows x d_col] in the layer's dtype.

    Workload 1 is a single 2048-row chunk drawn from ``default_rng(0)`` after W.
    """
    d = spec.d_col
    if spec.workload == 1:
        if chunk != 0:
            raise ValueError("workload 1 has one chunk")
        rng = np.random.default_rng(0)
        rng.standard_normal((spec.d_row, spec.d_col))          # W is drawn first
        z = rng.standard_normal((spec.n_rows, d))
        return _ar1_rows(z, 0.9).astype(spec.np_x_dtype)
    start = chunk * CHUNK_ROWS
    nr = rows if rows is not None else min(CHUNK_ROWS, spec.n_rows - start)
    if nr <= 0:
        raise ValueError("chunk out of range")
    rng = _rng(spec.workload, spec.layer, T_X, chunk)
    if spec.x_kind == "ar1":
        x = _ar1_rows(rng.standard_normal((nr, d)), 0.9)
    elif spec.x_kind == "lnorm":
        g = rng.standard_normal((nr, d))
        mu = g.mean(axis=1, keepdims=True)
        var = g.var(axis=1, keepdims=True)
        x = (g - mu) / np.sqrt(var + 1e-5)
        ch = _lnorm_params(spec)
        x[:, ch] = rng.standard_t(3.0, size=(nr, ch.size))
    elif spec.x_kind == "lowrank":
        a, ch = _lowrank_params(spec)
        x = rng.standard_normal((nr, a.shape[0])) @ a
        x[:, ch] *= 20.0
    elif spec.x_kind == "silu":
        a = rng.standard_normal((nr, d))
        b = rng.standard_normal((nr, d))
        x = a / (1.0 + np.exp(-a)) * b
    elif spec.x_kind == "powerlaw":
        m, s, signs, q3, perm = _powerlaw_params(spec)
        y = rng.standard_normal((nr, d)) * s * signs
        y = y.reshape(nr, 3, 1 << m)
        y = np.einsum("ab,rbk->rak", q3, y)
        y = _fwht_rows(y) * (2.0 ** (-m / 2.0))
        y = y.reshape(nr, d)
        x = np.empty_like(y)
        x[:, perm] = y
    else:
        raise ValueError(spec.x_kind)
    return x.astype(spec.np_x_dtype)


def n_chunks(spec: LayerSpec) -> int:
    if spec.workload == 1:
        return 1
    return (spec.n_rows + CHUNK_ROWS - 1) // CHUNK_ROWS


def iter_x_chunks(spec: LayerSpec) -> Iterator[np.ndarray]:
    for c in range(n_chunks(spec)):
        yield make_x_chunk(spec, c)


def make_x(spec: LayerSpec) -> np.ndarray:
    """All of X as one array (only for sizes that fit comfortably in host memory)."""
    if spec.workload == 1:
        return make_x_chunk(spec, 0)
    out = np.empty((spec.n_rows, spec.d_col), dtype=spec.np_x_dtype)
    for c in range(n_chunks(spec)):
        s = c * CHUNK_ROWS
        out[s:s + CHUNK_ROWS] = make_x_chunk(spec, c)
    return out


def tiny_case(seed: int, d_row: int, d_col: int, n_rows: int, corr: float = 0.8,
              dtype=np.float64):
    """Small correlated case for tests: W ~ 0.02 N(0,1), AR(1)-correlated X."""
    rng = np.random.default_rng(np.random.SeedSequence([1, seed, d_row, d_col, n_rows]))
    w = 0.02 * rng.standard_normal((d_row, d_col))
    x = _ar1_rows(rng.standard_normal((n_rows, d_col)), corr)
    return w.astype(dtype), x.astype(dtype)


# ---------------------------------------------------------------------------
# synthetic GPT-style model (random weights) for the model-level procedure
# ---------------------------------------------------------------------------
# The wiki page's description of the whole-model procedure (blocks one at a time,
# each quantized block's outputs feeding the next) needs a model; the nanoGPT
# post's model is a GPT-2-style stack.  Only the seeded parameters and the block-0
# inputs live here: the fp64 oracle and the GPU-side torch module each implement
# the block's forward pass on their own.

GPT_WORKLOAD = 6
GPT_LINEARS = ("attn", "attn_proj", "fc", "fc_proj")   # [out x in]: 3d x d, d x d, 4d x d, d x 4d


@dataclasses.dataclass(frozen=True)
class GPTSpec:
    """A pre-LayerNorm GPT-2-style stack: x += attn_proj(attention(attn(ln1(x))));
    x += fc_proj(gelu(fc(ln2(x)))), causal attention with n_head heads."""
    n_block: int = 6
    d: int = 384
    n_head: int = 6
    seq: int = 256
    n_seq: int = 64          # sequences per calibration batch
    n_batch: int = 10
    w_std: float = 0.02
    bits: int = 4
    group_size: int = 0
    block_size: int = 128
    percdamp: float = 0.01

    @property
    def tokens(self) -> int:
        return self.n_seq * self.seq * self.n_batch


def gpt_block_params(spec: GPTSpec, block: int) -> dict:
    """fp32 parameters of one block: linear weights w_std * N(0, 1), biases
    0.02 * N(0, 1), LayerNorm gains 1 + 0.1 * N(0, 1) and shifts 0.02 * N(0, 1)."""
    rng = _rng(GPT_WORKLOAD, block, T_W)
    d = spec.d
    shapes = {"attn": (3 * d, d), "attn_proj": (d, d), "fc": (4 * d, d), "fc_proj": (d, 4 * d)}
    p = {}
    for ln in ("ln1", "ln2"):
        p[ln + "_w"] = 1.0 + 0.1 * rng.standard_normal(d)
        p[ln + "_b"] = 0.02 * rng.standard_normal(d)
    for name in GPT_LINEARS:
        p[name + "_w"] = spec.w_std * rng.standard_normal(shapes[name])
        p[name + "_b"] = 0.02 * rng.standard_normal(shapes[name][0])
    return {k: v.astype(np.float32) for k, v in p.items()}


def gpt_embeddings(spec: GPTSpec, batch: int) -> np.ndarray:
    """Block-0 inputs of one calibration batch, fp32 [n_seq x seq x d]: the
    LayerNorm-like recipe with 2% Student-t(3) outlier channels."""
    layer = LayerSpec(GPT_WORKLOAD, 10_000, "emb", spec.d, spec.d, spec.n_seq * spec.seq, "f32", "f32",
                      0.0, spec.bits, 0, x_kind="lnorm")
    x = make_x_chunk(layer, batch, rows=spec.n_seq * spec.seq)
    return x.reshape(spec.n_seq, spec.seq, spec.d)
