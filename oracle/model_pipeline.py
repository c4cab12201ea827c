"""fp64 oracle of the whole-model procedure around the layer solver.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's
CPU-baseline leg, never by the GPU library or its binding.

Sources:
  itwiki "GPTQ", section "최소 구현" (the paragraph after the sketch): the whole
    model is processed one transformer block at a time, front to back; the
    calibration inputs are run through the block while H is accumulated for each
    of its layers, the layers are quantized, and the quantized block's outputs are
    the next block's inputs ("sequential").
  molayo1419.me, "GPTQ를 밑바닥부터 구현하며 배운 것들", section 3: forward hooks
    capture the inputs that reach every nn.Linear during calibration, and every
    linear layer is quantized independently ("independent": all inputs come from
    the unquantized model).

Readings (the pages leave these open):
  - Within a block, one pass with the block's original weights collects every
    layer's H; all its layers are then quantized; a second pass with the quantized
    weights gives the next block's inputs.
  - The model is the GPT-2-style pre-LayerNorm block of the nanoGPT post: causal
    multi-head attention, exact (erf) GELU, LayerNorm eps 1e-5 with the biased
    variance; linear layers keep their biases, which are not quantized.
  - Every layer uses the same solver settings (bits, group, block size, damping).

Pinned in tests/test_oracle_pipeline.py against torch's own CPU layer norm,
attention and GELU in fp64, causality, the zero-weight identity, and the layer
solver on the captured inputs.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
from scipy.special import erf

from .gptq_oracle import (act_order_perm, damp, gptq_quantize, gptq_quantize_act_order, hessian,
                          inv_hessian_factor, output_error)

LINEARS = ("attn", "attn_proj", "fc", "fc_proj")


def layer_norm(x: np.ndarray, w: np.ndarray, b: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) * w + b over the last axis, biased variance."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * w + b


def gelu(x: np.ndarray) -> np.ndarray:
    """x * Phi(x) with the normal CDF written through erf."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(dh)) v with position i attending to positions <= i;
    q, k, v [S x H x T x dh]."""
    T, dh = q.shape[2], q.shape[3]
    s = q @ np.swapaxes(k, 2, 3) / math.sqrt(dh)
    s = np.where(np.triu(np.ones((T, T), dtype=bool), 1), -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=-1, keepdims=True)) @ v


def block_forward(p: Dict[str, np.ndarray], x: np.ndarray, n_head: int,
                  capture: Optional[Dict[str, List[np.ndarray]]] = None) -> np.ndarray:
    """One block on x [S x T x d]; when capture is given, the rows that reach each
    linear layer ([S*T x in]) are appended to capture[name]."""
    S, T, d = x.shape

    def lin(name, a):
        if capture is not None:
            capture.setdefault(name, []).append(a.reshape(-1, a.shape[-1]))
        return a @ p[name + "_w"].T + p[name + "_b"]

    h = layer_norm(x, p["ln1_w"], p["ln1_b"])
    qkv = lin("attn", h)
    dh = d // n_head
    q, k, v = (qkv[..., i * d:(i + 1) * d].reshape(S, T, n_head, dh).transpose(0, 2, 1, 3) for i in range(3))
    y = causal_attention(q, k, v).transpose(0, 2, 1, 3).reshape(S, T, d)
    x = x + lin("attn_proj", y)
    h = layer_norm(x, p["ln2_w"], p["ln2_b"])
    return x + lin("fc_proj", gelu(lin("fc", h)))


@dataclasses.dataclass
class LayerOutcome:
    H: np.ndarray            # 2 X^T X of the rows that reached the layer
    lam: float
    result: object           # GPTQResult or ActOrderResult
    err: float               # ||X (W0 - What)^T||^2


@dataclasses.dataclass
class BlockOutcome:
    inputs: List[np.ndarray]             # the block's calibration inputs, one per batch
    layers: Dict[str, LayerOutcome]
    weights: Dict[str, np.ndarray]       # parameters with What in place of W


def quantize_model(blocks: Sequence[Dict[str, np.ndarray]], x_batches: Sequence[np.ndarray], n_head: int,
                   bits: int, group_size: int = 0, block_size: int = 128, percdamp: float = 0.01,
                   act_order: bool = False, sequential: bool = True):
    """Quantize every linear layer of the blocks, front to back.

    sequential=True: each block's calibration inputs are the previous quantized
    block's outputs (the wiki page's procedure); False: the unquantized block's
    outputs (every layer quantized independently, as in the nanoGPT post).
    Returns (per-block outcomes, the last block's outputs).
    """
    xs = [np.asarray(x, dtype=np.float64) for x in x_batches]
    outcomes = []
    for params in blocks:
        p = {k: np.asarray(v, dtype=np.float64) for k, v in params.items()}
        cap: Dict[str, List[np.ndarray]] = {}
        ys = [block_forward(p, x, n_head, capture=cap) for x in xs]
        qp = dict(p)
        layers = {}
        for name in LINEARS:
            H = hessian(cap[name])
            W0 = p[name + "_w"]
            if act_order:
                perm = act_order_perm(H)
                Hl, lam = damp(H[np.ix_(perm, perm)], percdamp)
                r = gptq_quantize_act_order(W0, inv_hessian_factor(Hl), perm, bits, group_size, block_size)
            else:
                Hl, lam = damp(H, percdamp)
                r = gptq_quantize(W0, inv_hessian_factor(Hl), bits, group_size, block_size)
            layers[name] = LayerOutcome(H=H, lam=lam, result=r, err=output_error(W0, r.w_hat, H))
            qp[name + "_w"] = r.w_hat
        outcomes.append(BlockOutcome(inputs=xs, layers=layers, weights=qp))
        xs = [block_forward(qp, x, n_head) for x in xs] if sequential else ys
    return outcomes, xs
