"""Whole-model quantization around the layer solver.

itwiki "GPTQ", section "최소 구현" (the paragraph after the sketch): the model is
processed one transformer block at a time, front to back; the calibration inputs
are run through the block while H is accumulated for each of its layers, the
layers are quantized, and the quantized block's outputs become the next block's
inputs.  molayo1419.me (nanoGPT post), section 3: forward hooks capture the inputs
of every nn.Linear and each layer is quantized independently -- the
``sequential=False`` mode here (every block sees the unquantized model's
activations).

Per block: one pass of every calibration batch with forward pre-hooks on the
block's nn.Linear layers, each hook adding 2 X^T X of that layer's input rows to
the layer's H on the device (gptq_hessian_accumulate -- the activations are never
stored); then for each layer the damped factor and the lazy-batch loop (or their
act-order forms), and What written back into the layer's weight
(gptq_dequantize); then, in sequential mode, a second pass with the quantized
weights whose outputs are the next block's inputs.  Every quantizer step runs in
the library's kernels on the current stream; the forward passes are the caller's
model.  Biases are left as they are.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

from . import (NotPositiveDefinite, _torch, gptq_act_order_perm, gptq_dequantize, gptq_hessian_accumulate,
               gptq_prepare_hinv, gptq_prepare_hinv_perm, gptq_quantize_layer, gptq_quantize_layer_perm)


@dataclasses.dataclass
class LayerQuant:
    codes: object            # uint8 [out x in], original column order
    scales: object           # fp32 [out x n_groups]
    zeros: object            # int32 [out x n_groups]
    err: object              # fp64 [1]: ||X (W0 - What)^T||^2 over the layer's calibration rows
    lam: object              # fp32 [1]
    perm: object = None      # act-order: the quantization order
    g_idx: object = None     # act-order: column -> group
    H: object = None         # the layer's H (kept on request)


@dataclasses.dataclass
class BlockQuant:
    layers: Dict[str, LayerQuant]
    inputs: Optional[List[object]] = None   # the block's calibration inputs (kept on request)


def linear_layers(block) -> List:
    """(name, module) of every nn.Linear in the block, in registration order."""
    torch = _torch()
    return [(n, m) for n, m in block.named_modules() if isinstance(m, torch.nn.Linear)]


def quantize_model(blocks: Sequence, x_batches: Sequence, bits: int, group_size: int = 0,
                   block_size: int = 128, percdamp: float = 0.01, act_order: bool = False,
                   sequential: bool = True, keep_inputs: bool = False, keep_hessians: bool = False,
                   stream=None):
    """Quantize every nn.Linear of ``blocks`` (torch modules on the GPU, each mapping
    a batch to the next block's input), front to back, with ``x_batches`` (device
    tensors) as the first block's calibration inputs.  The layers' weights are
    replaced by What in place.  Returns (per-block results, the last block's
    outputs for the batches).  Raises NotPositiveDefinite if a layer's damped H
    could not be factored (checked once per block, before any weight of that
    block is replaced, so the block's weights are then left as they were)."""
    torch = _torch()
    xs = list(x_batches)
    results = []
    with torch.no_grad():
        for block in blocks:
            lins = linear_layers(block)
            Hs = {n: torch.zeros(m.in_features, m.in_features, dtype=torch.float32, device=m.weight.device)
                  for n, m in lins}

            def hook_for(name, width):
                def hook(_mod, inp):
                    x = inp[0].reshape(-1, width)
                    gptq_hessian_accumulate(Hs[name], x if x.is_contiguous() else x.contiguous(), stream=stream)
                return hook

            handles = [m.register_forward_pre_hook(hook_for(n, m.in_features)) for n, m in lins]
            ys = []                    # the unquantized block's outputs, kept for independent mode
            try:
                for x in xs:
                    y = block(x)
                    if not sequential:
                        ys.append(y)
            finally:
                for h in handles:
                    h.remove()
            layers, infos = {}, []
            for n, m in lins:
                W0 = m.weight.data
                if act_order:
                    perm = gptq_act_order_perm(Hs[n], stream=stream)
                    U, lam, info = gptq_prepare_hinv_perm(Hs[n], perm, percdamp, stream=stream)
                    codes, scales, zeros, g_idx, err = gptq_quantize_layer_perm(
                        W0, U, lam, perm, bits, group_size, block_size, stream=stream)
                else:
                    perm = g_idx = None
                    U, lam, info = gptq_prepare_hinv(Hs[n], percdamp, stream=stream)
                    codes, scales, zeros, err = gptq_quantize_layer(W0, U, lam, bits, group_size, block_size,
                                                                    stream=stream)
                # What goes to a staging tensor: the weights are replaced only once every
                # layer of the block is known to have been factored (U is unspecified
                # when info != 0, and a caller may catch the error and retry)
                w_hat = gptq_dequantize(codes, scales, zeros, group_size, g_idx, out_dtype=W0.dtype,
                                        stream=stream)
                layers[n] = LayerQuant(codes, scales, zeros, err, lam, perm, g_idx, Hs[n] if keep_hessians else None)
                infos.append((n, info, W0, w_hat))
            (stream or torch.cuda.current_stream()).synchronize()
            for n, info, _, _ in infos:
                if int(info.item()) != 0:
                    raise NotPositiveDefinite(int(info.item()))
            for _, _, W0, w_hat in infos:
                W0.copy_(w_hat)
            results.append(BlockQuant(layers, xs if keep_inputs else None))
            xs = [block(x) for x in xs] if sequential else ys
    return results, xs
