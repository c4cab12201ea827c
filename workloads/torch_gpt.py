"""The synthetic GPT-style block as a torch module: the caller's model that the
whole-model procedure runs on the GPU (its forward pass is the model's, not the
quantizer's).  Used by the GPU tests and the benchmark only; the fp64 oracle has
its own forward pass and takes nothing from here but the seeded parameters of
``workloads.gpt_block_params``.

Pre-LayerNorm block: x += attn_proj(causal_attention(attn(ln1(x)))),
x += fc_proj(gelu(fc(ln2(x)))).  Attention is written out (fp32 matmuls with
contiguous operands, a causal mask, softmax) rather than through a fused kernel.
"""
from __future__ import annotations

import math

import torch
import torch.nn.functional as F

from . import GPT_LINEARS


class GPTBlock(torch.nn.Module):
    def __init__(self, params: dict, n_head: int, device="cuda", dtype=torch.float32):
        super().__init__()
        d = params["ln1_w"].shape[0]
        self.n_head = n_head
        self.ln1 = torch.nn.LayerNorm(d, eps=1e-5)
        self.attn = torch.nn.Linear(d, 3 * d)
        self.attn_proj = torch.nn.Linear(d, d)
        self.ln2 = torch.nn.LayerNorm(d, eps=1e-5)
        self.fc = torch.nn.Linear(d, 4 * d)
        self.fc_proj = torch.nn.Linear(4 * d, d)
        with torch.no_grad():
            for ln in ("ln1", "ln2"):
                getattr(self, ln).weight.copy_(torch.from_numpy(params[ln + "_w"]))
                getattr(self, ln).bias.copy_(torch.from_numpy(params[ln + "_b"]))
            for name in GPT_LINEARS:
                getattr(self, name).weight.copy_(torch.from_numpy(params[name + "_w"]))
                getattr(self, name).bias.copy_(torch.from_numpy(params[name + "_b"]))
        self.to(device=device, dtype=dtype)

    def forward(self, x):
        S, T, d = x.shape
        H, dh = self.n_head, d // self.n_head
        q, k, v = self.attn(self.ln1(x)).split(d, dim=-1)
        q = q.reshape(S, T, H, dh).transpose(1, 2).contiguous()
        k = k.reshape(S, T, H, dh).transpose(1, 2).contiguous()
        v = v.reshape(S, T, H, dh).transpose(1, 2).contiguous()
        s = torch.matmul(q, k.transpose(-2, -1).contiguous()) / math.sqrt(dh)
        s = s.masked_fill(torch.ones(T, T, dtype=torch.bool, device=x.device).triu(1), float("-inf"))
        y = torch.matmul(torch.softmax(s, dim=-1), v)
        x = x + self.attn_proj(y.transpose(1, 2).reshape(S, T, d))
        return x + self.fc_proj(F.gelu(self.fc(self.ln2(x))))


def build_model(spec, device="cuda", dtype=torch.float32):
    from . import gpt_block_params
    return [GPTBlock(gpt_block_params(spec, b), spec.n_head, device, dtype) for b in range(spec.n_block)]
