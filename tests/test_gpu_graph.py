"""A whole layer (H := 0, gptq_hessian_accumulate, gptq_prepare_hinv or the
act-order calls, the quantize loop) captured once in a HIP graph and replayed:
every replay, with unrelated eager work and a synchronization before it, gives
bitwise the outputs of the same calls launched eagerly.  The library issues
only kernels (no memsets or copies), so a captured layer replays the same
launches.  Shapes: a layer whose loop runs in pair launches (at most 4096 rows,
whole pairs of 128-column blocks), one on the grouped path with thin launches
(more rows), and the act-order calls.
"""
import numpy as np
import pytest

import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import post_weight_quantization_02_amd as G  # noqa: E402


def _buffers(d_row, d_col, n, group, B, x_dtype):
    ng = -(-d_col // group) if group else 1
    f = torch.float32
    dev = "cuda"
    return dict(
        H=torch.zeros(d_col, d_col, dtype=f, device=dev), U=torch.empty(d_col, d_col, dtype=f, device=dev),
        lam=torch.empty(1, dtype=f, device=dev), info=torch.empty(1, dtype=torch.int32, device=dev),
        codes=torch.empty(d_row, d_col, dtype=torch.uint8, device=dev),
        scales=torch.empty(d_row, ng, dtype=f, device=dev), zeros=torch.empty(d_row, ng, dtype=torch.int32, device=dev),
        err=torch.empty(1, dtype=torch.float64, device=dev), perm=torch.empty(d_col, dtype=torch.int32, device=dev),
        g_idx=torch.empty(d_col, dtype=torch.int32, device=dev),
        ws_h=torch.empty(G.gptq_hessian_accumulate_workspace_size(
            d_col, n, G.GPTQ_F16 if x_dtype == torch.float16 else G.GPTQ_F32), dtype=torch.uint8, device=dev),
        ws_f=torch.empty(G.gptq_prepare_hinv_workspace_size(d_col), dtype=torch.uint8, device=dev),
        ws_q=torch.empty(G.gptq_quantize_layer_workspace_size(d_row, d_col, B), dtype=torch.uint8, device=dev))


CASES = [
    ("pairs_4096x1024_g128", 4096, 1024, 8192, 4, 128, 128, torch.float16, False),
    ("grouped_5000x768_row", 5000, 768, 4096, 3, 0, 128, torch.float32, False),
    ("act_order_1024x512_g64", 1024, 512, 4096, 4, 64, 64, torch.float16, True),
]


@pytest.mark.parametrize("name,d_row,d_col,n,bits,group,B,x_dtype,act", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager(name, d_row, d_col, n, bits, group, B, x_dtype, act):
    w, x = wl.tiny_case(7, d_row, d_col, n, 0.85, dtype=np.float32)
    W = torch.from_numpy(w).cuda().to(x_dtype)
    X = torch.from_numpy(x).cuda().to(x_dtype)
    b = _buffers(d_row, d_col, n, group, B, x_dtype)

    def layer():
        s = torch.cuda.current_stream()
        b["H"].zero_()
        G.gptq_hessian_accumulate(b["H"], X, ws=b["ws_h"], stream=s)
        if act:
            G.gptq_act_order_perm(b["H"], b["perm"], stream=s)
            G.gptq_prepare_hinv_perm(b["H"], b["perm"], 0.01, b["U"], b["lam"], b["info"], ws=b["ws_f"], stream=s)
            G.gptq_quantize_layer_perm(W, b["U"], b["lam"], b["perm"], bits, group, B, b["codes"], b["scales"],
                                       b["zeros"], b["g_idx"], b["err"], ws=b["ws_q"], stream=s)
        else:
            G.gptq_prepare_hinv(b["H"], 0.01, b["U"], b["lam"], b["info"], ws=b["ws_f"], stream=s)
            G.gptq_quantize_layer(W, b["U"], b["lam"], bits, group, B, b["codes"], b["scales"], b["zeros"],
                                  b["err"], ws=b["ws_q"], stream=s)

    keys = ["H", "U", "lam", "info", "codes", "scales", "zeros", "err"] + (["perm", "g_idx"] if act else [])
    print(f"graph: {name}", flush=True)
    layer()
    torch.cuda.synchronize()
    assert int(b["info"].item()) == 0
    ref = {k: b[k].clone() for k in keys}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    torch.cuda.synchronize()
    for r in range(3):
        # unrelated eager work and a synchronization between replays
        for k in keys:
            b[k].fill_(0)
        junk = torch.randn(4096, device="cuda").cumsum(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in keys:
            assert torch.equal(b[k], ref[k]), (r, k)
        del junk
    del graph
