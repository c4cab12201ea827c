"""Pins of the whole-model oracle (itwiki "GPTQ", "최소 구현": blocks one at a time,
each quantized block's outputs feeding the next; the nanoGPT post, section 3:
hooks on every linear layer, layers quantized independently).  CPU only."""
import numpy as np
import pytest

import oracle as O
import workloads as wl

MP = O.model_pipeline
SPEC = wl.GPTSpec(n_block=2, d=32, n_head=4, seq=16, n_seq=4, n_batch=2, block_size=16)


def _model(spec=SPEC):
    blocks = [wl.gpt_block_params(spec, b) for b in range(spec.n_block)]
    xs = [wl.gpt_embeddings(spec, i) for i in range(spec.n_batch)]
    return blocks, xs


def test_block_forward_matches_torch_library_primitives():
    """The block through torch's own fp64 CPU layer norm, scaled-dot-product
    attention with a causal mask, exact GELU and linear layers."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    blocks, xs = _model()
    p = {k: torch.from_numpy(v.astype(np.float64)) for k, v in blocks[0].items()}
    x = torch.from_numpy(xs[0].astype(np.float64))
    S, T, d = x.shape
    h = F.layer_norm(x, (d,), p["ln1_w"], p["ln1_b"], eps=1e-5)
    q, k, v = F.linear(h, p["attn_w"], p["attn_b"]).split(d, dim=-1)
    heads = lambda t: t.reshape(S, T, SPEC.n_head, d // SPEC.n_head).transpose(1, 2)  # noqa: E731
    y = F.scaled_dot_product_attention(heads(q), heads(k), heads(v), is_causal=True)
    x1 = x + F.linear(y.transpose(1, 2).reshape(S, T, d), p["attn_proj_w"], p["attn_proj_b"])
    h2 = F.layer_norm(x1, (d,), p["ln2_w"], p["ln2_b"], eps=1e-5)
    ref = x1 + F.linear(F.gelu(F.linear(h2, p["fc_w"], p["fc_b"])), p["fc_proj_w"], p["fc_proj_b"])
    got = MP.block_forward({k: v.astype(np.float64) for k, v in blocks[0].items()}, xs[0].astype(np.float64),
                           SPEC.n_head)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_zero_layers_are_the_identity():
    blocks, xs = _model()
    p = {k: (np.zeros_like(v) if k.split("_")[0] in ("attn", "fc") else v) for k, v in blocks[0].items()}
    x = xs[0].astype(np.float64)
    np.testing.assert_array_equal(MP.block_forward(p, x, SPEC.n_head), x)


def test_attention_is_causal():
    """Changing tokens after position t leaves outputs at positions <= t unchanged."""
    blocks, xs = _model()
    p = {k: v.astype(np.float64) for k, v in blocks[0].items()}
    x = xs[0].astype(np.float64)
    x2 = x.copy()
    x2[:, 9:, :] = np.random.default_rng(3).standard_normal(x2[:, 9:, :].shape)
    a, b = MP.block_forward(p, x, SPEC.n_head), MP.block_forward(p, x2, SPEC.n_head)
    np.testing.assert_array_equal(a[:, :9], b[:, :9])
    assert not np.allclose(a[:, 9:], b[:, 9:])


@pytest.mark.parametrize("act_order", [False, True])
def test_each_layer_is_the_solver_on_its_captured_inputs(act_order):
    blocks, xs = _model()
    out, _ = MP.quantize_model(blocks[:1], xs, SPEC.n_head, 4, 8, 16, act_order=act_order)
    cap = {}
    for x in xs:
        MP.block_forward({k: v.astype(np.float64) for k, v in blocks[0].items()}, x.astype(np.float64),
                         SPEC.n_head, capture=cap)
    for name in MP.LINEARS:
        W0 = blocks[0][name + "_w"].astype(np.float64)
        sol = (O.solve_layer_act_order if act_order else O.solve_layer)(W0, cap[name], 4, 8, 16)
        got = out[0].layers[name]
        np.testing.assert_array_equal(got.result.codes, sol.result.codes)
        np.testing.assert_array_equal(got.result.w_hat, sol.result.w_hat)
        assert got.err == pytest.approx(sol.err, rel=1e-12)
        assert got.err == pytest.approx(O.output_error_direct(W0, got.result.w_hat, np.vstack(cap[name])),
                                        rel=1e-9)


def test_blocks_are_fed_in_order():
    """Sequential: block 1 sees block 0's outputs with What in place; independent:
    with the original weights.  Each is checked by running block 0 again."""
    blocks, xs = _model()
    seq, _ = MP.quantize_model(blocks, xs, SPEC.n_head, 3, 0, 16, sequential=True)
    ind, _ = MP.quantize_model(blocks, xs, SPEC.n_head, 3, 0, 16, sequential=False)
    p0 = {k: v.astype(np.float64) for k, v in blocks[0].items()}
    for i, x in enumerate(xs):
        x = x.astype(np.float64)
        np.testing.assert_array_equal(seq[1].inputs[i], MP.block_forward(seq[0].weights, x, SPEC.n_head))
        np.testing.assert_array_equal(ind[1].inputs[i], MP.block_forward(p0, x, SPEC.n_head))
    # block 0 is the same in both; block 1's Hessians differ (a wrong feed is caught)
    for name in MP.LINEARS:
        np.testing.assert_array_equal(seq[0].layers[name].H, ind[0].layers[name].H)
        assert not np.allclose(seq[1].layers[name].H, ind[1].layers[name].H, rtol=1e-6, atol=0)


def test_more_bits_bring_the_model_closer():
    """The quantized model's final outputs approach the unquantized model's as the
    grid gets finer; at 8 bits they agree to about 1e-3."""
    blocks, xs = _model()
    ref = [x.astype(np.float64) for x in xs]
    for p in blocks:
        ref = [MP.block_forward({k: v.astype(np.float64) for k, v in p.items()}, x, SPEC.n_head) for x in ref]
    dist = {}
    for bits in (2, 4, 8):
        _, ys = MP.quantize_model(blocks, xs, SPEC.n_head, bits, 0, 16)
        dist[bits] = max(float(np.linalg.norm(y - r) / np.linalg.norm(r)) for y, r in zip(ys, ref))
    assert dist[2] > dist[4] > dist[8]
    assert dist[8] < 1e-2
