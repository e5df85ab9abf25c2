"""Pins of the encoder-block oracle (``oracle/encoder.py``) against things other than itself.

* LayerNorm: torch's ``layer_norm`` in f64 (the textbook definition with the biased variance),
  rows with variance near eps (where eps placement matters), shift invariance, the affine
  identity, the moments of the output, constant rows and d = 1.
* RoPE table and rotation: the complex form (each pair ``(v_i, v_{i+rot/2})`` as
  ``v_i + i v_{i+rot/2}`` times ``e^{i theta}``), the relative-position identity of scores, norm
  preservation, frame 0 is the identity, dims past ``rot`` and the v third untouched, the
  angles' geometric progression and ``cos^2 + sin^2 = 1``.
* q/k norm: torch's ``layer_norm`` per head.
* attention: torch's ``scaled_dot_product_attention`` in f64 with a boolean key mask; one valid
  key, identical keys, a zero scale, masked keys' contents, frame permutation, no valid key.
* the block and the forward: a composition written with torch's functional ops in f64 (its own
  bf16 decode, complex RoPE, SDPA, exact GELU).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import encoder as enc
from oracle import reference as ref

T64 = torch.float64


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


# ---------------------------------------------------------------- LayerNorm

@pytest.mark.parametrize("d", [1, 3, 8, 100, 1024])
def test_layer_norm_matches_torch(d):
    g = synth.rng(300, d)
    x = g.standard_normal((6, d)) * g.uniform(0.001, 5.0, (6, 1)) + g.uniform(-3, 3, (6, 1))
    wb = g.standard_normal(2 * d)
    got = enc.layer_norm(x, wb)
    want = F.layer_norm(_t(x), (d,), _t(wb[:d]), _t(wb[d:]), eps=1e-5).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_layer_norm_eps_matters_at_small_variance():
    """Rows whose variance is comparable to eps: the eps inside the square root changes the
    result by a large factor, so a misplaced eps fails against torch."""
    g = synth.rng(301)
    d = 64
    x = g.standard_normal((4, d)) * np.array([[1e-3], [3e-3], [1e-2], [1.0]])
    wb = np.concatenate([np.ones(d), np.zeros(d)])
    got = enc.layer_norm(x, wb)
    want = F.layer_norm(_t(x), (d,), eps=1e-5).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # Without eps the first row would have unit mean square; with it, far less.
    assert np.mean(got[0] ** 2) < 0.2


def test_layer_norm_invariants():
    g = synth.rng(302)
    d = 37
    x = g.standard_normal((5, d)) * 2.0
    w, b = g.standard_normal(d), g.standard_normal(d)
    one = np.concatenate([np.ones(d), np.zeros(d)])
    y1 = enc.layer_norm(x, one)
    # shift invariance, affine identity
    np.testing.assert_allclose(enc.layer_norm(x + 7.25, one), y1, atol=1e-12)
    np.testing.assert_allclose(enc.layer_norm(x, np.concatenate([w, b])), y1 * w + b, atol=1e-12)
    # moments: mean 0, mean square var/(var+eps) with the biased variance
    var = x.var(axis=1)
    np.testing.assert_allclose(y1.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose((y1 ** 2).mean(axis=1), var / (var + 1e-5), rtol=1e-12)
    # a constant row and a single value give the bias
    np.testing.assert_allclose(enc.layer_norm(np.full((1, d), 3.0), np.concatenate([w, b])), b[None], atol=0)
    np.testing.assert_allclose(enc.layer_norm(np.array([[4.0]]), np.array([2.0, -1.5])), [[-1.5]], atol=0)


# ---------------------------------------------------------------- RoPE

def test_rope_table_closed_forms():
    n, rot = 50, 16
    cos, sin = enc.rope_table(n, rot)
    assert cos.shape == sin.shape == (n, rot // 2)
    np.testing.assert_array_equal(cos[0], 1.0)
    np.testing.assert_array_equal(sin[0], 0.0)
    np.testing.assert_allclose(cos ** 2 + sin ** 2, 1.0, atol=1e-15)
    # pair 0 turns by one radian per frame
    np.testing.assert_allclose(cos[:, 0], [math.cos(t) for t in range(n)], atol=1e-15)
    np.testing.assert_allclose(sin[:, 0], [math.sin(t) for t in range(n)], atol=1e-15)
    # frame 1: angles fall geometrically by 10000^(-2/rot) per pair, from 1 down to 10000^(-(rot-2)/rot)
    ang1 = np.arctan2(sin[1], cos[1])
    np.testing.assert_allclose(ang1[1:] / ang1[:-1], 10000.0 ** (-2.0 / rot), rtol=1e-12)
    np.testing.assert_allclose(ang1[-1], 10000.0 ** (-(rot - 2) / rot), rtol=1e-12)
    with pytest.raises(ValueError):
        enc.rope_table(4, 5)


def _qkv(g, n, heads, hd, scale=1.0):
    return g.standard_normal((n, 3 * heads * hd)) * scale


@pytest.mark.parametrize("heads,hd,rot", [(2, 8, 8), (3, 10, 6), (1, 128, 128), (2, 80, 32), (1, 4, 0)])
def test_rotation_is_complex_multiplication(heads, hd, rot):
    g = synth.rng(303, heads, hd, rot)
    n = 9
    d = heads * hd
    x = _qkv(g, n, heads, hd)
    cos, sin = enc.rope_table(n, rot)
    got = enc.qk_norm_rope(x, heads, hd, rot, cos, sin)
    half = rot // 2
    theta = np.arctan2(sin, cos)
    for which in (0, 1):
        for h in range(heads):
            base = which * d + h * hd
            z = (x[:, base:base + half] + 1j * x[:, base + half:base + rot]) * np.exp(1j * theta)
            np.testing.assert_allclose(got[:, base:base + half], z.real, atol=1e-13)
            np.testing.assert_allclose(got[:, base + half:base + rot], z.imag, atol=1e-13)
            np.testing.assert_array_equal(got[:, base + rot:base + hd], x[:, base + rot:base + hd])
    np.testing.assert_array_equal(got[:, 2 * d:], x[:, 2 * d:])
    np.testing.assert_array_equal(got[0], x[0])  # frame 0 turns by nothing


def test_rotation_scores_depend_on_frame_difference():
    """<R_t1 q, R_t2 k> = <R_(t1-t2) q, k> on fully rotated heads: checks that q and k share one
    convention and that the angle grows with the frame."""
    g = synth.rng(304)
    heads, hd, rot, n = 1, 16, 16, 12
    q, k = g.standard_normal(hd), g.standard_normal(hd)
    x = np.zeros((n, 3 * hd))
    x[:, :hd] = q
    x[:, hd:2 * hd] = k
    cos, sin = enc.rope_table(n, rot)
    r = enc.qk_norm_rope(x, heads, hd, rot, cos, sin)
    for t1, t2 in ((5, 2), (9, 0), (11, 7)):
        lhs = r[t1, :hd] @ r[t2, hd:2 * hd]
        rhs = r[t1 - t2, :hd] @ k
        assert abs(lhs - rhs) < 1e-12
        # and the norm of every pair is kept
        pairs = r[t1, :hd].reshape(2, -1)
        np.testing.assert_allclose(pairs[0] ** 2 + pairs[1] ** 2, q[:hd // 2] ** 2 + q[hd // 2:] ** 2, rtol=1e-12)


def test_qk_norm_is_layer_norm_per_head_before_rotation():
    g = synth.rng(305)
    heads, hd, rot, n = 3, 12, 8, 7
    d = heads * hd
    x = _qkv(g, n, heads, hd, 3.0) + 1.0
    qn, kn = g.standard_normal(2 * hd), g.standard_normal(2 * hd)
    cos, sin = enc.rope_table(n, rot)
    got = enc.qk_norm_rope(x, heads, hd, rot, cos, sin, qn, kn)
    # at frame 0 there is no rotation: the result is the per-head LayerNorm
    for which, nw in ((0, qn), (1, kn)):
        for h in range(heads):
            s = slice(which * d + h * hd, which * d + (h + 1) * hd)
            want = F.layer_norm(_t(x[:, s]), (hd,), _t(nw[:hd]), _t(nw[hd:]), eps=1e-5).numpy()
            np.testing.assert_allclose(got[0, s], want[0], atol=1e-12)
            # at other frames, undoing the rotation (complex conjugate) gives it back
            half = rot // 2
            theta = np.arctan2(sin, cos)
            z = (got[:, s][:, :half] + 1j * got[:, s][:, half:rot]) * np.exp(-1j * theta)
            np.testing.assert_allclose(z.real, want[:, :half], atol=1e-12)
            np.testing.assert_allclose(z.imag, want[:, half:rot], atol=1e-12)
            np.testing.assert_allclose(got[:, s][:, rot:], want[:, rot:], atol=1e-12)
    np.testing.assert_array_equal(got[:, 2 * d:], x[:, 2 * d:])
    with pytest.raises(ValueError):
        enc.qk_norm_rope(x, heads, hd, rot, cos, sin, qn, None)


# ---------------------------------------------------------------- attention

def _sdpa(x, valid, heads, hd, scale):
    n = x.shape[0]
    d = heads * hd
    t = _t(x).reshape(n, 3, heads, hd).permute(1, 2, 0, 3)  # [3][heads][n][hd]
    mask = torch.from_numpy(np.asarray(valid) != 0)[None, None, :].expand(heads, n, n)
    o = F.scaled_dot_product_attention(t[0], t[1], t[2], attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).reshape(n, d).numpy()


@pytest.mark.parametrize("n,heads,hd", [(1, 1, 4), (7, 2, 8), (33, 3, 10), (70, 2, 64)])
def test_attention_matches_torch_sdpa(n, heads, hd):
    g = synth.rng(306, n, heads, hd)
    x = _qkv(g, n, heads, hd, 2.0)
    valid = (g.random(n) > 0.3).astype(np.int32)
    valid[g.integers(0, n)] = 1
    scale = 1.0 / math.sqrt(hd)
    np.testing.assert_allclose(enc.attention(x, valid, heads, hd, scale), _sdpa(x, valid, heads, hd, scale),
                               rtol=1e-11, atol=1e-12)


def test_attention_special_cases():
    g = synth.rng(307)
    n, heads, hd = 10, 2, 6
    d = heads * hd
    x = _qkv(g, n, heads, hd)
    # one valid key: every query gets that key's value
    valid = np.zeros(n, np.int32)
    valid[4] = 1
    o = enc.attention(x, valid, heads, hd, 0.5)
    np.testing.assert_allclose(o, np.broadcast_to(x[4, 2 * d:], (n, d)), atol=1e-15)
    # identical keys, or a zero scale: the mean of the valid values
    valid = np.array([1, 0, 1, 1, 0, 1, 1, 1, 0, 1], np.int32)
    mean_v = x[valid != 0, 2 * d:].mean(axis=0)
    np.testing.assert_allclose(enc.attention(x, valid, heads, hd, 0.0), np.broadcast_to(mean_v, (n, d)), atol=1e-14)
    same = x.copy()
    same[:, d:2 * d] = x[0, d:2 * d]
    np.testing.assert_allclose(enc.attention(same, valid, heads, hd, 0.7), np.broadcast_to(mean_v, (n, d)),
                               atol=1e-14)
    # masked keys' contents do not matter
    junk = x.copy()
    junk[valid == 0, d:] = 1e6
    np.testing.assert_allclose(enc.attention(junk, valid, heads, hd, 0.3), enc.attention(x, valid, heads, hd, 0.3),
                               atol=1e-14)
    # permuting the frames (and the mask) permutes the outputs
    perm = g.permutation(n)
    np.testing.assert_allclose(enc.attention(x[perm], valid[perm], heads, hd, 0.3),
                               enc.attention(x, valid, heads, hd, 0.3)[perm], atol=1e-14)
    # no valid key: NaN everywhere
    assert np.isnan(enc.attention(x, np.zeros(n, np.int32), heads, hd, 0.3)).all()


def test_attention_weight_scale():
    g = synth.rng(308)
    n, heads, hd = 12, 2, 5
    d = heads * hd
    x = np.abs(_qkv(g, n, heads, hd))  # non-negative q, k, v
    valid = (g.random(n) > 0.2).astype(np.int32)
    valid[0] = 1
    pv, sqk = enc.attention_weight_scale(x, valid, heads, hd, 0.4)
    # with v >= 0 the weighted magnitudes are the outputs; with q, k >= 0 the largest score
    np.testing.assert_allclose(pv, enc.attention(x, valid, heads, hd, 0.4), rtol=1e-13)
    for h in range(heads):
        s = 0.4 * x[:, h * hd:(h + 1) * hd] @ x[valid != 0, d + h * hd:d + (h + 1) * hd].T
        np.testing.assert_allclose(sqk[:, h], s.max(axis=1), rtol=1e-13)


# ---------------------------------------------------------------- block and forward

def _bf16_to_torch(bits, rows, cols):
    """bf16 bit patterns to f64 through torch's own reinterpretation of the upper half."""
    b = torch.from_numpy(np.asarray(bits).astype(np.int32).reshape(rows, cols) << 16)
    return b.view(torch.float32).to(T64)


def _torch_rope(v, cos, sin, rot):
    half = rot // 2
    z = torch.complex(v[..., :half], v[..., half:rot]) * torch.complex(_t(cos), _t(sin))[:, None, :]
    return torch.cat([z.real, z.imag, v[..., rot:]], dim=-1)


def _torch_block(h, L, valid, heads, rot, cos, sin):
    n, d = h.shape
    hd = d // heads
    inter = len(L["fc1_b"])
    scale = float(np.float32(1.0) / np.sqrt(np.float32(hd)))
    a = F.layer_norm(h, (d,), _t(L["ln1"][:d]), _t(L["ln1"][d:]), eps=1e-5)
    qkv = F.linear(a, _bf16_to_torch(L["qkv_w"], 3 * d, d), None if L["qkv_b"] is None else _t(L["qkv_b"]))
    q, k, v = qkv.reshape(n, 3, heads, hd).unbind(1)
    if L["qn"] is not None:
        q = F.layer_norm(q, (hd,), _t(L["qn"][:hd]), _t(L["qn"][hd:]), eps=1e-5)
        k = F.layer_norm(k, (hd,), _t(L["kn"][:hd]), _t(L["kn"][hd:]), eps=1e-5)
    q, k = _torch_rope(q, cos, sin, rot), _torch_rope(k, cos, sin, rot)
    mask = torch.from_numpy(valid != 0)[None, None, :].expand(heads, n, n)
    att = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                         attn_mask=mask, scale=scale).transpose(0, 1).reshape(n, d)
    h = h + F.linear(att, _bf16_to_torch(L["out_w"], d, d), _t(L["out_b"]))
    a = F.layer_norm(h, (d,), _t(L["ln2"][:d]), _t(L["ln2"][d:]), eps=1e-5)
    f = F.gelu(F.linear(a, _bf16_to_torch(L["fc1_w"], inter, d), _t(L["fc1_b"])), approximate="none")
    return h + F.linear(f, _bf16_to_torch(L["fc2_w"], d, inter), _t(L["fc2_b"]))


def _layer(g, d, inter, hd, qk_norm, qkv_bias):
    ln = lambda: np.concatenate([1.0 + 0.1 * g.standard_normal(d), 0.1 * g.standard_normal(d)])  # noqa: E731
    return {
        "ln1": ln(), "ln2": ln(),
        "qkv_w": synth.bf16_weight(g, 3 * d, d, 0.3), "qkv_b": synth.normal_f32(g, (3 * d,), 0.1) if qkv_bias else None,
        "qn": np.concatenate([1.0 + 0.1 * g.standard_normal(hd), 0.1 * g.standard_normal(hd)]) if qk_norm else None,
        "kn": np.concatenate([1.0 + 0.1 * g.standard_normal(hd), 0.1 * g.standard_normal(hd)]) if qk_norm else None,
        "out_w": synth.bf16_weight(g, d, d, 0.2), "out_b": synth.normal_f32(g, (d,), 0.1),
        "fc1_w": synth.bf16_weight(g, inter, d, 0.2), "fc1_b": synth.normal_f32(g, (inter,), 0.1),
        "fc2_w": synth.bf16_weight(g, d, inter, 0.2), "fc2_b": synth.normal_f32(g, (d,), 0.1),
    }


@pytest.mark.parametrize("qk_norm,qkv_bias", [(True, False), (False, True)])
def test_encoder_layer_matches_torch_composition(qk_norm, qkv_bias):
    g = synth.rng(309, qk_norm, qkv_bias)
    n, d, heads, rot, inter = 11, 16, 2, 4, 24
    L = _layer(g, d, inter, d // heads, qk_norm, qkv_bias)
    h = g.standard_normal((n, d))
    valid = np.ones(n, np.int32)
    valid[[3, 9]] = 0
    cos, sin = enc.rope_table(n, rot)
    got = enc.encoder_layer(h, L, ref.W_BF16, valid, heads, rot, cos, sin)
    want = _torch_block(_t(h), L, valid, heads, rot, cos, sin).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-10)


def test_encoder_forward_matches_torch_composition():
    g = synth.rng(310)
    n, d, heads, rot, inter, stack_in = 9, 16, 2, 8, 20, 12
    layers = [_layer(g, d, inter, d // heads, True, False) for _ in range(2)]
    ln = lambda: np.concatenate([1.0 + 0.1 * g.standard_normal(d), 0.1 * g.standard_normal(d)])  # noqa: E731
    model = {"proj": synth.bf16_weight(g, d, stack_in, 0.3), "embed_norm": ln(), "final_norm": ln(), "layers": layers}
    x = g.standard_normal((n, stack_in))
    valid = np.ones(n, np.int32)
    valid[-2:] = 0
    got = enc.encoder_forward(x, model, ref.W_BF16, valid, heads, rot)
    cos, sin = enc.rope_table(n, rot)
    t = F.linear(_t(x), _bf16_to_torch(model["proj"], d, stack_in))
    t = F.layer_norm(t, (d,), _t(model["embed_norm"][:d]), _t(model["embed_norm"][d:]), eps=1e-5)
    for L in layers:
        t = _torch_block(t, L, valid, heads, rot, cos, sin)
    t = F.layer_norm(t, (d,), _t(model["final_norm"][:d]), _t(model["final_norm"][d:]), eps=1e-5)
    np.testing.assert_allclose(got, t.numpy(), rtol=1e-10, atol=1e-10)
