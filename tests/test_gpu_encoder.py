"""GPU parity of the encoder-block kernels (LayerNorm, q/k norm + rotation, attention) and of one
whole block, through the C ABI, against the f64 oracle (``oracle/encoder.py``), within the bounds
derived in ``tests/encoder_bounds.py``. Outputs are NaN-prefilled with canaries after them.
"""
import math

import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import synth
from oracle import encoder as enc
from oracle import reference as ref
from tests import encoder_bounds as eb
from tests.parity import assert_within, dev, guarded_out, read_guarded

pytestmark = pytest.mark.gpu


def _rows(g, n, d, spread=True):
    """Rows with their own offsets and scales (down to variances near eps)."""
    x = synth.normal_f32(g, (n, d), 1.0)
    if spread:
        scale = np.exp(g.uniform(np.log(1e-3), np.log(30.0), (n, 1))).astype(np.float32)
        shift = g.uniform(-5, 5, (n, 1)).astype(np.float32)
        x = (x * scale + shift).astype(np.float32)
    return x


# ---------------------------------------------------------------- LayerNorm

LN_SHAPES = [(1, 1), (5, 7), (3, 64), (37, 1000), (1500, 1024), (4, 1022), (9, 4096), (2, 5000), (300, 256)]


@pytest.mark.parametrize("n,d", LN_SHAPES)
def test_layer_norm(n, d):
    g = synth.rng(400, n, d)
    x = _rows(g, n, d)
    wb = synth.layer_norm_weights(g, d)
    buf, out = guarded_out(n, d)
    wq.layer_norm(dev(x), dev(wb), d=d, out=out)
    got = read_guarded(buf, n, d)
    assert_within(got, enc.layer_norm(x, wb), eb.ln_tol(x, wb), f"layer norm {n}x{d}")


@pytest.mark.parametrize("n,d", [(7, 1024), (3, 60)])
def test_layer_norm_in_place_and_unaligned(n, d):
    g = synth.rng(401, n, d)
    x = _rows(g, n, d)
    wb = synth.layer_norm_weights(g, d)
    want, tol = enc.layer_norm(x, wb), eb.ln_tol(x, wb)
    t = dev(x)
    wq.layer_norm(t, dev(wb), d=d, out=t)  # in place
    assert_within(t.cpu().numpy(), want, tol, "in place")
    # rows starting 4 bytes past a 16-byte boundary take the scalar kernel
    import torch
    big = torch.full((n * d + 1,), float("nan"), device="cuda")
    big[1:] = dev(x).reshape(-1)
    o = torch.full((n * d + 1,), float("nan"), device="cuda")
    wq.layer_norm(big[1:], dev(wb), d=d, out=o[1:])
    assert_within(o[1:].cpu().numpy().reshape(n, d), want, tol, "offset rows")
    assert math.isnan(o[0].item())


def test_bound_layer_norm_equals_the_plain_call():
    """The bound call (arguments marshalled once) launches the same kernel on the same buffers."""
    n, d = 1500, 1024
    g = synth.rng(402, n, d)
    x = _rows(g, n, d)
    wb = synth.layer_norm_weights(g, d)
    xt, wbt = dev(x), dev(wb)
    buf, out = guarded_out(n, d)
    call = wq.bind_layer_norm(xt, wbt, d=d, out=out)
    for _ in range(3):
        call()
    got = read_guarded(buf, n, d)
    plain = wq.layer_norm(xt, wbt, d=d).cpu().numpy()
    assert np.array_equal(got, plain)
    assert_within(got, enc.layer_norm(x, wb), eb.ln_tol(x, wb), "bound layer norm")


# ---------------------------------------------------------------- q/k norm + rotation

QK_CASES = [  # n, heads, hd, rot, norm
    (1, 1, 64, 64, True), (37, 8, 128, 128, True), (37, 8, 128, 64, False), (20, 3, 40, 16, True),
    (9, 2, 256, 256, True), (5, 4, 100, 0, True), (3, 2, 2, 2, False), (130, 2, 80, 32, True),
]


@pytest.mark.parametrize("n,heads,hd,rot,norm", QK_CASES)
def test_qk_norm_rope_synthetic_table(n, heads, hd, rot, norm):
    """Any table serves to check the arithmetic: both sides get the same f32 table."""
    g = synth.rng(402, n, heads, hd, rot, norm)
    d = heads * hd
    qkv = _rows(g, n, 3 * d, spread=False) * np.float32(2.0) + np.float32(0.5)
    qn = synth.layer_norm_weights(g, hd) if norm else None
    kn = synth.layer_norm_weights(g, hd) if norm else None
    half = rot // 2
    cs = synth.unit_circle_table(g, n, half)
    cos, sin = cs[:n * half].reshape(n, half), cs[n * half:].reshape(n, half)
    want, tol = eb.qk_bound(qkv, heads, hd, rot, cos, sin, qn, kn)
    buf, out = guarded_out(n, 3 * d, qkv)
    wq.qk_norm_rope(out, dev(cs) if rot else None, n=n, heads=heads, hd=hd, rot=rot,
                    qn=None if qn is None else dev(qn), kn=None if kn is None else dev(kn))
    got = read_guarded(buf, n, 3 * d)
    assert_within(got, want, tol, f"qk {n}x{heads}x{hd} rot {rot}")
    np.testing.assert_array_equal(got[:, 2 * d:], qkv[:, 2 * d:])  # v untouched, bit for bit


def test_qk_norm_rope_with_the_host_table():
    """The page's own table (host f32) against the oracle's exact table, at the workload's frames."""
    n, heads, hd, rot = 1500, 8, 128, 128
    g = synth.rng(403)
    d = heads * hd
    qkv = _rows(g, n, 3 * d, spread=False)
    qn, kn = synth.layer_norm_weights(g, hd), synth.layer_norm_weights(g, hd)
    cos, sin = enc.rope_table(n, rot)
    want, tol = eb.qk_bound(qkv, heads, hd, rot, cos, sin, qn, kn, table_err=eb.rope_table_err(n, rot))
    t = dev(qkv)
    wq.qk_norm_rope(t, wq.rope_table(n, rot).cuda(), n=n, heads=heads, hd=hd, rot=rot, qn=dev(qn), kn=dev(kn))
    assert_within(t.cpu().numpy(), want, tol, "qk with the host table")


# ---------------------------------------------------------------- attention

ATTN_CASES = [  # n, heads, hd, p_valid (None: all valid), score scale
    (1, 1, 32, None, 1.0), (63, 2, 64, 0.7, 1.0), (64, 2, 64, 0.7, 1.0), (65, 3, 40, 0.5, 1.0),
    (200, 4, 128, 0.8, 1.0), (130, 1, 100, 0.5, 3.0), (129, 2, 128, None, 3.0), (300, 5, 16, 0.9, 1.0),
]


def _attn_inputs(n, heads, hd, p_valid, amp, seed):
    g = synth.rng(404, n, heads, hd, seed)
    qkv = synth.normal_f32(g, (n, 3 * heads * hd), 1.0)
    qkv[:, :2 * heads * hd] *= np.float32(amp)  # q and k: larger scores make the softmax peakier
    valid = np.ones(n, np.int32) if p_valid is None else synth.random_key_mask(g, n, p_valid)
    valid[g.integers(0, n)] = 1
    return qkv, valid


def _run_attn(qkv, valid, n, heads, hd, scale):
    buf, out = guarded_out(n, heads * hd)
    wq.attention(dev(qkv), dev(valid), n=n, heads=heads, hd=hd, scale=scale, out=out)
    return read_guarded(buf, n, heads * hd)


@pytest.mark.parametrize("n,heads,hd,p_valid,amp", ATTN_CASES)
def test_attention(n, heads, hd, p_valid, amp):
    qkv, valid = _attn_inputs(n, heads, hd, p_valid, amp, 0)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(hd)))
    got = _run_attn(qkv, valid, n, heads, hd, scale)
    # Tight: the oracle on the bf16 values the kernel computes with.
    r = eb.bf16_round(qkv)
    assert_within(got, enc.attention(r, valid, heads, hd, scale), eb.attn_tol(r, valid, heads, hd, scale, True),
                  f"attention {n}x{heads}x{hd} (bf16 inputs)")
    # And against the f32 inputs themselves, with the rounding of q, k and v in the bound.
    assert_within(got, enc.attention(qkv, valid, heads, hd, scale),
                  eb.attn_tol(qkv, valid, heads, hd, scale, False), f"attention {n}x{heads}x{hd}")


def test_attention_workload_size():
    """1500 frames, 8 heads of 128, the last 100 frames masked: every output checked."""
    n, heads, hd = synth.ENCODER_N, synth.ENCODER_HEADS, synth.ENCODER_D // synth.ENCODER_HEADS
    g = synth.rng(405)
    qkv = synth.normal_f32(g, (n, 3 * heads * hd), 1.0)
    valid = synth.key_mask(n, synth.ENCODER_VALID)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(hd)))
    got = _run_attn(qkv, valid, n, heads, hd, scale)
    r = eb.bf16_round(qkv)
    assert_within(got, enc.attention(r, valid, heads, hd, scale), eb.attn_tol(r, valid, heads, hd, scale, True),
                  "attention 1500x8x128")


def test_attention_special_cases():
    n, heads, hd = 70, 2, 64
    d = heads * hd
    qkv, _ = _attn_inputs(n, heads, hd, None, 1.0, 1)
    # No valid key: NaN everywhere (the page's 0 * (1/0)).
    assert np.isnan(_run_attn(qkv, np.zeros(n, np.int32), n, heads, hd, 0.125)).all()
    # One valid key: every query gets that key's value, rounded to bf16, exactly.
    valid = np.zeros(n, np.int32)
    valid[41] = 1
    got = _run_attn(qkv, valid, n, heads, hd, 0.125)
    np.testing.assert_array_equal(got, np.broadcast_to(eb.bf16_round(qkv[41, 2 * d:]), (n, d)))
    # Zero scale: every weight is 1, the mean of the valid (rounded) values.
    valid = synth.random_key_mask(synth.rng(406), n, 0.6)
    got = _run_attn(qkv, valid, n, heads, hd, 0.0)
    mean = eb.bf16_round(qkv[valid != 0, 2 * d:]).mean(axis=0)
    np.testing.assert_allclose(got, np.broadcast_to(mean, (n, d)), rtol=0, atol=4 * n * 2.0 ** -24 * 4)
    # Masked keys' contents do not matter, bit for bit.
    junk = qkv.copy()
    junk[valid == 0, d:] = 1e30
    np.testing.assert_array_equal(_run_attn(junk, valid, n, heads, hd, 0.2), _run_attn(qkv, valid, n, heads, hd, 0.2))


def test_attention_is_deterministic():
    qkv, valid = _attn_inputs(500, 4, 128, 0.9, 1.0, 2)
    a = _run_attn(qkv, valid, 500, 4, 128, 0.09)
    b = _run_attn(qkv, valid, 500, 4, 128, 0.09)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- one block

def _layer_dev(L):
    return {k: (None if v is None else dev(v)) for k, v in L.items()}


def _layer_reference(h, L, valid, heads, rot, bf16, var_in=None):
    """The oracle's block and the variance of the propagated rounding errors
    (``encoder_bounds.layer_sigma``)."""
    n, d = h.shape
    h2, var = eb.layer_sigma(h, L, valid, heads, rot, bf16, var_in)
    cos, sin = enc.rope_table(n, rot)
    # The step-by-step value is the oracle's block.
    np.testing.assert_allclose(h2, enc.encoder_layer(h, L, ref.W_BF16, valid, heads, rot, cos, sin), rtol=1e-12,
                               atol=1e-12)
    return h2, var


LAYER_CASES = [  # n, d, heads, inter, rot, qk_norm, qkv_bias, path
    (70, 128, 2, 256, 64, True, False, wq.PATH_MFMA),
    (70, 128, 2, 256, 32, False, True, wq.PATH_MFMA),
    (33, 96, 3, 160, 32, True, False, wq.PATH_MFMA_F32),
    (130, 256, 4, 512, 64, True, True, wq.PATH_AUTO),
    (12, 128, 1, 128, 128, True, False, wq.PATH_AUTO),   # n <= 16: the products take the f32 matvec
    (50, 96, 3, 160, 32, True, True, wq.PATH_MFMA),       # d % 64 != 0: f32 hand-offs on the bf16 path
    (200, 192, 3, 640, 64, False, True, wq.PATH_MFMA),    # bf16 hand-offs, 64 x 64 product tiles
    (10, 128, 2, 256, 32, True, False, wq.PATH_MFMA),     # bf16 hand-offs with fewer frames than a tile
    (40, 192, 16, 256, 4, True, True, wq.PATH_MFMA),      # heads of 12 dims: element-wise bf16 stores
]


@pytest.mark.parametrize("n,d,heads,inter,rot,qk_norm,qkv_bias,path", LAYER_CASES)
def test_encoder_layer(n, d, heads, inter, rot, qk_norm, qkv_bias, path):
    L = synth.encoder_block_weights(0, seed=n, d=d, heads=heads, inter=inter, qk_norm=qk_norm, qkv_bias=qkv_bias,
                                    sigma=0.05)
    g = synth.rng(407, n, d)
    h = synth.normal_f32(g, (n, d), 1.0)
    valid = synth.random_key_mask(g, n, 0.85)
    valid[0] = 1
    bf16 = path == wq.PATH_MFMA or (path == wq.PATH_AUTO and n > wq.MATVEC_MAX_N)
    want, var = _layer_reference(h, L, valid, heads, rot, bf16)
    tol = eb.sigma_tol(want, var)
    t = dev(h)
    cs = wq.rope_table(n, rot).cuda()
    Ld = _layer_dev(L)
    wq.encoder_layer(t, Ld, wq.W_BF16, dev(valid), cs, n=n, d=d, heads=heads, rot=rot, inter=inter, path=path)
    got = t.cpu().numpy()
    assert_within(got, want, tol, f"encoder layer {n}x{d} heads {heads} path {path}")

    # The block is exactly its steps, called one by one.
    import torch
    hs = dev(h)
    a = wq.layer_norm(hs, Ld["ln1"], d=d)
    qkv = wq.gemm(a, Ld["qkv_w"], wq.W_BF16, m=3 * d, k=d, bias=Ld["qkv_b"], path=path)
    wq.qk_norm_rope(qkv, cs, n=n, heads=heads, hd=d // heads, rot=rot, qn=Ld["qn"], kn=Ld["kn"])
    att = wq.attention(qkv, dev(valid), n=n, heads=heads, hd=d // heads,
                       scale=float(np.float32(1.0) / np.sqrt(np.float32(d // heads))))
    wq.gemm(att, Ld["out_w"], wq.W_BF16, m=d, k=d, bias=Ld["out_b"], residual=True, out=hs, path=path)
    a = wq.layer_norm(hs, Ld["ln2"], d=d)
    f = wq.gemm(a, Ld["fc1_w"], wq.W_BF16, m=inter, k=d, bias=Ld["fc1_b"], gelu=True, path=path)
    wq.gemm(f, Ld["fc2_w"], wq.W_BF16, m=d, k=inter, bias=Ld["fc2_b"], residual=True, out=hs, path=path)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got, hs.cpu().numpy())


def test_encoder_forward_small():
    """Two blocks with the input projection, on the f32-accurate matrix-core path, against the
    oracle with the bound carried through every step (projection, embedding LayerNorm, each block,
    final LayerNorm)."""
    n, d, heads, inter, rot, stack_in = 40, 128, 2, 256, 64, 96
    model = synth.encoder_model(2, seed=1, d=d, heads=heads, inter=inter, stack_in=stack_in)
    g = synth.rng(408)
    x = synth.normal_f32(g, (n, stack_in), 1.0)
    valid = synth.key_mask(n, 35)
    md = {"proj": dev(model["proj"]), "embed_norm": dev(model["embed_norm"]),
          "final_norm": dev(model["final_norm"]), "layers": [_layer_dev(L) for L in model["layers"]]}
    got = wq.encoder_forward(dev(x), md, wq.W_BF16, dev(valid), heads=heads, rot=rot,
                             path=wq.PATH_MFMA_F32).cpu().numpy()
    want = enc.encoder_forward(x, model, ref.W_BF16, valid, heads, rot)
    # Tolerance: projection (f32-accurate), embedding LayerNorm, each block, final LayerNorm.
    x0, var = eb.gemm_sigma(x.astype(np.float64), np.zeros((n, stack_in)),
                            ref.decode(model["proj"], ref.W_BF16, d, stack_in), None, False)
    h, var = eb.ln_sigma(x0, model["embed_norm"], var)
    for L in model["layers"]:
        h, var = _layer_reference(h, L, valid, heads, rot, False, var)
    _, var = eb.ln_sigma(h, model["final_norm"], var)
    assert_within(got, want, eb.sigma_tol(want, var), "encoder forward")


def test_encoder_layer_workload_size():
    """One block at the workload's size (1500 frames, d = 1024, 8 heads of 128, MLP 4096, the last
    100 frames masked), on the bf16 matrix-core path the forward uses: every output against the
    oracle's block within the probabilistic bound."""
    n, d, heads, inter, rot = synth.ENCODER_N, synth.ENCODER_D, synth.ENCODER_HEADS, synth.ENCODER_FF, synth.ENCODER_ROT
    L = synth.encoder_block_weights(0)
    h = synth.normal_f32(synth.rng(409), (n, d), 1.0)
    valid = synth.key_mask(n, synth.ENCODER_VALID)
    t = dev(h)
    wq.encoder_layer(t, _layer_dev(L), wq.W_BF16, dev(valid), wq.rope_table(n, rot).cuda(), n=n, d=d, heads=heads,
                     rot=rot, inter=inter, path=wq.PATH_MFMA)
    got = t.cpu().numpy()
    want, var = eb.layer_sigma(h, L, valid, heads, rot, True)
    assert_within(got, want, eb.sigma_tol(want, var), "encoder layer 1500x1024")

    # The block hands its activations over in bf16 between its kernels; its steps called one by one
    # (f32 hand-offs, other product tiles) give the same bits.
    import torch
    Ld = _layer_dev(L)
    cs = wq.rope_table(n, rot).cuda()
    hs = dev(h)
    a = wq.layer_norm(hs, Ld["ln1"], d=d)
    qkv = wq.gemm(a, Ld["qkv_w"], wq.W_BF16, m=3 * d, k=d, bias=Ld["qkv_b"], path=wq.PATH_MFMA)
    wq.qk_norm_rope(qkv, cs, n=n, heads=heads, hd=d // heads, rot=rot, qn=Ld["qn"], kn=Ld["kn"])
    att = wq.attention(qkv, dev(valid), n=n, heads=heads, hd=d // heads,
                       scale=float(np.float32(1.0) / np.sqrt(np.float32(d // heads))))
    wq.gemm(att, Ld["out_w"], wq.W_BF16, m=d, k=d, bias=Ld["out_b"], residual=True, out=hs, path=wq.PATH_MFMA)
    a = wq.layer_norm(hs, Ld["ln2"], d=d)
    f = wq.gemm(a, Ld["fc1_w"], wq.W_BF16, m=inter, k=d, bias=Ld["fc1_b"], gelu=True, path=wq.PATH_MFMA)
    wq.gemm(f, Ld["fc2_w"], wq.W_BF16, m=d, k=inter, bias=Ld["fc2_b"], residual=True, out=hs, path=wq.PATH_MFMA)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got, hs.cpu().numpy())
