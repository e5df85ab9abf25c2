"""The encoder-block entry points on the host: argument checks that refuse a call before any HIP
call (fake, never dereferenced device addresses), the workspace sizes, and the host-built rotation
table against the oracle's f64 table within the bound of its f32 arithmetic.
"""
import ctypes

import numpy as np
import pytest
import torch

import gemv_wq_gemm_amd as wq
from oracle import encoder as enc

if torch.cuda.device_count() > 0:
    pytest.skip("host-side checks with fake device pointers: run where no GPU is visible",
                allow_module_level=True)

A, B, C, D, E = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000  # aligned, far apart
NULL = None


def _ln(**kw):
    a = dict(x=A, wb=B, y=C, n=4, d=64)
    a.update(kw)
    return wq.lib().wq_layer_norm(a["x"], a["wb"], a["y"], a["n"], a["d"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), -2), (dict(d=0), -2), (dict(x=NULL), -1), (dict(wb=NULL), -1), (dict(y=NULL), -1),
    (dict(x=A + 2), -5), (dict(y=C + 1), -5),
    (dict(y=A + 4), -6),           # partial overlap with x
    (dict(y=B), -6),               # y on wb
    (dict(n=1 << 31), -2),
])
def test_layer_norm_argument_errors(kw, code):
    assert _ln(**kw) == code
    assert wq.lib().wq_last_error().decode()


def test_layer_norm_empty_is_a_noop():
    assert _ln(n=0, x=NULL, wb=NULL, y=NULL) == 0


def _qk(**kw):
    a = dict(qkv=A, qn=B, kn=C, cs=D, n=8, heads=2, hd=64, rot=32)
    a.update(kw)
    return wq.lib().wq_qk_norm_rope(a["qkv"], a["qn"], a["kn"], a["cs"], a["n"], a["heads"], a["hd"], a["rot"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(hd=0), -2), (dict(hd=257), -2), (dict(heads=0), -2), (dict(rot=3), -2), (dict(rot=66), -2),
    (dict(rot=-2), -2), (dict(kn=NULL), -1), (dict(qkv=NULL), -1), (dict(cs=NULL), -1),
    (dict(qkv=A + 2), -5), (dict(cs=A + 64), -6), (dict(n=(1 << 22) + 1), -2),
])
def test_qk_norm_rope_argument_errors(kw, code):
    assert _qk(**kw) == code


def test_qk_norm_rope_accepts_no_norm_and_no_rotation_sizes():
    # Valid sizes with n = 0 return before touching any pointer.
    assert _qk(n=0, qn=NULL, kn=NULL, cs=NULL, rot=0) == 0


def _attn(**kw):
    a = dict(qkv=A, valid=B, o=C, ws=0x100000, wsb=1 << 30, n=100, heads=2, hd=64, scale=0.125)
    a.update(kw)
    return wq.lib().wq_attention(a["qkv"], a["valid"], a["o"], a["ws"], a["wsb"], a["n"], a["heads"], a["hd"],
                                 a["scale"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(hd=129), -2), (dict(hd=0), -2), (dict(heads=0), -2), (dict(n=-1), -2), (dict(n=(1 << 22) + 1), -2),
    (dict(scale=float("inf")), -4), (dict(scale=float("nan")), -4),
    (dict(qkv=NULL), -1), (dict(valid=NULL), -1), (dict(o=NULL), -1), (dict(ws=NULL), -1),
    (dict(ws=0x100000 + 128), -5), (dict(o=C + 2), -5),
    (dict(wsb=1000), -2),
    (dict(o=A + 64), -6),          # o inside qkv
])
def test_attention_argument_errors(kw, code):
    assert _attn(**kw) == code


def test_workspace_sizes():
    # K and V in bf16 over frames padded to 64 and head dims padded to 32/64/128, plus the key bias.
    assert wq.attention_workspace_bytes(1500, 8, 128) == 2 * 8 * 1536 * 128 * 2 + 1536 * 4
    assert wq.attention_workspace_bytes(1, 3, 40) == 2 * ((3 * 64 * 64 * 2 + 255) // 256 * 256) + 256
    assert wq.lib().wq_attention_workspace_bytes(10, 1, 129) == -1
    nd, n, d, inter = 1500 * 1024 * 4, 1500, 1024, 4096
    assert wq.encoder_workspace_bytes(n, d, 8, inter) == nd + 3 * nd + nd + n * inter * 4 + \
        wq.attention_workspace_bytes(n, 8, d // 8)
    for bad in ((10, 48, 2, 64), (10, 64, 3, 64), (10, 64, 2, 48), (10, 512, 2, 64)):
        assert wq.lib().wq_encoder_workspace_bytes(*bad) == -1, bad


def _layer_ptrs(**kw):
    fields = dict(ln1=A, qkv_w=B, qkv_b=None, qn=None, kn=None, out_w=C, out_b=D, ln2=E, fc1_w=0x60000,
                  fc1_b=0x70000, fc2_w=0x80000, fc2_b=0x90000)
    fields.update(kw)
    return wq.EncoderLayerDesc(**fields)


def _layer(desc=None, **kw):
    a = dict(wtype=wq.W_BF16, h=0x200000, valid=0x300000, cs=0x400000, ws=0x1000000, wsb=1 << 40, n=100, d=128,
             heads=2, rot=64, inter=256, path=wq.PATH_AUTO)
    a.update(kw)
    d = desc if desc is not None else _layer_ptrs()
    return wq.lib().wq_encoder_layer(ctypes.byref(d), a["wtype"], a["h"], a["valid"], a["cs"], a["ws"], a["wsb"],
                                     a["n"], a["d"], a["heads"], a["rot"], a["inter"], a["path"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=100), -2), (dict(inter=100), -2), (dict(heads=3), -2), (dict(d=512, heads=2), -2),
    (dict(rot=66), -2), (dict(rot=5), -2), (dict(path=wq.PATH_MATVEC), -2), (dict(wtype=9), -3),
    (dict(h=NULL), -1), (dict(valid=NULL), -1), (dict(ws=NULL), -1), (dict(cs=NULL), -1),
    (dict(h=0x200000 + 4), -5), (dict(ws=0x1000000 + 16), -5), (dict(wsb=100), -2),
    (dict(h=0x1000000 + 256), -6),
])
def test_encoder_layer_argument_errors(kw, code):
    assert _layer(**kw) == code


def test_encoder_layer_weight_checks():
    assert _layer(_layer_ptrs(ln1=None)) == -1
    assert _layer(_layer_ptrs(qn=A)) == -1  # qn without kn
    assert wq.lib().wq_encoder_layer(None, 0, 1, 1, 1, 1, 1, 10, 64, 1, 0, 64, 0, None) == -1
    assert _layer(n=0, h=NULL, valid=NULL, ws=NULL, cs=NULL) == 0


@pytest.mark.parametrize("desc_kw,kw,code", [
    (dict(fc2_w=0x80000 + 8), {}, -5),        # the last product's weight, misaligned
    (dict(qkv_b=0xA0002), {}, -5),            # a vector, misaligned
    (dict(fc1_w=0x200000), {}, -6),           # a weight on h
    (dict(out_b=0x1000000 + 1024), {}, -6),   # a vector inside the workspace
    ({}, dict(valid=0x200000 + 8), -6),       # valid inside h
    ({}, dict(cs=0x1000000), -6),             # cs on the workspace
    ({}, dict(wtype=wq.W_Q4_K, d=256, inter=512), -3),  # Q4_K at n = 100: the products take n <= 16 only
])
def test_encoder_layer_checks_every_step_before_launching(desc_kw, kw, code):
    """Each of these would be refused only at a later step if the steps were checked one at a
    time; here the call is refused before the first launch (without a GPU a launch would return
    WQ_ERR_HIP, -7), so h is left as it was."""
    assert _layer(_layer_ptrs(**desc_kw), **kw) == code
    assert wq.lib().wq_last_error().decode()


def test_encoder_layer_valid_call_reaches_the_launch():
    # Every check passes; the first launch then fails for want of a GPU.
    assert _layer() == -7
    assert "launch" in wq.lib().wq_last_error().decode().lower()


def test_rope_table_argument_errors():
    buf = (ctypes.c_float * 16)()
    assert wq.lib().wq_rope_table(buf, 4, 3) == -2
    assert wq.lib().wq_rope_table(buf, 4, 0) == -2
    assert wq.lib().wq_rope_table(buf, -1, 4) == -2
    assert wq.lib().wq_rope_table(None, 4, 4) == -1
    assert wq.lib().wq_rope_table(None, 0, 4) == 0


@pytest.mark.parametrize("n,rot", [(1, 2), (7, 6), (100, 64), (1500, 128)])
def test_rope_table_within_f32_bound(n, rot):
    """The host table computes 10000^(2i/rot), its inverse, the angle t * inv and its cosine and
    sine in f32. Each step rounds once (powf and the libm cos/sin are within an ulp or two), so the
    angle carries a relative error of at most 6 u (u = 2^-24) and each entry an absolute error of
    at most 6 u * angle + 2 u against the exact table."""
    cs = wq.rope_table(n, rot).numpy().astype(np.float64)
    half = rot // 2
    cos, sin = enc.rope_table(n, rot)
    u = 2.0 ** -24
    ang = np.arange(n)[:, None] * 10000.0 ** (-(2.0 * np.arange(half)) / rot)[None, :]
    bound = 6 * u * ang + 2 * u
    got_c = cs[:n * half].reshape(n, half)
    got_s = cs[n * half:].reshape(n, half)
    assert np.all(np.abs(got_c - cos) <= bound)
    assert np.all(np.abs(got_s - sin) <= bound)
    assert got_c[0].tolist() == [1.0] * half and got_s[0].tolist() == [0.0] * half
