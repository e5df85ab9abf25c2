"""Plain f64 CPU oracle of the rest of the encoder block around the linear layer.

TEST INFRASTRUCTURE, like the rest of this package: only the tests, the package's smoke check and
the bench's CPU-baseline leg may import or call it. It shares no code with the HIP path.

Written from cortiq-engine 0.8.49, ``src/gpu_wgpu/nemotron_audio.rs`` (the module comment, the
``AE_WGSL`` kernels ``ae_ln``, ``ae_qk`` and ``ae_attn`` with their parameter blocks, and
``AudioEncoder::run``):

* ``layer_norm``: a row LayerNorm over ``d`` values, eps 1e-5, with the variance taken as the mean
  square deviation (division by ``d``); weight and bias packed as one ``[w | b]`` vector.
* ``rope_table``, ``qk_norm_rope``: per head, an optional LayerNorm of q and of k (own ``[w | b]``
  of ``hd`` each, same eps), then a rotation of the first ``rot`` dims in two halves: dim ``i``
  pairs with dim ``i + rot/2``, at angle ``t * 10000^(-2i/rot)`` for frame ``t`` (frames count
  from 0). v is not touched.
* ``attention``: bidirectional attention per head over the packed ``[q | k | v]`` rows, with
  scores scaled by ``scale`` and keys masked by ``valid``.
* ``encoder_layer`` / ``encoder_forward``: the pre-norm block of ``AudioEncoder::run``:
  LayerNorm, fused q/k/v product, q/k norm + rotation, attention, output product with bias and
  residual, LayerNorm, GELU MLP with residual; the forward adds the optional input projection
  (no bias), the embedding LayerNorm before the blocks and the final LayerNorm after them.

Every step is f64 with plain numpy primitives; the products go through ``reference.linear``.
"""
from __future__ import annotations

import numpy as np

from .reference import FLAG_BIAS, FLAG_GELU, FLAG_RESIDUAL, linear

LN_EPS = 1e-5
ROPE_BASE = 10000.0


def layer_norm(x, wb) -> np.ndarray:
    """Row LayerNorm (``ae_ln``): for each row ``x`` of ``d`` values,
    ``mu = sum(x)/d``, ``var = sum((x - mu)^2)/d``, ``y = (x - mu) / sqrt(var + 1e-5) * w + b``
    with ``wb = [w | b]`` (``2d`` values)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    wb = np.asarray(wb, dtype=np.float64).reshape(2, d)
    mu = x.sum(axis=-1, keepdims=True) / d
    var = ((x - mu) ** 2).sum(axis=-1, keepdims=True) / d
    return (x - mu) / np.sqrt(var + LN_EPS) * wb[0] + wb[1]


def rope_table(n: int, rot: int):
    """``(cos, sin)``, each ``[n][rot/2]``: angle ``t * 10000^(-2i/rot)`` for frame ``t`` and pair
    ``i`` (``AudioEncoder::run`` builds this table on the host, frames from 0)."""
    if rot % 2:
        raise ValueError("rot must be even")
    half = rot // 2
    inv = ROPE_BASE ** (-(2.0 * np.arange(half)) / rot)
    ang = np.arange(n, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def _rotate(v, cos, sin, rot: int) -> np.ndarray:
    """Rotation of the first ``rot`` dims of ``v`` ``[n][hd]``: for ``i < rot/2``,
    ``o_i = v_i c_i - v_{i+rot/2} s_i`` and ``o_{i+rot/2} = v_{i+rot/2} c_i + v_i s_i``; dims from
    ``rot`` on pass through."""
    half = rot // 2
    out = v.copy()
    a, b = v[:, :half], v[:, half:rot]
    out[:, :half] = a * cos - b * sin
    out[:, half:rot] = b * cos + a * sin
    return out


def qk_norm_rope(qkv, heads: int, hd: int, rot: int, cos, sin, qn=None, kn=None) -> np.ndarray:
    """``ae_qk`` on ``[n][3 * heads * hd]`` rows ``[q | k | v]``: returns a copy with each head of
    q and of k LayerNormed over its ``hd`` dims (when ``qn`` / ``kn``, each ``[w | b]`` of ``2 hd``,
    are given) and then rotated on its first ``rot`` dims at the row's frame (``cos``/``sin``
    ``[n][rot/2]``). v is returned as it was."""
    if (qn is None) != (kn is None):
        raise ValueError("give both q and k norm weights or neither")
    if rot % 2 or not 0 <= rot <= hd:
        raise ValueError("rot must be even and in [0, hd]")
    x = np.array(qkv, dtype=np.float64, copy=True)
    n = x.shape[0]
    d = heads * hd
    x = x.reshape(n, 3 * d)
    cos = np.asarray(cos, dtype=np.float64).reshape(n, rot // 2)
    sin = np.asarray(sin, dtype=np.float64).reshape(n, rot // 2)
    for which, norm in ((0, qn), (1, kn)):
        for h in range(heads):
            cols = slice(which * d + h * hd, which * d + (h + 1) * hd)
            v = x[:, cols]
            if norm is not None:
                v = layer_norm(v, norm)
            x[:, cols] = _rotate(v, cos, sin, rot)
    return x


def attention(qkv, valid, heads: int, hd: int, scale: float) -> np.ndarray:
    """``ae_attn``: ``[n][heads * hd]`` outputs. For frame ``t`` and head ``h``, the scores over
    keys ``j`` with ``valid[j] != 0`` are ``scale * q[t,h] . k[j,h]``; their softmax weighs
    ``v[j,h]``. Masked keys take no weight. With no valid key the weights are all 0 and the sum
    is normalised by 1/0, so every output is NaN (0 * inf)."""
    x = np.asarray(qkv, dtype=np.float64)
    n = x.shape[0]
    d = heads * hd
    x = x.reshape(n, 3 * d)
    keep = np.asarray(valid).reshape(n) != 0
    out = np.empty((n, d))
    if not keep.any():
        out[:] = np.nan
        return out
    for h in range(heads):
        q = x[:, h * hd:(h + 1) * hd]
        k = x[keep, d + h * hd:d + (h + 1) * hd]
        v = x[keep, 2 * d + h * hd:2 * d + (h + 1) * hd]
        s = float(scale) * (q @ k.T)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h * hd:(h + 1) * hd] = (e @ v) / e.sum(axis=1, keepdims=True)
    return out


def attention_weight_scale(qkv, valid, heads: int, hd: int, scale: float):
    """``(P|v|, Sqk)`` beside ``attention``: ``P|v|[t, h*hd + c] = sum_j p_tj |v_jc|`` (the sum of
    the weighted magnitudes of the values) and ``Sqk[t, h] = max_j scale * sum_c |q_tc k_jc|`` over
    valid keys (the largest score magnitude before cancellation). The error bounds of the tests
    are stated in these."""
    x = np.asarray(qkv, dtype=np.float64)
    n = x.shape[0]
    d = heads * hd
    x = x.reshape(n, 3 * d)
    keep = np.asarray(valid).reshape(n) != 0
    pv = np.zeros((n, d))
    sqk = np.zeros((n, heads))
    if not keep.any():
        return pv, sqk
    for h in range(heads):
        q = x[:, h * hd:(h + 1) * hd]
        k = x[keep, d + h * hd:d + (h + 1) * hd]
        v = x[keep, 2 * d + h * hd:2 * d + (h + 1) * hd]
        s = float(scale) * (q @ k.T)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        pv[:, h * hd:(h + 1) * hd] = p @ np.abs(v)
        sqk[:, h] = (abs(float(scale)) * (np.abs(q) @ np.abs(k).T)).max(axis=1)
    return pv, sqk


def encoder_layer(h, layer: dict, wtype: int, valid, heads: int, rot: int, cos, sin) -> np.ndarray:
    """One pre-norm block of ``AudioEncoder::run`` on ``h`` ``[n][d]``; returns the new ``h``.

    ``layer`` holds ``ln1``, ``qkv_w`` (``[3d][d]``), ``qkv_b`` (or None: the page's block has
    none), ``qn``/``kn`` (or None), ``out_w``, ``out_b``, ``ln2``, ``fc1_w`` (``[inter][d]``),
    ``fc1_b``, ``fc2_w`` (``[d][inter]``), ``fc2_b``; weights in ``wtype``'s raw layout. The
    attention scale is ``1/sqrt(hd)``, rounded to f32 as the page computes it.
    """
    h = np.asarray(h, dtype=np.float64)
    n, d = h.shape
    hd = d // heads
    inter = np.asarray(layer["fc1_b"]).shape[0]
    scale = float(np.float32(1.0) / np.sqrt(np.float32(hd)))
    a = layer_norm(h, layer["ln1"])
    qkv_flags = FLAG_BIAS if layer.get("qkv_b") is not None else 0
    qkv, _ = linear(a, layer["qkv_w"], wtype, 3 * d, d, layer.get("qkv_b"), qkv_flags)
    qkv = qk_norm_rope(qkv, heads, hd, rot, cos, sin, layer.get("qn"), layer.get("kn"))
    att = attention(qkv, valid, heads, hd, scale)
    h, _ = linear(att, layer["out_w"], wtype, d, d, layer["out_b"], FLAG_BIAS | FLAG_RESIDUAL, h)
    a = layer_norm(h, layer["ln2"])
    f, _ = linear(a, layer["fc1_w"], wtype, inter, d, layer["fc1_b"], FLAG_BIAS | FLAG_GELU)
    h, _ = linear(f, layer["fc2_w"], wtype, d, inter, layer["fc2_b"], FLAG_BIAS | FLAG_RESIDUAL, h)
    return h


def encoder_forward(x, enc: dict, wtype: int, valid, heads: int, rot: int) -> np.ndarray:
    """``AudioEncoder::run``: ``x`` is ``[n][stack_in]`` stacked features when ``enc["proj"]`` is
    given (projected to ``d`` with no bias), else ``[n][d]`` embedded rows. Then the embedding
    LayerNorm, every block of ``enc["layers"]`` and the final LayerNorm; returns ``[n][d]``."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    d = np.asarray(enc["embed_norm"]).shape[0] // 2
    if enc.get("proj") is not None:
        x, _ = linear(x, enc["proj"], wtype, d, x.shape[1], None, 0)
    cos, sin = rope_table(n, rot)
    h = layer_norm(x, enc["embed_norm"])
    for layer in enc["layers"]:
        h = encoder_layer(h, layer, wtype, valid, heads, rot, cos, sin)
    return layer_norm(h, enc["final_norm"])
