"""Error bounds of the encoder-block kernels against the f64 oracle, derived from their arithmetic.

u = 2^-24 is the f32 unit roundoff. Every bound is elementwise and is computed from the oracle's own
values (never from the GPU's). Each kernel's own rounding is bounded term by term below (worst
case); a whole block is checked with the probabilistic model at the end of this file.

LayerNorm (one f32 pass for the mean, one for the squared deviations, rsqrt, then
(x - mu) * inv * w + b):
    e_mu  <= (d + 2) u mean|x|                      (d-term sum and the division)
    inv   relative <= ((d + 6) u var + e_mu^2) / (2 (var + eps)) + 3 u
    y     <= |w| inv (e_mu + |x - mu| (rel_inv + 4 u)) + 2 u (|y| + |b|)
and the whole is scaled by 1.25 for the second-order products of these terms.

Rotation (o = v_a c -/+ v_b s in f32): |c| E_a + |s| E_b + 3 u (|v_a c| + |v_b s|), plus
|v_a| dc + |v_b| ds when the table itself differs from the exact one by dc, ds.

Attention: q, k, v and the weights are rounded to bf16; scores and sums are f32.
  bf16 keeps 8 significant bits, so rounding to nearest moves a value by at most 2^-8 of itself.
  * scores: the bf16 products are exact, their f32 sum errs by at most (hd + 3) u Sqk (Sqk: the
    largest scale * sum_c |q_c k_c| of the query); from f32 inputs, rounding q and k adds
    (2^-7 + 2^-16) Sqk. A score error of at most delta moves each softmax weight by a factor
    within e^(+-2 delta).
  * weights rounded to bf16 (2^-8 each) and normalised by the sum of the rounded weights: each
    final weight within a factor 1 +- 2^-7 (1.01) of the unrounded one.
  * v rounded to bf16: 2^-8 relative (from f32 inputs only).
  * the weighted sum, the running sum of weights and the per-tile rescales: (2 npad + tiles + 10) u
    relative to sum_j p_j |v_j| (npad: frames padded to 64).
    So |o - o_ref| <= P|v| ((e^(2 delta) - 1) + 2^-7 (1.01) + [2^-8] + (2 npad + tiles + 10) u)
    e^(2 delta), times 1.1.
"""
from __future__ import annotations

import numpy as np

import synth
from oracle import encoder as enc

U = 2.0 ** -24
EPS = 1e-5


def bf16_round(a) -> np.ndarray:
    """f32 values rounded to bf16 (nearest even), as f64."""
    bits = synth.bf16_bits(np.asarray(a, np.float32)).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def _ln_parts(x, wb):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    wb = np.asarray(wb, np.float64).reshape(2, d)
    mu = x.mean(axis=-1, keepdims=True)
    c = x - mu
    var = (c * c).mean(axis=-1, keepdims=True)
    inv = 1.0 / np.sqrt(var + EPS)
    return d, wb[0], wb[1], mu, c, var, inv


def ln_tol(x, wb) -> np.ndarray:
    """Rounding bound of the f32 LayerNorm at exact inputs ``x`` (rows of the last axis)."""
    d, w, b, mu, c, var, inv = _ln_parts(x, wb)
    e_mu = (d + 2) * U * np.abs(np.asarray(x, np.float64)).mean(axis=-1, keepdims=True)
    rel_inv = 0.5 * ((d + 6) * U * var + e_mu ** 2) / (var + EPS) + 3 * U
    y = c * inv * w + b
    return 1.25 * (np.abs(w) * inv * (e_mu + np.abs(c) * (rel_inv + 4 * U)) + 2 * U * (np.abs(y) + np.abs(b)))


def ln_prop(x, wb, e_in) -> np.ndarray:
    """First-order bound on the change of LayerNorm's output when each input moves by at most
    ``e_in``: dy_i = w_i inv (dx_i - mean(dx) - xh_i mean(xh dx)), xh the normalised row."""
    d, w, b, mu, c, var, inv = _ln_parts(x, wb)
    xh = c * inv
    e = np.asarray(e_in, np.float64)
    return np.abs(w) * inv * (e + e.mean(axis=-1, keepdims=True) +
                              np.abs(xh) * (np.abs(xh) * e).mean(axis=-1, keepdims=True))


def rope_table_err(n: int, rot: int):
    """Bound on |table - exact table| of the host-built f32 table (6 u angle + 2 u)."""
    half = rot // 2
    ang = np.arange(n)[:, None] * 10000.0 ** (-(2.0 * np.arange(half)) / rot)[None, :]
    e = 6 * U * ang + 2 * U
    return e, e


def qk_bound(qkv, heads: int, hd: int, rot: int, cos, sin, qn=None, kn=None, e_in=None, table_err=None):
    """(reference, bound) of the q/k norm + rotation: the oracle's result for exact inputs, and
    the bound on |GPU - reference| given input errors ``e_in`` (None: exact inputs) and a table
    that differs from ``cos``/``sin`` by ``table_err`` (None: the same table)."""
    x = np.asarray(qkv, np.float64)
    n = x.shape[0]
    d = heads * hd
    ref = enc.qk_norm_rope(x, heads, hd, rot, cos, sin, qn, kn)
    e_all = np.zeros_like(x) if e_in is None else np.asarray(e_in, np.float64).copy()
    out = e_all.copy()
    half = rot // 2
    cos = np.asarray(cos, np.float64).reshape(n, half)
    sin = np.asarray(sin, np.float64).reshape(n, half)
    tc, ts = (np.zeros((n, half)), np.zeros((n, half))) if table_err is None else table_err
    for which, nw in ((0, qn), (1, kn)):
        for h in range(heads):
            cols = slice(which * d + h * hd, which * d + (h + 1) * hd)
            v, e = x[:, cols], e_all[:, cols]
            if nw is not None:
                e = ln_prop(v, nw, e) + ln_tol(v, nw)
                v = enc.layer_norm(v, nw)
            r = e.copy()
            a, b = v[:, :half], v[:, half:rot]
            ea, eb = e[:, :half], e[:, half:rot]
            r[:, :half] = (np.abs(cos) * ea + np.abs(sin) * eb + 3 * U * (np.abs(a * cos) + np.abs(b * sin)) +
                           np.abs(a) * tc + np.abs(b) * ts)
            r[:, half:rot] = (np.abs(cos) * eb + np.abs(sin) * ea + 3 * U * (np.abs(b * cos) + np.abs(a * sin)) +
                              np.abs(b) * tc + np.abs(a) * ts)
            out[:, cols] = r
    return ref, out


def _heads(x, keep, h, hd, d):
    q = x[:, h * hd:(h + 1) * hd]
    k = x[keep, d + h * hd:d + (h + 1) * hd]
    v = x[keep, 2 * d + h * hd:2 * d + (h + 1) * hd]
    return q, k, v


def _probs(q, k, scale):
    s = scale * (q @ k.T)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def attn_tol(qkv, valid, heads: int, hd: int, scale: float, rounded_inputs: bool) -> np.ndarray:
    """Rounding bound of the attention kernel at exact inputs ``qkv``; ``rounded_inputs`` when
    q, k and v are already bf16 values (then the kernel's own rounding of them is exact)."""
    x = np.asarray(qkv, np.float64)
    n = x.shape[0]
    pv, sqk = enc.attention_weight_scale(x, valid, heads, hd, scale)
    npad = -(-n // 64) * 64
    tiles = npad // 64
    delta = (hd + 3) * U * sqk * (1 + 2.0 ** -8)
    if not rounded_inputs:
        delta = delta + (2.0 ** -7 + 2.0 ** -16) * sqk
    grow = np.exp(2 * np.repeat(delta, hd, axis=1))
    rel = (grow - 1) + 2.0 ** -7 * 1.01 + (0 if rounded_inputs else 2.0 ** -8) + (2 * npad + tiles + 10) * U
    return 1.1 * pv * rel * grow


def attn_prop(qkv, valid, heads: int, hd: int, scale: float, e_in) -> np.ndarray:
    """First-order bound on the change of the attention output when each of q, k, v moves by at
    most ``e_in``: do = sum_j p_j dv_j + sum_j p_j (v_j - o)(dS_j - sum_l p_l dS_l), with
    |dS_j| <= scale (|q| . e_k_j + e_q . |k_j|) and |v_j - o| <= |v_j| + |o|."""
    x = np.asarray(qkv, np.float64)
    e = np.asarray(e_in, np.float64)
    n = x.shape[0]
    d = heads * hd
    keep = np.asarray(valid).reshape(n) != 0
    out = np.zeros((n, d))
    if not keep.any():
        return out
    for h in range(heads):
        q, k, v = _heads(x, keep, h, hd, d)
        eq, ek, ev = _heads(e, keep, h, hd, d)
        p = _probs(q, k, scale)
        o = p @ v
        es = abs(scale) * (np.abs(q) @ ek.T + eq @ np.abs(k).T)
        w = p * (es + (p * es).sum(axis=1, keepdims=True))
        out[:, h * hd:(h + 1) * hd] = p @ ev + w @ np.abs(v) + w.sum(axis=1, keepdims=True) * np.abs(o)
    return out


def gemm_step(x, e_x, w_f64, bias, bound):
    """(value, error bound) of ``x . W^T (+ bias)`` on a matrix-core path with the given bound B:
    B S for the call itself, |W| e_x carried from the input, u for the bias add."""
    v = x @ w_f64.T
    s = np.abs(x) @ np.abs(w_f64).T
    e = bound * s + e_x @ np.abs(w_f64).T
    if bias is not None:
        v = v + np.asarray(bias, np.float64)[None, :]
        e = e + U * (np.abs(v) + np.abs(np.asarray(bias, np.float64))[None, :])
    return v, e


# ---------------------------------------------------------------------------------------------
# A whole block: probabilistic propagation
# ---------------------------------------------------------------------------------------------
# Worst-case bounds do not compose usefully through a block: a product sums k input errors of
# either sign as if all had the same sign, and attention turns score errors into weight errors
# exponentially, so the worst case grows past the outputs themselves. The block test instead uses
# the standard probabilistic model of rounding: every rounding error is independent and of mean
# zero; one bounded by r has variance at most r^2 / 3. (Higham and Mary, "A new approach to
# probabilistic rounding error analysis", SIAM J. Sci. Comput. 2019, bound sums of such errors
# under the same assumption.) Each step adds the variance of its own roundings -- the worst-case
# bound of a step's own f32 roundings (the functions above) counted as one such error -- to that of
# its inputs carried through its derivative. An output is accepted when its error is within
# LAMBDA = 8 standard deviations, plus 4 u of its magnitude.

R_BF16 = 2.0 ** -8    # unit roundoff of bf16 (8 significant bits) rounding to nearest
LAMBDA = 8.0


def gemm_sigma(x, var_x, w_f64, bias, bf16: bool):
    """(value, variance) of ``x . W^T (+ bias)``: on the bf16 path each x is rounded (variance
    R_BF16^2/3 x^2 each); the f32 sum of k terms adds about u^2/3 * k/2 * sum (x w)^2, the bias add
    u^2/3 |v|^2."""
    k = x.shape[1]
    v = x @ w_f64.T
    sq = (x * x) @ (w_f64 * w_f64).T
    var = (var_x @ (w_f64 * w_f64).T) + (U * U / 3.0) * (k / 2.0) * sq
    if bf16:
        var = var + (R_BF16 ** 2 / 3.0) * sq
    if bias is not None:
        v = v + np.asarray(bias, np.float64)[None, :]
        var = var + (U * U / 3.0) * v * v
    return v, var


def ln_sigma(x, wb, var_x):
    """(value, variance) of LayerNorm: dy_i = w_i inv (dx_i - mean(dx) - xh_i mean(xh dx)); with
    independent input errors the last two terms add at most (1 + xh_i^2) mean(var) to dx_i's
    variance. Its own f32 roundings: ``ln_tol`` as one bounded error."""
    d, w, b, mu, c, var, inv = _ln_parts(x, wb)
    xh = c * inv
    v = xh * w + b
    out = (w * inv) ** 2 * (var_x + (1 + xh * xh) * var_x.mean(axis=-1, keepdims=True))
    return v, out + ln_tol(x, wb) ** 2 / 3.0


def qk_sigma(qkv, var_in, heads: int, hd: int, rot: int, cos, sin, qn, kn, table_err):
    """(value, variance) of the q/k norm and rotation, with the table's own error bound."""
    x = np.asarray(qkv, np.float64)
    n = x.shape[0]
    d = heads * hd
    val = x.copy()
    var = np.asarray(var_in, np.float64).copy()
    half = rot // 2
    cos = np.asarray(cos, np.float64).reshape(n, half)
    sin = np.asarray(sin, np.float64).reshape(n, half)
    tc, ts = table_err
    for which, nw in ((0, qn), (1, kn)):
        for h in range(heads):
            cols = slice(which * d + h * hd, which * d + (h + 1) * hd)
            v, s2 = x[:, cols], var[:, cols]
            if nw is not None:
                v, s2 = ln_sigma(v, nw, s2)
            a, b = v[:, :half], v[:, half:rot]
            ra, rb = s2[:, :half], s2[:, half:rot]
            out_v, out_s = v.copy(), s2.copy()
            out_v[:, :half] = a * cos - b * sin
            out_v[:, half:rot] = b * cos + a * sin
            own = (3 * U * (np.abs(a * cos) + np.abs(b * sin)) + np.abs(a) * tc + np.abs(b) * ts) ** 2 / 3.0
            out_s[:, :half] = cos ** 2 * ra + sin ** 2 * rb + own
            out_s[:, half:rot] = cos ** 2 * rb + sin ** 2 * ra + own
            val[:, cols], var[:, cols] = out_v, out_s
    return val, var


def attn_sigma(qkv, var_in, valid, heads: int, hd: int, scale: float):
    """(value, variance) of attention. The kernel's bf16 roundings of q, k and v join their input
    variances; the rounding of each weight p_j (relative, normalised by the rounded sum) moves o by
    sum_j p_j eta_j (v_j - o). To first order
        do = sum_j p_j dv_j + sum_j p_j (v_j - o) dS_j        (sum_j p_j (v_j - o) = 0)
        dS_j = scale (q . dk_j + dq . k_j),
    where dk_j differs from key to key but dq is shared by all of a query's scores:
        var(o_c) = sum_j p_j^2 var(v_jc)
                 + scale^2 sum_j p_j^2 (v_jc - o_c)^2 sum_c' q_c'^2 var(k_jc')
                 + scale^2 sum_c' var(q_c') (sum_j p_j (v_jc - o_c) k_jc')^2
                 + R_BF16^2/3 sum_j p_j^2 (v_jc - o_c)^2,
    plus the f32 sums, (2 npad + tiles + 14) u sum_j p_j |v_j| as one bounded error."""
    x = np.asarray(qkv, np.float64)
    n = x.shape[0]
    d = heads * hd
    keep = np.asarray(valid).reshape(n) != 0
    var_x = np.asarray(var_in, np.float64) + (R_BF16 ** 2 / 3.0) * x * x
    val = enc.attention(x, valid, heads, hd, scale)
    npad = -(-n // 64) * 64
    pv, _ = enc.attention_weight_scale(x, valid, heads, hd, scale)
    var = ((2 * npad + npad // 64 + 14) * U * pv) ** 2 / 3.0
    for h in range(heads):
        q, k, v = _heads(x, keep, h, hd, d)
        sq, sk, sv = _heads(var_x, keep, h, hd, d)
        p = _probs(q, k, scale)
        o = val[:, h * hd:(h + 1) * hd]
        p2 = p * p
        dev2 = lambda wts: wts @ (v * v) - 2 * o * (wts @ v) + o * o * wts.sum(axis=1, keepdims=True)  # noqa: E731
        term_v = p2 @ sv
        term_k = scale * scale * dev2(p2 * ((q * q) @ sk.T))
        term_p = (R_BF16 ** 2 / 3.0) * dev2(p2)
        # shared dq: M[t, c, c'] = sum_j p_tj v_jc k_jc' - o_tc (p_t . k)_c', as one matrix product
        # over the keys' outer products v_j k_j^T (row j of `outer`)
        outer = (v[:, :, None] * k[:, None, :]).reshape(v.shape[0], hd * hd)
        m = (p @ outer).reshape(-1, hd, hd) - o[:, :, None] * (p @ k)[:, None, :]
        term_q = scale * scale * np.einsum("tce,te->tc", m * m, sq)
        del outer, m
        var[:, h * hd:(h + 1) * hd] += np.maximum(term_v + term_k + term_q + term_p, 0.0)
    return val, var


def gelu_slope(v):
    from scipy.special import erf
    return np.abs(0.5 * (1 + erf(v / np.sqrt(2))) + v * np.exp(-v * v / 2) / np.sqrt(2 * np.pi))


def layer_sigma(h, L, valid, heads: int, rot: int, bf16: bool, var_in=None):
    """(value, variance) of one block by the oracle, step by step; ``var_in`` is the variance the
    input ``h`` already carries."""
    from oracle import reference as ref
    h = np.asarray(h, np.float64)
    n, d = h.shape
    hd = d // heads
    inter = np.asarray(L["fc1_b"]).shape[0]
    var_h = np.zeros_like(h) if var_in is None else var_in
    dec = lambda w, m, k: ref.decode(w, ref.W_BF16, m, k)  # noqa: E731
    scale = float(np.float32(1.0) / np.sqrt(np.float32(hd)))
    cos, sin = enc.rope_table(n, rot)
    a1, var = ln_sigma(h, L["ln1"], var_h)
    qkv, var = gemm_sigma(a1, var, dec(L["qkv_w"], 3 * d, d), L.get("qkv_b"), bf16)
    qr, var = qk_sigma(qkv, var, heads, hd, rot, cos, sin, L.get("qn"), L.get("kn"), rope_table_err(n, rot))
    att, var = attn_sigma(qr, var, valid, heads, hd, scale)
    o, var = gemm_sigma(att, var, dec(L["out_w"], d, d), L["out_b"], bf16)
    h1 = h + o
    var_h1 = var_h + var + (U * U / 3.0) * h1 * h1
    a2, var = ln_sigma(h1, L["ln2"], var_h1)
    fpre, var = gemm_sigma(a2, var, dec(L["fc1_w"], inter, d), L["fc1_b"], bf16)
    f = ref.gelu_erf(fpre)
    var = gelu_slope(fpre) ** 2 * var + (4 * U * f) ** 2 / 3.0
    o2, var = gemm_sigma(f, var, dec(L["fc2_w"], d, inter), L["fc2_b"], bf16)
    h2 = h1 + o2
    return h2, var_h1 + var + (U * U / 3.0) * h2 * h2


def sigma_tol(value, var) -> np.ndarray:
    """The acceptance band of the probabilistic model: LAMBDA standard deviations plus 4 u."""
    return LAMBDA * np.sqrt(var) + 4 * U * np.abs(value)
