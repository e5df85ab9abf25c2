"""Plain f64 CPU oracle of the weight-dequantizing linear layer.

TEST INFRASTRUCTURE. Only the tests, the package's smoke check and the
bench's CPU-baseline leg may import or call this module; the product path
never does. It shares no code with the HIP path and imports nothing from it.

What it computes, written out from the pages it follows:

* ``Y = epilogue(X . W^T + b)`` with X ``[n x k]``, W ``[m x k]``, Y ``[n x m]``
  -- the kernel contract stated at the top of cortiq-engine
  ``nemotron_audio.rs`` (``AE_WGSL``, the ``ae_gemm`` comment and its
  ``GmP`` parameter block), with the epilogue of its ``ae_put``: add the bias
  (flag 1), then erf-GELU (flag 2), then add the value already in Y (flag 4).
  wavo ``gpu/mod.rs`` ``Epilogue`` (``Residual``/``GeluResidual``) describes
  the same accumulate-into-output step, and adds the other activations
  (SiLU, ReLU, tanh: flags 8, 16, 32 here) and a factor alpha on the
  accumulated value (``Residual(alpha)``).
* Weights are decoded exactly before the product: bf16 is the upper half of
  an f32 (``ae_gemm``'s weight-pair unpacking); f32 and f16 are IEEE values
  (wavo's ``Linear`` types 0 and 1); Q8_0 is ``d * q`` with an f16
  ``d`` and int8 ``q`` (wavo ``Gpu::upload_linear`` and the test helper
  ``weights``); Q4_0 is ``d * (q - 8)`` with 4-bit ``q`` (format named by
  hanzo-ml ``wgpu_backend.rs`` ``matvec_q4_0_gpu``; nibble order: low nibbles
  are elements 0-15, high nibbles 16-31). Q4_K (hanzo-ml ``matvec_q4k_gpu``:
  144-byte super-blocks of 256 weights, k a multiple of 256) is
  ``d * sc_j * q - dmin * m_j`` per 32-element sub-block ``j``; the pages name
  the type but do not print its bytes, so its layout is GGML's published
  k-quant super-block (``decode_q4_k``).
* The MoE matvec of hanzo-ml ``moe_matvec_gpu``: for routed slot ``s`` and
  output row ``r``, ``y[s, r] = sum_k W[ids[s], r, k] * x[s, k]`` over one
  weight bank ``[E, m, k]``; with gate weights the slots of a token are summed,
  each times its gate.

Every step uses f64 and a plain library primitive (numpy matmul, scipy erf);
nothing is blocked, fused or reordered. The error scale
``S[t, j] = sum_k |x[t, k] * w[j, k]|`` that the acceptance bounds use is
returned beside every result.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

W_BF16, W_Q8_0, W_Q4_0, W_F32, W_F16, W_Q4_K = 0, 1, 2, 3, 4, 5
FLAG_BIAS, FLAG_GELU, FLAG_RESIDUAL = 1, 2, 4
FLAG_SILU, FLAG_RELU, FLAG_TANH = 8, 16, 32
QBLOCK = 32
QBYTES = {W_Q8_0: 34, W_Q4_0: 18}
# Q4_K super-block: 256 weights in 144 bytes (hanzo-ml ``matvec_q4k_gpu`` states both sizes).
QK_K = 256
Q4K_BYTES = 144


# ---------------------------------------------------------------------------
# Scalar formats
# ---------------------------------------------------------------------------

def f16_bits_to_f64(bits) -> np.ndarray:
    """Value of IEEE-754 binary16 bit patterns: 1 sign, 5 exponent (bias 15), 10 fraction bits.

    Written from the format's definition: normal numbers are
    ``(-1)^s * 2^(e-15) * (1 + f/1024)``, subnormals (e = 0) are
    ``(-1)^s * 2^-14 * f/1024``, e = 31 is infinity (f = 0) or NaN.
    """
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    s = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = s * np.ldexp(1.0 + f / 1024.0, (e - 15).astype(np.int64))
    sub = s * np.ldexp(f / 1024.0, -14)
    special = np.where(f == 0, s * np.inf, np.nan)
    return np.where(e == 0, sub, np.where(e == 31, special, normal))


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Value of bfloat16 bit patterns: 1 sign, 8 exponent (bias 127), 7 fraction bits.

    A bf16 is the upper half of an f32 (the ``ae_gemm`` weight unpack shifts it
    into the high 16 bits), so it has f32's exponent range: normals are
    ``(-1)^s * 2^(e-127) * (1 + f/128)``, subnormals ``(-1)^s * 2^-126 * f/128``.
    """
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    s = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    f = (b & 0x7F).astype(np.float64)
    normal = s * np.ldexp(1.0 + f / 128.0, (e - 127).astype(np.int64))
    sub = s * np.ldexp(f / 128.0, -126)
    special = np.where(f == 0, s * np.inf, np.nan)
    return np.where(e == 0, sub, np.where(e == 255, special, normal))


def f32_bits_to_f64(bits) -> np.ndarray:
    """Value of IEEE-754 binary32 bit patterns: 1 sign, 8 exponent (bias 127), 23 fraction bits.

    Normals are ``(-1)^s * 2^(e-127) * (1 + f/2^23)``, subnormals (e = 0)
    ``(-1)^s * 2^-126 * f/2^23``, e = 255 is infinity (f = 0) or NaN. (wavo's
    ``Linear`` F32 weights, type 0 of ``Gpu::upload_linear``, are these values.)
    """
    b = np.asarray(bits).astype(np.int64) & 0xFFFFFFFF
    s = np.where(b >> 31, -1.0, 1.0)
    e = (b >> 23) & 0xFF
    f = (b & 0x7FFFFF).astype(np.float64)
    normal = s * np.ldexp(1.0 + f / 2.0 ** 23, (e - 127).astype(np.int64))
    sub = s * np.ldexp(f / 2.0 ** 23, -126)
    special = np.where(f == 0, s * np.inf, np.nan)
    return np.where(e == 0, sub, np.where(e == 255, special, normal))


# ---------------------------------------------------------------------------
# Weight decode
# ---------------------------------------------------------------------------

# Bytes per weight of the plain (unblocked) types: bf16, wavo's F32 (type 0) and F16 (type 1).
PLAIN_BYTES = {W_BF16: 2, W_F32: 4, W_F16: 2}


def weight_nbytes(wtype: int, m: int, k: int) -> int:
    if wtype in PLAIN_BYTES:
        return PLAIN_BYTES[wtype] * m * k
    if wtype == W_Q4_K:
        return Q4K_BYTES * m * (k // QK_K)
    return QBYTES[wtype] * m * (k // QBLOCK)


def _blocks(raw: np.ndarray, wtype: int, m: int, k: int) -> np.ndarray:
    if k % QBLOCK:
        raise ValueError(f"k = {k} is not a multiple of {QBLOCK}")
    a = np.ascontiguousarray(raw).view(np.uint8).reshape(-1)
    need = weight_nbytes(wtype, m, k)
    if a.size < need:
        raise ValueError(f"weight has {a.size} bytes, needs {need}")
    return a[:need].reshape(m, k // QBLOCK, QBYTES[wtype])


def decode_q8_0(raw: np.ndarray, m: int, k: int) -> np.ndarray:
    """Q8_0 rows -> ``f64[m][k]``: block = little-endian f16 ``d``, then 32 int8 ``q``; w = d*q."""
    blk = _blocks(raw, W_Q8_0, m, k)
    d = f16_bits_to_f64(blk[:, :, 0].astype(np.int64) | (blk[:, :, 1].astype(np.int64) << 8))
    q = blk[:, :, 2:].view(np.int8).astype(np.float64)
    return (d[:, :, None] * q).reshape(m, k)


def decode_q4_0(raw: np.ndarray, m: int, k: int) -> np.ndarray:
    """Q4_0 rows -> ``f64[m][k]``: block = LE f16 ``d``, then 16 bytes; w = d*(q-8).

    Byte j of the 16 holds element j in its low nibble and element j+16 in its
    high nibble.
    """
    blk = _blocks(raw, W_Q4_0, m, k)
    d = f16_bits_to_f64(blk[:, :, 0].astype(np.int64) | (blk[:, :, 1].astype(np.int64) << 8))
    qs = blk[:, :, 2:].astype(np.int64)
    q = np.concatenate([qs & 0xF, qs >> 4], axis=2).astype(np.float64)
    return (d[:, :, None] * (q - 8.0)).reshape(m, k)


def q4_k_scale_min(scales) -> tuple:
    """``(sc, mn)``, each ``int64[..., 8]``: the 6-bit scale and 6-bit min of the eight sub-blocks
    of a Q4_K super-block, from its 12 packed bytes ``scales[..., 0:12]``.

    GGML's k-quant packing: for sub-blocks j = 0..3 the scale is the low 6 bits of byte j and the
    min the low 6 bits of byte j + 4. For j = 4..7 byte j + 4 carries the low 4 bits of the scale
    (its low nibble) and of the min (its high nibble), and the top 2 bits of the scale and of the
    min sit in the top 2 bits of bytes j - 4 and j.
    """
    b = np.asarray(scales).astype(np.int64)
    sc = np.empty(b.shape[:-1] + (8,), np.int64)
    mn = np.empty_like(sc)
    for j in range(4):
        sc[..., j] = b[..., j] & 63
        mn[..., j] = b[..., j + 4] & 63
    for j in range(4, 8):
        sc[..., j] = (b[..., j + 4] & 15) | ((b[..., j - 4] >> 6) << 4)
        mn[..., j] = (b[..., j + 4] >> 4) | ((b[..., j] >> 6) << 4)
    return sc, mn


def decode_q4_k_parts(raw: np.ndarray, m: int, k: int):
    """``(P, N)``, both ``f64[m][k]``: the two products a Q4_K weight is the difference of,
    ``P = d * sc_j * q`` and ``N = dmin * m_j`` (so ``W = P - N``, ``decode_q4_k``). A layer that
    computes with the two parts rounds relative to ``|P| + |N|`` rather than ``|W|``."""
    if k % QK_K:
        raise ValueError(f"k = {k} is not a multiple of {QK_K}")
    a = np.ascontiguousarray(raw).view(np.uint8).reshape(-1)
    need = weight_nbytes(W_Q4_K, m, k)
    if a.size < need:
        raise ValueError(f"weight has {a.size} bytes, needs {need}")
    sb = a[:need].reshape(m, k // QK_K, Q4K_BYTES).astype(np.int64)
    d = f16_bits_to_f64(sb[:, :, 0] | (sb[:, :, 1] << 8))
    dmin = f16_bits_to_f64(sb[:, :, 2] | (sb[:, :, 3] << 8))
    sc, mn = q4_k_scale_min(sb[:, :, 4:16])
    qs = sb[:, :, 16:].reshape(m, k // QK_K, 4, 32)          # [row][super][c][byte]
    q = np.stack([qs & 0xF, qs >> 4], axis=3)                # [row][super][c][nibble][l]
    q = q.reshape(m, k // QK_K, 8, 32).astype(np.float64)    # sub-block j = 2c + nibble
    pos = d[:, :, None, None] * sc[:, :, :, None] * q
    neg = np.broadcast_to(dmin[:, :, None, None] * mn[:, :, :, None], pos.shape)
    return pos.reshape(m, k), np.ascontiguousarray(neg).reshape(m, k)


def decode_q4_k(raw: np.ndarray, m: int, k: int) -> np.ndarray:
    """Q4_K rows -> ``f64[m][k]``: ``k/256`` super-blocks of 144 bytes per row.

    Super-block bytes (GGML's published k-quant layout; the pages give only the sizes):
    0-1 little-endian f16 ``d``, 2-3 little-endian f16 ``dmin``, 4-15 the packed 6-bit scales
    and mins of the eight 32-element sub-blocks (``q4_k_scale_min``), 16-143 the 4-bit quants.
    Sub-blocks 2c and 2c+1 (c = 0..3) share quant bytes 32c .. 32c+31: element l of sub-block
    2c is the low nibble of byte 32c + l, element l of sub-block 2c+1 its high nibble.
    Weight = ``d * sc_j * q - dmin * m_j`` for element of sub-block j, with unsigned ``q``.
    """
    pos, neg = decode_q4_k_parts(raw, m, k)
    return pos - neg


def q4_k_part_scale(x, raw, m: int, k: int, rows=None) -> np.ndarray:
    """``S2[t, j] = sum_k |x[t, k]| * (|P[j, k]| + |N[j, k]|)`` for a Q4_K weight (``P``, ``N`` of
    ``decode_q4_k_parts``): the scale of the roundings of a product computed from the two parts."""
    a = np.ascontiguousarray(raw).view(np.uint8).reshape(m, -1)
    if rows is not None:
        a = a[np.asarray(rows)]
    pos, neg = decode_q4_k_parts(a, a.shape[0], k)
    return np.abs(np.asarray(x, dtype=np.float64).reshape(-1, k)) @ (np.abs(pos) + np.abs(neg)).T


def decode(raw: np.ndarray, wtype: int, m: int, k: int, rows=None) -> np.ndarray:
    """Exact f64 values of an ``m x k`` weight (optionally only the listed rows).

    bf16 and f16 rows are 16-bit patterns, f32 rows 32-bit patterns, all
    little-endian (wavo ``Gpu::upload_linear`` copies F32 / F16 tensor bytes as
    stored); Q8_0 / Q4_0 rows are 34- / 18-byte blocks, Q4_K rows 144-byte super-blocks.
    """
    if wtype in PLAIN_BYTES:
        dt = np.uint32 if wtype == W_F32 else np.uint16
        a = np.ascontiguousarray(raw).view(np.uint8).reshape(-1)[: PLAIN_BYTES[wtype] * m * k].view(dt)
        a = a.reshape(m, k)
        if rows is not None:
            a = a[np.asarray(rows)]
        fn = {W_BF16: bf16_bits_to_f64, W_F32: f32_bits_to_f64, W_F16: f16_bits_to_f64}[wtype]
        return fn(a)
    if wtype not in QBYTES and wtype != W_Q4_K:
        raise ValueError(f"unknown weight type {wtype}")
    a = np.ascontiguousarray(raw).view(np.uint8).reshape(-1)[: weight_nbytes(wtype, m, k)].reshape(m, -1)
    mm = m
    if rows is not None:
        a = a[np.asarray(rows)]
        mm = a.shape[0]
    dec = {W_Q8_0: decode_q8_0, W_Q4_0: decode_q4_0, W_Q4_K: decode_q4_k}[wtype]
    return dec(a, mm, k)


def padded_k(k: int) -> int:
    """The inner size a weight with ``k`` columns is padded to: the next multiple of 32 (the
    GEMM's k step; wavo ``Gpu::upload_linear``, ``kp = k.next_multiple_of(32)``)."""
    return -(-int(k) // QBLOCK) * QBLOCK


def pad_weight(raw, wtype: int, m: int, k: int):
    """``(W_padded, kp)``: an ``m x k`` weight of a plain type (f32, f16 or bf16), decoded to its
    exact values and zero-padded to ``kp = padded_k(k)`` columns.

    This is wavo ``Gpu::upload_linear``'s load path for conv weights (``Gpu::conv``) whose inner
    size is not a multiple of 32: the rows are converted to f32, each row gets zero columns up to
    the next multiple of 32, and the result is stored as an f32 (type 0) linear layer, which then
    multiplies im2col rows that are zero past ``k`` as well. Every decoded value is exact in f32.
    """
    if wtype not in PLAIN_BYTES:
        raise ValueError("only f32, f16 and bf16 weights are padded (block types need k % 32 == 0)")
    kp = padded_k(k)
    w = decode(raw, wtype, m, k)
    out = np.zeros((m, kp), dtype=np.float64)
    out[:, :k] = w
    return out, kp


# ---------------------------------------------------------------------------
# Epilogue
# ---------------------------------------------------------------------------

def gelu_erf(v) -> np.ndarray:
    """erf-GELU: ``0.5 * v * (1 + erf(v / sqrt(2)))`` (``ae_put``'s flag-2 step, exact erf)."""
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * v * (1.0 + erf(v / np.sqrt(2.0)))


def silu(v) -> np.ndarray:
    """SiLU: ``v / (1 + exp(-v))`` (wavo ``gpu/mod.rs`` test reference ``silu``, ``Epilogue::Silu``)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def relu(v) -> np.ndarray:
    """ReLU: ``max(v, 0)`` (wavo ``Epilogue::Relu``)."""
    return np.maximum(np.asarray(v, dtype=np.float64), 0.0)


def tanh(v) -> np.ndarray:
    """Hyperbolic tangent (wavo ``Epilogue::Tanh``), numpy's f64 ``tanh``."""
    return np.tanh(np.asarray(v, dtype=np.float64))


ACTIVATIONS = {FLAG_GELU: gelu_erf, FLAG_SILU: silu, FLAG_RELU: relu, FLAG_TANH: tanh}


def epilogue(v: np.ndarray, flags: int, bias=None, y_old=None, alpha: float = 1.0) -> np.ndarray:
    """bias -> activation -> times alpha -> + old output, in that order.

    The order and flag bits 1/2/4 are ``ae_put``'s (cortiq-engine); the other
    activations (flag 8 SiLU, 16 ReLU, 32 tanh; at most one activation) and the
    factor ``alpha`` on the accumulated value are wavo's ``Epilogue`` modes
    (``Residual(alpha)``: ``c + alpha * (a.W^T + b)``, ``GeluResidual``:
    ``c + GELU(a.W^T + b)``). ``alpha = 1`` is the cortiq-engine epilogue.
    """
    out = np.array(v, dtype=np.float64, copy=True)
    if flags & FLAG_BIAS:
        out = out + np.asarray(bias, dtype=np.float64)[None, :]
    acts = [f for f in ACTIVATIONS if flags & f]
    if len(acts) > 1:
        raise ValueError("at most one activation flag")
    if acts:
        out = ACTIVATIONS[acts[0]](out)
    out = float(alpha) * out
    if flags & FLAG_RESIDUAL:
        out = out + np.asarray(y_old, dtype=np.float64)
    return out


# ---------------------------------------------------------------------------
# The layer
# ---------------------------------------------------------------------------

def linear_dual(x, w_raw, wtype: int, m: int, k: int, dual: int, bias=None, flags: int = 0, y_old=None,
                alpha: float = 1.0):
    """``(Y_ref, S)`` with wavo's dual outputs: ``Y`` is ``[n][m + dual]``; columns ``0..m-1``
    are the layer with ``bias[0..m-1]``, and columns ``m + j`` (``j < dual``) repeat output ``j``
    with its own bias ``bias[m + j]`` (wavo ``Linear.dual`` and ``Gpu::upload_linear``: the first
    ``dual`` outputs written again after the others, with the extra bias values). ``y_old`` is
    ``[n][m + dual]`` too; ``S`` is that of each column's product.
    """
    if not 0 <= dual <= m:
        raise ValueError("dual must be in [0, m]")
    n = np.asarray(x).reshape(-1, k).shape[0]
    b = None if bias is None else np.asarray(bias, dtype=np.float64).reshape(-1)
    yo = None if y_old is None else np.asarray(y_old, dtype=np.float64).reshape(n, m + dual)
    main, s = linear(x, w_raw, wtype, m, k, None if b is None else b[:m], flags,
                     None if yo is None else yo[:, :m], alpha=alpha)
    if dual == 0:
        return main, s
    rows = np.arange(dual)
    bias2 = None if b is None else np.concatenate([b[m:m + dual], np.zeros(m - dual)])
    yo2 = None if yo is None else np.concatenate([yo[:, m:], np.zeros((n, m - dual))], axis=1)
    second, s2 = linear(x, w_raw, wtype, m, k, bias2, flags, yo2, rows=rows, alpha=alpha)
    return np.concatenate([main, second], axis=1), np.concatenate([s, s2], axis=1)


def linear(x, w_raw, wtype: int, m: int, k: int, bias=None, flags: int = 0, y_old=None,
           rows=None, alpha: float = 1.0):
    """``(Y_ref, S)`` for ``Y = epilogue(X . W^T + b)``; both ``f64[n][len(rows) or m]``.

    ``rows`` restricts the output columns (rows of W) to a subset, so that a
    sample of a large product can be checked one output at a time; ``bias``
    and ``y_old`` are then given for the full width and sliced here.
    """
    x64 = np.asarray(x, dtype=np.float64).reshape(-1, k)
    w = decode(w_raw, wtype, m, k, rows)
    v = x64 @ w.T
    s = np.abs(x64) @ np.abs(w).T
    b = None if bias is None else np.asarray(bias, dtype=np.float64)
    yo = None if y_old is None else np.asarray(y_old, dtype=np.float64).reshape(x64.shape[0], m)
    if rows is not None:
        r = np.asarray(rows)
        b = None if b is None else b[r]
        yo = None if yo is None else yo[:, r]
    return epilogue(v, flags, b, yo, alpha), s


def moe(x, bank_raw, wtype: int, ids, n_exp: int, m: int, k: int, gates=None, rows=None):
    """MoE matvec over one weight bank ``[E][m][k]``.

    Without ``gates``: ``Y[s] = W[ids[s]] . x[token(s)]`` per routed slot
    ``s = t*top_k + j`` (``[n_tok*top_k][m]``). With ``gates``:
    ``Y[t] = sum_j gates[t, j] * W[ids[t, j]] . x[t]`` (``[n_tok][m]``), and
    ``S[t] = sum_j |gates[t, j]| * (|W[ids[t, j]]| . |x[t]|)``.
    """
    ids = np.asarray(ids).astype(np.int64)
    n_tok, top_k = ids.shape
    x64 = np.asarray(x, dtype=np.float64).reshape(n_tok, k)
    nb = weight_nbytes(wtype, m, k)
    bank = np.ascontiguousarray(bank_raw).view(np.uint8).reshape(-1)
    width = m if rows is None else len(rows)
    slot_y = np.zeros((n_tok, top_k, width))
    slot_s = np.zeros((n_tok, top_k, width))
    for e in np.unique(ids):
        if not 0 <= e < n_exp:
            raise ValueError(f"expert id {e} outside [0, {n_exp})")
        w = decode(bank[e * nb:(e + 1) * nb], wtype, m, k, rows)
        t_idx, j_idx = np.nonzero(ids == e)
        slot_y[t_idx, j_idx] = x64[t_idx] @ w.T
        slot_s[t_idx, j_idx] = np.abs(x64[t_idx]) @ np.abs(w).T
    if gates is None:
        return slot_y.reshape(n_tok * top_k, width), slot_s.reshape(n_tok * top_k, width)
    g = np.asarray(gates, dtype=np.float64).reshape(n_tok, top_k)
    return ((g[:, :, None] * slot_y).sum(axis=1),
            (np.abs(g)[:, :, None] * slot_s).sum(axis=1))


# ---------------------------------------------------------------------------
# Q8_0 test encoder (wavo gpu/mod.rs, test helper ``weights``)
# ---------------------------------------------------------------------------

def encode_q8_0(w) -> np.ndarray:
    """Q8_0 bytes of f32 rows, as the wavo test helper builds them.

    Per block of 32: ``d = max|x| / 127`` (in f32), ``q = round(x / d)``
    (rounded half away from zero) cast to int8, and ``d`` stored as f16.
    """
    w = np.asarray(w, dtype=np.float32)
    m, k = w.shape
    blocks = w.reshape(m, k // QBLOCK, QBLOCK)
    d = (np.abs(blocks).max(axis=2) / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = blocks / d[:, :, None]
    r = np.where(np.isfinite(r), r, 0.0)
    q = (np.sign(r) * np.floor(np.abs(r) + np.float32(0.5))).astype(np.int8)
    dh = d.astype(np.float16).view(np.uint16)
    out = np.empty((m, k // QBLOCK, 34), np.uint8)
    out[:, :, 0] = dh & 0xFF
    out[:, :, 1] = dh >> 8
    out[:, :, 2:] = q.view(np.uint8)
    return out.reshape(m, -1)
