"""Python binding of ``libwq.so``, the weight-dequantizing linear layer for MI355X.

Argument marshalling only: every function checks tensor dtypes, devices and
sizes, then passes raw device pointers and torch's current HIP stream to the C
ABI declared in ``include/wq.h``. All arithmetic happens in the HIP kernels;
there is no fallback. If the library is not built, every call raises.

    import gemv_wq_gemm_amd as wq
    y = wq.gemm(x, w, wq.W_Q8_0, m=4096, k=4096)              # n <= 16: f32 matvec path
    y = wq.gemm(x, w, wq.W_BF16, bias=b, gelu=True)           # n > 16: bf16 MFMA path
    y = wq.moe_matvec(x, bank, wq.W_Q4_0, ids, gates, n_experts=8, m=14336, k=4096)
"""
from __future__ import annotations

import ctypes
import os

W_BF16, W_Q8_0, W_Q4_0, W_F32, W_F16, W_Q4_K = 0, 1, 2, 3, 4, 5
BIAS, GELU, RESIDUAL, SILU, RELU, TANH = 1, 2, 4, 8, 16, 32
ACTIVATIONS = {None: 0, "gelu": GELU, "silu": SILU, "relu": RELU, "tanh": TANH}
PATH_AUTO, PATH_MATVEC, PATH_MFMA, PATH_MFMA_F32 = 0, 1, 2, 3
MATVEC_MAX_N = 16

STATUS = {
    0: "WQ_OK", -1: "WQ_ERR_NULL", -2: "WQ_ERR_SHAPE", -3: "WQ_ERR_WTYPE", -4: "WQ_ERR_FLAGS",
    -5: "WQ_ERR_ALIGN", -6: "WQ_ERR_ALIAS", -7: "WQ_ERR_HIP",
}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwq.so")

# (name, restype, argtypes) of every function include/wq.h declares.
_P, _I64, _I, _U = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint
SIGNATURES = [
    ("wq_gemm", _I, [_P, _P, _I, _P, _U, _P, _I64, _I64, _I64, _P]),
    ("wq_gemm_ex", _I, [_P, _P, _I, _P, _U, _P, _I64, _I64, _I64, _I, _P]),
    ("wq_linear", _I, [_P, _P, _I, _P, _U, ctypes.c_float, _P, _I64, _I64, _I64, _I, _P]),
    ("wq_linear_dual", _I, [_P, _P, _I, _P, _U, ctypes.c_float, _P, _I64, _I64, _I64, _I64, _I, _P]),
    ("wq_moe_matvec", _I, [_P, _P, _I, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P]),
    ("wq_moe_matvec_noalloc", _I, [_P, _P, _I, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P]),
    ("wq_dequantize", _I, [_P, _I, _P, _I64, _I64, _P]),
    ("wq_pad_weight", _I, [_P, _I, _P, _I64, _I64, _P]),
    ("wq_padded_k", _I64, [_I64]),
    ("wq_weight_bytes", _I64, [_I, _I64, _I64]),
    ("wq_gemm_path", _I, [_I64, _I64, _I64, _I]),
    ("wq_layer_norm", _I, [_P, _P, _P, _I64, _I64, _P]),
    ("wq_rope_table", _I, [_P, _I64, _I64]),
    ("wq_qk_norm_rope", _I, [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]),
    ("wq_attention_workspace_bytes", _I64, [_I64, _I64, _I64]),
    ("wq_attention", _I, [_P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_float, _P]),
    ("wq_encoder_workspace_bytes", _I64, [_I64, _I64, _I64, _I64]),
    ("wq_encoder_layer", _I, [_P, _I, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I, _P]),
    ("wq_last_error", ctypes.c_char_p, []),
    ("wq_version", ctypes.c_char_p, []),
]


class WqError(RuntimeError):
    """A nonzero status from the C ABI, with the library's message."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded ``libwq.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gemv_wq_gemm_amd.build`")
        # torch ships its own HIP runtime under another file name. Importing it
        # first makes the library's libamdhip64.so.7 resolve (by soname) to that
        # same runtime; otherwise the process would hold two HIP runtimes and
        # the second one sees no device.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        handle = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise WqError(status, lib().wq_last_error().decode())


def version() -> str:
    return lib().wq_version().decode()


def weight_bytes(wtype: int, m: int, k: int) -> int:
    return int(lib().wq_weight_bytes(wtype, m, k))


def gemm_path(n: int, m: int, k: int, wtype: int) -> int:
    r = lib().wq_gemm_path(n, m, k, wtype)
    _check(min(r, 0))
    return r


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _f32(t, name, numel=None):
    import torch
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return _dev(t, name)


def _weight(w, wtype, nbytes, name="w"):
    if w.numel() * w.element_size() < nbytes:
        raise ValueError(f"{name} has {w.numel() * w.element_size()} bytes, needs {nbytes}")
    return _dev(w, name)


def _flags(bias, gelu: bool, act, residual: bool) -> int:
    if act not in ACTIVATIONS:
        raise ValueError(f"act must be one of {sorted(a for a in ACTIVATIONS if a)} or None, got {act!r}")
    if gelu and act not in (None, "gelu"):
        raise ValueError("gelu=True and another act")
    a = GELU if gelu else ACTIVATIONS[act]
    return (BIAS if bias is not None else 0) | a | (RESIDUAL if residual else 0)


def gemm(x, w, wtype: int, *, m: int, k: int, bias=None, gelu: bool = False, residual: bool = False,
         out=None, path: int = PATH_AUTO, act=None, alpha: float = 1.0, dual: int = 0):
    """``out[n][m] = alpha * act(x[n][k] . W^T + bias) (+ out)`` via ``wq_linear_dual``.

    ``w`` holds the weight in its storage format (any dtype; its bytes are
    used). ``act`` is None, "gelu", "silu", "relu" or "tanh" (``gelu=True`` is
    ``act="gelu"``). With ``residual=True``, ``out`` is required and
    accumulated into. With ``dual > 0``, ``out`` is ``[n][m + dual]`` and
    ``bias`` has ``m + dual`` values: outputs ``0..dual-1`` are written again
    at ``m + j`` with ``bias[m + j]``.
    """
    import torch
    n = x.numel() // k if k else 0
    if x.numel() != n * k:
        raise ValueError("x must hold n*k elements")
    if out is None:
        if residual:
            raise ValueError("residual=True needs out= (the values to accumulate into)")
        out = torch.empty((n, m + dual), dtype=torch.float32, device=x.device)
    flags = _flags(bias, gelu, act, residual)
    nbytes = weight_bytes(wtype, m, k)
    if nbytes < 0:
        _check(lib().wq_gemm_path(n, m, k, wtype))
    st = lib().wq_linear_dual(
        _f32(x, "x"), _weight(w, wtype, nbytes), wtype,
        None if bias is None else _f32(bias, "bias", m + dual), flags, float(alpha),
        _f32(out, "out", n * (m + dual)), n, m, k, dual, path, _stream())
    _check(st)
    return out


class BoundGemm:
    """One ``wq_linear`` (or ``wq_layer_norm``) call with every argument resolved up front.

    For loops that call the same layer on the same buffers again and again (a
    timing loop, a decode step): calling the object costs one ctypes call, with
    no tensor inspection. The tensors given to :func:`bind_gemm` or
    :func:`bind_layer_norm` must stay alive and in place for as long as the
    object is used, and the stream it was bound to must still be the one to
    launch on.
    """

    def __init__(self, fn, args):
        self._fn, self._args = fn, args

    def __call__(self) -> None:
        _check(self._fn(*self._args))


def bind_gemm(x, w, wtype: int, *, m: int, k: int, out, bias=None, gelu: bool = False,
              residual: bool = False, path: int = PATH_AUTO, act=None, alpha: float = 1.0) -> BoundGemm:
    """Checks the arguments as :func:`gemm` does and returns a :class:`BoundGemm`."""
    n = x.numel() // k if k else 0
    if x.numel() != n * k:
        raise ValueError("x must hold n*k elements")
    flags = _flags(bias, gelu, act, residual)
    nbytes = weight_bytes(wtype, m, k)
    if nbytes < 0:
        _check(lib().wq_gemm_path(n, m, k, wtype))
    args = (_f32(x, "x"), _weight(w, wtype, nbytes), wtype, None if bias is None else _f32(bias, "bias", m),
            flags, ctypes.c_float(alpha), _f32(out, "out", n * m), n, m, k, path, _stream())
    return BoundGemm(lib().wq_linear, args)


def moe_matvec(x, w_experts, wtype: int, ids, gates=None, *, n_experts: int, m: int, k: int, out=None,
               noalloc: bool = False):
    """Expert-major MoE matvec via ``wq_moe_matvec`` (``wq_moe_matvec_noalloc`` with ``noalloc``).

    ``ids`` int32 ``[n_tok][top_k]``. Without ``gates`` the result is per slot
    ``[n_tok*top_k][m]``; with ``gates`` (f32 ``[n_tok][top_k]``) it is the
    gate-weighted sum per token, ``[n_tok][m]``. ``noalloc`` takes the entry point
    that never allocates device memory (give ``out`` as well, so this call allocates nothing).
    """
    import torch
    if ids.dtype != torch.int32:
        raise ValueError("ids must be int32")
    n_tok, top_k = ids.shape
    rows = n_tok if gates is not None else n_tok * top_k
    if out is None:
        out = torch.empty((rows, m), dtype=torch.float32, device=x.device)
    nbytes = weight_bytes(wtype, m, k)
    fn = lib().wq_moe_matvec_noalloc if noalloc else lib().wq_moe_matvec
    st = fn(
        _f32(x, "x", n_tok * k), _weight(w_experts, wtype, max(nbytes, 0) * n_experts, "w_experts"), wtype,
        _dev(ids, "ids"), None if gates is None else _f32(gates, "gates", n_tok * top_k),
        _f32(out, "out", rows * m), n_tok, top_k, n_experts, m, k, _stream())
    _check(st)
    return out


def dequantize(w, wtype: int, *, m: int, k: int, out=None):
    """``out[m][k]`` = exact f32 values of the weight, via ``wq_dequantize``."""
    import torch
    if out is None:
        out = torch.empty((m, k), dtype=torch.float32, device=w.device)
    nbytes = weight_bytes(wtype, m, k)
    st = lib().wq_dequantize(_weight(w, wtype, max(nbytes, 0)), wtype, _f32(out, "out", m * k), m, k, _stream())
    _check(st)
    return out


def padded_k(k: int) -> int:
    """The inner size :func:`pad_weight` pads ``k`` to (the next multiple of 32)."""
    r = int(lib().wq_padded_k(k))
    if r < 0:
        raise ValueError(f"k = {k} is outside [1, 2^29 - 1]")
    return r


def pad_weight(w, wtype: int, *, m: int, k: int, out=None):
    """``out[m][kp]`` f32: the f32/f16/bf16 weight ``w[m][k]`` zero-padded to ``kp = padded_k(k)``
    columns, via ``wq_pad_weight`` (wavo's conv weights with k % 32 != 0)."""
    import torch
    kp = padded_k(k)
    if out is None:
        out = torch.empty((m, kp), dtype=torch.float32, device=w.device)
    width = 4 if wtype == W_F32 else 2
    if w.numel() * w.element_size() < m * k * width:
        raise ValueError(f"w has {w.numel() * w.element_size()} bytes, needs {m * k * width}")
    st = lib().wq_pad_weight(_dev(w, "w"), wtype, _f32(out, "out", m * kp), m, k, _stream())
    _check(st)
    return out


# ---- the encoder block -----------------------------------------------------------------------

class EncoderLayerDesc(ctypes.Structure):
    """``wq_encoder_layer_t``: device pointers of one block's weights (NULL where absent)."""
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("ln1", "qkv_w", "qkv_b", "qn", "kn", "out_w", "out_b", "ln2", "fc1_w", "fc1_b", "fc2_w", "fc2_b")]


def layer_norm(x, wb, *, d: int, out=None):
    """Row LayerNorm (eps 1e-5) of ``x[n][d]`` with ``wb = [w | b]`` via ``wq_layer_norm``;
    ``out`` may be ``x`` (in place)."""
    import torch
    n = x.numel() // d
    if x.numel() != n * d:
        raise ValueError("x must hold n*d elements")
    if out is None:
        out = torch.empty((n, d), dtype=torch.float32, device=x.device)
    _check(lib().wq_layer_norm(_f32(x, "x"), _f32(wb, "wb", 2 * d), _f32(out, "out", n * d), n, d, _stream()))
    return out


def bind_layer_norm(x, wb, *, d: int, out) -> BoundGemm:
    """Checks the arguments as :func:`layer_norm` does and returns the bound call."""
    n = x.numel() // d
    if x.numel() != n * d:
        raise ValueError("x must hold n*d elements")
    args = (_f32(x, "x"), _f32(wb, "wb", 2 * d), _f32(out, "out", n * d), n, d, _stream())
    return BoundGemm(lib().wq_layer_norm, args)


def rope_table(n: int, rot: int):
    """The host-built f32 rotation table ``[cos n*rot/2 | sin n*rot/2]`` (``wq_rope_table``), as a
    CPU tensor."""
    import torch
    cs = torch.empty(n * rot, dtype=torch.float32)
    _check(lib().wq_rope_table(ctypes.c_void_p(cs.data_ptr()), n, rot))
    return cs


def qk_norm_rope(qkv, cs, *, n: int, heads: int, hd: int, rot: int, qn=None, kn=None):
    """In place on ``qkv[n][3*heads*hd]``: per-head q/k LayerNorm (when ``qn``/``kn``) and the
    rotation of the first ``rot`` dims by the table ``cs`` (a device tensor), via
    ``wq_qk_norm_rope``. Returns ``qkv``."""
    _check(lib().wq_qk_norm_rope(
        _f32(qkv, "qkv", n * 3 * heads * hd), None if qn is None else _f32(qn, "qn", 2 * hd),
        None if kn is None else _f32(kn, "kn", 2 * hd), None if cs is None else _f32(cs, "cs", n * rot),
        n, heads, hd, rot, _stream()))
    return qkv


def attention_workspace_bytes(n: int, heads: int, hd: int) -> int:
    r = int(lib().wq_attention_workspace_bytes(n, heads, hd))
    if r < 0:
        raise ValueError(f"invalid attention sizes n={n}, heads={heads}, hd={hd}")
    return r


def _workspace(nbytes: int, device, workspace):
    import torch
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace has {workspace.numel() * workspace.element_size()} bytes, needs {nbytes}")
    return workspace


def attention(qkv, valid, *, n: int, heads: int, hd: int, scale: float, out=None, workspace=None):
    """Masked bidirectional attention over ``qkv[n][3*heads*hd]`` (``valid`` int32 ``[n]``) via
    ``wq_attention``; returns ``out[n][heads*hd]``. ``workspace`` (device bytes, 256-byte aligned)
    is allocated when not given."""
    import torch
    if valid.dtype != torch.int32:
        raise ValueError("valid must be int32")
    if out is None:
        out = torch.empty((n, heads * hd), dtype=torch.float32, device=qkv.device)
    ws = _workspace(attention_workspace_bytes(n, heads, hd), qkv.device, workspace)
    _check(lib().wq_attention(_f32(qkv, "qkv", n * 3 * heads * hd), _dev(valid, "valid"),
                              _f32(out, "out", n * heads * hd), _dev(ws, "workspace"),
                              ws.numel() * ws.element_size(), n, heads, hd, float(scale), _stream()))
    return out


def encoder_workspace_bytes(n: int, d: int, heads: int, inter: int) -> int:
    r = int(lib().wq_encoder_workspace_bytes(n, d, heads, inter))
    if r < 0:
        raise ValueError(f"invalid encoder sizes n={n}, d={d}, heads={heads}, inter={inter}")
    return r


def encoder_layer_desc(layer: dict) -> EncoderLayerDesc:
    """The C descriptor of one block from a dict of device tensors (keys as the struct's fields;
    ``qkv_b``, ``qn`` and ``kn`` may be missing or None). The tensors must outlive its use."""
    def ptr(key):
        t = layer.get(key)
        return None if t is None else _dev(t, key).value
    return EncoderLayerDesc(*[ptr(name) for name, _ in EncoderLayerDesc._fields_])


def encoder_layer(h, layer, wtype: int, valid, cs, *, n: int, d: int, heads: int, rot: int, inter: int,
                  path: int = PATH_AUTO, workspace=None):
    """One pre-norm block in place on ``h[n][d]`` via ``wq_encoder_layer``. ``layer`` is a dict of
    device tensors or an :class:`EncoderLayerDesc`; ``cs`` the device rotation table."""
    desc = layer if isinstance(layer, EncoderLayerDesc) else encoder_layer_desc(layer)
    ws = _workspace(encoder_workspace_bytes(n, d, heads, inter), h.device, workspace)
    _check(lib().wq_encoder_layer(
        ctypes.byref(desc), wtype, _f32(h, "h", n * d), _dev(valid, "valid"),
        None if cs is None else _f32(cs, "cs", n * rot), _dev(ws, "workspace"), ws.numel() * ws.element_size(),
        n, d, heads, rot, inter, path, _stream()))
    return h


def encoder_forward(x, model: dict, wtype: int, valid, *, heads: int, rot: int, path: int = PATH_AUTO,
                    workspace=None):
    """``AudioEncoder::run``: optional input projection ``model["proj"]`` (no bias), the embedding
    LayerNorm, every block of ``model["layers"]`` (dicts of device tensors) and the final LayerNorm.
    Returns ``[n][d]``. Every step is a library call; nothing is computed here."""
    import torch
    n = x.shape[0]
    d = model["embed_norm"].numel() // 2
    inter = model["layers"][0]["fc1_b"].numel() if model["layers"] else 32
    if model.get("proj") is not None:
        x = gemm(x, model["proj"], wtype, m=d, k=x.shape[1], path=path)
    cs = rope_table(n, rot).to(x.device) if rot > 0 else None
    h = layer_norm(x, model["embed_norm"], d=d)
    ws = _workspace(encoder_workspace_bytes(n, d, heads, inter), x.device, workspace)
    for layer in model["layers"]:
        encoder_layer(h, layer, wtype, valid, cs, n=n, d=d, heads=heads, rot=rot, inter=inter, path=path,
                      workspace=ws)
    return layer_norm(h, model["final_norm"], d=d, out=torch.empty_like(h))

