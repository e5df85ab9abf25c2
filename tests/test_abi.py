"""The C ABI on the host: the library loads, exports what include/wq.h declares,
and rejects bad arguments before any HIP call (so these run without a GPU).

Every call below fails one of the host-side checks; none reaches a kernel
launch, which is why fake (never dereferenced) pointers are safe here.
"""
import ctypes
import os
import re

import pytest

import gemv_wq_gemm_amd as wq
from tests.conftest import ROOT

# The calls below pass fake device addresses and rely on the host checks to refuse them. With a GPU
# present a slip in one of them would launch a kernel on those addresses, so the module runs only
# where no GPU is visible (device_count does not initialise the runtime).
import torch  # noqa: E402

if torch.cuda.device_count() > 0:
    pytest.skip("host-side checks with fake device pointers: run where no GPU is visible",
                allow_module_level=True)

HEADER = os.path.join(ROOT, "include", "wq.h")

# Aligned fake addresses, never dereferenced (every call here fails validation).
X, W, B, Y = 0x10000, 0x20000, 0x30000, 0x40000


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wq_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = wq.lib()
    declared = _declared()
    assert declared == sorted(name for name, _, _ in wq.SIGNATURES)
    for name in declared:
        assert hasattr(lib, name), name


def test_header_constants_match_binding():
    src = open(HEADER).read()
    consts = dict(re.findall(r"#define\s+(WQ_[A-Z_0-9]+)\s+\(?(-?\d+)u?\)?", src))
    assert int(consts["WQ_W_BF16"]) == wq.W_BF16
    assert int(consts["WQ_W_Q8_0"]) == wq.W_Q8_0
    assert int(consts["WQ_W_Q4_0"]) == wq.W_Q4_0
    assert int(consts["WQ_W_F32"]) == wq.W_F32 and int(consts["WQ_W_F16"]) == wq.W_F16
    assert int(consts["WQ_W_Q4_K"]) == wq.W_Q4_K
    assert int(consts["WQ_BIAS"]) == wq.BIAS and int(consts["WQ_GELU"]) == wq.GELU
    assert int(consts["WQ_RESIDUAL"]) == wq.RESIDUAL
    assert [int(consts[f"WQ_{a}"]) for a in ("SILU", "RELU", "TANH")] == [wq.SILU, wq.RELU, wq.TANH]
    assert int(consts["WQ_MATVEC_MAX_N"]) == wq.MATVEC_MAX_N
    assert [int(consts[f"WQ_PATH_{p}"]) for p in ("AUTO", "MATVEC", "MFMA", "MFMA_F32")] == [
        wq.PATH_AUTO, wq.PATH_MATVEC, wq.PATH_MFMA, wq.PATH_MFMA_F32]
    for name, code in consts.items():
        if name.startswith("WQ_ERR_") or name == "WQ_OK":
            assert wq.STATUS[int(code)] == name


def test_version():
    assert "gfx950" in wq.version()


@pytest.mark.parametrize("wtype,m,k,want", [
    (0, 4096, 4096, 2 * 4096 * 4096),
    (1, 4096, 4096, 17825792),
    (2, 14336, 4096, 33030144),
    (1, 3, 32, 102),
    (2, 1, 32, 18),
    (0, 0, 64, 0),
    (1, 5, 33, -1),
    (3, 5, 32, 640),
    (4, 5, 32, 320),
    (3, 5, 48, -1),
    (5, 5, 32, -1),
    (5, 5, 768, 5 * 3 * 144),
    (5, 14336, 4096, 33030144),
    (5, 1, 512, 288),
    (5, 2, 1024 + 32, -1),
    (6, 5, 256, -1),
    (0, -1, 32, -1),
])
def test_weight_bytes(wtype, m, k, want):
    assert wq.weight_bytes(wtype, m, k) == want


def test_path_selection():
    assert wq.gemm_path(0, 8, 32, 0) == wq.PATH_MATVEC
    assert wq.gemm_path(16, 8, 32, 1) == wq.PATH_MATVEC
    assert wq.gemm_path(17, 8, 32, 2) == wq.PATH_MFMA
    assert wq.gemm_path(1500, 1024, 4096, 0) == wq.PATH_MFMA
    with pytest.raises(wq.WqError):
        wq.gemm_path(4, 8, 40, 0)
    assert wq.gemm_path(16, 8, 256, wq.W_Q4_K) == wq.PATH_MATVEC
    with pytest.raises(wq.WqError, match="matvec path"):
        wq.gemm_path(17, 8, 256, wq.W_Q4_K)
    with pytest.raises(wq.WqError, match="256"):
        wq.gemm_path(4, 8, 32, wq.W_Q4_K)


def _gemm(x=X, w=W, wtype=0, bias=None, flags=0, y=Y, n=4, m=8, k=32, path=0):
    lib = wq.lib()
    st = lib.wq_gemm_ex(x, w, wtype, bias, flags, y, n, m, k, path, None)
    return st, lib.wq_last_error().decode()


@pytest.mark.parametrize("kwargs,code,msg", [
    (dict(wtype=6), -3, "weight type"),
    (dict(wtype=-1), -3, "weight type"),
    (dict(wtype=5), -2, "256"),
    (dict(wtype=5, k=256, n=17), -3, "matvec path"),
    (dict(wtype=5, k=256, path=2), -3, "matvec path"),
    (dict(wtype=5, k=256, path=3), -3, "matvec path"),
    (dict(flags=64), -4, "flag"),
    (dict(flags=2 | 8), -4, "at most one activation"),
    (dict(flags=16 | 32 | 4), -4, "at most one activation"),
    (dict(flags=1), -4, "WQ_BIAS"),
    (dict(bias=B), -4, "WQ_BIAS"),
    (dict(k=40), -2, "multiple of 32"),
    (dict(k=0), -2, "multiple of 32"),
    (dict(n=-1), -2, "negative"),
    (dict(m=-5), -2, "negative"),
    (dict(n=17, path=1), -2, "n <= 16"),
    (dict(path=7), -2, "path"),
    (dict(path=-1), -2, "path"),
    (dict(path=3, flags=128), -4, "flag"),
    (dict(path=3, k=48), -2, "multiple of 32"),
    (dict(path=3, y=X), -6, "overlaps"),
    (dict(x=None), -1, "NULL"),
    (dict(w=None), -1, "NULL"),
    (dict(y=None), -1, "NULL"),
    (dict(x=X + 4), -5, "aligned"),
    (dict(w=W + 2), -5, "aligned"),
    (dict(y=Y + 2), -5, "aligned"),
    (dict(y=Y + 1), -5, "aligned"),
    (dict(bias=B + 2, flags=1), -5, "aligned"),
    (dict(y=X), -6, "overlaps"),
    (dict(y=W + 16), -6, "overlaps"),
    (dict(bias=Y + 16, flags=1), -6, "overlaps"),
])
def test_gemm_argument_errors(kwargs, code, msg):
    st, err = _gemm(**kwargs)
    assert st == code, err
    assert msg in err


@pytest.mark.parametrize("alpha", [float("nan"), float("inf"), float("-inf")])
def test_linear_refuses_non_finite_alpha(alpha):
    lib = wq.lib()
    st = lib.wq_linear(X, W, 0, None, 4, ctypes.c_float(alpha), Y, 4, 8, 32, 0, None)
    assert st == -4 and "alpha" in lib.wq_last_error().decode()


def test_linear_checks_like_gemm_ex():
    lib = wq.lib()
    assert lib.wq_linear(X, W, 6, None, 0, ctypes.c_float(1.0), Y, 4, 8, 32, 0, None) == -3
    assert lib.wq_linear(X, W, 5, None, 0, ctypes.c_float(1.0), Y, 4, 8, 32, 0, None) == -2
    assert lib.wq_linear(X, W, 0, None, 2 | 16, ctypes.c_float(0.5), Y, 4, 8, 32, 2, None) == -4
    assert lib.wq_linear(X, W, 0, None, 0, ctypes.c_float(0.5), Y, 4, 8, 40, 0, None) == -2
    assert lib.wq_linear(None, None, 0, None, 0, ctypes.c_float(2.0), None, 0, 8, 32, 0, None) == 0


def test_linear_dual_checks():
    lib = wq.lib()
    one = ctypes.c_float(1.0)
    assert lib.wq_linear_dual(X, W, 0, None, 0, one, Y, 4, 8, 32, -1, 0, None) == -2
    assert lib.wq_linear_dual(X, W, 0, None, 0, one, Y, 4, 8, 32, 9, 0, None) == -2
    assert "dual" in lib.wq_last_error().decode()
    # y [4][8 + 8] f32 is 256 bytes, [4][8] would be 128: a bias 200 bytes on overlaps y only
    # through the dual columns. (Every call here must fail a host check: none may reach a launch.)
    assert lib.wq_linear_dual(X, W, 0, Y + 200, 1, one, Y, 4, 8, 32, 8, 0, None) == -6
    assert lib.wq_linear_dual(None, None, 0, None, 0, one, None, 0, 8, 32, 3, 0, None) == 0


def test_binding_refuses_unknown_or_double_activation():
    import torch
    x = torch.zeros(2, 32)
    with pytest.raises(ValueError):
        wq.gemm(x, x, wq.W_BF16, m=2, k=32, act="swish")
    with pytest.raises(ValueError):
        wq.gemm(x, x, wq.W_BF16, m=2, k=32, gelu=True, act="tanh")


def test_empty_shapes_are_noops_even_with_null_pointers():
    # n == 0 or m == 0: nothing to do, WQ_OK, and no pointer is touched.
    assert _gemm(x=None, w=None, y=None, n=0)[0] == 0
    assert _gemm(x=None, w=None, y=None, m=0)[0] == 0
    lib = wq.lib()
    assert lib.wq_moe_matvec(None, None, 2, None, None, None, 0, 2, 8, 16, 32, None) == 0
    assert lib.wq_dequantize(None, 1, None, 0, 32, None) == 0


def _moe(x=X, w=W, wtype=2, ids=B, gates=None, y=Y, n_tok=4, top_k=2, n_exp=8, m=16, k=32):
    lib = wq.lib()
    st = lib.wq_moe_matvec(x, w, wtype, ids, gates, y, n_tok, top_k, n_exp, m, k, None)
    return st, lib.wq_last_error().decode()


@pytest.mark.parametrize("kwargs,code", [
    (dict(wtype=6), -3),
    (dict(wtype=5), -2),
    (dict(top_k=0), -2),
    (dict(top_k=9), -2),
    (dict(n_exp=0), -2),
    (dict(k=48), -2),
    (dict(n_tok=4097, top_k=1), -2),
    (dict(ids=None), -1),
    (dict(x=None), -1),
    (dict(ids=B + 2), -5),
    (dict(gates=B + 0x1002), -5),
    (dict(x=X + 8), -5),
    (dict(y=B), -6),
])
def test_moe_argument_errors(kwargs, code):
    st, err = _moe(**kwargs)
    assert st == code, err


def test_moe_noalloc_checks_like_moe():
    lib = wq.lib()
    for kwargs, code in [(dict(wtype=6), -3), (dict(wtype=5), -2), (dict(top_k=0), -2), (dict(ids=None), -1),
                         (dict(y=B), -6)]:
        a = dict(x=X, w=W, wtype=2, ids=B, gates=None, y=Y, n_tok=4, top_k=2, n_exp=8, m=16, k=32)
        a.update(kwargs)
        st = lib.wq_moe_matvec_noalloc(a["x"], a["w"], a["wtype"], a["ids"], a["gates"], a["y"], a["n_tok"],
                                       a["top_k"], a["n_exp"], a["m"], a["k"], None)
        assert st == code, lib.wq_last_error().decode()
    # Gated calls beyond the 2^23-float scratch are refused on the host.
    st = lib.wq_moe_matvec_noalloc(X, W, 1, B, B + 0x10000, 0x10000000, 4096, 1, 1, 4096, 32, None)
    assert st == -2 and "scratch" in lib.wq_last_error().decode()
    assert lib.wq_moe_matvec_noalloc(None, None, 2, None, None, None, 0, 2, 8, 16, 32, None) == 0


@pytest.mark.parametrize("args,code", [
    ((W, 9, Y, 4, 32), -3),
    ((W, 5, Y, 4, 32), -2),
    ((W, 1, Y, 4, 31), -2),
    ((None, 1, Y, 4, 32), -1),
    ((W + 2, 1, Y, 4, 32), -5),
    ((W, 0, W, 4, 32), -6),
])
def test_dequantize_argument_errors(args, code):
    lib = wq.lib()
    assert lib.wq_dequantize(*args, None) == code


@pytest.mark.parametrize("k,kp", [(1, 32), (40, 64), (64, 64), (100, 128), (0, -1), (-3, -1)])
def test_padded_k(k, kp):
    assert wq.lib().wq_padded_k(k) == kp


@pytest.mark.parametrize("args,code", [
    ((W, 1, Y, 4, 40), -3),            # Q8_0 cannot be padded
    ((W, 2, Y, 4, 40), -3),
    ((W, 9, Y, 4, 40), -3),
    ((W, 3, Y, 4, 0), -2),
    ((W, 3, Y, -1, 40), -2),
    ((None, 3, Y, 4, 40), -1),
    ((W + 2, 3, Y, 4, 40), -5),        # f32 weight on a 2-byte boundary
    ((W + 1, 4, Y, 4, 40), -5),
    ((W, 3, Y + 2, 4, 40), -5),
    ((W, 3, W + 64, 4, 40), -6),
])
def test_pad_weight_argument_errors(args, code):
    lib = wq.lib()
    assert lib.wq_pad_weight(*args, None) == code, lib.wq_last_error().decode()
    assert lib.wq_pad_weight(None, 3, None, 0, 40, None) == 0


def test_error_message_is_per_call():
    st, err = _gemm(k=40)
    assert st == -2 and err
    assert wq.lib().wq_gemm_path(4, 8, 32, 0) == wq.PATH_MATVEC
    assert wq.lib().wq_last_error().decode() == ""


def test_binding_rejects_host_tensors_before_calling():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 32)
    w = torch.zeros(8, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        wq.gemm(x, w, wq.W_BF16, m=8, k=32, out=torch.zeros(4, 8))


def test_one_hip_runtime_in_the_process():
    """Loading the library must not bring a second HIP runtime beside torch's."""
    import subprocess
    import sys
    code = ("import gemv_wq_gemm_amd as wq, re; wq.gemm_path(1, 1, 32, 0); import torch; "
            "print(len(set(re.findall(r'\\S*libamdhip64\\S*', open('/proc/self/maps').read()))))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert out.stdout.strip() == "1", out.stdout + out.stderr
