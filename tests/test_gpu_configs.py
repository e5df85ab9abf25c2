"""GPU parity at the five workloads' full sizes, in the launch configuration the
bench times (the same C-ABI calls), checked on every output: the small cases and
the large matvecs (C2, C3 and the MoE, C4) element by element against the oracle
(C3 and C4 in row chunks), and the 24-layer encoder chain (C5) on frames at every
tile edge plus random ones, with all of its outputs required finite. Every output
buffer is NaN-prefilled with canaries after it. Each test prints the literal
ratio err / (B * S) beside err / tol.
"""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import oracle
import synth
from tests.parity import (B_F32, B_MFMA, GELU_SLOPE, ULP_SLACK, assert_within, dev, guarded_out,
                          literal_ratio, oracle_with_tol, read_guarded)

pytestmark = pytest.mark.gpu


def _call(cfg, path=wq.PATH_AUTO):
    n, m, k = cfg["n"], cfg["m"], cfg["k"]
    buf, out = guarded_out(n, m)
    bias = cfg["bias"]
    wq.gemm(dev(cfg["x"]), dev(cfg["w"]), cfg["wtype"], m=m, k=k,
            bias=None if bias is None else dev(bias), gelu=bool(cfg["flags"] & wq.GELU), out=out, path=path)
    return read_guarded(buf, n, m)


def _report(what, got, y_ref, S, bound, ratio_tol):
    print(f"{what}: err/tol = {ratio_tol:.4f}, err/(B*S) = {literal_ratio(got, y_ref, S, bound):.4f}")


def test_bf16_gemm_64x256x256_bias_gelu():
    cfg = synth.config_gemm_small()
    assert wq.gemm_path(cfg["n"], cfg["m"], cfg["k"], cfg["wtype"]) == wq.PATH_MFMA
    got = _call(cfg)
    y_ref, tol = oracle_with_tol(cfg["x"], cfg["w"], cfg["wtype"], cfg["m"], cfg["k"], cfg["bias"],
                                 cfg["flags"], None, B_MFMA)
    r = assert_within(got, y_ref, tol, "64x256x256")
    # The literal ratio compares the pre-activation error; GELU's slope may stretch it by up to 1.13.
    v, S = oracle.linear(cfg["x"], cfg["w"], cfg["wtype"], cfg["m"], cfg["k"], cfg["bias"], wq.BIAS)
    _report("C1 64x256x256 bias+GELU", got, y_ref, S, B_MFMA, r)


@pytest.mark.parametrize("n", [1, 4])
def test_q8_0_matvec_4096(n):
    cfg = synth.config_q8_matvec(n)
    got = _call(cfg)
    y_ref, S = oracle.linear(cfg["x"], cfg["w"], cfg["wtype"], cfg["m"], cfg["k"])
    r = assert_within(got, y_ref, B_F32 * S + ULP_SLACK * np.abs(y_ref), f"q8_0 n={n}")
    _report(f"C2 Q8_0 4096x4096 n={n}", got, y_ref, S, B_F32, r)


def _check_chunked(got, oracle_rows, m, bound, what, chunk=4096):
    """Every output column j of `got` against the oracle, computed on row chunks of W."""
    worst_tol = worst_lit = 0.0
    for j0 in range(0, m, chunk):
        rows = np.arange(j0, min(m, j0 + chunk))
        y_ref, S = oracle_rows(rows)
        part = got[:, rows]
        worst_tol = max(worst_tol, assert_within(part, y_ref, bound * S + ULP_SLACK * np.abs(y_ref),
                                                 f"{what} rows {rows[0]}..{rows[-1]}"))
        worst_lit = max(worst_lit, literal_ratio(part, y_ref, S, bound))
    print(f"{what}: err/tol = {worst_tol:.4f}, err/(B*S) = {worst_lit:.4f} over all {got.size} outputs")


def test_q4_0_matvec_14336x4096():
    cfg = synth.config_q4_matvec()
    got = _call(cfg)
    _check_chunked(got, lambda rows: oracle.linear(cfg["x"], cfg["w"], cfg["wtype"], cfg["m"], cfg["k"], rows=rows),
                   cfg["m"], B_F32, "C3 Q4_0 14336x4096")


@pytest.mark.parametrize("gated", [True, False])
def test_moe_q4_0_16_tokens_top2_of_8(gated):
    cfg = synth.config_moe()
    n_tok, top_k, E, m, k = cfg["n_tok"], cfg["top_k"], cfg["n_exp"], cfg["m"], cfg["k"]
    rows = n_tok if gated else n_tok * top_k
    buf, out = guarded_out(rows, m)
    wq.moe_matvec(dev(cfg["x"]), dev(cfg["w"]), cfg["wtype"], dev(cfg["ids"]),
                  dev(cfg["gates"]) if gated else None, n_experts=E, m=m, k=k, out=out)
    got = read_guarded(buf, rows, m)
    _check_chunked(got, lambda r: oracle.moe(cfg["x"], cfg["w"], cfg["wtype"], cfg["ids"], E, m, k,
                                             cfg["gates"] if gated else None, rows=r),
                   m, B_F32, f"C4 MoE 16 tokens top-2 of 8 ({'gated' if gated else 'per slot'})")


# ---------------------------------------------------------------- encoder chain

# Frames on both sides of every 32-, 64-, 96-, 128- and 256-row tile edge in a spread of places,
# the first and last frames, and random ones.
SAMPLE_FRAMES = sorted(set(
    [0, 1, 2, 1497, 1498, 1499]
    + [e + d for e in (32, 64, 96, 128, 192, 256, 384, 512, 768, 1024, 1152, 1280, 1408, 1472) for d in (-1, 0)]
    + list(np.random.default_rng(5).choice(1500, 24, replace=False))))


@pytest.fixture(scope="module")
def encoder():
    acts = synth.encoder_activations()
    layers = [synth.encoder_layer_weights(layer) for layer in range(synth.ENCODER_LAYERS)]
    return acts, layers


def _gpu_chain(acts, layers):
    """The workload as the bench runs it: per layer QKV(+bias), out(+bias,+=h), fc1(+bias,GELU),
    fc2(+bias,+=h). qkv and f are NaN-prefilled and h starts as h0; canaries follow all three."""
    n, d, ff = synth.ENCODER_N, synth.ENCODER_D, synth.ENCODER_FF
    a1, a2, a3 = (dev(acts[name]) for name in ("a1", "a2", "a3"))
    hbuf, h = guarded_out(n, d, acts["h0"])
    qbuf, qkv = guarded_out(n, 3 * d)
    fbuf, f = guarded_out(n, ff)
    for lw in layers:
        W = {name: (dev(v["w"]), dev(v["bias"])) for name, v in lw.items()}
        wq.gemm(a1, W["qkv"][0], wq.W_BF16, m=3 * d, k=d, bias=W["qkv"][1], out=qkv)
        wq.gemm(a2, W["out"][0], wq.W_BF16, m=d, k=d, bias=W["out"][1], residual=True, out=h)
        wq.gemm(a3, W["fc1"][0], wq.W_BF16, m=ff, k=d, bias=W["fc1"][1], gelu=True, out=f)
        wq.gemm(f, W["fc2"][0], wq.W_BF16, m=d, k=ff, bias=W["fc2"][1], residual=True, out=h)
    return read_guarded(qbuf, n, 3 * d), read_guarded(fbuf, n, ff), read_guarded(hbuf, n, d)


def test_encoder_chain_24_layers(encoder):
    acts, layers = encoder
    qkv, f, h = _gpu_chain(acts, layers)
    for name, arr in (("qkv", qkv), ("f", f), ("h", h)):
        assert np.isfinite(arr).all(), f"{name}: non-finite outputs"
    t = np.array(SAMPLE_FRAMES)
    a1, a2, a3 = (acts[name][t] for name in ("a1", "a2", "a3"))
    h_ref = acts["h0"][t].astype(np.float64)
    h_tol = np.zeros_like(h_ref)
    bf = wq.W_BF16
    for lw in layers:
        qkv_w, out_w, fc1_w, fc2_w = lw["qkv"], lw["out"], lw["fc1"], lw["fc2"]
        q_ref, q_tol = oracle_with_tol(a1, qkv_w["w"], bf, qkv_w["m"], qkv_w["k"], qkv_w["bias"], 1, None, B_MFMA)
        o_ref, o_S = oracle.linear(a2, out_w["w"], bf, out_w["m"], out_w["k"], out_w["bias"], 1)
        f_ref, f_tol = oracle_with_tol(a3, fc1_w["w"], bf, fc1_w["m"], fc1_w["k"], fc1_w["bias"], 3, None, B_MFMA)
        # fc2 sees the GPU's f, which differs from f_ref by at most f_tol per element:
        # that difference reaches the output through |W2|.
        w2 = oracle.decode(fc2_w["w"], bf, fc2_w["m"], fc2_w["k"])
        c_ref, c_S = oracle.linear(f_ref, fc2_w["w"], bf, fc2_w["m"], fc2_w["k"], fc2_w["bias"], 1)
        carried = f_tol @ np.abs(w2).T
        h_new = h_ref + o_ref + c_ref
        h_tol = (h_tol + B_MFMA * (o_S + c_S) + carried * (1 + B_MFMA)
                 + ULP_SLACK * (np.abs(h_ref) + np.abs(o_ref) + np.abs(c_ref) + np.abs(h_new)))
        h_ref = h_new
    rq = assert_within(qkv[t], q_ref, q_tol, "last layer qkv")
    _, q_S = oracle.linear(a1, layers[-1]["qkv"]["w"], bf, 3 * synth.ENCODER_D, synth.ENCODER_D)
    _report("C5 last layer QKV", qkv[t], q_ref, q_S, B_MFMA, rq)
    rf = assert_within(f[t], f_ref, f_tol, "last layer fc1+GELU")
    _, f_S = oracle.linear(a3, layers[-1]["fc1"]["w"], bf, synth.ENCODER_FF, synth.ENCODER_D)
    _report("C5 last layer fc1+GELU (vs pre-activation S)", f[t], f_ref, f_S, B_MFMA, rf)
    worst = assert_within(h[t], h_ref, h_tol, "residual stream after 24 layers")
    print(f"C5 residual stream after 24 layers on {len(t)} frames: err/tol = {worst:.4f}")
