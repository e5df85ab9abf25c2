"""GPU parity at the five workloads' full sizes, in the launch configuration the
bench times (the same C-ABI calls), checked on every output the oracle can
afford: all of them for the small cases, sampled output columns for the large
matvecs, and sampled frames (rows) of the 24-layer encoder chain.
"""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import oracle
import synth
from tests.parity import (B_F32, B_MFMA, GELU_SLOPE, ULP_SLACK, assert_within, dev, guarded_out,
                          oracle_with_tol, read_guarded)

pytestmark = pytest.mark.gpu


def _call(cfg, path=wq.PATH_AUTO):
    n, m, k = cfg["n"], cfg["m"], cfg["k"]
    buf, out = guarded_out(n, m)
    bias = cfg["bias"]
    wq.gemm(dev(cfg["x"]), dev(cfg["w"]), cfg["wtype"], m=m, k=k,
            bias=None if bias is None else dev(bias), gelu=bool(cfg["flags"] & wq.GELU), out=out, path=path)
    return read_guarded(buf, n, m)


def test_bf16_gemm_64x256x256_bias_gelu():
    cfg = synth.config_gemm_small()
    assert wq.gemm_path(cfg["n"], cfg["m"], cfg["k"], cfg["wtype"]) == wq.PATH_MFMA
    got = _call(cfg)
    y_ref, tol = oracle_with_tol(cfg["x"], cfg["w"], cfg["wtype"], cfg["m"], cfg["k"], cfg["bias"],
                                 cfg["flags"], None, B_MFMA)
    assert_within(got, y_ref, tol, "64x256x256")


@pytest.mark.parametrize("n", [1, 4])
def test_q8_0_matvec_4096(n):
    cfg = synth.config_q8_matvec(n)
    got = _call(cfg)
    y_ref, tol = oracle_with_tol(cfg["x"], cfg["w"], cfg["wtype"], cfg["m"], cfg["k"], None, 0, None, B_F32)
    assert_within(got, y_ref, tol, f"q8_0 n={n}")


def _sample_cols(m, count, seed):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(64), np.arange(m - 64, m), g.choice(m, count, replace=False)]))


def test_q4_0_matvec_14336x4096():
    cfg = synth.config_q4_matvec()
    got = _call(cfg)
    cols = _sample_cols(cfg["m"], 1024, 1)
    y_ref, tol = oracle_with_tol(cfg["x"], cfg["w"], cfg["wtype"], cfg["m"], cfg["k"], None, 0, None, B_F32,
                                 rows=cols)
    assert_within(got[:, cols], y_ref, tol, "q4_0 14336x4096")


@pytest.mark.parametrize("gated", [True, False])
def test_moe_q4_0_16_tokens_top2_of_8(gated):
    cfg = synth.config_moe()
    n_tok, top_k, E, m, k = cfg["n_tok"], cfg["top_k"], cfg["n_exp"], cfg["m"], cfg["k"]
    rows = n_tok if gated else n_tok * top_k
    buf, out = guarded_out(rows, m)
    wq.moe_matvec(dev(cfg["x"]), dev(cfg["w"]), cfg["wtype"], dev(cfg["ids"]),
                  dev(cfg["gates"]) if gated else None, n_experts=E, m=m, k=k, out=out)
    got = read_guarded(buf, rows, m)
    cols = _sample_cols(m, 256, 2)
    y_ref, S = oracle.moe(cfg["x"], cfg["w"], cfg["wtype"], cfg["ids"], E, m, k,
                          cfg["gates"] if gated else None, rows=cols)
    assert_within(got[:, cols], y_ref, B_F32 * S + ULP_SLACK * np.abs(y_ref), "moe 16x top2/8")


# ---------------------------------------------------------------- encoder chain

SAMPLE_FRAMES = [0, 1, 777, 1499]


@pytest.fixture(scope="module")
def encoder():
    acts = synth.encoder_activations()
    layers = [synth.encoder_layer_weights(layer) for layer in range(synth.ENCODER_LAYERS)]
    return acts, layers


def _gpu_chain(acts, layers):
    """The workload as the bench runs it: per layer QKV(+bias), out(+bias,+=h), fc1(+bias,GELU), fc2(+bias,+=h)."""
    import torch
    n, d, ff = synth.ENCODER_N, synth.ENCODER_D, synth.ENCODER_FF
    a1, a2, a3 = (dev(acts[name]) for name in ("a1", "a2", "a3"))
    h = dev(acts["h0"]).clone()
    qkv = torch.empty((n, 3 * d), device="cuda")
    f = torch.empty((n, ff), device="cuda")
    for lw in layers:
        W = {name: (dev(v["w"]), dev(v["bias"])) for name, v in lw.items()}
        wq.gemm(a1, W["qkv"][0], wq.W_BF16, m=3 * d, k=d, bias=W["qkv"][1], out=qkv)
        wq.gemm(a2, W["out"][0], wq.W_BF16, m=d, k=d, bias=W["out"][1], residual=True, out=h)
        wq.gemm(a3, W["fc1"][0], wq.W_BF16, m=ff, k=d, bias=W["fc1"][1], gelu=True, out=f)
        wq.gemm(f, W["fc2"][0], wq.W_BF16, m=d, k=ff, bias=W["fc2"][1], residual=True, out=h)
    torch.cuda.synchronize()
    return qkv.cpu().numpy(), f.cpu().numpy(), h.cpu().numpy()


def test_encoder_chain_24_layers_sampled_frames(encoder):
    acts, layers = encoder
    qkv, f, h = _gpu_chain(acts, layers)
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
    assert_within(qkv[t], q_ref, q_tol, "last layer qkv")
    assert_within(f[t], f_ref, f_tol, "last layer fc1+GELU")
    worst = assert_within(h[t], h_ref, h_tol, "residual stream after 24 layers")
    print(f"encoder chain: worst err/tol = {worst:.3f}")
