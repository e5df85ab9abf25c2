"""Seeded synthetic inputs for the weight-dequantizing linear layer.

This module only draws numbers and lays them out in the storage formats the
layer consumes; it computes nothing the layer computes. Both the HIP path (via
the tests and the bench) and the CPU oracle receive the arrays it returns, and
neither of them imports the other.

Storage formats (what the bytes mean is defined by the pages this project
follows, and restated here only to lay the bytes out):

* bf16 weights: ``uint16[m][k]``, the upper half of the f32 bit pattern
  (cortiq-engine ``nemotron_audio.rs``, the ``ae_gemm`` kernel's weight pairs).
* Q8_0 weights: ``m`` rows of ``k/32`` blocks of 34 bytes -- a little-endian
  f16 scale followed by 32 signed bytes (wavo ``gpu/mod.rs``,
  ``Gpu::upload_linear`` and the test helper ``weights``; hanzo-ml
  ``wgpu_backend.rs``, ``matvec_q8_0_gpu``).
* f32 / f16 weights: ``float32[m][k]`` / IEEE ``float16[m][k]`` bit patterns
  (wavo ``gpu/mod.rs`` ``Linear``: GEMM types 0 and 1, copied as stored by
  ``Gpu::upload_linear``).
* Q4_0 weights: ``m`` rows of ``k/32`` blocks of 18 bytes -- a little-endian
  f16 scale followed by 16 bytes whose low nibbles are elements 0-15 and high
  nibbles elements 16-31 (hanzo-ml ``wgpu_backend.rs`` names the format in
  ``matvec_q4_0_gpu``; the nibble order is the plain GGML reading).
* Q4_K weights: ``m`` rows of ``k/256`` super-blocks of 144 bytes (hanzo-ml
  ``matvec_q4k_gpu`` names the type and both sizes); the bytes hold two f16
  factors, packed 6-bit sub-block fields and 4-bit quants in GGML's published
  k-quant layout. Only the two f16 factors are drawn as numbers; the rest are
  uniform random bytes.

Every tensor gets its own generator ``numpy.random.default_rng([seed, cfg,
tensor])`` so that its values do not depend on the shapes of other tensors.
"""
from __future__ import annotations

import numpy as np

W_BF16, W_Q8_0, W_Q4_0, W_F32, W_F16, W_Q4_K = 0, 1, 2, 3, 4, 5
BLOCK = 32
BLOCK_BYTES = {W_Q8_0: 34, W_Q4_0: 18}
SUPER = 256        # Q4_K super-block: 256 weights
SUPER_BYTES = 144  # in 144 bytes


def rng(*key: int) -> np.random.Generator:
    """A generator keyed by a tuple of non-negative integers."""
    return np.random.default_rng([int(v) for v in key])


def normal_f32(g: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """f32 samples of N(0, sigma^2): a standard normal drawn in f32, times sigma."""
    return g.standard_normal(shape, dtype=np.float32) * np.float32(sigma)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round f32 values to bf16 (round to nearest, ties to even) and return the bits.

    Only finite inputs are expected (the generators draw normals).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_weight(g: np.random.Generator, m: int, k: int, sigma: float) -> np.ndarray:
    """``uint16[m][k]`` bf16 bits of N(0, sigma^2) samples."""
    return bf16_bits(normal_f32(g, (m, k), sigma))


def _scales_f16_bits(g: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """f16 bits of |N(0, sigma^2)| (f32 draw, then numpy's round-to-nearest f16)."""
    return np.abs(normal_f32(g, shape, sigma)).astype(np.float16).view(np.uint16)


def q8_0_weight(g: np.random.Generator, m: int, k: int, dsigma: float = 0.01) -> np.ndarray:
    """``uint8[m][k/32*34]``: scales |N(0, dsigma^2)| as f16, quants uniform in [-127, 127]."""
    assert k % BLOCK == 0
    nb = k // BLOCK
    d = _scales_f16_bits(g, (m, nb), dsigma)
    q = g.integers(-127, 128, size=(m, nb, BLOCK), dtype=np.int8)
    out = np.empty((m, nb, 34), dtype=np.uint8)
    out[:, :, 0] = (d & 0xFF).astype(np.uint8)
    out[:, :, 1] = (d >> 8).astype(np.uint8)
    out[:, :, 2:] = q.view(np.uint8)
    return out.reshape(m, nb * 34)


def q4_0_weight(g: np.random.Generator, m: int, k: int, dsigma: float = 0.01) -> np.ndarray:
    """``uint8[m][k/32*18]``: scales |N(0, dsigma^2)| as f16, 4-bit quants uniform in [0, 15].

    Every element is an independent uniform nibble, so each quant byte is a
    uniform byte; drawing the bytes directly gives exactly that distribution.
    """
    assert k % BLOCK == 0
    nb = k // BLOCK
    d = _scales_f16_bits(g, (m, nb), dsigma)
    qs = g.integers(0, 256, size=(m, nb, 16), dtype=np.uint8)
    out = np.empty((m, nb, 18), dtype=np.uint8)
    out[:, :, 0] = (d & 0xFF).astype(np.uint8)
    out[:, :, 1] = (d >> 8).astype(np.uint8)
    out[:, :, 2:] = qs
    return out.reshape(m, nb * 18)


def q4_k_weight(g: np.random.Generator, m: int, k: int, dsigma: float = 0.01) -> np.ndarray:
    """``uint8[m][k/256*144]``: Q4_K super-blocks with random fields.

    Bytes 0-1 and 2-3 of each 144-byte super-block are the f16 bits of |N(0, (dsigma/16)^2)| and
    |N(0, (dsigma/2)^2)| (the super-block's scale and min factors); the other 140 bytes (the packed
    6-bit sub-block scales and mins, and the 4-bit quants) are uniform random bytes, so every
    6-bit field and every nibble is uniform. With these factors the weights of a sub-block
    straddle zero, as trained weights do.
    """
    assert k % SUPER == 0
    ns = k // SUPER
    d = _scales_f16_bits(g, (m, ns), dsigma / 16)
    dmin = _scales_f16_bits(g, (m, ns), dsigma / 2)
    rest = g.integers(0, 256, size=(m, ns, SUPER_BYTES - 4), dtype=np.uint8)
    out = np.empty((m, ns, SUPER_BYTES), dtype=np.uint8)
    out[:, :, 0] = (d & 0xFF).astype(np.uint8)
    out[:, :, 1] = (d >> 8).astype(np.uint8)
    out[:, :, 2] = (dmin & 0xFF).astype(np.uint8)
    out[:, :, 3] = (dmin >> 8).astype(np.uint8)
    out[:, :, 4:] = rest
    return out.reshape(m, ns * SUPER_BYTES)


def weight(g: np.random.Generator, wtype: int, m: int, k: int, sigma: float = 0.02,
           dsigma: float = 0.01) -> np.ndarray:
    """A weight of the given storage type, as the raw array the layer reads."""
    if wtype == W_BF16:
        return bf16_weight(g, m, k, sigma)
    if wtype == W_Q8_0:
        return q8_0_weight(g, m, k, dsigma)
    if wtype == W_Q4_0:
        return q4_0_weight(g, m, k, dsigma)
    if wtype == W_F32:
        return normal_f32(g, (m, k), sigma)
    if wtype == W_F16:
        return f16_weight(g, m, k, sigma)
    if wtype == W_Q4_K:
        return q4_k_weight(g, m, k, dsigma)
    raise ValueError(f"unknown weight type {wtype}")


def f16_weight(g: np.random.Generator, m: int, k: int, sigma: float) -> np.ndarray:
    """``uint16[m][k]`` f16 bits of N(0, sigma^2) samples (numpy's round-to-nearest f16)."""
    return normal_f32(g, (m, k), sigma).astype(np.float16).view(np.uint16)


def weight_nbytes(wtype: int, m: int, k: int) -> int:
    """Bytes of one ``m x k`` weight in its storage format."""
    if wtype in (W_BF16, W_F16):
        return 2 * m * k
    if wtype == W_F32:
        return 4 * m * k
    if wtype == W_Q4_K:
        return SUPER_BYTES * m * (k // SUPER)
    return BLOCK_BYTES[wtype] * m * (k // BLOCK)


def moe_routing(g: np.random.Generator, n_tok: int, n_exp: int, top_k: int):
    """Per token ``top_k`` distinct expert ids (uniform, without replacement) and gate weights.

    The gate weights are the softmax of ``top_k`` N(0,1) logits drawn per token
    (one per routed expert, in draw order), taken in f64 and rounded to f32.
    """
    ids = np.stack([g.choice(n_exp, top_k, replace=False) for _ in range(n_tok)]).astype(np.int32)
    logits = g.standard_normal((n_tok, top_k))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    gates = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids.reshape(n_tok, top_k), gates


# ---------------------------------------------------------------------------
# The five workloads (seed 0; tensor index = position in the list below).
# ---------------------------------------------------------------------------

def config_gemm_small(seed: int = 0):
    """bf16 GEMM: X[64x256] ~N(0,1), W[256x256] bf16 ~N(0,0.02), bias[256] ~N(0,0.1), bias+GELU."""
    cfg = 1
    n, m, k = 64, 256, 256
    return dict(
        n=n, m=m, k=k, wtype=W_BF16, flags=1 | 2,
        x=normal_f32(rng(seed, cfg, 0), (n, k), 1.0),
        w=bf16_weight(rng(seed, cfg, 1), m, k, 0.02),
        bias=normal_f32(rng(seed, cfg, 2), (m,), 0.1),
    )


def config_q8_matvec(n: int, seed: int = 0, copy: int = 0):
    """Q8_0 decode matvec: X[n x 4096] ~N(0,1), W 4096x4096 Q8_0, no bias."""
    cfg = 2
    m = k = 4096
    return dict(
        n=n, m=m, k=k, wtype=W_Q8_0, flags=0,
        x=normal_f32(rng(seed, cfg, 0, n), (n, k), 1.0),
        w=q8_0_weight(rng(seed, cfg, 1, copy), m, k),
        bias=None,
    )


def config_q4_matvec(seed: int = 0, copy: int = 0):
    """Q4_0 matvec: X[1 x 4096] ~N(0,1), W 14336x4096 Q4_0, no bias."""
    cfg = 3
    n, m, k = 1, 14336, 4096
    return dict(
        n=n, m=m, k=k, wtype=W_Q4_0, flags=0,
        x=normal_f32(rng(seed, cfg, 0), (n, k), 1.0),
        w=q4_0_weight(rng(seed, cfg, 1, copy), m, k),
        bias=None,
    )


def config_moe(seed: int = 0, n_exp: int = 8, m: int = 14336, k: int = 4096, bank: int = 0):
    """MoE Q4_0 matvec: 16 tokens, top-2 of 8 experts, each expert W_e[14336x4096] Q4_0."""
    cfg = 4
    n_tok, top_k = 16, 2
    ids, gates = moe_routing(rng(seed, cfg, 2), n_tok, n_exp, top_k)
    return dict(
        n_tok=n_tok, top_k=top_k, n_exp=n_exp, m=m, k=k, wtype=W_Q4_0,
        x=normal_f32(rng(seed, cfg, 0), (n_tok, k), 1.0),
        w=np.stack([q4_0_weight(rng(seed, cfg, 1, e, bank), m, k) for e in range(n_exp)]),
        ids=ids, gates=gates,
    )


ENCODER_LAYERS = 24
ENCODER_N, ENCODER_D, ENCODER_FF = 1500, 1024, 4096


def encoder_layer_weights(layer: int, seed: int = 0):
    """One encoder layer's four bf16 weights and biases (wqkv, wo, w1, w2)."""
    cfg = 5
    d, ff = ENCODER_D, ENCODER_FF
    shapes = [("qkv", 3 * d, d), ("out", d, d), ("fc1", ff, d), ("fc2", d, ff)]
    out = {}
    for i, (name, m, k) in enumerate(shapes):
        out[name] = dict(
            m=m, k=k,
            w=bf16_weight(rng(seed, cfg, 100 + layer, 2 * i), m, k, 0.02),
            bias=normal_f32(rng(seed, cfg, 100 + layer, 2 * i + 1), (m,), 0.1),
        )
    return out


def encoder_activations(seed: int = 0):
    """The stand-ins for the LayerNorm/attention outputs A1..A3 and the residual stream h0."""
    cfg = 5
    n, d = ENCODER_N, ENCODER_D
    return {name: normal_f32(rng(seed, cfg, i), (n, d), 1.0)
            for i, name in enumerate(["a1", "a2", "a3", "h0"])}


# ---- the rest of the encoder block (LayerNorm, q/k norm + rotation, attention) ----------------
# Heads, rotated dims and padding are not fixed by the pages for this encoder: 8 heads of 128
# (the largest head its kernels take, d = 1024), every dim of a head rotated, and the last 100 of
# the 1500 frames marked as padding (masked keys).
ENCODER_HEADS, ENCODER_ROT, ENCODER_VALID = 8, 128, 1400


def layer_norm_weights(g: np.random.Generator, d: int) -> np.ndarray:
    """f32 [2d]: weights 1 + N(0, 0.1^2), then biases N(0, 0.1^2)."""
    return np.concatenate([1.0 + normal_f32(g, (d,), 0.1), normal_f32(g, (d,), 0.1)]).astype(np.float32)


def unit_circle_table(g: np.random.Generator, n: int, half: int) -> np.ndarray:
    """f32 [2 * n * half]: cosines then sines of angles drawn uniformly in [0, 2 pi), laid out as a
    rotation table (any table serves to test the rotation's arithmetic)."""
    theta = g.uniform(0.0, 2.0 * np.pi, (n, half))
    return np.concatenate([np.cos(theta).reshape(-1), np.sin(theta).reshape(-1)]).astype(np.float32)


def key_mask(n: int, n_valid: int) -> np.ndarray:
    """int32 [n]: the first n_valid frames valid (1), the rest padding (0)."""
    v = np.zeros(n, np.int32)
    v[:n_valid] = 1
    return v


def random_key_mask(g: np.random.Generator, n: int, p_valid: float) -> np.ndarray:
    """int32 [n]: each frame valid with probability p_valid."""
    return (g.random(n) < p_valid).astype(np.int32)


def encoder_block_weights(layer: int, seed: int = 0, d: int = ENCODER_D, heads: int = ENCODER_HEADS,
                          inter: int = ENCODER_FF, qk_norm: bool = True, qkv_bias: bool = False,
                          sigma: float = 0.02):
    """One pre-norm block: LayerNorm weights, bf16 matrices N(0, sigma^2), biases N(0, 0.1^2);
    q/k norm weights when qk_norm, a q/k/v bias when qkv_bias (the pages' block has none)."""
    cfg = 6
    hd = d // heads
    r = lambda i: rng(seed, cfg, layer, d, inter, i)  # noqa: E731
    return {
        "ln1": layer_norm_weights(r(0), d),
        "qkv_w": bf16_weight(r(1), 3 * d, d, sigma),
        "qkv_b": normal_f32(r(2), (3 * d,), 0.1) if qkv_bias else None,
        "qn": layer_norm_weights(r(3), hd) if qk_norm else None,
        "kn": layer_norm_weights(r(4), hd) if qk_norm else None,
        "out_w": bf16_weight(r(5), d, d, sigma), "out_b": normal_f32(r(6), (d,), 0.1),
        "ln2": layer_norm_weights(r(7), d),
        "fc1_w": bf16_weight(r(8), inter, d, sigma), "fc1_b": normal_f32(r(9), (inter,), 0.1),
        "fc2_w": bf16_weight(r(10), d, inter, sigma), "fc2_b": normal_f32(r(11), (d,), 0.1),
    }


def encoder_model(n_layers: int, seed: int = 0, d: int = ENCODER_D, heads: int = ENCODER_HEADS,
                  inter: int = ENCODER_FF, stack_in: int | None = None, qk_norm: bool = True):
    """Embedding and final LayerNorms, an optional input projection [d][stack_in] (bf16, no bias)
    and n_layers blocks."""
    cfg = 7
    return {
        "proj": None if stack_in is None else bf16_weight(rng(seed, cfg, 0), d, stack_in, 0.05),
        "embed_norm": layer_norm_weights(rng(seed, cfg, 1, d), d),
        "final_norm": layer_norm_weights(rng(seed, cfg, 2, d), d),
        "layers": [encoder_block_weights(i, seed, d, heads, inter, qk_norm) for i in range(n_layers)],
    }
