/*
 * wq.h -- C ABI of the weight-dequantizing linear layer for AMD MI355X (gfx950).
 *
 *   Y[n x m] = epilogue( X[n x k] . W[m x k]^T + bias )
 *
 * X is f32, W is stored as bf16 or as GGML-style 32-element Q8_0 / Q4_0
 * blocks, accumulation is f32, and the epilogue adds a bias, applies erf-GELU
 * and/or accumulates into Y. The operation and its flag bits are those of the
 * GEMM kernel on the cortiq-engine 0.8.49 page src/gpu_wgpu/nemotron_audio.rs
 * (the `AE_WGSL` source: `ae_gemm`, its `GmP` parameter block and `ae_put`);
 * the quantized weight formats and the MoE matvec are those of the hanzo-ml
 * 0.11.13 page src/wgpu_backend.rs (`upload_qweight`, `matvec_q8_0_gpu`,
 * `matvec_q4_0_gpu`, `moe_matvec_gpu`); wavo 0.3.0 src/gpu/mod.rs describes
 * the same layer (`Linear`, `Epilogue`, `Pass::gemm`, `Pass::gemv`) and the
 * requirement k % 32 == 0 (`Gpu::upload_linear`).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, owned by the caller. The
 *     library keeps no reference to them after the call returns; the caller
 *     keeps them alive until the work enqueued on `stream` has completed.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call is asynchronous on it; nothing synchronizes the host.
 *   - Tensors are contiguous and row-major; there are no strides.
 *   - Arguments are checked on the host before any HIP call; a failed check
 *     returns a negative status, enqueues nothing and leaves the outputs
 *     untouched. `wq_last_error()` then describes it (per thread).
 *   - Faults of the enqueued work itself surface at the caller's next
 *     synchronization, as for any HIP kernel.
 *   - The library allocates device memory only for the MoE gate combine
 *     (a per-device, per-stream workspace, grown on demand and kept until
 *     the process ends). Growing it is the one place a call waits and
 *     allocates: it synchronizes the stream (work already queued there may
 *     still read the old buffer), frees that buffer and calls hipMalloc. A
 *     gated wq_moe_matvec call that grows the workspace therefore cannot be
 *     captured into a HIP graph; make one uncaptured call of the largest size
 *     first, or use wq_moe_matvec_noalloc, which never allocates.
 *   - Every entry point may be called from several host threads at once, on
 *     the same stream or on different ones.
 *   - Alignment: x and w must be 16-byte aligned (the kernels move them with
 *     16-byte vector loads and 16-byte direct-to-LDS loads); y, bias, the
 *     MoE ids and gates need only 4 bytes (they are read and written one f32
 *     or int32 at a time), so y may start at any element of a larger buffer.
 *   - Sizes: n, m (and m + dual) at most 2^31 - 513 and n * (m + dual) at
 *     most 2^40, so that every tile and grid count the kernels form fits in
 *     32 bits. Byte offsets into W are 64-bit (a weight may pass 2 GiB).
 *   - Determinism: every route sums in a fixed order and gives bit-identical
 *     results run to run, except one: the quantized, f16 and f32 weight
 *     types on the matrix cores, when the output has too few tiles to fill
 *     the chip and the epilogue is WQ_RESIDUAL with no activation. That call
 *     splits k across workgroups that add their partial sums into Y with f32
 *     atomics, so the order of those additions (and the last bits of Y) may
 *     differ between runs. bf16 weights take it only when X or W reaches
 *     4 GiB: operands that large run on the same kernel as the other types.
 */
#ifndef WQ_H
#define WQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- weight storage types ------------------------------------------------
 * WQ_W_BF16: uint16[m][k]; each value is the upper 16 bits of an f32
 *            (little-endian), decoded exactly by a 16-bit shift -- the weight
 *            pairs of `ae_gemm` on the cortiq-engine page.
 * WQ_W_Q8_0: m rows of k/32 blocks of 34 bytes: a little-endian f16 scale d,
 *            then 32 int8 quants q; value = d*q (wavo `Gpu::upload_linear`,
 *            hanzo-ml `matvec_q8_0_gpu`).
 * WQ_W_Q4_0: m rows of k/32 blocks of 18 bytes: a little-endian f16 scale d,
 *            then 16 bytes; byte j holds element j in its low nibble and
 *            element j+16 in its high nibble; value = d*(q-8) (hanzo-ml
 *            `matvec_q4_0_gpu`). Rows follow each other with no padding.
 * WQ_W_F32:  float[m][k], IEEE binary32, little-endian (wavo `Linear` GEMM
 *            type 0, copied as stored by `Gpu::upload_linear`).
 * WQ_W_F16:  uint16[m][k], IEEE binary16, little-endian (wavo `Linear` GEMM
 *            type 1).
 * WQ_W_Q4_K: m rows of k/256 super-blocks of 144 bytes, k a multiple of 256
 *            (hanzo-ml `matvec_q4k_gpu` names the type and both sizes; the
 *            byte layout is GGML's published k-quant super-block): bytes 0-1
 *            f16 d, 2-3 f16 dmin, 4-15 the 6-bit scale sc_j and 6-bit min m_j
 *            of each 32-element sub-block j (j < 4: low 6 bits of bytes 4+j
 *            and 8+j; j >= 4: low and high nibble of byte 8+j, their top two
 *            bits in the top bits of bytes j and 4+j), 16-143 the 4-bit quants
 *            (sub-blocks 2c and 2c+1 in the low and high nibbles of bytes
 *            16+32c .. 16+32c+31); value = d*sc_j*q - dmin*m_j. Q4_K takes the
 *            matvec path only (n <= WQ_MATVEC_MAX_N, and wq_moe_matvec); the
 *            matrix-core paths refuse it with WQ_ERR_WTYPE.
 * Every type enters every path exactly: the f32 paths decode each weight to
 * its f32 value; the matrix cores take bf16 as stored, the integer quants with
 * the block scale applied in f32, and f16 / f32 weights as two / three bf16
 * parts that add up to the weight (two / three times the MFMA work). */
#define WQ_W_BF16 0
#define WQ_W_Q8_0 1
#define WQ_W_Q4_0 2
#define WQ_W_F32 3
#define WQ_W_F16 4
#define WQ_W_Q4_K 5

/* ---- epilogue flags ---------------------------------------------------------
 * Applied to each output in this order: + bias[j] (WQ_BIAS); then at most one
 * activation; then times alpha (wq_linear; 1 for every other entry point);
 * then + the value Y held before the call (WQ_RESIDUAL; Y is read and written
 * in place). Bits 1, 2, 4 and that order are those of `GmP.flags` / `ae_put`
 * (cortiq-engine). The activations and alpha are the modes of wavo's
 * `Epilogue` (src/gpu/mod.rs: Silu, Relu, Tanh, Gelu, GeluResidual,
 * Residual(alpha) = c + alpha * (a.W^T + b)):
 *   WQ_GELU  erf-GELU 0.5*v*(1+erf(v/sqrt 2));
 *   WQ_SILU  v / (1 + exp(-v));
 *   WQ_RELU  max(v, 0);
 *   WQ_TANH  tanh(v).
 * Two activation bits together are refused (WQ_ERR_FLAGS). */
#define WQ_BIAS 1u
#define WQ_GELU 2u
#define WQ_RESIDUAL 4u
#define WQ_SILU 8u
#define WQ_RELU 16u
#define WQ_TANH 32u

/* ---- contraction paths ----------------------------------------------------
 * WQ_PATH_MATVEC: all-f32 FMA path for n <= 16 (weights streamed once for all
 *   n rows of X). Error: |y - y_ref| <= 1e-5 * sum_k |x_k * w_k|.
 * WQ_PATH_MFMA: bf16 matrix-core path for any n: X rounded to bf16 (to
 *   nearest even), W fed exactly (bf16 as stored; Q8_0/Q4_0 as their integer
 *   quants, with the f16 scale applied in f32 per 32-element block), f32
 *   accumulation. Error: |y - y_ref| <= 2^-8 * sum_k |x_k * w_k|.
 * WQ_PATH_MFMA_F32: the matrix-core path with f32 accuracy for any n: the
 *   arithmetic of the encoder on the cortiq-engine page (nemotron_audio.rs,
 *   module doc: bf16 weights, f32 activations and f32 accumulation, as its
 *   fp32 reference tower computes). Each x is split into three bf16 parts,
 *   p1 = bf16(x), p2 = bf16(x - p1), p3 = bf16(x - p1 - p2) (nearest even),
 *   which add up to x exactly; each part is multiplied by the exact weights
 *   on the matrix cores (three times the MFMA work of WQ_PATH_MFMA). The
 *   products are thus exact and only the f32 running sums round, as in an f32
 *   GEMM; the result is held to the WQ_PATH_MATVEC bound,
 *   |y - y_ref| <= 1e-5 * sum_k |x_k * w_k|. Never chosen by WQ_PATH_AUTO.
 * WQ_PATH_AUTO: MATVEC when n <= 16, else MFMA (`wq_gemm_path` tells which). */
#define WQ_PATH_AUTO 0
#define WQ_PATH_MATVEC 1
#define WQ_PATH_MFMA 2
#define WQ_PATH_MFMA_F32 3
#define WQ_MATVEC_MAX_N 16

/* ---- status codes ---------------------------------------------------------- */
#define WQ_OK 0
#define WQ_ERR_NULL (-1)   /* a required pointer is NULL */
#define WQ_ERR_SHAPE (-2)  /* negative size, k % 32 != 0, n too large for the path, ... */
#define WQ_ERR_WTYPE (-3)  /* unknown weight type */
#define WQ_ERR_FLAGS (-4)  /* unknown flag bits, two activations, WQ_BIAS without a bias (or a bias
                              without WQ_BIAS), or a non-finite alpha */
#define WQ_ERR_ALIGN (-5)  /* x or w not 16-byte aligned; y, bias, ids or gates not 4-byte aligned */
#define WQ_ERR_ALIAS (-6)  /* y overlaps x, w, bias, ids or gates */
#define WQ_ERR_HIP (-7)    /* a HIP call failed (launch, allocation, device query) */

/*
 * wq_gemm: Y = epilogue(X . W^T + bias) on `stream`, path chosen by n.
 *   x     f32 [n][k], 16-byte aligned.
 *   w     weight [m][k] in `wtype` storage (wq_weight_bytes bytes), 16-byte aligned.
 *   bias  f32 [m] when flags & WQ_BIAS, else NULL; 4-byte aligned.
 *   y     f32 [n][m], 4-byte aligned (wavo's `Pass::gemv` writes its output from an offset into
 *         a larger buffer); read first when flags & WQ_RESIDUAL.
 *   n, m  >= 0 (n == 0 or m == 0: nothing to do, WQ_OK); k > 0, k % 32 == 0 (Q4_K: k % 256 == 0,
 *         and n <= WQ_MATVEC_MAX_N, else WQ_ERR_SHAPE / WQ_ERR_WTYPE).
 * Returns WQ_OK or a WQ_ERR_* code.
 */
int wq_gemm(const float* x, const void* w, int wtype, const float* bias, unsigned flags,
            float* y, int64_t n, int64_t m, int64_t k, void* stream);

/* wq_gemm with the path forced (WQ_PATH_*). WQ_PATH_MATVEC requires n <= 16;
 * WQ_PATH_MFMA_F32 (f32 accuracy on the matrix cores) is reached only here. */
int wq_gemm_ex(const float* x, const void* w, int wtype, const float* bias, unsigned flags,
               float* y, int64_t n, int64_t m, int64_t k, int path, void* stream);

/*
 * wq_linear: wq_gemm_ex with a factor on the activated value:
 *   Y = alpha * act(X . W^T + bias) (+ Y_old when flags & WQ_RESIDUAL),
 * wavo's `Epilogue::Residual(alpha)` (with WQ_BIAS | WQ_RESIDUAL) and its
 * activations at any scale. alpha must be finite (WQ_ERR_FLAGS otherwise);
 * alpha = 1 is exactly wq_gemm_ex. Every other argument as for wq_gemm_ex.
 */
int wq_linear(const float* x, const void* w, int wtype, const float* bias, unsigned flags, float alpha,
              float* y, int64_t n, int64_t m, int64_t k, int path, void* stream);

/*
 * wq_linear_dual: wq_linear with wavo's dual outputs (`Linear.dual`, set up by
 * `Gpu::upload_linear` from a bias with `dual` extra values): the first `dual`
 * outputs are written a second time, after the m others, each with its own
 * bias -- for one projection that needs two position biases.
 *   bias  f32 [m + dual] when flags & WQ_BIAS (bias[m + j] is the second bias
 *         of output j), else NULL.
 *   y     f32 [n][m + dual]: y[t][j] for j < m as wq_linear; y[t][m + j] for
 *         j < dual is the same product with bias[m + j], the same activation
 *         and alpha, and (WQ_RESIDUAL) its own old value.
 *   dual  0 <= dual <= m (WQ_ERR_SHAPE otherwise); 0 is exactly wq_linear.
 * Every other argument as for wq_linear.
 */
int wq_linear_dual(const float* x, const void* w, int wtype, const float* bias, unsigned flags, float alpha,
                   float* y, int64_t n, int64_t m, int64_t k, int64_t dual, int path, void* stream);

/*
 * wq_moe_matvec: the MoE matvec of hanzo-ml `moe_matvec_gpu`, expert-major.
 *   x          f32 [n_tok][k], 16-byte aligned. Every routed slot of token t reads row t
 *              (one activation row per token, shared by its top_k slots); hanzo-ml's page
 *              gives x per routed slot, which is this with top_k = 1 or with the rows repeated.
 *   w_experts  one bank of n_experts weights, expert e at byte offset
 *              e * wq_weight_bytes(wtype, m, k); 16-byte aligned.
 *   expert_ids int32 [n_tok][top_k]: expert of slot s = t*top_k + j.
 *              Precondition 0 <= id < n_experts (not checked on the host:
 *              the ids live on the device). A slot with an id outside that
 *              range is never read from the bank; its output is NaN.
 *   gate_w     f32 [n_tok][top_k] or NULL.
 *   y          4-byte aligned.
 *              gate_w == NULL: f32 [n_tok*top_k][m], y[s] = W[ids[s]] . x[t].
 *              gate_w != NULL: f32 [n_tok][m], y[t] = sum_j gate_w[t][j] * W[ids[t][j]] . x[t],
 *              summed in j order.
 *   1 <= top_k <= n_experts <= 65534; n_tok*top_k <= 4096 (every workgroup scans all routed
 *   slots' ids; callers with more slots split the call); k % 32 == 0.
 * With gate_w, the per-slot products go to the library's workspace first (see the workspace
 * note at the top), then the combine sums them per token.
 * Each expert's weights are streamed once per call for all tokens routed to
 * it; all arithmetic is f32 (the WQ_PATH_MATVEC bound per slot).
 */
int wq_moe_matvec(const float* x, const void* w_experts, int wtype, const int32_t* expert_ids,
                  const float* gate_w, float* y, int64_t n_tok, int64_t top_k,
                  int64_t n_experts, int64_t m, int64_t k, void* stream);

/*
 * wq_moe_matvec_noalloc: wq_moe_matvec for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same arguments,
 * checks and results (bit for bit: the same kernels). It never allocates or frees: a gated
 * call's per-slot products go to a fixed scratch array that the library holds per GPU (32 MiB,
 * kept until the process ends) instead of the grown workspace.
 *   - A gated call needs n_tok * top_k * m <= 8,388,608 (2^23 floats); a larger one returns
 *     WQ_ERR_SHAPE. Ungated calls use no scratch and have no extra limit.
 *   - Every call on a GPU shares that GPU's scratch array: calls of this entry point that overlap
 *     on one GPU (on different streams, or from several threads without ordering) race on it.
 *     Calls on one stream are ordered and safe. Nothing in the scratch must start at zero: every
 *     value the combine reads is written by the same call first.
 *   - The first call on a device looks up the array's device address (hipGetSymbolAddress).
 */
int wq_moe_matvec_noalloc(const float* x, const void* w_experts, int wtype, const int32_t* expert_ids,
                          const float* gate_w, float* y, int64_t n_tok, int64_t top_k,
                          int64_t n_experts, int64_t m, int64_t k, void* stream);

/*
 * wq_dequantize: out[m][k] = the exact f32 value of every weight (bf16: the
 * upper-half bit pattern; Q8_0: d*q; Q4_0: d*(q-8); f32 as stored; f16
 * widened; all exact in f32; Q4_K: d*sc_j*q - dmin*m_j rounded once to f32, since the
 * difference of the two exact products need not fit in f32) -- the per-type unpacking of the formats above
 * (cortiq-engine `ae_gemm`'s weight pairs, wavo `Gpu::upload_linear`, hanzo-ml
 * `upload_qweight`), written out in full so it can be compared bit for bit.
 *   w    weight in `wtype` storage, 16-byte aligned; out f32 [m][k], 16-byte aligned
 *        (written with 16-byte stores).
 */
int wq_dequantize(const void* w, int wtype, float* out, int64_t m, int64_t k, void* stream);

/*
 * wq_pad_weight: out[m][kp] = w[m][k] as exact f32 values, each row followed by kp - k zeros,
 * kp = wq_padded_k(k). wavo's load path for conv weights whose inner size is not a multiple of
 * 32 (`Gpu::upload_linear` with its `kp != k` branch, reached through `Gpu::conv`): the rows are
 * converted to f32 and zero-padded, and the layer then runs as an f32 weight of inner size kp on
 * input rows that are zero past k (wavo's im2col rows). wq_gemm itself still refuses
 * k % 32 != 0; pad once at load, then call wq_gemm(..., WQ_W_F32, ..., k = kp).
 *   w     f32, f16 or bf16 [m][k] (WQ_W_F32, WQ_W_F16, WQ_W_BF16; other types WQ_ERR_WTYPE),
 *         aligned to its element size.
 *   out   f32 [m][kp], 4-byte aligned, not overlapping w.
 *   k     1 <= k <= 2^29 - 1, any value (a multiple of 32 just copies).
 */
int wq_pad_weight(const void* w, int wtype, float* out, int64_t m, int64_t k, void* stream);

/* The inner size wq_pad_weight pads k to: the next multiple of 32 (the GEMM's k step), or -1 for
 * k outside [1, 2^29 - 1]. */
int64_t wq_padded_k(int64_t k);

/* Bytes of one m x k weight: bf16 2*m*k; Q8_0 34*m*(k/32); Q4_0 18*m*(k/32); f32 4*m*k; f16 2*m*k;
 * Q4_K 144*m*(k/256); -1 for an unknown type, negative sizes, k % 32 != 0 or (Q4_K) k % 256 != 0. The block sizes are those of the formats
 * above (wavo `Gpu::upload_linear` sizes a Q8_0 row as k/32 blocks of 34 bytes; hanzo-ml
 * `matvec_q4_0_gpu` / `matvec_q8_0_gpu` refuse a buffer shorter than the blocks of nout rows). */
int64_t wq_weight_bytes(int wtype, int64_t m, int64_t k);

/* The path wq_gemm takes for these sizes: WQ_PATH_MATVEC or WQ_PATH_MFMA
 * (negative WQ_ERR_* for invalid sizes or type, and for Q4_K with n > WQ_MATVEC_MAX_N). The pages put the split between
 * a matrix path for many rows of X (cortiq-engine `ae_gemm`, wavo `Pass::gemm`) and
 * a vector path for a few (wavo `Pass::gemv`, hanzo-ml `matvec_*_gpu`) without a
 * number; the reading taken is n <= 16 (WQ_MATVEC_MAX_N) on the f32 matvec. */
int wq_gemm_path(int64_t n, int64_t m, int64_t k, int wtype);

/* ---- the encoder block around the layer -----------------------------------------------------
 * The rest of the pre-norm block of cortiq-engine's audio encoder (src/gpu_wgpu/nemotron_audio.rs:
 * the kernels `ae_ln`, `ae_qk`, `ae_attn` and the order `AudioEncoder::run` runs them in). All
 * arithmetic is f32 except the two attention products (see wq_attention). Sizes: d = heads * hd;
 * frames n; a q/k/v row is [q | k | v] of d floats each, head h at columns h*hd .. h*hd+hd-1 of
 * each third. */

/*
 * wq_layer_norm: y[t] = (x[t] - mu) / sqrt(var + 1e-5) * w + b for each of n rows of d floats,
 * with mu the row mean and var the mean squared deviation from it (division by d) -- `ae_ln`.
 *   x   f32 [n][d], 4-byte aligned.
 *   wb  f32 [2d]: w then b (the page's packed LayerNorm weights), 4-byte aligned.
 *   y   f32 [n][d], 4-byte aligned; y == x (in place) is allowed, any other overlap with x or wb
 *       is WQ_ERR_ALIAS.
 *   n >= 0 (0: nothing to do), d >= 1, n * d <= 2^40. Rows with d % 4 == 0, d <= 4096 and x, y,
 *   wb 16-byte aligned are held in registers; others take a slower kernel, same arithmetic.
 */
int wq_layer_norm(const float* x, const float* wb, float* y, int64_t n, int64_t d, void* stream);

/*
 * wq_rope_table: the rotation table `AudioEncoder::run` builds on the host, written to host
 * memory: cs[t*(rot/2) + i] = cos(a), cs[n*(rot/2) + t*(rot/2) + i] = sin(a) with
 * a = t * (1 / 10000^(2i/rot)), every step in f32 (the page's own arithmetic; the angle is
 * rounded to f32 before its cosine is taken), frames t = 0 .. n-1.
 *   cs   host float [n * rot]; rot even, 2 <= rot; n >= 0.
 */
int wq_rope_table(float* cs, int64_t n, int64_t rot);

/*
 * wq_qk_norm_rope: in place on qkv f32 [n][3d], for each frame t and head h of q and of k (v is
 * not touched) -- `ae_qk`:
 *   1. with qn / kn given: LayerNorm of the head's hd values as wq_layer_norm, weights
 *      qn (for q) or kn (for k), each f32 [2*hd] (w then b);
 *   2. rotation of its first rot dims: for i < rot/2, with c = cs[t*(rot/2) + i] and
 *      s = cs[n*(rot/2) + t*(rot/2) + i],
 *        v'[i] = v[i]*c - v[i + rot/2]*s,   v'[i + rot/2] = v[i + rot/2]*c + v[i]*s;
 *      dims rot .. hd-1 pass through.
 *   qkv   device f32, 4-byte aligned.
 *   qn,kn device f32 [2*hd] each, or both NULL (no norm); one without the other: WQ_ERR_NULL.
 *   cs    device f32 [n * rot] (the table above, or any other); may be NULL when rot == 0.
 *   1 <= hd <= 256, heads >= 1, rot even and 0 <= rot <= hd, n >= 0.
 * qn, kn and cs must not overlap qkv (WQ_ERR_ALIAS).
 */
int wq_qk_norm_rope(float* qkv, const float* qn, const float* kn, const float* cs, int64_t n,
                    int64_t heads, int64_t hd, int64_t rot, void* stream);

/* Bytes of device workspace wq_attention needs for these sizes (bf16 copies of K and of V laid
 * out for the attention kernel, and the key mask as a bias), or -1 for invalid sizes. */
int64_t wq_attention_workspace_bytes(int64_t n, int64_t heads, int64_t hd);

/*
 * wq_attention: bidirectional attention with masked keys -- `ae_attn`. For frame t and head h:
 * scores s_j = scale * q[t,h] . k[j,h] over the keys j with valid[j] != 0, weights
 * p_j = exp(s_j - max) / sum exp(s - max), output o[t, h*hd + c] = sum_j p_j v[j,h,c].
 * Masked keys take no weight. With no valid key at all the sum of weights is 0 and every output is
 * NaN (the page's 0 * (1/0)).
 *   qkv        device f32 [n][3d] (the q/k/v rows after wq_qk_norm_rope), 4-byte aligned.
 *   valid      device int32 [n], 4-byte aligned.
 *   o          device f32 [n][d], 4-byte aligned, not overlapping qkv, valid or the workspace.
 *   workspace  device, 256-byte aligned, at least wq_attention_workspace_bytes(n, heads, hd)
 *              bytes (workspace_bytes says how many it has; fewer: WQ_ERR_SHAPE). Overwritten.
 *   scale      finite; the page's is 1/sqrt(hd) in f32.
 *   1 <= hd <= 128, 1 <= heads <= 4096, 0 <= n <= 2^22.
 * Arithmetic: q, k and v are rounded to bf16 (nearest even) and both products run on the bf16
 * matrix cores with f32 accumulation; the softmax runs in f32 (base-2 exponentials of scores
 * pre-multiplied by scale*log2(e)), and the weights are rounded to bf16 for the second product,
 * normalised by the sum of the rounded weights. The page's kernel keeps q, k and v in f32; the
 * error bound this gives is stated with the tests.
 */
int wq_attention(const float* qkv, const int32_t* valid, float* o, void* workspace,
                 int64_t workspace_bytes, int64_t n, int64_t heads, int64_t hd, float scale,
                 void* stream);

/* One pre-norm block's weights (`AeLayerDesc` on the page). Weight matrices are in the layer's
 * storage type (wq_encoder_layer's wtype) and 16-byte aligned; vectors are f32, 4-byte aligned. */
typedef struct wq_encoder_layer {
  const float* ln1;   /* [2d] LayerNorm before attention: w then b */
  const void* qkv_w;  /* [3d][d] fused q/k/v weights */
  const float* qkv_b; /* [3d] or NULL (the page's block has no q/k/v bias) */
  const float* qn;    /* [2*hd] q LayerNorm, or NULL (then kn is NULL too: no q/k norm) */
  const float* kn;    /* [2*hd] k LayerNorm, or NULL */
  const void* out_w;  /* [d][d] output projection */
  const float* out_b; /* [d] */
  const float* ln2;   /* [2d] LayerNorm before the MLP */
  const void* fc1_w;  /* [inter][d] */
  const float* fc1_b; /* [inter] */
  const void* fc2_w;  /* [d][inter] */
  const float* fc2_b; /* [d] */
} wq_encoder_layer_t;

/* Bytes of device workspace wq_encoder_layer needs (its activations a, qkv, att and f, and the
 * attention workspace), or -1 for invalid sizes. */
int64_t wq_encoder_workspace_bytes(int64_t n, int64_t d, int64_t heads, int64_t inter);

/*
 * wq_encoder_layer: one block of `AudioEncoder::run`, in place on h f32 [n][d]:
 *   a = LayerNorm(h; ln1);  qkv = a . qkv_w^T (+ qkv_b);  wq_qk_norm_rope(qkv; qn, kn, cs);
 *   att = wq_attention(qkv, valid, scale = 1/sqrt(hd) in f32);
 *   h = h + att . out_w^T + out_b;  a = LayerNorm(h; ln2);
 *   f = GELU(a . fc1_w^T + fc1_b);  h = h + f . fc2_w^T + fc2_b.
 * The products are wq_linear calls on `path` (WQ_PATH_AUTO, WQ_PATH_MFMA or WQ_PATH_MFMA_F32).
 *   h          device f32 [n][d], 16-byte aligned.
 *   valid, cs  as for wq_attention / wq_qk_norm_rope (cs [n * rot]).
 *   workspace  device, 256-byte aligned, >= wq_encoder_workspace_bytes(n, d, heads, inter).
 *   d % 32 == 0, inter % 32 == 0, d % heads == 0 with hd = d / heads <= 128, rot as for
 *   wq_qk_norm_rope, 0 <= n <= 2^22.
 * Every step's argument checks run before the first launch, so a refused call leaves h as it
 * was. The layer's weights and vectors, valid and cs must not overlap h or the workspace
 * (WQ_ERR_ALIAS). Only a launch that fails (WQ_ERR_HIP) returns with h partly updated.
 */
int wq_encoder_layer(const wq_encoder_layer_t* layer, int wtype, float* h, const int32_t* valid,
                     const float* cs, void* workspace, int64_t workspace_bytes, int64_t n, int64_t d,
                     int64_t heads, int64_t rot, int64_t inter, int path, void* stream);

/* Message of the last failed call on this thread ("" when none): the text of the
 * checks above, in the manner of the messages hanzo-ml's host functions return
 * on a refused call (`bail!` with the offending sizes). */
const char* wq_last_error(void);

/* Library version string. */
const char* wq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
