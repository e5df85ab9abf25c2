// Internal interface between the host API (wq_api.cpp) and the kernel files.
// Not installed; the public ABI is include/wq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

enum WType : int { kBF16 = 0, kQ8_0 = 1, kQ4_0 = 2, kF32 = 3, kF16 = 4, kQ4_K = 5 };

// Bytes of one 32-element block in each storage type (bf16, f16: 32 x 2 bytes; f32: 32 x 4).
// Q4_K is stored in 256-element super-blocks (kQ4KBytes each): 18 bytes per 32 elements on
// average, but its 32-element sub-blocks are not self-contained, so only the Q4_K kernels read it.
__host__ __device__ constexpr int block_bytes(int wt) {
  return wt == kBF16 || wt == kF16 ? 64 : wt == kF32 ? 128 : wt == kQ8_0 ? 34 : 18;
}
constexpr int kQ4KElems = 256;  // weights per Q4_K super-block
constexpr int kQ4KBytes = 144;  // bytes per Q4_K super-block

// Types stored value by value (no per-block scale): bf16, f16, f32.
__host__ __device__ constexpr bool plain_type(int wt) { return wt == kBF16 || wt == kF16 || wt == kF32; }

// Exact bf16 parts one weight splits into on the matrix cores: bf16 and the integer quants 1,
// f16 2 (11 significant bits), f32 3 (24 bits).
__host__ __device__ constexpr int weight_parts(int wt) { return wt == kF32 ? 3 : wt == kF16 ? 2 : 1; }

// ---- matvec / MoE (f32 FMA path) ---------------------------------------------------------------
struct MatvecParams {
  const float* x;           // activations, rows of k floats
  const uint8_t* w;         // weight, or the first expert of a bank
  long long expert_bytes;   // byte distance between experts (0 for a single weight)
  const float* bias;        // [m] or null
  float* y;                 // outputs, rows of m floats
  const int32_t* ids;       // MoE: expert of each slot; null for the plain layer
  int n_slots;              // plain: rows of x (<= 16); MoE: n_tok * top_k
  int top_k;                // MoE: slots per token (x row of slot s = s / top_k); plain: 1
  int n_exp;                // experts in the bank (plain: 1)
  int m, k;
  long long rowbytes;       // bytes of one weight row
  unsigned flags;           // epilogue flags (plain layer only)
  float alpha;              // factor on the activated value (plain layer only)
  int ystride;              // floats from one row of y to the next: m + dual (MoE: m); the sliced
                            // and matrix-core kernels take only dual == 0 (stride m)
  int dual;                 // plain layer: outputs 0..dual-1 stored again at m + j (bias[m + j])
  int moe_compact;          // MoE: 1 when the grid is dealt over the touched experts (wq_moe_sched.hpp)
};

// Picks the kernel variant (tokens per pass, rows per wave) and launches it.
// For MoE (ids != null) the grid has one extra expert row that writes NaN for
// slots whose id is out of range.
hipError_t launch_matvec(int wtype, const MatvecParams& p, int max_tokens_per_expert,
                         hipStream_t stream);

// The sliced kernel (k a multiple of 1024, at most 8192), which launch_matvec
// prefers when it applies; the general kernel takes every other k.
bool matvec_sliced_supports(int k);
hipError_t launch_matvec_sliced(int wtype, const MatvecParams& p, int max_tokens_per_expert,
                                hipStream_t stream);

// The matrix-core kernel for 2..16 tokens per pass and MoE (Q8_0 / Q4_0, k a multiple of 512
// in 2048..4096), which launch_matvec prefers when it applies.
bool matvec_mfma_supports(int wtype, int k);
// Whether a plain call (no ids) of n tokens on m rows goes to the matrix-core kernel: from 9
// tokens, and from 5 when the weight has at least two 16-row tiles per CU (three for Q4_K).
bool matvec_mfma_takes_plain(int wtype, int m, int n);
hipError_t launch_matvec_mfma(int wtype, const MatvecParams& p, hipStream_t stream);

// Q4_K weights (k a multiple of 256): the sliced kernel where it applies (no dual outputs), else
// the Q4_K general kernel (wq_matvec_q4k.hip). launch_matvec sends Q4_K here.
hipError_t launch_matvec_q4k(const MatvecParams& p, int max_tokens_per_expert, hipStream_t stream);
hipError_t launch_dequantize_q4k(const uint8_t* w, float* out, int m, int k, hipStream_t stream);

// y[t][j] = sum_s gate[t*top_k + s] * slots[(t*top_k + s)][j], summed in s order.
hipError_t launch_moe_combine(const float* slots, const float* gates, float* y, int n_tok,
                              int top_k, int m, hipStream_t stream);

// out[m][k] = exact f32 value of every weight.
hipError_t launch_dequantize(int wtype, const uint8_t* w, float* out, int m, int k,
                             hipStream_t stream);

// out[m][kp] f32 = w[m][k] (f32, f16 or bf16) decoded and zero-padded to kp columns.
hipError_t launch_pad_weight(int wtype, const uint8_t* w, float* out, long long m, int k, int kp,
                             hipStream_t stream);

// ---- MFMA GEMM ---------------------------------------------------------------------------------
struct GemmParams {
  const float* x;     // [n][k]
  const uint8_t* w;   // [m][k] in storage type
  const float* bias;  // [m] or null
  float* y;           // [n][m]
  int n, m, k;
  long long rowbytes;
  unsigned flags;
  float alpha;        // factor on the activated value, before the old output is added
  int ystride;        // floats from one row of y to the next: m + dual
  int dual;           // outputs 0..dual-1 stored again at columns m + j, with bias[m + j]
  int x_parts;        // 3: X enters as three exact bf16 parts (three MFMAs per product); 1: as bf16(X)
  int x_bf16;         // 1: x holds bf16 bit patterns [n][k] (already rounded; bf16 weights, x_parts 1)
  int y_bf16;         // 1: y receives bf16 bit patterns [n][ystride], each output rounded to nearest
                      // even (bf16 weights, no residual, no dual outputs)
};

hipError_t launch_gemm(int wtype, const GemmParams& p, hipStream_t stream);

// ---- encoder block (wq_encoder.hip) ---------------------------------------------------------
hipError_t launch_layer_norm(const float* x, const float* wb, float* y, int n, int d, hipStream_t stream);
// The same with y as bf16 bit patterns (8-byte aligned for the vector kernel), each output rounded to
// nearest even: the encoder block's input to a product that rounds it so anyway.
hipError_t launch_layer_norm_bf16(const float* x, const float* wb, uint16_t* y, int n, int d, hipStream_t stream);
hipError_t launch_qk_norm_rope(float* qkv, const float* qn, const float* kn, const float* cs, int n, int heads,
                               int hd, int rot, hipStream_t stream);
long long attention_workspace_bytes(long long n, long long heads, long long hd);
hipError_t launch_attention(const float* qkv, const int32_t* valid, float* o, void* ws, int n, int heads, int hd,
                            float scale, hipStream_t stream);
// q/k norm + rotation fused with the attention's pack (k is not written back to qkv), then the
// attention: the block's path. Same workspace as launch_attention. o_bf16: o receives bf16 bit
// patterns (rounded to nearest even) instead of f32.
hipError_t launch_qk_attention(float* qkv, const float* qn, const float* kn, const float* cs, const int32_t* valid,
                               void* o, void* ws, int n, int heads, int hd, int rot, float scale,
                               hipStream_t stream, int o_bf16);

}  // namespace wq
