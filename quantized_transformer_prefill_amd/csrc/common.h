// Internal declarations shared by the HIP sources of the Q8_0 prefill library.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/mi_prefill.h"

namespace mi {

// ------------------------------------------------------------------ errors
int set_error(int code, const char* fmt, ...);
int hip_check(hipError_t e, const char* what);

#define MI_HIP(call)                                          \
  do {                                                        \
    hipError_t e_ = (call);                                   \
    if (e_ != hipSuccess) return ::mi::hip_check(e_, #call);  \
  } while (0)

#define MI_LAUNCH_CHECK(name)                                 \
  do {                                                        \
    hipError_t e_ = hipGetLastError();                        \
    if (e_ != hipSuccess) return ::mi::hip_check(e_, name);   \
  } while (0)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ------------------------------------------------------------------ device helpers
constexpr int QK = 32;  // values per Q8_0 block

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  _Float16 h = (_Float16)v;  // v_cvt_f16_f32: round to nearest even, subnormals kept
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// Q8_0 of one block of 32 f32 values spread over 8 consecutive lanes (lane group
// aligned to 8), 4 consecutive values per lane.  amax exact; d = f32(amax/127);
// id = f32(1/d) or 0; code = round half away from zero of f32(x*id), clamped.
// Returns the 4 codes packed little-endian; d_out = f32 scale (before fp16).
__device__ __forceinline__ uint32_t q8_block_quant4(float4 v, float& d_out) {
  float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  m = fmaxf(m, __shfl_xor(m, 1));
  m = fmaxf(m, __shfl_xor(m, 2));
  m = fmaxf(m, __shfl_xor(m, 4));
  const float d = m / 127.0f;
  const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
  auto code = [&](float x) -> uint32_t {
    float r = roundf(x * id);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (uint32_t)(uint8_t)(int8_t)(int)r;
  };
  d_out = d;
  return code(v.x) | (code(v.y) << 8) | (code(v.z) << 16) | (code(v.w) << 24);
}

// ------------------------------------------------------------------ launchers (internal)
// All take device pointers, assume validated shapes, launch on `s`.
int launch_quantize(const float* x, int64_t rows, int cols, int64_t ld_x, int8_t* codes,
                    uint16_t* scales, hipStream_t s);
int launch_rmsnorm_quant(const float* x, const float* gamma, int64_t rows, int cols, float eps,
                         int8_t* codes, uint16_t* scales, float* y, hipStream_t s);
int launch_swiglu_quant(const float* gate, const float* up, int64_t rows, int cols, int64_t ld_in,
                        int8_t* codes, uint16_t* scales, hipStream_t s);
int launch_embed(const int8_t* codes, const uint16_t* scales, int cols, const int32_t* ids, int n,
                 float* out, hipStream_t s);
int launch_qk_norm(float* x, int64_t ld, const float* gamma, int64_t rows, int n_heads, int head_dim,
                   float eps, hipStream_t s);
int launch_rope_kvstore(float* q, int64_t ld_q, const float* k, const float* v, int64_t ld_kv,
                        const int32_t* pos, int n_tokens, int n_head, int n_head_kv, int head_dim,
                        const double* table, float* k_region, float* v_region, hipStream_t s);
int launch_attention(const float* q, int64_t ld_q, const float* k_region, const float* v_region,
                     const int32_t* pos, int n_tokens, int max_pos, int n_head, int n_head_kv,
                     int head_dim, float* out, int64_t ld_out, hipStream_t s);

// Exact Q8_0 GEMM.  Epilogue modes:
enum GemmEpi { EPI_F32 = 0, EPI_SWIGLU_Q8 = 1 };
struct GemmArgs {
  const int8_t* a_codes; const uint16_t* a_scales; int m;   // activations [m][k]
  const int8_t* w_codes; const uint16_t* w_scales; int n;   // weights [n][k]
  int k;
  const float* bias;      // [n] or null (EPI_F32)
  const float* residual;  // [m][ld_out] or null (EPI_F32)
  float* out; int64_t ld_out;                                // EPI_F32 output
  int8_t* q_codes; uint16_t* q_scales;                       // EPI_SWIGLU_Q8 output [m][n/2]
  void* workspace; size_t workspace_bytes;                   // split-K partials
  int split_k;            // 0 = choose
};
int launch_gemm_q8(const GemmArgs& a, hipStream_t s);
size_t gemm_workspace_bytes(int m, int n, int k);
int launch_lm_head(const int8_t* xq, const uint16_t* xs, int cols, const int8_t* w_codes,
                   const uint16_t* w_scales, int rows, float* logits, hipStream_t s);

}  // namespace mi
