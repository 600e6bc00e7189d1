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

// ---- cross-lane maxima of non-negative f32 values without LDS round trips: DPP row
// permutations inside 16-lane rows, one bit-mode swizzle across the two rows of a 32-lane half.
// For non-negative floats the unsigned order of the bit patterns is the numeric order, so the
// maxima run as integer maxima (no NaN canonicalization, and the DPP move folds into the max).
// Lanes whose DPP source is unavailable read 0, which leaves the maximum unchanged.
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;  // lane i <- 15 - i within a row of 16
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <- 7 - i within each 8 lanes

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
  return v > o ? v : o;
}

// max over each aligned group of 8 lanes (v >= 0)
__device__ __forceinline__ float max8_nonneg(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  u = dpp_umax<DPP_XOR1>(u);
  u = dpp_umax<DPP_XOR2>(u);
  u = dpp_umax<DPP_HALF_MIRROR>(u);  // quad 0 <-> quad 1 of the 8
  return __builtin_bit_cast(float, u);
}

// max over each aligned group of 32 lanes (v >= 0)
__device__ __forceinline__ float max32_nonneg(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, max8_nonneg(v));
  u = dpp_umax<DPP_ROW_MIRROR>(u);  // 8-lane halves of a row
  // ds_swizzle bit mode (offset bit 15 = 0): lane <- ((lane & 0x1F) | 0) ^ 0x10 within 32 lanes
  const uint32_t o = (uint32_t)__builtin_amdgcn_ds_swizzle((int)u, 0x401F);
  return __builtin_bit_cast(float, u > o ? u : o);
}

// f32(m / 127), correctly rounded, from one f64 product.  The f64 result is within 2^-52
// (relative) of m/127, while m/127 for an f32 m is never closer than about 2^-32 (relative) to a
// rounding midpoint of the f32 grid (m - 127*midpoint is a nonzero multiple of the midpoint
// spacing), so rounding the f64 value to f32 gives the correctly rounded quotient.
__device__ __forceinline__ float div127_f32(float m) { return (float)((double)m * (1.0 / 127.0)); }

// f32(1 / d), correctly rounded, for an f32 d != 0: the hardware f64 reciprocal refined by two
// Newton steps (error below 2^-52 relative), rounded to f32; 1/d is never closer than 2^-46
// (relative) to an f32 rounding midpoint, so the result equals the IEEE f32 division.
__device__ __forceinline__ float recip_f32(float d) {
  const double x = d;
  double r = __builtin_amdgcn_rcp(x);
  r = fma(r, fma(-x, r, 1.0), r);
  r = fma(r, fma(-x, r, 1.0), r);
  return (float)r;
}

// Q8_0 of one block of 32 f32 values spread over 8 consecutive lanes (lane group
// aligned to 8), 4 consecutive values per lane.  amax exact; d = f32(amax/127);
// id = f32(1/d) or 0; code = round half away from zero of f32(x*id), clamped.
// Returns the 4 codes packed little-endian; d_out = f32 scale (before fp16).
__device__ __forceinline__ int q8_code(float x, float id) {
  float r = roundf(x * id);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

__device__ __forceinline__ uint32_t q8_block_quant4(float4 v, float& d_out) {
  float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  m = max8_nonneg(m);
  const float d = div127_f32(m);
  const float id = (d != 0.0f) ? recip_f32(d) : 0.0f;
  d_out = d;
  return (uint32_t)(uint8_t)q8_code(v.x, id) | ((uint32_t)(uint8_t)q8_code(v.y, id) << 8) |
         ((uint32_t)(uint8_t)q8_code(v.z, id) << 16) | ((uint32_t)(uint8_t)q8_code(v.w, id) << 24);
}

// ---- e^x and SiLU in f64: the softmax of the attention node and the activation of the SwiGLU
// node, silu(g) = g / (1 + e^-g).  e^x by Tang's table-driven method: x = (64k + j) ln2/64 + r
// with |r| <= ln2/128, so e^x = 2^k * 2^(j/64) * e^r; e^r from its degree-5 Taylor polynomial
// (truncation below 4e-17 relative).  ln2/64 is split into a 36-bit head (k * head exact for
// |64k + j| < 2^17) and a tail.  Quotients use the f64 reciprocal with two Newton steps.  Error: a
// few f64 ulps, far below the f32 rounding the callers apply.  `tab` holds 2^(j/64), j = 0..63
// (exp2_table_fill, in LDS).
__device__ __forceinline__ void exp2_table_fill(double* tab, int tid) {
  if (tid < 64) tab[tid] = exp2((double)tid * (1.0 / 64.0));
}

// e^x for x <= 709 (x below -745 gives 0 or a subnormal), from the 2^(j/64) table `tab`.
__device__ __forceinline__ double exp_f64(double x, const double* tab) {
  constexpr double INV_LN2_64 = 0x1.71547652b82fep+6;   // 64 / ln2
  constexpr double LN2_64_HI = 0x1.62e42fefa0000p-7;    // ln2/64, first 36 bits
  constexpr double LN2_64_LO = 0x1.cf79abc9e3b3ap-46;   // ln2/64 - LN2_64_HI
  x = fmin(fmax(x, -746.0), 709.0);
  const double kf = rint(x * INV_LN2_64);
  double r = fma(-kf, LN2_64_HI, x);
  r = fma(-kf, LN2_64_LO, r);
  const double p = fma(fma(fma(fma(fma(1.0 / 120.0, r, 1.0 / 24.0), r, 1.0 / 6.0), r, 0.5), r, 1.0), r, 1.0);
  const int k = (int)kf;
  return ldexp(tab[k & 63] * p, k >> 6);
}

// 1/x for x >= 1 (or any normal x): hardware f64 reciprocal plus two Newton steps.
__device__ __forceinline__ double recip_f64(double x) {
  double rc = __builtin_amdgcn_rcp(x);
  rc = fma(rc, fma(-x, rc, 1.0), rc);
  return fma(rc, fma(-x, rc, 1.0), rc);
}

__device__ __forceinline__ double silu_f64(double g, const double* tab) {
  // e^-g overflows past 709.78 (silu(g) is then -0 or a tiny negative that rounds to 0 in f32)
  // and underflows below -745 (silu(g) = g): exp_f64's clamp keeps every step finite
  return g * recip_f64(1.0 + exp_f64(-g, tab));
}

// SwiGLU of one element: f32(silu(g) * u), silu and the product in f64.
__device__ __forceinline__ float swiglu_f32(float g, float u, const double* tab) {
  return (float)(silu_f64((double)g, tab) * (double)u);
}

// ------------------------------------------------------------------ launchers (internal)
// All take device pointers, assume validated shapes, launch on `s`.
int launch_quantize(const float* x, int64_t rows, int cols, int64_t ld_x, int8_t* codes,
                    uint16_t* scales, hipStream_t s);
// canonical 34-byte Q8_0 blocks (fp16 scale bits, 32 codes) -> the two planes; codes 16-byte aligned
int launch_pack_q8_0(const void* blocks, int64_t rows, int cols, int8_t* codes, uint16_t* scales, hipStream_t s);
// x [rows][cols]; with n_split > 1, x += f32(sum of the split-K partials [n_split][rows][cols]) first
// (written back), as the deferred reduction of the matmul that produced them.
int launch_rmsnorm_quant(float* x, const float* gamma, int64_t rows, int cols, float eps,
                         int8_t* codes, uint16_t* scales, float* y, hipStream_t s,
                         const double* partial = nullptr, int n_split = 0);
int launch_swiglu_quant(const float* gate, const float* up, int64_t rows, int cols, int64_t ld_in,
                        int8_t* codes, uint16_t* scales, hipStream_t s);
int launch_embed(const int8_t* codes, const uint16_t* scales, int cols, const int32_t* ids, int n,
                 float* out, hipStream_t s);
// bytes (a multiple of 4) from a pinned host buffer to device memory, read by a kernel
int launch_stage_in(void* dst, const void* host_src, size_t bytes, hipStream_t s);
// out[r] = x[rows[r]] for r < n (rows of cols floats; rows: device int32 [n])
int launch_gather_rows(const float* x, int cols, const int32_t* rows, int n, float* out, hipStream_t s);
int launch_qk_norm(float* x, int64_t ld, const float* gamma, int64_t rows, int n_heads, int head_dim,
                   float eps, hipStream_t s);
int launch_rope_kvstore(float* q, int64_t ld_q, const float* k, const float* v, int64_t ld_kv,
                        const int32_t* pos, int n_tokens, int n_head, int n_head_kv, int head_dim,
                        const double* table, float* k_region, float* v_region, hipStream_t s);
// out f32 [n_tokens][ld_out], or, with q_codes non-null, the output rows quantized to Q8_0
// (codes [n_tokens][n_head*head_dim], scales [n_tokens][n_head*head_dim/32]) and out unused.
// max_pos: the call's largest position, read from device memory when max_pos_dev is non-null.
// One query tile of a call with several sequences: rows t0 .. t0+count-1 (count <= 16) of one
// sequence, whose regions and largest position these are.
struct AttnSlotTile {
  const float* k_region;
  const float* v_region;
  int t0, count, max_pos, pad;
};
// tiles: device [n_tiles] (several sequences; n_tokens is then the total row count), or null
int launch_attention(const float* q, int64_t ld_q, const float* k_region, const float* v_region,
                     const int32_t* pos, int n_tokens, const int32_t* max_pos_dev, int max_pos, int n_head, int n_head_kv,
                     int head_dim, float* out, int64_t ld_out, hipStream_t s,
                     int8_t* q_codes = nullptr, uint16_t* q_scales = nullptr, const AttnSlotTile* tiles = nullptr,
                     int n_tiles = 0);

// Exact Q8_0 GEMM.  Epilogue modes:
enum GemmEpi { EPI_F32 = 0, EPI_SWIGLU_Q8 = 1, EPI_QKV = 2 };

// EPI_QKV: the stacked Q|K|V matmul of a layer finishes the attention inputs in its epilogue:
// [per-head QK RMSNorm] and NeoX RoPE of the Q and K heads, Q written to `out`, rotated K and raw
// V stored into the layer's regions at row pos[t].  Every head lies inside one tile.
struct QkvEpi {
  const int32_t* pos;      // device [m]
  const double* rope;      // device [n_ctx][head_dim/2] of (cos, sin)
  int n_q, n_kv, head_dim; // Q columns, K (= V) columns, head size
  float* k_region;         // device [n_ctx][n_kv]
  float* v_region;
  // several sequences in one call: row t stores into the regions of slot slot_of_row[t]
  // (k_slots / v_slots: device arrays of region pointers); null = the one region above
  const int32_t* slot_of_row;
  float* const* k_slots;
  float* const* v_slots;
  const float* q_norm;     // [head_dim] gains of the QK norm, or null (no QK norm)
  const float* k_norm;
  float eps;
};
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
  // EPI_F32 only: when split K is used, leave the f64 partials [split][m][n] in workspace
  // and skip the reduction (the consumer reduces them); *split_out receives the split (1 = none)
  int* split_out;
  QkvEpi qkv;             // EPI_QKV parameters (used when qkv.pos is non-null)
};
int launch_gemm_q8(const GemmArgs& a, hipStream_t s);
size_t gemm_workspace_bytes(int m, int n, int k);
// the current device's address of the library's static scratch array (MI_STATIC_SCRATCH_BYTES)
int static_scratch(void** ptr);
int launch_lm_head(const int8_t* xq, const uint16_t* xs, int cols, const int8_t* w_codes,
                   const uint16_t* w_scales, int rows, float* logits, hipStream_t s);

// ---- decode step (one activation row): exact Q8_0 matrix-vector products and single-query attention
enum GemvEpi { GV_RES = 0, GV_F32 = 1, GV_SWIGLU = 3 };
// the one-row kernels stage their Q8_0 input row in LDS (K codes + K/32 f64 scales, 64 KB at most)
constexpr int GV_MAX_K = 49152;
struct GemvArgs {
  // input row: with x non-null, RMSNorm(x; gamma, eps) + Q8_0 inside the kernel; else xq/xs
  const float* x; const float* gamma; float eps;
  const int8_t* xq; const uint16_t* xs;
  int k;
  const int8_t* w_codes; const uint16_t* w_scales; int n;   // weights [n][k]
  const float* bias;                                         // GV_F32: [n] or null
  const float* residual; float* out;                         // GV_RES: out = residual + y; GV_F32: out = y
  int8_t* q_codes; uint16_t* q_scales;                       // GV_SWIGLU: Q8_0 [n/2]
  int epi;
};
int launch_gemv_q8(const GemvArgs& g, hipStream_t s);
// attention of one query per head over keys 0..*pos_dev: partial states per key range in `part`
// (n_head * n_range * (head_dim + 2) f64, n_range <= AD_MAX_RANGES), merged by launch_attn_merge
constexpr int AD_MAX_RANGES = 64;
int attn_decode_ranges(int n_ctx, int* keys_per_range);
// With `fin` (the decode step), q is the raw Q|K|V row: the per-head QK norm and RoPE at *pos_dev are
// applied in the kernel, and the new K and V rows are stored at row *pos_dev of the regions.
// Without it, q holds finished queries and the regions hold row *pos_dev already.
struct AttnFinish {
  const double* rope;  // [rows][head_dim / 2] (cos, sin)
  const float* q_norm; const float* k_norm;  // per-head RMSNorm weights, or null
  float eps;
};
int launch_attn_decode(const float* q, float* k_region, float* v_region, const int32_t* pos_dev, int n_ctx,
                       int n_head, int n_head_kv, int head_dim, double* part, const AttnFinish* fin, hipStream_t s);
// the ranges of `part` merged per head, normalized and quantized: the Q8_0 row [n_head * head_dim]
int launch_attn_merge(const double* part, int n_ctx, const int32_t* pos_dev, int n_head, int head_dim, int8_t* codes,
                      uint16_t* scales, hipStream_t s);

// ---- sampler (sampler.hip)
size_t sampler_workspace_bytes();
// window: host ids [n_window <= 64], passed to the kernel by value
int launch_sample(const float* logits, int vocab, const int32_t* window, int n_window, const mi_sampler_params& p,
                  uint64_t seed, uint64_t step, void* workspace, int32_t* token_out, hipStream_t s);

}  // namespace mi
