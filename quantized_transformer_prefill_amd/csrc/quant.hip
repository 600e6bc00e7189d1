// Elementwise and row-wise kernels that end in (or feed) Q8_0:
//   quantize, RMSNorm + quantize, SwiGLU + quantize, embedding rows, per-head QK RMSNorm.
//
// Every kernel reads each input element once and writes each output once, with
// 16-byte accesses laid out so that consecutive lanes touch consecutive addresses
// (these kernels are HBM-bound).  Floating-point node math runs in f64 and rounds
// once to f32; the Q8_0 step is the bit-exact f32 quantizer of common.h.
#include <algorithm>

#include "common.h"

namespace mi {

// ---------------------------------------------------------------- plain quantizer
// One lane per 4 values; 8 lanes per Q8_0 block; flat grid over all float4 of the
// matrix (cols % 32 == 0 so a block never straddles rows).
__global__ void __launch_bounds__(256) k_quantize(const float* __restrict__ x, int64_t rows, int cols,
                                                  int64_t ld_x, int8_t* __restrict__ codes,
                                                  uint16_t* __restrict__ scales) {
  const int64_t nvec_row = cols / 4;
  const int64_t total = rows * nvec_row;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total + 0; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nvec_row, c4 = i - r * nvec_row;
    const float4 v = *reinterpret_cast<const float4*>(x + r * ld_x + c4 * 4);
    float d;
    const uint32_t q = q8_block_quant4(v, d);
    reinterpret_cast<uint32_t*>(codes + r * cols)[c4] = q;
    if ((c4 & 7) == 0) scales[r * (cols / QK) + c4 / 8] = f32_to_f16_bits(d);
  }
}

// ---------------------------------------------------------------- canonical blocks -> planes
// One thread per 34-byte block (fp16 scale bits, then 32 codes; 2-byte aligned): 17 two-byte
// loads, the scale to its plane, the codes as two 16-byte stores (code rows are 32-byte multiples).
__global__ void __launch_bounds__(256) k_pack_q8_0(const uint16_t* __restrict__ blocks, int64_t n_blocks,
                                                   int8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < n_blocks; b += (int64_t)gridDim.x * blockDim.x) {
    const uint16_t* src = blocks + b * 17;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = (uint32_t)src[1 + 2 * i] | ((uint32_t)src[2 + 2 * i] << 16);
    scales[b] = src[0];
    uint4* dst = reinterpret_cast<uint4*>(codes + b * QK);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

int launch_pack_q8_0(const void* blocks, int64_t rows, int cols, int8_t* codes, uint16_t* scales, hipStream_t s) {
  const int64_t n_blocks = rows * (cols / QK);
  const int64_t wg = std::min<int64_t>((n_blocks + 255) / 256, 65536);
  hipLaunchKernelGGL(k_pack_q8_0, dim3((unsigned)wg), dim3(256), 0, s, reinterpret_cast<const uint16_t*>(blocks),
                     n_blocks, codes, scales);
  MI_LAUNCH_CHECK("k_pack_q8_0");
  return MI_OK;
}

// The shuffle inside q8_block_quant4 needs all 8 lanes of a block active, so grid-stride
// loops must keep whole lane groups together: total % 8 == 0 always holds (cols % 32 == 0)
// and the stride is a multiple of 64, so a group is either fully in range or fully out.

int launch_quantize(const float* x, int64_t rows, int cols, int64_t ld_x, int8_t* codes,
                    uint16_t* scales, hipStream_t s) {
  if (rows == 0) return MI_OK;
  const int64_t total = rows * (cols / 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)blocks), dim3(256), 0, s, x, rows, cols, ld_x, codes, scales);
  MI_LAUNCH_CHECK("k_quantize");
  return MI_OK;
}

// ---------------------------------------------------------------- block reductions
__device__ __forceinline__ double wave_sum_f64(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ---------------------------------------------------------------- RMSNorm + quantize
// One workgroup per row.  y = f32(x / sqrt(mean(x^2) + eps) * gamma) with the mean, sqrt,
// reciprocal and gain in f64; then Q8_0 per 32-block.  A row of up to NV float4 per thread is held
// in registers between the two passes, indexed only by unrolled (compile-time) loop counters so it
// stays in VGPRs; the gains are requested together with the row.  Longer rows take the NV = 0
// variant, which reads the row again in the second pass.
//
// Pending split-K partials (partial != null): the row first becomes
// x + f32(sum_z partial[z][r]) (the residual add of the matmul that produced the partials, summed
// in the fixed order z = 0..n_split-1 exactly as the split-K reduction would), which is written
// back to x before the norm.
constexpr int RN_THREADS = 256;

template <int NV>
__global__ void __launch_bounds__(RN_THREADS) k_rmsnorm_quant(float* __restrict__ x,
                                                             const float* __restrict__ gamma, int cols,
                                                             float eps, int8_t* __restrict__ codes,
                                                             uint16_t* __restrict__ scales,
                                                             float* __restrict__ y_out,
                                                             const double* __restrict__ partial, int n_split,
                                                             int64_t rows) {
  __shared__ double sh[RN_THREADS / 64];
  const int64_t r = blockIdx.x;
  float* xr = x + r * cols;
  const int nvec = cols / 4;
  auto load = [&](int c4) -> float4 {
    float4 v = reinterpret_cast<const float4*>(xr)[c4];
    if (partial) {
      double a = 0.0, b = 0.0, c = 0.0, d = 0.0;
      for (int z = 0; z < n_split; ++z) {
        const double* pz = partial + ((int64_t)z * rows + r) * cols + 4 * c4;
        const double2 p0 = reinterpret_cast<const double2*>(pz)[0];
        const double2 p1 = reinterpret_cast<const double2*>(pz)[1];
        a += p0.x; b += p0.y; c += p1.x; d += p1.y;
      }
      v.x = v.x + (float)a; v.y = v.y + (float)b; v.z = v.z + (float)c; v.w = v.w + (float)d;
      reinterpret_cast<float4*>(xr)[c4] = v;
    }
    return v;
  };
  auto sq = [](float4 v) {
    const double a = v.x, b = v.y, c = v.z, d = v.w;
    return a * a + b * b + c * c + d * d;
  };
  // rows are a multiple of 32 values; lane groups of 8 cover one block, and all 8 lanes of a group
  // are in or out of range together, so the cross-lane maxima see a full group
  auto emit = [&](int c4, float4 v, float4 g, double inv_rms) {
    float4 o;
    o.x = (float)((double)v.x * inv_rms * (double)g.x);
    o.y = (float)((double)v.y * inv_rms * (double)g.y);
    o.z = (float)((double)v.z * inv_rms * (double)g.z);
    o.w = (float)((double)v.w * inv_rms * (double)g.w);
    if (y_out) reinterpret_cast<float4*>(y_out + r * cols)[c4] = o;
    float d;
    const uint32_t q = q8_block_quant4(o, d);
    reinterpret_cast<uint32_t*>(codes + r * cols)[c4] = q;
    if ((c4 & 7) == 0) scales[r * (cols / QK) + c4 / 8] = f32_to_f16_bits(d);
  };
  const float4* g4 = reinterpret_cast<const float4*>(gamma);
  double ss = 0.0;
  float4 keep[NV > 0 ? NV : 1], gk[NV > 0 ? NV : 1];
  if constexpr (NV > 0) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int c4 = threadIdx.x + j * RN_THREADS;
      if (c4 < nvec) {
        keep[j] = load(c4);
        gk[j] = g4[c4];
      }
    }
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (threadIdx.x + j * RN_THREADS < nvec) ss += sq(keep[j]);
  } else {
    for (int c4 = threadIdx.x; c4 < nvec; c4 += RN_THREADS) ss += sq(load(c4));
  }
  // the row's sum: wave sums, then every thread adds the 4 wave sums in a fixed order
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = ss;
  __syncthreads();
  double total = 0.0;
#pragma unroll
  for (int w = 0; w < RN_THREADS / 64; ++w) total += sh[w];
  const double inv_rms = recip_f64(sqrt(total / (double)cols + (double)eps));
  if constexpr (NV > 0) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int c4 = threadIdx.x + j * RN_THREADS;
      if (c4 < nvec) emit(c4, keep[j], gk[j], inv_rms);
    }
  } else {
    for (int c4 = threadIdx.x; c4 < nvec; c4 += RN_THREADS)
      emit(c4, reinterpret_cast<const float4*>(xr)[c4], g4[c4], inv_rms);
  }
}

int launch_rmsnorm_quant(float* x, const float* gamma, int64_t rows, int cols, float eps,
                         int8_t* codes, uint16_t* scales, float* y, hipStream_t s, const double* partial,
                         int n_split) {
  if (rows == 0) return MI_OK;
  const double* pp = n_split > 1 ? partial : nullptr;
  const int per_thread = (cols / 4 + RN_THREADS - 1) / RN_THREADS;  // float4 per thread
#define MI_RN(NV)                                                                                        \
  hipLaunchKernelGGL(k_rmsnorm_quant<NV>, dim3((unsigned)rows), dim3(RN_THREADS), 0, s, x, gamma, cols, eps, \
                     codes, scales, y, pp, n_split, rows)
  if (per_thread <= 1) MI_RN(1);
  else if (per_thread <= 2) MI_RN(2);
  else if (per_thread <= 4) MI_RN(4);
  else if (per_thread <= 8) MI_RN(8);
  else MI_RN(0);
#undef MI_RN
  MI_LAUNCH_CHECK("k_rmsnorm_quant");
  return MI_OK;
}

// ---------------------------------------------------------------- SwiGLU + quantize
// s = f32(silu(g) * u) in f64 (common.h), then Q8_0.  Flat grid over float4s.
__global__ void __launch_bounds__(256) k_swiglu_quant(const float* __restrict__ gate,
                                                      const float* __restrict__ up, int64_t rows, int cols,
                                                      int64_t ld_in, int8_t* __restrict__ codes,
                                                      uint16_t* __restrict__ scales) {
  __shared__ double exp_tab[64];
  exp2_table_fill(exp_tab, threadIdx.x);
  __syncthreads();
  const int64_t nvec_row = cols / 4;
  const int64_t total = rows * nvec_row;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nvec_row, c4 = i - r * nvec_row;
    const float4 g = *reinterpret_cast<const float4*>(gate + r * ld_in + c4 * 4);
    const float4 u = *reinterpret_cast<const float4*>(up + r * ld_in + c4 * 4);
    float4 o;
    o.x = swiglu_f32(g.x, u.x, exp_tab);
    o.y = swiglu_f32(g.y, u.y, exp_tab);
    o.z = swiglu_f32(g.z, u.z, exp_tab);
    o.w = swiglu_f32(g.w, u.w, exp_tab);
    float d;
    const uint32_t q = q8_block_quant4(o, d);
    reinterpret_cast<uint32_t*>(codes + r * cols)[c4] = q;
    if ((c4 & 7) == 0) scales[r * (cols / QK) + c4 / 8] = f32_to_f16_bits(d);
  }
}

int launch_swiglu_quant(const float* gate, const float* up, int64_t rows, int cols, int64_t ld_in,
                        int8_t* codes, uint16_t* scales, hipStream_t s) {
  if (rows == 0) return MI_OK;
  const int64_t total = rows * (cols / 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_swiglu_quant, dim3((unsigned)blocks), dim3(256), 0, s, gate, up, rows, cols, ld_in,
                     codes, scales);
  MI_LAUNCH_CHECK("k_swiglu_quant");
  return MI_OK;
}

// ---------------------------------------------------------------- staging from pinned host memory
// words [0, n) of a pinned (device-mapped, coherent) host buffer -> device memory: the kernel reads
// the host buffer over the bus itself, so the ids and positions of a call reach the device without
// a copy-engine transfer (and the queue switch it costs) in front of the first kernel.
__global__ void __launch_bounds__(256) k_stage_in(uint32_t* __restrict__ dst, const uint32_t* __restrict__ src,
                                                  int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

int launch_stage_in(void* dst, const void* host_src, size_t bytes, hipStream_t s) {
  if (bytes % 4) return set_error(MI_ERR_INVALID_ARG, "stage: %zu bytes is not a whole number of words", bytes);
  const int64_t n = (int64_t)(bytes / 4);
  if (n == 0) return MI_OK;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 256);
  hipLaunchKernelGGL(k_stage_in, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<uint32_t*>(dst),
                     reinterpret_cast<const uint32_t*>(host_src), n);
  MI_LAUNCH_CHECK("k_stage_in");
  return MI_OK;
}

// ---------------------------------------------------------------- embedding rows
// out[t][c] = scale[id][c/32] * code[id][c]  (exact in f32).  One lane per 4 values.
__global__ void __launch_bounds__(256) k_embed(const int8_t* __restrict__ codes,
                                               const uint16_t* __restrict__ scales, int cols,
                                               const int32_t* __restrict__ ids, int n, float* __restrict__ out) {
  const int64_t nvec_row = cols / 4;
  const int64_t total = (int64_t)n * nvec_row;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / nvec_row, c4 = i - t * nvec_row;
    const int64_t row = ids[t];
    const uint32_t q = reinterpret_cast<const uint32_t*>(codes + row * cols)[c4];
    const float d = f16_bits_to_f32(scales[row * (cols / QK) + c4 / 8]);
    float4 o;
    o.x = d * (float)(int8_t)(q & 0xff);
    o.y = d * (float)(int8_t)((q >> 8) & 0xff);
    o.z = d * (float)(int8_t)((q >> 16) & 0xff);
    o.w = d * (float)(int8_t)(q >> 24);
    reinterpret_cast<float4*>(out + t * cols)[c4] = o;
  }
}

int launch_embed(const int8_t* codes, const uint16_t* scales, int cols, const int32_t* ids, int n,
                 float* out, hipStream_t s) {
  if (n == 0) return MI_OK;
  const int64_t total = (int64_t)n * (cols / 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_embed, dim3((unsigned)blocks), dim3(256), 0, s, codes, scales, cols, ids, n, out);
  MI_LAUNCH_CHECK("k_embed");
  return MI_OK;
}

// ---------------------------------------------------------------- per-head QK RMSNorm
// One wave per (row, head); head_dim <= 128 so each lane holds at most 2 values.
__global__ void __launch_bounds__(256) k_qk_norm(float* __restrict__ x, int64_t ld, const float* __restrict__ gamma,
                                                 int64_t rows, int n_heads, int head_dim, float eps) {
  const int64_t wave = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / 64;
  const int lane = threadIdx.x % 64;
  if (wave >= rows * n_heads) return;  // whole waves exit together
  const int64_t r = wave / n_heads;
  const int h = (int)(wave - r * n_heads);
  float* p = x + r * ld + (int64_t)h * head_dim;
  const bool has0 = lane < head_dim, has1 = lane + 64 < head_dim;
  const float v0 = has0 ? p[lane] : 0.0f, v1 = has1 ? p[lane + 64] : 0.0f;
  double ss = (double)v0 * v0 + (double)v1 * v1;
  ss = wave_sum_f64(ss);
  const double rms = sqrt(ss / (double)head_dim + (double)eps);
  if (has0) p[lane] = (float)((double)v0 / rms * (double)gamma[lane]);
  if (has1) p[lane + 64] = (float)((double)v1 / rms * (double)gamma[lane + 64]);
}

int launch_qk_norm(float* x, int64_t ld, const float* gamma, int64_t rows, int n_heads, int head_dim,
                   float eps, hipStream_t s) {
  if (rows == 0) return MI_OK;
  const int64_t waves = rows * n_heads;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL(k_qk_norm, dim3((unsigned)blocks), dim3(256), 0, s, x, ld, gamma, rows, n_heads,
                     head_dim, eps);
  MI_LAUNCH_CHECK("k_qk_norm");
  return MI_OK;
}

}  // namespace mi

namespace mi {

// out[r][:] = x[rows[r]][:] (cols a multiple of 4): the last rows of several sequences, gathered
__global__ void __launch_bounds__(256) k_gather_rows(const float* __restrict__ x, int cols,
                                                     const int32_t* __restrict__ rows, int n,
                                                     float* __restrict__ out) {
  const int nvec = cols / 4;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < (int64_t)n * nvec;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nvec, c4 = i - r * nvec;
    reinterpret_cast<float4*>(out + r * cols)[c4] = reinterpret_cast<const float4*>(x + (int64_t)rows[r] * cols)[c4];
  }
}

int launch_gather_rows(const float* x, int cols, const int32_t* rows, int n, float* out, hipStream_t s) {
  if (n == 0) return MI_OK;
  const int64_t total = (int64_t)n * (cols / 4);
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(k_gather_rows, dim3(blocks), dim3(256), 0, s, x, cols, rows, n, out);
  MI_LAUNCH_CHECK("k_gather_rows");
  return MI_OK;
}

}  // namespace mi
