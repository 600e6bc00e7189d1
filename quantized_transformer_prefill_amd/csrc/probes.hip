// Rate probes: what one MI355X sustains for the instruction mixes that bound the Q8_0 matmul, with
// no memory traffic.  They give the ceilings the matmul's roofline fraction is read against:
//   - the f64 FMA rate of the vector ALU (the exact scale epilogue runs on it);
//   - the int8 MFMA rate (v_mfma_i32_32x32x32_i8, the matmul's contraction);
//   - the matmul's inner loop per Q8_0 block with the exact f64 epilogue: one MFMA per 16 real rows
//     x 32 columns, then two f64 FMAs per output (q8_epilogue.h), as the matmul kernel issues them,
//     operands in registers -- the loop-only bound of the exact matmul;
//   - the same loop with an f32 epilogue (all 32 MFMA rows real; per output: convert, multiply,
//     fused add in f32): what the matmul would reach if f32 accumulation were enough.
// Every kernel keeps its work alive by writing one value per thread.
#include "../../include/mi_probes.h"
#include "common.h"
#include "q8_epilogue.h"

namespace mi {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef double v8d __attribute__((ext_vector_type(8)));

constexpr int P_THREADS = 256;

__global__ void __launch_bounds__(P_THREADS) k_probe_f64_fma(double* out, int iters, double a, double b) {
  double x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 1e-3 * threadIdx.x + i;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fma(x[i], a, b);  // 8 independent chains per lane
  }
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * (int64_t)P_THREADS + threadIdx.x] = s;
}

__global__ void __launch_bounds__(P_THREADS) k_probe_mfma_i8(double* out, int iters, int seed) {
  v4i a = {seed, seed + 1, seed + 2, (int)threadIdx.x}, b = {seed + 3, seed + 4, (int)threadIdx.x, seed};
  v16i c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) c[j][i] = 0;
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(a), "+v"(b));  // operands the compiler cannot hoist
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[j][i];
  out[blockIdx.x * (int64_t)P_THREADS + threadIdx.x] = (double)s;
}

// The exact matmul's block loop for an RG x CG wave tile: per block RG*CG MFMAs, each followed by
// 8 exact products I*dw and 8 DPP-broadcast f64 accumulations (q8_epilogue.h).  Each iteration is one
// stage of 4 Q8_0 blocks of K; fragments and scales come from registers the compiler treats as new
// at every block.
template <int RG, int CG>
__global__ void __launch_bounds__(P_THREADS, RG == 1 ? 3 : 2) k_probe_loop_exact(double* out, int iters, int seed) {
  v4i fa[RG], fb[CG];
#pragma unroll
  for (int r = 0; r < RG; ++r) fa[r] = v4i{seed + r, (int)threadIdx.x, seed ^ r, 7};
#pragma unroll
  for (int c = 0; c < CG; ++c) fb[c] = v4i{seed - c, 3, (int)threadIdx.x, seed};
  v16i cinit;
#pragma unroll
  for (int i = 0; i < 16; ++i) cinit[i] = (i & 1) ? 0x43380000 : (int)0x80000000;
  double acc[RG][CG][8];
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[r][c][j] = 0.0;
  double da0 = 1.0 + 1e-3 * (threadIdx.x & 15), da1 = 2.0, dw[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) dw[c] = 0.5 + c;
  // one iteration = one stage of 4 blocks, unrolled as in the matmul (blocks 2p, 2p+1 take their
  // row scales from the two halves of register da_p)
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      asm volatile("" : "+v"(da0), "+v"(da1));
#pragma unroll
      for (int r = 0; r < RG; ++r) asm volatile("" : "+v"(fa[r]));
#pragma unroll
      for (int c = 0; c < CG; ++c) asm volatile("" : "+v"(fb[c]), "+v"(dw[c]));
      const double da = (jb >> 1) ? da1 : da0;
#pragma unroll
      for (int r = 0; r < RG; ++r)
#pragma unroll
        for (int c = 0; c < CG; ++c) {
          const v16i d = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[r], fb[c], cinit, 0, 0, 0);
          const v8d xv = __builtin_bit_cast(v8d, d);
          const double cdw = -G_MAGIC * dw[c];
          double x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = fma(xv[j], dw[c], cdw);
          if (jb & 1) fmac8_bcast<1>(acc[r][c], x, da);
          else fmac8_bcast<0>(acc[r][c], x, da);
        }
    }
  }
  double s = 0.0;
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) s += acc[r][c][j];
  out[blockIdx.x * (int64_t)P_THREADS + threadIdx.x] = s;
}

// The same loop with an f32 epilogue: all 32 MFMA rows real (accumulator starts at 0); per output
// and block acc += f32(I) * dw * da in f32 (convert, multiply, fused multiply-add).
template <int RG, int CG>
__global__ void __launch_bounds__(P_THREADS, 2) k_probe_loop_f32(double* out, int iters, int seed) {
  v4i fa[RG], fb[CG];
#pragma unroll
  for (int r = 0; r < RG; ++r) fa[r] = v4i{seed + r, (int)threadIdx.x, seed ^ r, 7};
#pragma unroll
  for (int c = 0; c < CG; ++c) fb[c] = v4i{seed - c, 3, (int)threadIdx.x, seed};
  v16i zero;
#pragma unroll
  for (int i = 0; i < 16; ++i) zero[i] = 0;
  float acc[RG][CG][16];
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[r][c][j] = 0.0f;
  float da = 1.0f + 1e-3f * (threadIdx.x & 15), dw[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) dw[c] = 0.5f + c;
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(da));
#pragma unroll
    for (int r = 0; r < RG; ++r) asm volatile("" : "+v"(fa[r]));
#pragma unroll
    for (int c = 0; c < CG; ++c) asm volatile("" : "+v"(fb[c]), "+v"(dw[c]));
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        const v16i d = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[r], fb[c], zero, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[r][c][j] = fmaf((float)d[j] * dw[c], da, acc[r][c][j]);
      }
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
      for (int j = 0; j < 16; ++j) s += acc[r][c][j];
  out[blockIdx.x * (int64_t)P_THREADS + threadIdx.x] = (double)s;
}

}  // namespace mi

using namespace mi;

// work per launch: f64 FMAs (probe 0); int8 ops counted as 2 x multiply-adds of the real MFMA rows
// (probes 1-5)
extern "C" int mi_probe_run(int32_t probe, int32_t n_workgroups, int32_t iters, double* out, double* work,
                            void* stream) {
  if (!out || !work || n_workgroups < 1 || iters < 1) return MI_ERR_INVALID_ARG;
  hipStream_t s = as_stream(stream);
  const double waves = (double)n_workgroups * (P_THREADS / 64);
  const double mfma_ops = 2.0 * 32 * 32 * 32;  // one v_mfma_i32_32x32x32_i8
  switch (probe) {
    case MI_PROBE_F64_FMA:
      hipLaunchKernelGGL(k_probe_f64_fma, dim3(n_workgroups), dim3(P_THREADS), 0, s, out, iters, 0.999999, 1e-9);
      *work = waves * 64 * 8 * (double)iters;
      break;
    case MI_PROBE_MFMA_I8:
      hipLaunchKernelGGL(k_probe_mfma_i8, dim3(n_workgroups), dim3(P_THREADS), 0, s, out, iters, 5);
      *work = waves * 4 * mfma_ops * (double)iters;
      break;
    case MI_PROBE_LOOP_EXACT_1X2:
      hipLaunchKernelGGL((k_probe_loop_exact<1, 2>), dim3(n_workgroups), dim3(P_THREADS), 0, s, out, iters, 5);
      *work = waves * 4 * 2 * (mfma_ops / 2) * (double)iters;  // 4 blocks; 16 of the 32 rows carry data
      break;
    case MI_PROBE_LOOP_EXACT_4X2:
      hipLaunchKernelGGL((k_probe_loop_exact<4, 2>), dim3(n_workgroups), dim3(P_THREADS), 0, s, out, iters, 5);
      *work = waves * 4 * 8 * (mfma_ops / 2) * (double)iters;
      break;
    case MI_PROBE_LOOP_F32_2X2:
      hipLaunchKernelGGL((k_probe_loop_f32<2, 2>), dim3(n_workgroups), dim3(P_THREADS), 0, s, out, iters, 5);
      *work = waves * 4 * mfma_ops * (double)iters;
      break;
    default:
      return MI_ERR_INVALID_ARG;
  }
  return hipGetLastError() == hipSuccess ? MI_OK : MI_ERR_HIP;
}
