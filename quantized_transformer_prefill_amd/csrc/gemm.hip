// Q8_0 x Q8_0 matmul on int8 MFMA with an exact per-block scale epilogue.
//
// out[m][n] = sum_kb da[m][kb] * dw[n][kb] * I[m][n][kb],  I = sum over the 32 values of the
// block of qa * qw (the matmul node of the Qwen2 layer; activations quantized to Q8_0 on the
// fly, weights stored [out][in]).
//
// * I comes from v_mfma_i32_32x32x32_i8: K = 32 is exactly one Q8_0 block, so every MFMA
//   yields the integer block sums of one block.
// * The scale epilogue is exact.  Only the even rows of each 32x32 MFMA carry data; the odd
//   rows have all-zero A rows, so the accumulator initial value passes through them
//   unchanged.  The initial value is 0x80000000 on even rows and 0x43380000 on odd rows, so
//   each (even, odd) output register pair is directly the f64 number 1.5*2^52 + 2^31 + I.
//   Then t = fma(x, dw, -(1.5*2^52 + 2^31)*dw) is exactly I*dw, and acc = fma(t, da, acc)
//   adds the exact product I*dw*da with a single f64 rounding.  With f64 accumulation the
//   rounded f32 result matches f32(exact sum) except for f64 rounding at ties.
// * The VALU f64 epilogue (2 f64 FMAs per output per block) bounds this kernel, not the
//   MFMA: half-used MFMAs cost nothing extra.
//
// Tiling: 256 threads = 4 waves (2 x 2); workgroup tile 64 real rows x 128 weight rows; wave
// tile 32 x 64 = 2 x 2 MFMAs per block.  A/B codes and the f64 scales of each block are
// staged through LDS, double-buffered.  Split-K writes f64 partials that a second kernel
// reduces in a fixed order (deterministic).
#include "common.h"

namespace mi {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int G_THREADS = 256;
constexpr int G_BM = 64;    // real activation rows per workgroup
constexpr int G_BN = 128;   // weight rows (output columns) per workgroup
constexpr double G_MAGIC = 0x1.8p+52 + 0x1p+31;  // 1.5*2^52 + 2^31, exact

struct GemmSmem {
  int8_t a[2][G_BM][QK];     // 4 KB
  int8_t b[2][G_BN][QK];     // 8 KB
  double as[2][G_BM];        // 1 KB
  double bs[2][G_BN];        // 2 KB
};

__device__ __forceinline__ double pair_f64(int lo, int hi) {
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}

__device__ __forceinline__ float swiglu_f32(float g, float u) {
  const double gd = g;
  const double sg = gd / (1.0 + exp(-gd));
  return (float)(sg * (double)u);
}

template <int EPI, bool SPLIT>
__global__ void __launch_bounds__(G_THREADS, 2)
k_gemm_q8(const int8_t* __restrict__ a_codes, const uint16_t* __restrict__ a_scales, int M,
          const int8_t* __restrict__ w_codes, const uint16_t* __restrict__ w_scales, int N, int K,
          const float* __restrict__ bias, const float* residual, float* out, int64_t ld_out,
          int8_t* __restrict__ q_codes, uint16_t* __restrict__ q_scales,
          double* __restrict__ partial, int kb_per_split) {
  __shared__ __align__(16) GemmSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * G_BN, m0 = blockIdx.y * G_BM;
  const int KB = K / QK;
  const int kb0 = blockIdx.z * kb_per_split;
  const int kb1 = min(KB, kb0 + kb_per_split);

  // ---- global -> register prefetch mapping
  const int ld_row = tid >> 1, ld_half = tid & 1;  // 128 rows x 2 halves of 16 bytes
  const bool a_ld = tid < 2 * G_BM;
  const int a_row = m0 + ld_row;
  const bool a_ok = a_ld && a_row < M;
  const int b_row = n0 + ld_row;  // N % 32 == 0 and n0 + 128 may exceed N
  const bool b_ok = b_row < N;
  const int8_t* a_src = a_codes + (int64_t)(a_ok ? a_row : 0) * K + ld_half * 16;
  const int8_t* b_src = w_codes + (int64_t)(b_ok ? b_row : 0) * K + ld_half * 16;
  const uint16_t* as_src = a_scales + (int64_t)(m0 + tid < M ? m0 + tid : 0) * KB;
  const uint16_t* bs_src = w_scales + (int64_t)(n0 + tid < N ? n0 + tid : 0) * KB;
  const bool as_ok = tid < G_BM && m0 + tid < M;
  const bool bs_ok = tid < G_BN && n0 + tid < N;

  v4i pa = {0, 0, 0, 0}, pb = {0, 0, 0, 0};
  uint16_t pas = 0, pbs = 0;
  auto fetch = [&](int kb) {
    if (a_ok) pa = *reinterpret_cast<const v4i*>(a_src + (int64_t)kb * QK);
    if (b_ok) pb = *reinterpret_cast<const v4i*>(b_src + (int64_t)kb * QK);
    if (as_ok) pas = as_src[kb];
    if (bs_ok) pbs = bs_src[kb];
  };
  auto stash = [&](int st) {
    if (a_ld) *reinterpret_cast<v4i*>(&sm.a[st][ld_row][ld_half * 16]) = pa;
    *reinterpret_cast<v4i*>(&sm.b[st][ld_row][ld_half * 16]) = pb;
    if (tid < G_BM) sm.as[st][tid] = as_ok ? (double)f16_bits_to_f32(pas) : 0.0;
    if (tid < G_BN) sm.bs[st][tid] = bs_ok ? (double)f16_bits_to_f32(pbs) : 0.0;
  };

  v16i cinit;
#pragma unroll
  for (int i = 0; i < 16; ++i) cinit[i] = (i & 1) ? 0x43380000 : (int)0x80000000;

  double acc[2][2][8];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg)
#pragma unroll
    for (int cg = 0; cg < 2; ++cg)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[rg][cg][j] = 0.0;

  const bool a_lane = (lane & 1) == 0;          // even MFMA rows carry data
  const int a_rrow = wm * 32 + ((lane & 31) >> 1);  // + rg*16
  const int koff = (lane >> 5) * 16;
  const int b_rrow = wn * 64 + (lane & 31);         // + cg*32
  const int da_row = wm * 32 + 2 * (lane >> 5);     // + rg*16 + 4c + e

  if (kb0 < kb1) {
    fetch(kb0);
    stash(0);
  }
  __syncthreads();
  for (int kb = kb0; kb < kb1; ++kb) {
    const int st = (kb - kb0) & 1;
    if (kb + 1 < kb1) fetch(kb + 1);
    v4i fa[2], fb[2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
      fa[rg] = a_lane ? *reinterpret_cast<const v4i*>(&sm.a[st][a_rrow + rg * 16][koff]) : v4i{0, 0, 0, 0};
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) fb[cg] = *reinterpret_cast<const v4i*>(&sm.b[st][b_rrow + cg * 32][koff]);
    v16i d[2][2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) d[rg][cg] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[rg], fb[cg], cinit, 0, 0, 0);
    double dw[2], cdw[2];
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
      dw[cg] = sm.bs[st][b_rrow + cg * 32];
      cdw[cg] = -G_MAGIC * dw[cg];
    }
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      double da[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const double2 v2 = *reinterpret_cast<const double2*>(&sm.as[st][da_row + rg * 16 + 4 * c]);
        da[2 * c] = v2.x;
        da[2 * c + 1] = v2.y;
      }
#pragma unroll
      for (int cg = 0; cg < 2; ++cg)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const double x = pair_f64(d[rg][cg][2 * j], d[rg][cg][2 * j + 1]);
          const double t = fma(x, dw[cg], cdw[cg]);
          acc[rg][cg][j] = fma(t, da[j], acc[rg][cg][j]);
        }
    }
    if (kb + 1 < kb1) stash(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  Lane holds, for each (rg, cg, j): real row rr, column cc.
#pragma unroll
  for (int rg = 0; rg < 2; ++rg)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = m0 + wm * 32 + rg * 16 + 4 * (j >> 1) + 2 * (lane >> 5) + (j & 1);
      if (SPLIT) {
        if (row < M) {
#pragma unroll
          for (int cg = 0; cg < 2; ++cg) {
            const int col = n0 + wn * 64 + cg * 32 + (lane & 31);
            if (col < N) partial[((int64_t)blockIdx.z * M + row) * N + col] = acc[rg][cg][j];
          }
        }
      } else if (EPI == EPI_F32) {
        if (row < M) {
#pragma unroll
          for (int cg = 0; cg < 2; ++cg) {
            const int col = n0 + wn * 64 + cg * 32 + (lane & 31);
            if (col < N) {
              double v = acc[rg][cg][j];
              if (bias) v += (double)bias[col];
              float y = (float)v;
              const int64_t o = (int64_t)row * ld_out + col;
              if (residual) y = residual[o] + y;
              out[o] = y;
            }
          }
        }
      } else {  // EPI_SWIGLU_Q8: cg 0 = gate, cg 1 = up of the same ffn column
        const int gcol = n0 + wn * 64;               // multiple of 64: 32 gate rows, 32 up rows
        const float g = (float)acc[rg][0][j];
        const float u = (float)acc[rg][1][j];
        const float sv = swiglu_f32(g, u);
        float m = fabsf(sv);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
        const float dq = m / 127.0f;
        const float id = (dq != 0.0f) ? 1.0f / dq : 0.0f;
        float r = roundf(sv * id);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        const int ncols = N / 2;
        const int scol = gcol / 2 + (lane & 31);
        if (row < M && gcol < N) {
          q_codes[(int64_t)row * ncols + scol] = (int8_t)(int)r;
          if ((lane & 31) == 0) q_scales[(int64_t)row * (ncols / QK) + scol / QK] = f32_to_f16_bits(dq);
        }
      }
    }
}

// ---- split-K reductions (fixed order over the splits)
__global__ void __launch_bounds__(256) k_splitk_f32(const double* __restrict__ partial, int S, int M, int N,
                                                    const float* __restrict__ bias, const float* residual,
                                                    float* out, int64_t ld_out) {
  const int64_t total = (int64_t)M * N;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / N;
    const int col = (int)(i - row * N);
    double v = 0.0;
    for (int z = 0; z < S; ++z) v += partial[(int64_t)z * total + i];
    if (bias) v += (double)bias[col];
    float y = (float)v;
    const int64_t o = row * ld_out + col;
    if (residual) y = residual[o] + y;
    out[o] = y;
  }
}

__global__ void __launch_bounds__(256) k_splitk_swiglu(const double* __restrict__ partial, int S, int M, int N,
                                                       int8_t* __restrict__ q_codes, uint16_t* __restrict__ q_scales) {
  const int ncols = N / 2;
  const int64_t nvec_row = ncols / 4;
  const int64_t total = (int64_t)M * nvec_row;
  const int64_t plane = (int64_t)M * N;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / nvec_row;
    const int c4 = (int)(i - row * nvec_row);
    float s[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int sc = c4 * 4 + e;
      const int gcol = (sc / 32) * 64 + (sc % 32);
      double g = 0.0, u = 0.0;
      for (int z = 0; z < S; ++z) {
        g += partial[z * plane + row * N + gcol];
        u += partial[z * plane + row * N + gcol + 32];
      }
      s[e] = swiglu_f32((float)g, (float)u);
    }
    float d;
    const uint32_t q = q8_block_quant4(make_float4(s[0], s[1], s[2], s[3]), d);
    reinterpret_cast<uint32_t*>(q_codes + row * ncols)[c4] = q;
    if ((c4 & 7) == 0) q_scales[row * (ncols / QK) + c4 / 8] = f32_to_f16_bits(d);
  }
}

static int choose_split(int m, int n, int k) {
  const int tiles = ((m + G_BM - 1) / G_BM) * ((n + G_BN - 1) / G_BN);
  const int KB = k / QK;
  int split = 1;
  const int target = 2 * 256;  // two workgroups per CU
  while (split < 16 && tiles * split < target && KB / (split * 2) >= 8) split *= 2;
  return split;
}

size_t gemm_workspace_bytes(int m, int n, int k) {
  const int s = choose_split(m, n, k);
  return s > 1 ? (size_t)s * m * n * sizeof(double) : 0;
}

int launch_gemm_q8(const GemmArgs& g, hipStream_t s) {
  if (g.m == 0) return MI_OK;
  const int KB = g.k / QK;
  int split = g.split_k > 0 ? g.split_k : choose_split(g.m, g.n, g.k);
  if (split > KB) split = KB;
  const size_t need = split > 1 ? (size_t)split * g.m * g.n * sizeof(double) : 0;
  if (need > g.workspace_bytes || (need && !g.workspace)) split = 1;
  const int kb_per = (KB + split - 1) / split;
  split = (KB + kb_per - 1) / kb_per;
  dim3 grid((g.n + G_BN - 1) / G_BN, (g.m + G_BM - 1) / G_BM, split);
  double* partial = reinterpret_cast<double*>(g.workspace);
  if (split == 1) {
    if (g.q_codes)
      hipLaunchKernelGGL((k_gemm_q8<EPI_SWIGLU_Q8, false>), grid, dim3(G_THREADS), 0, s, g.a_codes, g.a_scales,
                         g.m, g.w_codes, g.w_scales, g.n, g.k, g.bias, g.residual, g.out, g.ld_out, g.q_codes,
                         g.q_scales, nullptr, kb_per);
    else
      hipLaunchKernelGGL((k_gemm_q8<EPI_F32, false>), grid, dim3(G_THREADS), 0, s, g.a_codes, g.a_scales, g.m,
                         g.w_codes, g.w_scales, g.n, g.k, g.bias, g.residual, g.out, g.ld_out, g.q_codes,
                         g.q_scales, nullptr, kb_per);
    MI_LAUNCH_CHECK("k_gemm_q8");
    return MI_OK;
  }
  hipLaunchKernelGGL((k_gemm_q8<EPI_F32, true>), grid, dim3(G_THREADS), 0, s, g.a_codes, g.a_scales, g.m,
                     g.w_codes, g.w_scales, g.n, g.k, g.bias, g.residual, g.out, g.ld_out, g.q_codes,
                     g.q_scales, partial, kb_per);
  MI_LAUNCH_CHECK("k_gemm_q8 (split)");
  if (g.q_codes) {
    const int64_t total = (int64_t)g.m * (g.n / 2 / 4);
    const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
    hipLaunchKernelGGL(k_splitk_swiglu, dim3((unsigned)blocks), dim3(256), 0, s, partial, split, g.m, g.n,
                       g.q_codes, g.q_scales);
  } else {
    const int64_t total = (int64_t)g.m * g.n;
    const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
    hipLaunchKernelGGL(k_splitk_f32, dim3((unsigned)blocks), dim3(256), 0, s, partial, split, g.m, g.n, g.bias,
                       g.residual, g.out, g.ld_out);
  }
  MI_LAUNCH_CHECK("k_splitk_reduce");
  return MI_OK;
}

// ---------------------------------------------------------------- last-row lm_head
// logits[v] = f32( sum_kb dx[kb] * dw[v][kb] * sum_32 qx * qw ), one row of activations.
// HBM-bound: every weight byte is read once.  One wave per weight row at a time; a lane
// takes 16-byte chunks (half a block), sdot4 gives the integer half-block sums, lane pairs
// combine to the block sum, and the exact f64 epilogue accumulates per lane.
constexpr int LM_MAXC = 4;  // 16-byte activation chunks held per lane (K <= 4096)

__global__ void __launch_bounds__(256) k_lm_head(const int8_t* __restrict__ xq, const uint16_t* __restrict__ xs,
                                                 int K, const int8_t* __restrict__ w_codes,
                                                 const uint16_t* __restrict__ w_scales, int rows,
                                                 float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const int nchunk = K / 16;
  const int KB = K / QK;
  v4i xc[LM_MAXC];
  double xd[LM_MAXC];
#pragma unroll
  for (int c = 0; c < LM_MAXC; ++c) {
    const int ch = lane + 64 * c;
    xc[c] = ch < nchunk ? *reinterpret_cast<const v4i*>(xq + ch * 16) : v4i{0, 0, 0, 0};
    xd[c] = ch < nchunk ? (double)f16_bits_to_f32(xs[ch / 2]) : 0.0;
  }
  for (int64_t r = wave; r < rows; r += nwaves) {
    const int8_t* wr = w_codes + r * K;
    const uint16_t* wsr = w_scales + r * KB;
    double acc = 0.0;
#pragma unroll
    for (int c = 0; c < LM_MAXC; ++c) {
      const int ch = lane + 64 * c;
      int isum = 0;
      double dw = 0.0;
      if (ch < nchunk) {
        const v4i wv = *reinterpret_cast<const v4i*>(wr + ch * 16);
        isum = __builtin_amdgcn_sdot4(xc[c][0], wv[0], isum, false);
        isum = __builtin_amdgcn_sdot4(xc[c][1], wv[1], isum, false);
        isum = __builtin_amdgcn_sdot4(xc[c][2], wv[2], isum, false);
        isum = __builtin_amdgcn_sdot4(xc[c][3], wv[3], isum, false);
        dw = (double)f16_bits_to_f32(wsr[ch / 2]);
      }
      isum += __shfl_xor(isum, 1);  // both lanes of the pair now hold the block sum
      if ((lane & 1) == 0 && ch < nchunk) acc = fma((double)isum * dw, xd[c], acc);
    }
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) logits[r] = (float)acc;
  }
}

int launch_lm_head(const int8_t* xq, const uint16_t* xs, int cols, const int8_t* w_codes,
                   const uint16_t* w_scales, int rows, float* logits, hipStream_t s) {
  if (cols > 64 * 16 * LM_MAXC) return set_error(MI_ERR_UNSUPPORTED, "lm_head: cols %d > %d", cols, 64 * 16 * LM_MAXC);
  const int blocks = 256 * 8;
  hipLaunchKernelGGL(k_lm_head, dim3(blocks), dim3(256), 0, s, xq, xs, cols, w_codes, w_scales, rows, logits);
  MI_LAUNCH_CHECK("k_lm_head");
  return MI_OK;
}

}  // namespace mi
