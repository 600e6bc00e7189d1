// Decode step (one token at one position through the same layer sequence and KV regions as the
// prefill; the two-act engine of the walkthrough index, act two).  With one activation row every
// matmul is a matrix-vector product bound by HBM, and the attention has one query per head.
//
// k_gemv_q8: y[n] = sum_kb dx[kb] * dw[n][kb] * sum_32 qx * qw, one activation row.
//  * 16 waves per workgroup, RPW weight rows per wave in flight at once; a lane takes 16-byte
//    chunks (half a block) of every row, sdot4 gives the integer half-block sums, lane pairs
//    combine them to the block sum, and the exact f64 epilogue (block sum times dw, times dx,
//    one rounding per block) accumulates per lane; the lanes' partial sums then reduce in f64.
//  * The activation row is staged in LDS as codes + f64 scales.  With NORM the workgroup builds
//    it itself from the f32 residual stream: RMSNorm in f64, one rounding to f32, Q8_0 -- the
//    same arithmetic as the prefill's k_rmsnorm_quant -- so the decode step has no separate
//    normalization kernels.
//  * Epilogues: residual add (output projection, down projection), plain f32 (lm_head), the
//    attention inputs (bias, per-head QK RMSNorm, NeoX RoPE, K/V rows stored at the position; a
//    workgroup holds one head), SwiGLU + Q8_0 (a workgroup holds one interleaved group of 32
//    gate and 32 up rows, i.e. one Q8_0 block of the SwiGLU output).
//
// k_attn_decode + k_attn_decode_merge: the query's keys 0..pos are split into fixed ranges (the
// grid depends only on n_ctx, so the launch can be captured once and replayed for any position);
// each workgroup computes the partial softmax state (max, sum, unnormalized output) of one head
// over one range in f64, and the merge combines the ranges in order, normalizes, and writes the
// head's output row as Q8_0 (the input of the output projection).
#include "common.h"

namespace mi {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int GV_THREADS = 1024;  // 16 waves
constexpr int GV_WAVES = GV_THREADS / 64;

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}

template <int RPW, int EPI, bool NORM>
__global__ void __launch_bounds__(GV_THREADS) k_gemv_q8(const float* __restrict__ x, const float* __restrict__ gamma,
                                                       float eps, const int8_t* __restrict__ xq,
                                                       const uint16_t* __restrict__ xs, int K,
                                                       const int8_t* __restrict__ w_codes,
                                                       const uint16_t* __restrict__ w_scales, int N,
                                                       const float* __restrict__ bias, const float* residual,
                                                       float* out, int8_t* __restrict__ q_codes,
                                                       uint16_t* __restrict__ q_scales, GemvQkv qe) {
  constexpr int RWG = RPW * GV_WAVES;  // weight rows per workgroup
  extern __shared__ __align__(16) unsigned char gv_lds[];
  const int KB = K / QK;
  int8_t* a_codes = reinterpret_cast<int8_t*>(gv_lds);                           // [K]
  double* a_d = reinterpret_cast<double*>(gv_lds + ((K + 15) & ~15));             // [KB]
  float* y = reinterpret_cast<float*>(a_d + KB);                                   // [RWG]
  double* red = reinterpret_cast<double*>(y + RWG + (RWG & 1));                    // [GV_WAVES + 1]
  __shared__ double exp_tab[EPI == GV_SWIGLU ? 64 : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (EPI == GV_SWIGLU) exp2_table_fill(exp_tab, tid);

  // ---- the activation row -> LDS (codes, f64 scales)
  const int nvec = K / 4;
  if constexpr (NORM) {
    double ss = 0.0;
    for (int c4 = tid; c4 < nvec; c4 += GV_THREADS) {
      const float4 v = reinterpret_cast<const float4*>(x)[c4];
      const double a = v.x, b = v.y, c = v.z, d = v.w;
      ss += a * a + b * b + c * c + d * d;
    }
    ss = wave_sum_d(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    if (wave == 0) {
      double t = lane < GV_WAVES ? red[lane] : 0.0;
      t = wave_sum_d(t);
      if (lane == 0) red[GV_WAVES] = t;
    }
    __syncthreads();
    const double inv_rms = recip_f64(sqrt(red[GV_WAVES] / (double)K + (double)eps));
    // groups of 8 lanes cover one block; all 8 share the loop trip count (K is a multiple of 32)
    for (int c4 = tid; c4 < nvec; c4 += GV_THREADS) {
      const float4 v = reinterpret_cast<const float4*>(x)[c4];
      const float4 g = reinterpret_cast<const float4*>(gamma)[c4];
      float4 o;
      o.x = (float)((double)v.x * inv_rms * (double)g.x);
      o.y = (float)((double)v.y * inv_rms * (double)g.y);
      o.z = (float)((double)v.z * inv_rms * (double)g.z);
      o.w = (float)((double)v.w * inv_rms * (double)g.w);
      float d;
      const uint32_t q = q8_block_quant4(o, d);
      reinterpret_cast<uint32_t*>(a_codes)[c4] = q;
      if ((c4 & 7) == 0) a_d[c4 / 8] = (double)f16_bits_to_f32(f32_to_f16_bits(d));
    }
  } else {
    for (int c4 = tid; c4 < nvec; c4 += GV_THREADS)
      reinterpret_cast<uint32_t*>(a_codes)[c4] = reinterpret_cast<const uint32_t*>(xq)[c4];
    for (int b = tid; b < KB; b += GV_THREADS) a_d[b] = (double)f16_bits_to_f32(xs[b]);
  }
  __syncthreads();

  // ---- RPW rows per wave, all of their loads in flight together
  const int nchunk = K / 16;
  const int r0 = blockIdx.x * RWG + wave * RPW;
  const int8_t* wrow[RPW];
  const uint16_t* srow[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int r = min(r0 + i, N - 1);  // rows past N re-read the last row; never stored
    wrow[i] = w_codes + (int64_t)r * K;
    srow[i] = w_scales + (int64_t)r * KB;
  }
  double acc[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) acc[i] = 0.0;
  for (int c0 = 0; c0 < nchunk; c0 += 64) {
    const int ch = c0 + lane;
    const bool on = ch < nchunk;
    v4i xa = {0, 0, 0, 0};
    double da = 0.0;
    int isum[RPW];
    double dw[RPW];
    if (on) {
      xa = *reinterpret_cast<const v4i*>(a_codes + ch * 16);
      da = a_d[ch >> 1];
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      isum[i] = 0;
      dw[i] = 0.0;
      if (on) {
        const v4i wv = *reinterpret_cast<const v4i*>(wrow[i] + ch * 16);
        isum[i] = __builtin_amdgcn_sdot4(xa[0], wv[0], 0, false);
        isum[i] = __builtin_amdgcn_sdot4(xa[1], wv[1], isum[i], false);
        isum[i] = __builtin_amdgcn_sdot4(xa[2], wv[2], isum[i], false);
        isum[i] = __builtin_amdgcn_sdot4(xa[3], wv[3], isum[i], false);
        dw[i] = (double)f16_bits_to_f32(srow[i][ch >> 1]);
      }
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      isum[i] += __shfl_xor(isum[i], 1);  // both lanes of the pair hold the block sum
      if (on && (lane & 1) == 0) acc[i] = fma((double)isum[i] * dw[i], da, acc[i]);  // I*dw exact
    }
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) acc[i] = wave_sum_d(acc[i]);

  if constexpr (EPI == GV_RES || EPI == GV_F32) {
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int r = r0 + i;
        if (r < N) {
          float v = (float)acc[i];
          if (EPI == GV_RES) v = residual[r] + v;
          out[r] = v;
        }
      }
    }
    return;
  } else {
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        double v = acc[i];
        if (EPI == GV_QKV && bias) v += (double)bias[min(r0 + i, N - 1)];
        y[wave * RPW + i] = (float)v;
      }
    }
    __syncthreads();
    if constexpr (EPI == GV_SWIGLU) {
      // rows 64p..64p+31 are gate rows 32p.., rows 64p+32..64p+63 up rows 32p..: one Q8_0 block
      if (tid < 8) {
        float4 s;
        s.x = swiglu_f32(y[4 * tid + 0], y[32 + 4 * tid + 0], exp_tab);
        s.y = swiglu_f32(y[4 * tid + 1], y[32 + 4 * tid + 1], exp_tab);
        s.z = swiglu_f32(y[4 * tid + 2], y[32 + 4 * tid + 2], exp_tab);
        s.w = swiglu_f32(y[4 * tid + 3], y[32 + 4 * tid + 3], exp_tab);
        float d;
        const uint32_t q = q8_block_quant4(s, d);
        reinterpret_cast<uint32_t*>(q_codes + (int64_t)blockIdx.x * QK)[tid] = q;
        if (tid == 0) q_scales[blockIdx.x] = f32_to_f16_bits(d);
      }
    } else {  // GV_QKV: this workgroup's rows are one head of Q, K or V
      const int hd = qe.head_dim, half = hd / 2;
      const int c0 = blockIdx.x * RWG;
      const int64_t p = *qe.pos;
      if (c0 >= qe.n_q + qe.n_kv) {  // V head: stored as is
        for (int i = tid; i < hd; i += GV_THREADS) qe.v_region[p * qe.n_kv + (c0 - qe.n_q - qe.n_kv) + i] = y[i];
        return;
      }
      const bool isq = c0 < qe.n_q;
      const float* gam = isq ? qe.q_norm : qe.k_norm;
      if (gam) {  // per-head RMSNorm in f64, one rounding (wave 0)
        if (wave == 0) {
          double ss = 0.0;
          for (int i = lane; i < hd; i += 64) ss += (double)y[i] * (double)y[i];
          ss = wave_sum_d(ss);
          const double ir = recip_f64(sqrt(ss / (double)hd + (double)qe.eps));
          float t[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int i = lane + 64 * k;
            if (i < hd) t[k] = (float)((double)y[i] * ir * (double)gam[i]);
          }
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int i = lane + 64 * k;
            if (i < hd) y[i] = t[k];
          }
        }
        __syncthreads();
      }
      for (int i = tid; i < half; i += GV_THREADS) {
        const float a = y[i], b = y[i + half];
        const double2 cs = reinterpret_cast<const double2*>(qe.rope)[p * half + i];
        const float o0 = (float)((double)a * cs.x - (double)b * cs.y);
        const float o1 = (float)((double)a * cs.y + (double)b * cs.x);
        float* dst = isq ? qe.q_out + c0 : qe.k_region + p * qe.n_kv + (c0 - qe.n_q);
        dst[i] = o0;
        dst[i + half] = o1;
      }
    }
  }
}

int launch_gemv_q8(const GemvArgs& g, hipStream_t s) {
  const bool norm = g.x != nullptr;
  const int KB = g.k / QK;
  const size_t lds = (size_t)((g.k + 15) & ~15) + sizeof(double) * KB + sizeof(float) * 130 +
                     sizeof(double) * (GV_WAVES + 1);
  if (g.k % QK || g.k <= 0 || lds > 64 * 1024)
    return set_error(MI_ERR_UNSUPPORTED, "gemv: K %d (multiple of 32, LDS %zu bytes)", g.k, lds);
  GemvQkv qe = g.qkv;
#define GV_LAUNCH(RPW, EPI, NORM)                                                                        \
  hipLaunchKernelGGL((k_gemv_q8<RPW, EPI, NORM>), dim3((unsigned)((g.n + RPW * GV_WAVES - 1) / (RPW * GV_WAVES))), \
                     dim3(GV_THREADS), lds, s, g.x, g.gamma, g.eps, g.xq, g.xs, g.k, g.w_codes, g.w_scales, g.n,  \
                     g.bias, g.residual, g.out, g.q_codes, g.q_scales, qe)
  switch (g.epi) {
    case GV_RES:
      if (norm) GV_LAUNCH(4, GV_RES, true); else GV_LAUNCH(4, GV_RES, false);
      break;
    case GV_F32:
      if (norm) GV_LAUNCH(4, GV_F32, true); else GV_LAUNCH(4, GV_F32, false);
      break;
    case GV_SWIGLU:
      if (g.n % 64) return set_error(MI_ERR_UNSUPPORTED, "gemv: SwiGLU rows %d not a multiple of 64", g.n);
      if (norm) GV_LAUNCH(4, GV_SWIGLU, true); else GV_LAUNCH(4, GV_SWIGLU, false);
      break;
    case GV_QKV:
      if (qe.head_dim == 64 && g.n % 64 == 0) {
        if (norm) GV_LAUNCH(4, GV_QKV, true); else GV_LAUNCH(4, GV_QKV, false);
      } else if (qe.head_dim == 128 && g.n % 128 == 0) {
        if (norm) GV_LAUNCH(8, GV_QKV, true); else GV_LAUNCH(8, GV_QKV, false);
      } else {
        return set_error(MI_ERR_UNSUPPORTED, "gemv: attention inputs need head_dim 64 or 128 (got %d)", qe.head_dim);
      }
      break;
    default:
      return set_error(MI_ERR_INVALID_ARG, "gemv: epilogue %d", g.epi);
  }
#undef GV_LAUNCH
  MI_LAUNCH_CHECK("k_gemv_q8");
  return MI_OK;
}

// ---------------------------------------------------------------- single-query attention
constexpr int AD_THREADS = 256;  // 4 waves, 64 keys each per range tile

// Partial state of (head h, range r): part[((h * n_range + r) * (HD + 2))] = m, l, o[HD] (f64).
// m = max of the range's scores (-1e300 for an empty range), l = sum of e^(s - m), o = sum of
// e^(s - m) v.  Scores s = (q * 1/sqrt(hd)) . k in f64, as in the prefill kernel.
template <int HD>
__global__ void __launch_bounds__(AD_THREADS) k_attn_decode(const float* __restrict__ q,
                                                            const float* __restrict__ k_region,
                                                            const float* __restrict__ v_region,
                                                            const int32_t* __restrict__ pos_dev, int n_head,
                                                            int n_head_kv, int keys_per_range,
                                                            double* __restrict__ part) {
  constexpr int DPL = HD / 64;  // output dims per lane
  __shared__ double qs[HD];
  __shared__ double pw[AD_THREADS / 64][64];
  __shared__ double wst[AD_THREADS / 64][HD + 2];
  __shared__ double exp_tab[64];
  const int h = blockIdx.x, r = blockIdx.y, n_range = gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = h / (n_head / n_head_kv);
  const int n_kv = n_head_kv * HD;
  const int n_keys = *pos_dev + 1;
  const int j0 = r * keys_per_range, j1 = min(j0 + keys_per_range, n_keys);
  double* out = part + ((int64_t)h * n_range + r) * (HD + 2);
  if (j0 >= j1) {  // empty range (uniform for the workgroup)
    for (int i = tid; i < HD + 2; i += AD_THREADS) out[i] = i == 0 ? -1e300 : 0.0;
    return;
  }
  exp2_table_fill(exp_tab, tid);
  const double scale = 1.0 / sqrt((double)HD);
  for (int i = tid; i < HD; i += AD_THREADS) qs[i] = (double)q[h * HD + i] * scale;
  __syncthreads();
  double m_w = -1e300, l_w = 0.0, o_w[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) o_w[k] = 0.0;
  // wave w takes tiles w, w + 4, ... of 64 keys; lane <-> key for the scores, lane <-> dims for PV
  for (int t0 = j0 + 64 * wave; t0 < j1; t0 += 64 * (AD_THREADS / 64)) {
    const int j = t0 + lane;
    const int nk = min(64, j1 - t0);
    double s = -1e300;
    if (lane < nk) {
      const float4* kr = reinterpret_cast<const float4*>(k_region + (int64_t)j * n_kv + g * HD);
      double a = 0.0;
#pragma unroll 8
      for (int d4 = 0; d4 < HD / 4; ++d4) {
        const float4 kv = kr[d4];
        a = fma(qs[4 * d4], (double)kv.x, a);
        a = fma(qs[4 * d4 + 1], (double)kv.y, a);
        a = fma(qs[4 * d4 + 2], (double)kv.z, a);
        a = fma(qs[4 * d4 + 3], (double)kv.w, a);
      }
      s = a;
    }
    const double mt = wave_max_d(s);
    const double m_new = fmax(m_w, mt);
    const double p = lane < nk ? exp_f64(s - m_new, exp_tab) : 0.0;
    const double resc = exp_f64(m_w - m_new, exp_tab);  // 0 for the first tile (m_w = -1e300)
    l_w = l_w * resc + wave_sum_d(p);
#pragma unroll
    for (int k = 0; k < DPL; ++k) o_w[k] *= resc;
    m_w = m_new;
    pw[wave][lane] = p;  // the wave's own LDS row: its accesses complete in order
    for (int kk = 0; kk < nk; ++kk) {
      const double pk = pw[wave][kk];
      const float* vr = v_region + (int64_t)(t0 + kk) * n_kv + g * HD;
#pragma unroll
      for (int k = 0; k < DPL; ++k) o_w[k] = fma(pk, (double)vr[lane + 64 * k], o_w[k]);
    }
  }
  // merge the waves (fixed order)
  if (lane == 0) {
    wst[wave][0] = m_w;
    wst[wave][1] = l_w;
  }
#pragma unroll
  for (int k = 0; k < DPL; ++k) wst[wave][2 + lane + 64 * k] = o_w[k];
  __syncthreads();
  if (wave == 0) {
    double m = -1e300;
    for (int w = 0; w < AD_THREADS / 64; ++w) m = fmax(m, wst[w][0]);
    double l = 0.0, o[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] = 0.0;
    for (int w = 0; w < AD_THREADS / 64; ++w) {
      const double f = exp_f64(wst[w][0] - m, exp_tab);
      l = fma(wst[w][1], f, l);
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[k] = fma(wst[w][2 + lane + 64 * k], f, o[k]);
    }
    if (lane == 0) {
      out[0] = m;
      out[1] = l;
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) out[2 + lane + 64 * k] = o[k];
  }
}

// Merge the ranges of head h in order, normalize, round to f32, Q8_0 the head's output row.
template <int HD>
__global__ void __launch_bounds__(64) k_attn_decode_merge(const double* __restrict__ part, int n_range,
                                                          int8_t* __restrict__ q_codes, uint16_t* __restrict__ q_scales) {
  __shared__ double exp_tab[64];
  const int h = blockIdx.x, lane = threadIdx.x;
  exp2_table_fill(exp_tab, lane);
  __syncthreads();
  const double* ph = part + (int64_t)h * n_range * (HD + 2);
  double m = -1e300;
  for (int r = 0; r < n_range; ++r) m = fmax(m, ph[r * (HD + 2)]);
  // lane holds dims 4*lane .. 4*lane+3 (HD/4 lanes active)
  double l = 0.0, o[4] = {0.0, 0.0, 0.0, 0.0};
  for (int r = 0; r < n_range; ++r) {
    const double* pr = ph + r * (HD + 2);
    if (pr[1] == 0.0) continue;  // empty range
    const double f = exp_f64(pr[0] - m, exp_tab);
    l = fma(pr[1], f, l);
    if (lane < HD / 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = fma(pr[2 + 4 * lane + k], f, o[k]);
    }
  }
  const double inv = recip_f64(l);
  if (lane < HD / 4) {  // HD/4 = 16 or 32 lanes: whole groups of 8 per Q8_0 block
    float4 v;
    v.x = (float)(o[0] * inv);
    v.y = (float)(o[1] * inv);
    v.z = (float)(o[2] * inv);
    v.w = (float)(o[3] * inv);
    float d;
    const uint32_t qv = q8_block_quant4(v, d);
    reinterpret_cast<uint32_t*>(q_codes + (int64_t)h * HD)[lane] = qv;
    if ((lane & 7) == 0) q_scales[(int64_t)h * (HD / QK) + lane / 8] = f32_to_f16_bits(d);
  }
}

int attn_decode_ranges(int n_ctx, int* keys_per_range) {
  int kpr = 256;
  while ((n_ctx + kpr - 1) / kpr > AD_MAX_RANGES) kpr *= 2;
  *keys_per_range = kpr;
  return (n_ctx + kpr - 1) / kpr;
}

int launch_attn_decode(const float* q, const float* k_region, const float* v_region, const int32_t* pos_dev,
                       int n_ctx, int n_head, int n_head_kv, int head_dim, double* part, int8_t* q_codes,
                       uint16_t* q_scales, hipStream_t s) {
  int kpr = 0;
  const int n_range = attn_decode_ranges(n_ctx, &kpr);
  if (head_dim == 64) {
    hipLaunchKernelGGL(k_attn_decode<64>, dim3(n_head, n_range), dim3(AD_THREADS), 0, s, q, k_region, v_region,
                       pos_dev, n_head, n_head_kv, kpr, part);
    MI_LAUNCH_CHECK("k_attn_decode");
    hipLaunchKernelGGL(k_attn_decode_merge<64>, dim3(n_head), dim3(64), 0, s, part, n_range, q_codes, q_scales);
  } else if (head_dim == 128) {
    hipLaunchKernelGGL(k_attn_decode<128>, dim3(n_head, n_range), dim3(AD_THREADS), 0, s, q, k_region, v_region,
                       pos_dev, n_head, n_head_kv, kpr, part);
    MI_LAUNCH_CHECK("k_attn_decode");
    hipLaunchKernelGGL(k_attn_decode_merge<128>, dim3(n_head), dim3(64), 0, s, part, n_range, q_codes, q_scales);
  } else {
    return set_error(MI_ERR_UNSUPPORTED, "attention decode: head_dim %d", head_dim);
  }
  MI_LAUNCH_CHECK("k_attn_decode_merge");
  return MI_OK;
}

}  // namespace mi
