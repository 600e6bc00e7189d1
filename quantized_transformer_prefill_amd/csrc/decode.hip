// Decode step (one token at one position through the same layer sequence and KV regions as the
// prefill; the two-act engine of the walkthrough index, act two).  With one activation row every
// matmul is a matrix-vector product bound by HBM, and the attention has one query per head.
//
// k_gemv_q8: y[n] = sum_kb dx[kb] * dw[n][kb] * sum_32 qx * qw, one activation row.
//  * 16 waves per workgroup, RPW weight rows per wave in flight at once; a lane takes 16-byte
//    chunks (half a block) of every row, sdot4 gives the integer half-block sums, lane pairs
//    combine them to the block sum, and the exact f64 epilogue (block sum times dw, times dx,
//    one rounding per block) accumulates per lane; the lanes' partial sums then reduce in f64.
//  * The activation row is staged in LDS as codes + f64 scales.  The workgroup can build it
//    itself: from the f32 residual stream (RMSNorm in f64, one rounding to f32, Q8_0 -- the same
//    arithmetic as the prefill's k_rmsnorm_quant), or, for the output projection, by merging the
//    attention's per-range partial states -- so the decode step has no normalization or merge
//    kernels.  The weight loads of the first rows go out before this prologue.
//  * Epilogues: residual add (output projection, down projection), plain f32 (lm_head), the
//    attention inputs (bias, per-head QK RMSNorm, NeoX RoPE, K/V rows stored at the position; a
//    workgroup holds one head), SwiGLU + Q8_0 (a workgroup holds one interleaved group of 32
//    gate and 32 up rows, i.e. one Q8_0 block of the SwiGLU output).
//
// k_attn_decode: the query's keys 0..pos are split into fixed ranges (the grid depends only on
// n_ctx, so the launch can be captured once and replayed for any position); each workgroup
// computes the partial softmax state (max, sum, unnormalized output) of one head over one range in
// f64.  The output projection's prologue combines the ranges in order, normalizes, and quantizes
// each head's output row to Q8_0.
#include <algorithm>

#include "common.h"

namespace mi {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int GV_THREADS = 1024;  // 16 waves
constexpr int GV_WAVES = GV_THREADS / 64;

// f64 cross-lane reduction over a wave, every lane receiving the result: DPP row permutations for
// the 16-lane rows (each 32-bit half moved separately), a bit-mode swizzle across the two rows of a
// 32-lane half, then the two halves through scalar registers.  Each step combines a lane with its
// partner symmetrically, so every lane ends with the same value.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double swz16_f64(double v) {  // lane ^ 16 inside each 32-lane half
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)b, 0x401F);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)(b >> 32), 0x401F);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double lane_f64(double v, int l) {  // lane l's value, in every lane
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
template <bool MAX>
__device__ __forceinline__ double wave_reduce_f64(double v) {
  auto op = [](double a, double b) { return MAX ? fmax(a, b) : a + b; };
  v = op(v, dpp_f64<DPP_XOR1>(v));
  v = op(v, dpp_f64<DPP_XOR2>(v));
  v = op(v, dpp_f64<DPP_HALF_MIRROR>(v));
  v = op(v, dpp_f64<DPP_ROW_MIRROR>(v));
  v = op(v, swz16_f64(v));
  return op(lane_f64(v, 0), lane_f64(v, 32));
}

__device__ __forceinline__ double wave_sum_d(double v) { return wave_reduce_f64<false>(v); }
__device__ __forceinline__ double wave_max_d(double v) { return wave_reduce_f64<true>(v); }

// Prologue modes: the activation row comes as Q8_0 (GV_IN_Q8), is built from the f32 residual
// stream by RMSNorm + Q8_0 (GV_IN_NORM), or is the attention output merged from the per-range
// partial states of k_attn_decode, normalized and quantized per head (GV_IN_ATTN).
enum { GV_IN_Q8 = 0, GV_IN_NORM = 1, GV_IN_ATTN = 2 };

template <int HD>
__device__ __forceinline__ void attn_merge_head(const double* __restrict__ part, int n_range, int n_ne, int h, int lane,
                                                const double* exp_tab, int8_t* a_codes, double* a_d);

template <int RPW, int EPI, int PRO>
__global__ void __launch_bounds__(GV_THREADS) k_gemv_q8(const float* __restrict__ x, const float* __restrict__ gamma,
                                                       float eps, const int8_t* __restrict__ xq,
                                                       const uint16_t* __restrict__ xs, int K,
                                                       const int8_t* __restrict__ w_codes,
                                                       const uint16_t* __restrict__ w_scales, int N,
                                                       const float* __restrict__ bias, const float* residual,
                                                       float* out, int8_t* __restrict__ q_codes,
                                                       uint16_t* __restrict__ q_scales, GemvQkv qe, GemvAttnIn ai) {
  constexpr int RWG = RPW * GV_WAVES;  // weight rows per group
  constexpr int B = (RPW >= 8 || EPI == GV_QKV || EPI == GV_SWIGLU) ? 1 : (RPW >= 4 ? 2 : 4);  // 64-chunk steps of K in flight together
  extern __shared__ __align__(16) unsigned char gv_lds[];
  const int KB = K / QK;
  int8_t* a_codes = reinterpret_cast<int8_t*>(gv_lds);                           // [K]
  double* a_d = reinterpret_cast<double*>(gv_lds + ((K + 15) & ~15));             // [KB]
  float* y = reinterpret_cast<float*>(a_d + KB);                                   // [RWG]
  double* red = reinterpret_cast<double*>(y + RWG + (RWG & 1));                    // [GV_WAVES + 1]
  __shared__ double exp_tab[(EPI == GV_SWIGLU || PRO == GV_IN_ATTN) ? 64 : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunk = K / 16;
  const int n_groups = (N + RWG - 1) / RWG;

  // ---- requests that do not depend on the activation row go out first
  int64_t qpos = 0;
  if constexpr (EPI == GV_QKV) qpos = *qe.pos;
  constexpr int RS = RPW < 4 ? RPW : 4;  // rows of a wave whose loads are in flight together
  v4i wv[B][RS];
  uint16_t sv[B][RS];
  float bias_r[RPW];
  // 32-bit offsets from the uniform matrix bases (rows * K < 2^31 is checked by the launcher);
  // rows ib..ib+RS-1 of the wave's RPW
  auto load_batch = [&](int grp, int c0, int ib) {
    const int r0 = grp * RWG + wave * RPW + ib;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int ch = c0 + 64 * b + lane;
#pragma unroll
      for (int i = 0; i < RS; ++i) {
        const uint32_t r = (uint32_t)min(r0 + i, N - 1);  // rows past N re-read the last row; never stored
        if (ch < nchunk) {
          wv[b][i] = *reinterpret_cast<const v4i*>(w_codes + (r * (uint32_t)K + (uint32_t)ch * 16u));
          sv[b][i] = w_scales[r * (uint32_t)KB + (uint32_t)(ch >> 1)];
        }
      }
    }
  };
  load_batch(blockIdx.x, 0, 0);
  if constexpr (EPI == GV_QKV) {
    const int r0 = blockIdx.x * RWG + wave * RPW;
#pragma unroll
    for (int i = 0; i < RPW; ++i) bias_r[i] = bias ? bias[min(r0 + i, N - 1)] : 0.0f;
  }
  if constexpr (EPI == GV_SWIGLU || PRO == GV_IN_ATTN) exp2_table_fill(exp_tab, tid);

  // ---- the activation row -> LDS (codes, f64 scales)
  const int nvec = K / 4;
  if constexpr (PRO == GV_IN_ATTN) {  // wave w merges heads w, w + 16, ...
    __syncthreads();  // exp_tab
    const int n_ne = (*ai.pos + 1 + ai.keys_per_range - 1) / ai.keys_per_range;
    for (int h = wave; h < ai.n_head; h += GV_WAVES) {
      if (ai.head_dim == 64) attn_merge_head<64>(ai.part, ai.n_range, n_ne, h, lane, exp_tab, a_codes, a_d);
      else attn_merge_head<128>(ai.part, ai.n_range, n_ne, h, lane, exp_tab, a_codes, a_d);
    }
  } else if constexpr (PRO == GV_IN_NORM) {  // K <= GV_THREADS * 4: one float4 of x per thread, kept across both passes
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f), g = v;
    if (tid < nvec) {
      v = reinterpret_cast<const float4*>(x)[tid];
      g = reinterpret_cast<const float4*>(gamma)[tid];
    }
    const double a = v.x, b = v.y, c = v.z, d = v.w;
    double ss = wave_sum_d(a * a + b * b + c * c + d * d);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    if (wave == 0) {
      double t = lane < GV_WAVES ? red[lane] : 0.0;
      t = wave_sum_d(t);
      if (lane == 0) red[GV_WAVES] = t;
    }
    __syncthreads();
    const double inv_rms = recip_f64(sqrt(red[GV_WAVES] / (double)K + (double)eps));
    // groups of 8 lanes cover one block; a group is entirely inside or outside [0, nvec)
    if (tid < nvec) {
      float4 o;
      o.x = (float)((double)v.x * inv_rms * (double)g.x);
      o.y = (float)((double)v.y * inv_rms * (double)g.y);
      o.z = (float)((double)v.z * inv_rms * (double)g.z);
      o.w = (float)((double)v.w * inv_rms * (double)g.w);
      float dq;
      const uint32_t qv = q8_block_quant4(o, dq);
      reinterpret_cast<uint32_t*>(a_codes)[tid] = qv;
      if ((tid & 7) == 0) a_d[tid / 8] = (double)f16_bits_to_f32(f32_to_f16_bits(dq));
    }
  } else {
    for (int c4 = tid; c4 < nvec; c4 += GV_THREADS)
      reinterpret_cast<uint32_t*>(a_codes)[c4] = reinterpret_cast<const uint32_t*>(xq)[c4];
    for (int b = tid; b < KB; b += GV_THREADS) a_d[b] = (double)f16_bits_to_f32(xs[b]);
  }
  __syncthreads();

  for (int grp = blockIdx.x; grp < n_groups; grp += gridDim.x) {
    const int r0 = grp * RWG + wave * RPW;
    double acc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) acc[i] = 0.0;
#pragma unroll
    for (int ib = 0; ib < RPW; ib += RS) {
    if (ib || grp != (int)blockIdx.x) load_batch(grp, 0, ib);
#pragma unroll 1
    for (int c0 = 0; c0 < nchunk; c0 += 64 * B) {
      if (c0) load_batch(grp, c0, ib);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int ch = c0 + 64 * b + lane;
        const bool on = ch < nchunk;
        v4i xa = {0, 0, 0, 0};
        double da = 0.0;
        if (on) {
          xa = *reinterpret_cast<const v4i*>(a_codes + ch * 16);
          da = a_d[ch >> 1];
        }
#pragma unroll
        for (int i = 0; i < RS; ++i) {
          int isum = 0;
          double dw = 0.0;
          if (on) {
            isum = __builtin_amdgcn_sdot4(xa[0], wv[b][i][0], 0, false);
            isum = __builtin_amdgcn_sdot4(xa[1], wv[b][i][1], isum, false);
            isum = __builtin_amdgcn_sdot4(xa[2], wv[b][i][2], isum, false);
            isum = __builtin_amdgcn_sdot4(xa[3], wv[b][i][3], isum, false);
            dw = (double)f16_bits_to_f32(sv[b][i]);
          }
          isum += __builtin_amdgcn_update_dpp(0, isum, DPP_XOR1, 0xF, 0xF, false);  // both lanes of the pair: the block sum
          if (on && (lane & 1) == 0) acc[ib + i] = fma((double)isum * dw, da, acc[ib + i]);  // I*dw exact
        }
      }
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
    } else {
      if (lane == 0) {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          double v = acc[i];
          if (EPI == GV_QKV) v += (double)bias_r[i];
          y[wave * RPW + i] = (float)v;
        }
      }
      __syncthreads();
      if constexpr (EPI == GV_SWIGLU) {
        // rows 64p..64p+31 are gate rows 32p.., rows 64p+32..64p+63 up rows 32p..: one Q8_0 block
        if (tid < 8) {
          float4 sw;
          sw.x = swiglu_f32(y[4 * tid + 0], y[32 + 4 * tid + 0], exp_tab);
          sw.y = swiglu_f32(y[4 * tid + 1], y[32 + 4 * tid + 1], exp_tab);
          sw.z = swiglu_f32(y[4 * tid + 2], y[32 + 4 * tid + 2], exp_tab);
          sw.w = swiglu_f32(y[4 * tid + 3], y[32 + 4 * tid + 3], exp_tab);
          float d;
          const uint32_t q = q8_block_quant4(sw, d);
          reinterpret_cast<uint32_t*>(q_codes + (int64_t)grp * QK)[tid] = q;
          if (tid == 0) q_scales[grp] = f32_to_f16_bits(d);
        }
      } else {  // GV_QKV: this group's rows are one head of Q, K or V (one group per workgroup)
        const int hd = qe.head_dim, half = hd / 2;
        const int c0 = grp * RWG;
        if (c0 >= qe.n_q + qe.n_kv) {  // V head: stored as is
          for (int i = tid; i < hd; i += GV_THREADS) qe.v_region[qpos * qe.n_kv + (c0 - qe.n_q - qe.n_kv) + i] = y[i];
        } else {
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
            const double2 cs = reinterpret_cast<const double2*>(qe.rope)[qpos * half + i];
            const float o0 = (float)((double)a * cs.x - (double)b * cs.y);
            const float o1 = (float)((double)a * cs.y + (double)b * cs.x);
            float* dst = isq ? qe.q_out + c0 : qe.k_region + qpos * qe.n_kv + (c0 - qe.n_q);
            dst[i] = o0;
            dst[i + half] = o1;
          }
        }
      }
      __syncthreads();  // y is rewritten by the next group
    }
  }
}

int launch_gemv_q8(const GemvArgs& g, hipStream_t s) {
  const bool norm = g.x != nullptr;
  if (g.attn.part) {  // the output projection: its input is the merged attention row
    if (g.epi != GV_RES || norm || g.k != g.attn.n_head * g.attn.head_dim)
      return set_error(MI_ERR_INVALID_ARG, "gemv: attention-merge input needs the residual epilogue");
  }
  const int KB = g.k / QK;
  const size_t lds = (size_t)((g.k + 15) & ~15) + sizeof(double) * KB + sizeof(float) * 130 +
                     sizeof(double) * (GV_WAVES + 1);
  if (g.k % QK || g.k <= 0 || lds > 64 * 1024 || ((norm || g.attn.part) && g.k > GV_THREADS * 4) ||
      (int64_t)g.n * g.k >= ((int64_t)1 << 31))
    return set_error(MI_ERR_UNSUPPORTED, "gemv: K %d (multiple of 32, LDS %zu bytes, <= %d with the norm)", g.k, lds,
                     GV_THREADS * 4);
  GemvQkv qe = g.qkv;
  // enough workgroups to keep every CU busy, looping over row groups beyond that
  const int max_wg = 2 * 256;
  auto grid = [&](int rwg) { return dim3((unsigned)std::min((g.n + rwg - 1) / rwg, max_wg)); };
#define GV_LAUNCH(RPW, EPI, NORM)                                                                          \
  hipLaunchKernelGGL((k_gemv_q8<RPW, EPI, NORM>), grid(RPW * GV_WAVES), dim3(GV_THREADS), lds, s, g.x, g.gamma, \
                     g.eps, g.xq, g.xs, g.k, g.w_codes, g.w_scales, g.n, g.bias, g.residual, g.out, g.q_codes,     \
                     g.q_scales, qe, g.attn)
  switch (g.epi) {
    case GV_RES:
    case GV_F32: {
      // one row per wave while that gives fewer groups than CUs x 2, else four
      const bool small = g.n <= 16 * max_wg;
      if (g.epi == GV_RES) {
        if (g.attn.part) {
          if (small) GV_LAUNCH(1, GV_RES, GV_IN_ATTN); else GV_LAUNCH(4, GV_RES, GV_IN_ATTN);
        } else if (small) {
          if (norm) GV_LAUNCH(1, GV_RES, GV_IN_NORM); else GV_LAUNCH(1, GV_RES, GV_IN_Q8);
        } else {
          if (norm) GV_LAUNCH(4, GV_RES, GV_IN_NORM); else GV_LAUNCH(4, GV_RES, GV_IN_Q8);
        }
      } else {
        if (small) { if (norm) GV_LAUNCH(1, GV_F32, GV_IN_NORM); else GV_LAUNCH(1, GV_F32, GV_IN_Q8); }
        else { if (norm) GV_LAUNCH(4, GV_F32, GV_IN_NORM); else GV_LAUNCH(4, GV_F32, GV_IN_Q8); }
      }
      break;
    }
    case GV_SWIGLU:
      if (g.n % 64) return set_error(MI_ERR_UNSUPPORTED, "gemv: SwiGLU rows %d not a multiple of 64", g.n);
      if (norm) GV_LAUNCH(4, GV_SWIGLU, GV_IN_NORM); else GV_LAUNCH(4, GV_SWIGLU, GV_IN_Q8);
      break;
    case GV_QKV:
      if (g.n / (qe.head_dim > 0 ? qe.head_dim : 1) > max_wg)
        return set_error(MI_ERR_UNSUPPORTED, "gemv: more than %d heads", max_wg);
      if (qe.head_dim == 64 && g.n % 64 == 0) {
        if (norm) GV_LAUNCH(4, GV_QKV, GV_IN_NORM); else GV_LAUNCH(4, GV_QKV, GV_IN_Q8);
      } else if (qe.head_dim == 128 && g.n % 128 == 0) {
        if (norm) GV_LAUNCH(8, GV_QKV, GV_IN_NORM); else GV_LAUNCH(8, GV_QKV, GV_IN_Q8);
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
constexpr int AD_THREADS = 256;  // 4 waves; a wave takes 64 keys of its range per step

// Keys 0..pos of head h are split into ranges of keys_per_range; workgroup (h, r) takes range r
// and writes its partial state to part[(h * n_range + r) * (HD + 2)] = m, l, o[HD] (f64): m the
// range's largest score, l = sum e^(s - m), o = sum e^(s - m) v, with s = (q * 1/sqrt(hd)) . k as
// in the prefill kernel.  Ranges past pos write nothing.  The output projection merges the ranges.
//
// A wave takes 64-key tiles.  Scores: lane <-> key, the dot product in four independent f64 chains.
// Weighted sum: each V load instruction brings KG keys x all HD dims as float4s (lane <-> key group
// kg, dim quad), so a lane accumulates 4 dims over the keys kg, kg + KG, ... of the tile in four
// chains; the key groups and the waves are summed in the final merge through LDS (fixed order).
template <int HD>
__global__ void __launch_bounds__(AD_THREADS) k_attn_decode(const float* __restrict__ q,
                                                            const float* __restrict__ k_region,
                                                            const float* __restrict__ v_region,
                                                            const int32_t* __restrict__ pos_dev, int n_head,
                                                            int n_head_kv, int keys_per_range,
                                                            double* __restrict__ part) {
  constexpr int NW = AD_THREADS / 64;
  constexpr int DQ = HD / 4;        // dim quads
  constexpr int KG = 64 / DQ;       // keys per V load instruction: 4 (HD 64), 2 (HD 128)
  constexpr int VI = 64 / KG;       // V load instructions per 64-key tile
  constexpr bool V_EARLY = HD == 64;  // V requested together with K (registers allow it)
  // wave-private LDS: the query (f64, scaled), the e^x table and the tile's weights, so no wave
  // waits for another before the final merge (a wave's own LDS accesses complete in order)
  __shared__ double qs[NW][HD];
  __shared__ double etab[NW][64];
  __shared__ double pw[NW][64];
  __shared__ double wst[NW][KG][HD];
  __shared__ double wml[NW][2];
  const int h = blockIdx.x, r = blockIdx.y, n_range = gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = h / (n_head / n_head_kv);
  const int n_kv = n_head_kv * HD;
  const int n_keys = *pos_dev + 1;
  const int j0 = r * keys_per_range, j1 = min(j0 + keys_per_range, n_keys);
  if (j0 >= j1) return;  // uniform for the workgroup
  const int kg = lane / DQ, dq = lane % DQ;
  const float* kbase = k_region + g * HD;
  const float* vbase = v_region + g * HD + 4 * dq;
  double* qw = qs[wave];
  const double* tab = etab[wave];
  exp2_table_fill(etab[wave], lane);
  double m_w = -1e300, l_w = 0.0, o[4] = {0.0, 0.0, 0.0, 0.0};
  const int t_first = j0 + 64 * wave;
  for (int t0 = t_first; t0 < j1; t0 += 64 * NW) {
    const int nk = min(64, j1 - t0);
    // rows past the tile's keys re-read its last key (their weights are 0; the row is one this call
    // or an earlier one wrote)
    float4 kreg[DQ];
    {
      const float4* kr = reinterpret_cast<const float4*>(kbase + (int64_t)(t0 + min(lane, nk - 1)) * n_kv);
#pragma unroll
      for (int d4 = 0; d4 < DQ; ++d4) kreg[d4] = kr[d4];
    }
    float4 vreg[VI];
    auto load_v = [&]() {
#pragma unroll
      for (int i = 0; i < VI; ++i)
        vreg[i] = *reinterpret_cast<const float4*>(vbase + (int64_t)(t0 + min(KG * i + kg, nk - 1)) * n_kv);
    };
    if constexpr (V_EARLY) load_v();
    if (t0 == t_first) {  // the query, scaled by 1/sqrt(hd) in f64, while the loads are in flight
      const double scale = 1.0 / sqrt((double)HD);
      for (int i = lane; i < HD; i += 64) qw[i] = (double)q[h * HD + i] * scale;
    }
    double a[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int d4 = 0; d4 < DQ; ++d4) {
      const double2 q01 = *reinterpret_cast<const double2*>(&qw[4 * d4]);
      const double2 q23 = *reinterpret_cast<const double2*>(&qw[4 * d4 + 2]);
      a[0] = fma(q01.x, (double)kreg[d4].x, a[0]);
      a[1] = fma(q01.y, (double)kreg[d4].y, a[1]);
      a[2] = fma(q23.x, (double)kreg[d4].z, a[2]);
      a[3] = fma(q23.y, (double)kreg[d4].w, a[3]);
    }
    if constexpr (!V_EARLY) {
      asm volatile("" ::: "memory");  // the V loads reuse the K registers: issued after the scores
      load_v();
    }
    const double s = lane < nk ? (a[0] + a[1]) + (a[2] + a[3]) : -1e300;
    const double m_new = fmax(m_w, wave_reduce_f64<true>(s));
    const double p = lane < nk ? exp_f64(s - m_new, tab) : 0.0;
    const double resc = exp_f64(m_w - m_new, tab);  // 0 for the first tile (m_w = -1e300)
    l_w = l_w * resc + wave_reduce_f64<false>(p);
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] *= resc;
    m_w = m_new;
    pw[wave][lane] = p;
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const double pk = pw[wave][KG * i + kg];
      o[0] = fma(pk, (double)vreg[i].x, o[0]);
      o[1] = fma(pk, (double)vreg[i].y, o[1]);
      o[2] = fma(pk, (double)vreg[i].z, o[2]);
      o[3] = fma(pk, (double)vreg[i].w, o[3]);
    }
  }
  // merge the waves and key groups (fixed order)
#pragma unroll
  for (int c = 0; c < 4; ++c) wst[wave][kg][4 * dq + c] = o[c];
  if (lane == 0) {
    wml[wave][0] = m_w;
    wml[wave][1] = l_w;
  }
  __syncthreads();
  if (wave == 0) {
    double m = -1e300;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = fmax(m, wml[w][0]);
    double f[NW], l = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      f[w] = exp_f64(wml[w][0] - m, tab);
      l = fma(wml[w][1], f[w], l);
    }
    double* out = part + ((int64_t)h * n_range + r) * (HD + 2);
    if (lane == 0) {
      out[0] = m;
      out[1] = l;
    }
#pragma unroll
    for (int k = 0; k < HD / 64; ++k) {
      const int d = lane + 64 * k;
      double od = 0.0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        double ow = 0.0;
#pragma unroll
        for (int gg = 0; gg < KG; ++gg) ow += wst[w][gg][d];
        od = fma(ow, f[w], od);
      }
      out[2 + d] = od;
    }
  }
}

// Merge head h's n_ne ranges in order, normalize, round to f32 and Q8_0 into the LDS row (one
// wave; lane holds dims 4*lane..4*lane+3, HD/4 lanes = whole groups of 8 per block).
template <int HD>
__device__ __forceinline__ void attn_merge_head(const double* __restrict__ part, int n_range, int n_ne, int h, int lane,
                                                const double* exp_tab, int8_t* a_codes, double* a_d) {
  const double* ph = part + (int64_t)h * n_range * (HD + 2);
  double mr = -1e300, lr = 0.0;
  if (lane < n_ne) {  // one range per lane (n_ne <= AD_MAX_RANGES <= 64)
    mr = ph[lane * (HD + 2)];
    lr = ph[lane * (HD + 2) + 1];
  }
  const double m = wave_max_d(mr);
  const double f_own = lane < n_ne ? exp_f64(mr - m, exp_tab) : 0.0;
  const double l = wave_sum_d(lr * f_own);
  double o[4] = {0.0, 0.0, 0.0, 0.0};
  for (int rr = 0; rr < n_ne; ++rr) {
    const double f = lane_f64(f_own, rr);
    if (lane < HD / 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = fma(ph[rr * (HD + 2) + 2 + 4 * lane + k], f, o[k]);
    }
  }
  const double inv = recip_f64(l);
  if (lane < HD / 4) {
    float4 v;
    v.x = (float)(o[0] * inv);
    v.y = (float)(o[1] * inv);
    v.z = (float)(o[2] * inv);
    v.w = (float)(o[3] * inv);
    float d;
    const uint32_t qv = q8_block_quant4(v, d);
    reinterpret_cast<uint32_t*>(a_codes + h * HD)[lane] = qv;
    if ((lane & 7) == 0) a_d[h * (HD / QK) + lane / 8] = (double)f16_bits_to_f32(f32_to_f16_bits(d));
  }
}

int attn_decode_ranges(int n_ctx, int* keys_per_range) {
  int kpr = 256;  // one 64-key tile per wave
  while ((n_ctx + kpr - 1) / kpr > AD_MAX_RANGES) kpr *= 2;
  *keys_per_range = kpr;
  return (n_ctx + kpr - 1) / kpr;
}

int launch_attn_decode(const float* q, const float* k_region, const float* v_region, const int32_t* pos_dev,
                       int n_ctx, int n_head, int n_head_kv, int head_dim, double* part, hipStream_t s) {
  int kpr = 0;
  const int n_range = attn_decode_ranges(n_ctx, &kpr);
  if (head_dim == 64)
    hipLaunchKernelGGL(k_attn_decode<64>, dim3(n_head, n_range), dim3(AD_THREADS), 0, s, q, k_region, v_region,
                       pos_dev, n_head, n_head_kv, kpr, part);
  else if (head_dim == 128)
    hipLaunchKernelGGL(k_attn_decode<128>, dim3(n_head, n_range), dim3(AD_THREADS), 0, s, q, k_region, v_region,
                       pos_dev, n_head, n_head_kv, kpr, part);
  else
    return set_error(MI_ERR_UNSUPPORTED, "attention decode: head_dim %d", head_dim);
  MI_LAUNCH_CHECK("k_attn_decode");
  return MI_OK;
}

}  // namespace mi
