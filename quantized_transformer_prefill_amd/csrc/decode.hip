// Decode step (one token at one position through the same layer sequence and KV regions as the
// prefill; the two-act engine of the walkthrough index, act two).  With one activation row every
// matmul is a matrix-vector product bound by HBM, and the attention has one query per head.
//
// k_gemv_q8: y[n] = sum_kb dx[kb] * dw[n][kb] * sum_32 qx * qw, one activation row.
//  * 16 waves per workgroup, RPW weight rows per wave (up to 4 in flight at once); a lane takes
//    16-byte chunks (half a block) of every row, sdot4 gives the integer half-block sums, lane
//    pairs combine them to the block sum, and the exact f64 epilogue (block sum times dw, times
//    dx, one rounding per block) accumulates per lane; the lanes' partial sums then reduce in f64.
//    The weight loads are double buffered: the next step's requests go out before this step's
//    math, and are unconditional (clamped addresses) so that the wait for one buffer never
//    includes the other's requests.
//  * The activation row is staged in LDS as codes + f64 scales.  The workgroup can build it
//    itself from the f32 residual stream (RMSNorm in f64, one rounding to f32, Q8_0 -- the same
//    arithmetic as the prefill's k_rmsnorm_quant), so the decode step has no normalization
//    kernels.  The weight loads of the first rows go out before this prologue.
//  * Epilogues: residual add (output projection, down projection), plain f32 with an optional
//    bias (lm_head; the Q|K|V rows), SwiGLU + Q8_0 (a workgroup holds one interleaved group of 32
//    gate and 32 up rows, i.e. one Q8_0 block of the SwiGLU output).  Every epilogue is per row,
//    so a workgroup takes 16 or 64 rows and even the small matrices spread over the chip.
//
// k_qkv_finish: the per-head steps after the Q|K|V rows (per-head QK RMSNorm, NeoX RoPE at the
// position, the K and V rows stored in the regions), one single-wave workgroup per head.
//
// k_attn_decode: the query's keys 0..pos are split into fixed ranges (the grid depends only on
// n_ctx, so the launch can be captured once and replayed for any position); each workgroup
// computes the partial softmax state (max, sum, unnormalized output) of one head over one range in
// f64.  k_attn_merge combines a head's ranges in order, normalizes, and quantizes the head's
// output row to Q8_0, the output projection's input.
#include <algorithm>

#include "common.h"

namespace mi {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int GV_THREADS = 1024;  // 16 waves
constexpr int GV_WAVES = GV_THREADS / 64;
constexpr int GV_NORM_K = 4096;                                  // widest row the norm prologue takes
constexpr int GV_NV = (GV_NORM_K / 4 + GV_THREADS - 1) / GV_THREADS;  // float4s of the row per thread
constexpr int GV_RPW_SWIGLU = 64 / GV_WAVES;                       // a SwiGLU group is 64 rows
constexpr int GV_MAX_WG = (2048 / GV_THREADS) * 256;               // grid cap: two workgroups per CU

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

// Prologue modes: the activation row comes as Q8_0 (GV_IN_Q8) or is built from the f32 residual
// stream by RMSNorm + Q8_0 (GV_IN_NORM).
enum { GV_IN_Q8 = 0, GV_IN_NORM = 1 };

// The plain-epilogue one-row-per-wave instance (the Q|K|V rows: 288 workgroups at the 7B shape) is
// held to 64 registers, so that two workgroups fit a CU and the whole grid is resident at once.
template <int RPW, int EPI, int PRO>
__global__ void __launch_bounds__(GV_THREADS, (RPW == 1 && EPI == GV_F32) ? 8 : 1) k_gemv_q8(const float* __restrict__ x, const float* __restrict__ gamma,
                                                       float eps, const int8_t* __restrict__ xq,
                                                       const uint16_t* __restrict__ xs, int K,
                                                       const int8_t* __restrict__ w_codes,
                                                       const uint16_t* __restrict__ w_scales, int N,
                                                       const float* __restrict__ bias, const float* residual,
                                                       float* out, int8_t* __restrict__ q_codes,
                                                       uint16_t* __restrict__ q_scales) {
  constexpr int RWG = RPW * GV_WAVES;  // weight rows per group
  // 64-chunk steps of K per load batch; two batches are in flight (double buffered)
  constexpr int B = (EPI == GV_SWIGLU || RPW >= 4) ? 1 : 2;
  extern __shared__ __align__(16) unsigned char gv_lds[];
  const int KB = K / QK;
  int8_t* a_codes = reinterpret_cast<int8_t*>(gv_lds);                           // [K]
  double* a_d = reinterpret_cast<double*>(gv_lds + ((K + 15) & ~15));             // [KB]
  float* y = reinterpret_cast<float*>(a_d + KB);                                   // [RWG]
  double* red = reinterpret_cast<double*>(y + RWG + (RWG & 1));                    // [GV_WAVES + 1]
  __shared__ double exp_tab[EPI == GV_SWIGLU ? 64 : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunk = K / 16;
  const int n_groups = (N + RWG - 1) / RWG;

  // ---- requests that do not depend on the activation row go out first
  constexpr int RS = RPW < 4 ? RPW : 4;  // rows of a wave whose loads are in flight together
  struct Buf {
    v4i wv[B][RS];
    uint16_t sv[B][RS];
  };
  Buf buf0, buf1;  // two steps of K in flight: the next step's loads go out before this step's math
  // 32-bit offsets from the uniform matrix bases (rows * K < 2^31 is checked by the launcher);
  // rows ib..ib+RS-1 of the wave's RPW
  auto load_batch = [&](Buf& bf, int grp, int c0, int ib) {
    const int r0 = grp * RWG + wave * RPW + ib;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int ch = c0 + 64 * b + lane;
#pragma unroll
      for (int i = 0; i < RS; ++i) {
        // rows past N re-read the last row and chunks past the row its last chunk (never used):
        // the loads are unconditional, so the waits for one buffer never cover the other's
        const uint32_t r = (uint32_t)min(r0 + i, N - 1);
        const uint32_t c = (uint32_t)min(ch, nchunk - 1);
        bf.wv[b][i] = *reinterpret_cast<const v4i*>(w_codes + (r * (uint32_t)K + c * 16u));
        bf.sv[b][i] = w_scales[r * (uint32_t)KB + (c >> 1)];
      }
    }
  };
  load_batch(buf0, blockIdx.x, 0, 0);
  if constexpr (EPI == GV_SWIGLU) exp2_table_fill(exp_tab, tid);

  // ---- the activation row -> LDS (codes, f64 scales)
  const int nvec = K / 4;
  if constexpr (PRO == GV_IN_NORM) {  // K <= GV_NORM_K: NV float4s of x per thread, kept across both passes
    float4 v[GV_NV], g[GV_NV];
    double sq = 0.0;
#pragma unroll
    for (int j = 0; j < GV_NV; ++j) {
      const int c4 = tid + j * GV_THREADS;
      v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      g[j] = v[j];
      if (c4 < nvec) {
        v[j] = reinterpret_cast<const float4*>(x)[c4];
        g[j] = reinterpret_cast<const float4*>(gamma)[c4];
      }
      const double a = v[j].x, b = v[j].y, c = v[j].z, d = v[j].w;
      sq += a * a + b * b + c * c + d * d;
    }
    double ss = wave_sum_d(sq);
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
#pragma unroll
    for (int j = 0; j < GV_NV; ++j) {
      const int c4 = tid + j * GV_THREADS;
      if (c4 < nvec) {
        float4 o;
        o.x = (float)((double)v[j].x * inv_rms * (double)g[j].x);
        o.y = (float)((double)v[j].y * inv_rms * (double)g[j].y);
        o.z = (float)((double)v[j].z * inv_rms * (double)g[j].z);
        o.w = (float)((double)v[j].w * inv_rms * (double)g[j].w);
        float dq;
        const uint32_t qv = q8_block_quant4(o, dq);
        reinterpret_cast<uint32_t*>(a_codes)[c4] = qv;
        if ((c4 & 7) == 0) a_d[c4 / 8] = (double)f16_bits_to_f32(f32_to_f16_bits(dq));
      }
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
    // one step: B chunks of 16 bytes per lane of RS rows, the block sums in the exact f64 epilogue
    auto step = [&](const Buf& bf, int c0, double* a) {
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
            isum = __builtin_amdgcn_sdot4(xa[0], bf.wv[b][i][0], 0, false);
            isum = __builtin_amdgcn_sdot4(xa[1], bf.wv[b][i][1], isum, false);
            isum = __builtin_amdgcn_sdot4(xa[2], bf.wv[b][i][2], isum, false);
            isum = __builtin_amdgcn_sdot4(xa[3], bf.wv[b][i][3], isum, false);
            dw = (double)f16_bits_to_f32(bf.sv[b][i]);
          }
          isum += __builtin_amdgcn_update_dpp(0, isum, DPP_XOR1, 0xF, 0xF, false);  // both lanes of the pair: the block sum
          if (on && (lane & 1) == 0) a[i] = fma((double)isum * dw, da, a[i]);  // I*dw exact
        }
      }
    };
    constexpr int STEP = 64 * B;
#pragma unroll
    for (int ib = 0; ib < RPW; ib += RS) {
      if (ib || grp != (int)blockIdx.x) load_batch(buf0, grp, 0, ib);
#pragma unroll 1
      for (int c0 = 0;; c0 += 2 * STEP) {
        load_batch(buf1, grp, c0 + STEP, ib);
        step(buf0, c0, acc + ib);
        if (c0 + 2 * STEP >= nchunk) {  // uniform
          step(buf1, c0 + STEP, acc + ib);
          break;
        }
        load_batch(buf0, grp, c0 + 2 * STEP, ib);
        step(buf1, c0 + STEP, acc + ib);
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
            float v;
            if (EPI == GV_RES) v = residual[r] + (float)acc[i];
            else v = (float)(bias ? acc[i] + (double)bias[r] : acc[i]);  // one rounding
            out[r] = v;
          }
        }
      }
    } else {  // GV_SWIGLU
      if (lane == 0) {
#pragma unroll
        for (int i = 0; i < RPW; ++i) y[wave * RPW + i] = (float)acc[i];
      }
      __syncthreads();
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
      __syncthreads();  // y is rewritten by the next group
    }
  }
}

int launch_gemv_q8(const GemvArgs& g, hipStream_t s) {
  const bool norm = g.x != nullptr;
  const int KB = g.k / QK;
  const size_t lds = (size_t)((g.k + 15) & ~15) + sizeof(double) * KB + sizeof(float) * 130 +
                     sizeof(double) * (GV_WAVES + 1);
  if (g.k % QK || g.k <= 0 || lds > 64 * 1024 || (norm && g.k > GV_NORM_K) ||
      (int64_t)g.n * g.k >= ((int64_t)1 << 31))
    return set_error(MI_ERR_UNSUPPORTED, "gemv: K %d (multiple of 32, LDS %zu bytes, <= %d with the norm)", g.k, lds,
                     GV_NORM_K);
  if (g.bias && g.epi != GV_F32) return set_error(MI_ERR_INVALID_ARG, "gemv: a bias needs the plain f32 epilogue");
  // enough workgroups to keep every CU busy, looping over row groups beyond that
  const int max_wg = GV_MAX_WG;
  auto grid = [&](int rwg) { return dim3((unsigned)std::min((g.n + rwg - 1) / rwg, max_wg)); };
#define GV_LAUNCH(RPW, EPI, NORM)                                                                          \
  hipLaunchKernelGGL((k_gemv_q8<RPW, EPI, NORM>), grid(RPW * GV_WAVES), dim3(GV_THREADS), lds, s, g.x, g.gamma, \
                     g.eps, g.xq, g.xs, g.k, g.w_codes, g.w_scales, g.n, g.bias, g.residual, g.out, g.q_codes,     \
                     g.q_scales)
  switch (g.epi) {
    case GV_RES:
    case GV_F32: {
      // one row per wave while that gives fewer groups than CUs x 2, else four
      const bool small = g.n <= GV_WAVES * max_wg;
      if (g.epi == GV_RES) {
        if (small) {
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
      if (norm) GV_LAUNCH(GV_RPW_SWIGLU, GV_SWIGLU, GV_IN_NORM); else GV_LAUNCH(GV_RPW_SWIGLU, GV_SWIGLU, GV_IN_Q8);
      break;
    default:
      return set_error(MI_ERR_INVALID_ARG, "gemv: epilogue %d", g.epi);
  }
#undef GV_LAUNCH
  MI_LAUNCH_CHECK("k_gemv_q8");
  return MI_OK;
}

// The steps after the Q|K|V rows of one token (bias already added, one rounding): workgroup b < n_head
// takes Q head b, then the K heads, then the V heads.  Q and K: [per-head RMSNorm in f64, one
// rounding to f32], NeoX RoPE of the pair (i, i + hd/2) in f64 at the position, one rounding; Q in
// place, K to its region row.  V: copied to its region row.  One wave; lane i < hd/2 takes pair i.
template <int HD>
__global__ void __launch_bounds__(64) k_qkv_finish(float* __restrict__ qkv, const int32_t* __restrict__ pos_dev,
                                                   const double2* __restrict__ rope, int n_head, int n_head_kv,
                                                   const float* __restrict__ q_norm, const float* __restrict__ k_norm,
                                                   float eps, float* __restrict__ k_region,
                                                   float* __restrict__ v_region) {
  constexpr int HALF = HD / 2;
  static_assert(HALF <= 64, "one pair per lane");
  const int b = blockIdx.x, lane = threadIdx.x;
  const int64_t p = *pos_dev;
  const int n_kv = n_head_kv * HD;
  const int nq = n_head * HD;
  if (b >= n_head + n_head_kv) {  // V head
    const int c = (b - n_head - n_head_kv) * HD;
    for (int i = lane; i < HD; i += 64) v_region[p * n_kv + c + i] = qkv[nq + n_kv + c + i];
    return;
  }
  const bool isq = b < n_head;
  const int c = isq ? b * HD : nq + (b - n_head) * HD;  // the head's offset in the Q|K|V row
  const float* gam = isq ? q_norm : k_norm;
  const bool on = lane < HALF;
  float a = on ? qkv[c + lane] : 0.0f, bb = on ? qkv[c + lane + HALF] : 0.0f;
  if (gam) {  // per-head RMSNorm in f64, one rounding
    const double ss = wave_sum_d((double)a * (double)a + (double)bb * (double)bb);
    const double ir = recip_f64(sqrt(ss / (double)HD + (double)eps));
    if (on) {
      a = (float)((double)a * ir * (double)gam[lane]);
      bb = (float)((double)bb * ir * (double)gam[lane + HALF]);
    }
  }
  if (on) {
    float* dst = isq ? qkv + c : k_region + p * n_kv + (b - n_head) * HD;
    const double2 cs = rope[p * HALF + lane];
    dst[lane] = (float)((double)a * cs.x - (double)bb * cs.y);
    dst[lane + HALF] = (float)((double)a * cs.y + (double)bb * cs.x);
  }
}

int launch_qkv_finish(float* qkv, const int32_t* pos_dev, const double* rope, int n_head, int n_head_kv,
                      int head_dim, const float* q_norm, const float* k_norm, float eps, float* k_region,
                      float* v_region, hipStream_t s) {
  const dim3 grid(n_head + 2 * n_head_kv);
  const double2* r = reinterpret_cast<const double2*>(rope);
  if (head_dim == 64)
    hipLaunchKernelGGL(k_qkv_finish<64>, grid, dim3(64), 0, s, qkv, pos_dev, r, n_head, n_head_kv, q_norm, k_norm,
                       eps, k_region, v_region);
  else if (head_dim == 128)
    hipLaunchKernelGGL(k_qkv_finish<128>, grid, dim3(64), 0, s, qkv, pos_dev, r, n_head, n_head_kv, q_norm, k_norm,
                       eps, k_region, v_region);
  else
    return set_error(MI_ERR_UNSUPPORTED, "attention inputs: head_dim %d (supported: 64, 128)", head_dim);
  MI_LAUNCH_CHECK("k_qkv_finish");
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

// Merge head h's n_ne ranges in order, normalize, round to f32 and Q8_0 (one wave; lane holds dims
// 4*lane..4*lane+3, HD/4 lanes = whole groups of 8 per block).
template <int HD>
__device__ __forceinline__ void attn_merge_head(const double* __restrict__ part, int n_range, int n_ne, int h, int lane,
                                                const double* exp_tab, int8_t* a_codes, uint16_t* a_scales) {
  const double* ph = part + (int64_t)h * n_range * (HD + 2);
  double mr = -1e300, lr = 0.0;
  if (lane < n_ne) {  // one range per lane (n_ne <= AD_MAX_RANGES <= 64)
    mr = ph[lane * (HD + 2)];
    lr = ph[lane * (HD + 2) + 1];
  }
  const double m = wave_max_d(mr);
  const double f_own = lane < n_ne ? exp_f64(mr - m, exp_tab) : 0.0;
  const double l = wave_sum_d(lr * f_own);
  // every range's partial output requested at once (they do not depend on the max), then summed
  // in range order
  double2 po[AD_MAX_RANGES][2];
#pragma unroll
  for (int rr = 0; rr < AD_MAX_RANGES; ++rr) {
    const int r = rr < n_ne ? rr : 0;  // ranges past n_ne re-read range 0 (unused)
    const double2* src = reinterpret_cast<const double2*>(ph + r * (HD + 2) + 2) + 2 * (lane & (HD / 4 - 1));
    po[rr][0] = src[0];
    po[rr][1] = src[1];
  }
  double o[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int rr = 0; rr < AD_MAX_RANGES; ++rr) {
    if (rr < n_ne) {  // uniform
      const double f = lane_f64(f_own, rr);
      o[0] = fma(po[rr][0].x, f, o[0]);
      o[1] = fma(po[rr][0].y, f, o[1]);
      o[2] = fma(po[rr][1].x, f, o[2]);
      o[3] = fma(po[rr][1].y, f, o[3]);
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
    if ((lane & 7) == 0) a_scales[h * (HD / QK) + lane / 8] = f32_to_f16_bits(d);
  }
}

// The output projection's input row: wave w of workgroup b merges head 4b + w.
template <int HD>
__global__ void __launch_bounds__(256) k_attn_merge(const double* __restrict__ part, int n_range, int keys_per_range,
                                                    const int32_t* __restrict__ pos_dev, int n_head,
                                                    int8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  __shared__ double exp_tab[64];
  exp2_table_fill(exp_tab, threadIdx.x);
  __syncthreads();
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n_ne = (*pos_dev + keys_per_range) / keys_per_range;  // ranges holding keys 0..pos
  if (h < n_head) attn_merge_head<HD>(part, n_range, n_ne, h, threadIdx.x & 63, exp_tab, codes, scales);
}

int launch_attn_merge(const double* part, int n_ctx, const int32_t* pos_dev, int n_head, int head_dim, int8_t* codes,
                      uint16_t* scales, hipStream_t s) {
  int kpr = 0;
  const int n_range = attn_decode_ranges(n_ctx, &kpr);
  const dim3 grid((n_head + 3) / 4);
  if (head_dim == 64)
    hipLaunchKernelGGL(k_attn_merge<64>, grid, dim3(256), 0, s, part, n_range, kpr, pos_dev, n_head, codes, scales);
  else if (head_dim == 128)
    hipLaunchKernelGGL(k_attn_merge<128>, grid, dim3(256), 0, s, part, n_range, kpr, pos_dev, n_head, codes, scales);
  else
    return set_error(MI_ERR_UNSUPPORTED, "attention merge: head_dim %d", head_dim);
  MI_LAUNCH_CHECK("k_attn_merge");
  return MI_OK;
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
