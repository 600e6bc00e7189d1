// Decode step (one token at one position through the same layer sequence and KV regions as the
// prefill; the two-act engine of the walkthrough index, act two).  With one activation row every
// matmul is a matrix-vector product bound by HBM, and the attention has one query per head.
//
// k_gemv_q8: y[n] = sum_kb dx[kb] * dw[n][kb] * sum_32 qx * qw, one activation row.
//  * 16 waves per workgroup, RPW weight rows per wave (up to 4 in flight at once, 2 for the SwiGLU
//    rows); a lane takes 16-byte chunks (half a block) of every row, sdot4 gives the integer
//    half-block sums, lane pairs combine them to the block sum, and the exact f64 epilogue (block
//    sum times dw, times dx, one rounding per block) accumulates per lane; the lanes' partial sums
//    then reduce in f64.
//    The weight loads are double buffered: the next step's requests go out before this step's
//    math, and are unconditional (clamped addresses) so that the wait for one buffer never
//    includes the other's requests.
//  * The activation row is staged in LDS as codes + f64 scales.  The workgroup can build it
//    itself from the f32 residual stream (RMSNorm in f64, one rounding to f32, Q8_0 -- the same
//    arithmetic as the prefill's k_rmsnorm_quant), so the decode step has no normalization
//    kernels.  The prologue's inputs, then the first weight loads, go out before it.
//  * Epilogues: residual add (output projection, down projection), plain f32 with an optional
//    bias (lm_head; the Q|K|V rows), SwiGLU + Q8_0 (a workgroup holds one interleaved group of 32
//    gate and 32 up rows, i.e. one Q8_0 block of the SwiGLU output).  Every epilogue is per row,
//    so a workgroup takes 16 or 64 rows and even the small matrices spread over the chip.
//
// k_attn_decode: the query's keys 0..pos are split into fixed ranges (the grid depends only on
// n_ctx, so the launch can be captured once and replayed for any position); each workgroup
// computes the partial softmax states (max, sum, unnormalized output) of the query heads of one KV
// head (up to 4 of them) over one range in f64, reading each K and V row once for all of them.  In
// the decode step it also applies the per-head steps after the Q|K|V row (per-head QK RMSNorm, NeoX
// RoPE at the position) to its queries and, in the range holding the position, to the new K row,
// and stores the new K and V rows in the regions.
// k_attn_merge combines a head's ranges (in a fixed order), normalizes, and quantizes the head's
// output row to Q8_0, the output projection's input.
#include <algorithm>

#include "common.h"

namespace mi {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int GV_THREADS = 1024;  // 16 waves
constexpr int GV_WAVES = GV_THREADS / 64;
constexpr int GV_NORM_K = 4096;                                  // widest row the norm prologue takes
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

// The one-row-per-wave instances (the Q|K|V rows: 288 workgroups at the 7B shape; the output and
// down projections) and the SwiGLU instance are held to 64 registers, so that two workgroups fit a
// CU.  (The lm_head instance, with all four rows in flight, measured faster at one per CU.)
template <int RPW, int EPI, int PRO>
__global__ void __launch_bounds__(GV_THREADS, (EPI == GV_SWIGLU || RPW == 1) ? 8 : 1) k_gemv_q8(const float* __restrict__ x, const float* __restrict__ gamma,
                                                       float eps, const int8_t* __restrict__ xq,
                                                       const uint16_t* __restrict__ xs, int K,
                                                       const int8_t* __restrict__ w_codes,
                                                       const uint16_t* __restrict__ w_scales, int N,
                                                       const float* __restrict__ bias, const float* residual,
                                                       float* out, int8_t* __restrict__ q_codes,
                                                       uint16_t* __restrict__ q_scales) {
  constexpr int TH = GV_THREADS, WAVES = TH / 64;
  constexpr int NV = (GV_NORM_K / 4 + TH - 1) / TH;  // float4s of the row per thread (norm prologue)
  constexpr int RWG = RPW * WAVES;  // weight rows per group
  // 64-chunk steps of K per load batch; two batches are in flight (double buffered)
  constexpr int B = (EPI == GV_SWIGLU || RPW >= 4) ? 1 : 2;
  extern __shared__ __align__(16) unsigned char gv_lds[];
  const int KB = K / QK;
  int8_t* a_codes = reinterpret_cast<int8_t*>(gv_lds);                           // [K]
  double* a_d = reinterpret_cast<double*>(gv_lds + ((K + 15) & ~15));             // [KB]
  float* y = reinterpret_cast<float*>(a_d + KB);                                   // [RWG]
  double* red = reinterpret_cast<double*>(y + RWG + (RWG & 1));                    // [WAVES + 1]
  __shared__ double exp_tab[EPI == GV_SWIGLU ? 64 : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunk = K / 16;
  const int n_groups = (N + RWG - 1) / RWG;

  // ---- every request that depends on nothing goes out first: the activation row (the prologue's
  // input; K <= GV_NORM_K with the norm, K <= GV_MAX_K without), then the first load batches of
  // weights, so the prologue's waits never cover the weights and its latency overlaps them
  const int nvec = K / 4;
  constexpr int QW = (GV_MAX_K / 4 + TH - 1) / TH;   // code words of the Q8_0 row per thread
  constexpr int QS = (GV_MAX_K / 32 + TH - 1) / TH;  // scales of the Q8_0 row per thread
  float4 v[PRO == GV_IN_NORM ? NV : 1], gm[PRO == GV_IN_NORM ? NV : 1];
  uint32_t xw[PRO == GV_IN_NORM ? 1 : QW];
  uint16_t xsw[PRO == GV_IN_NORM ? 1 : QS];
  if constexpr (PRO == GV_IN_NORM) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int c4 = tid + j * TH;
      v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      gm[j] = v[j];
      if (c4 < nvec) {
        v[j] = reinterpret_cast<const float4*>(x)[c4];
        gm[j] = reinterpret_cast<const float4*>(gamma)[c4];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < QW; ++j)
      if (tid + j * TH < nvec) xw[j] = reinterpret_cast<const uint32_t*>(xq)[tid + j * TH];
#pragma unroll
    for (int j = 0; j < QS; ++j)
      if (tid + j * TH < KB) xsw[j] = xs[tid + j * TH];
  }

  // rows of a wave whose loads are in flight together; the SwiGLU rows two at a time, which keeps
  // that instance within 64 registers (two workgroups per CU: the 7B-shaped gate|up 32.5 -> 29.6 us)
  constexpr int RS = EPI == GV_SWIGLU ? 2 : (RPW < 4 ? RPW : 4);
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
  constexpr int STEP = 64 * B;  // chunks per load batch
  // one row per wave: both batches before the prologue (with more rows per wave the second batch
  // waits for the loop, which keeps the registers live across the prologue to 64)
  constexpr bool PRE2 = RPW == 1;
  load_batch(buf0, blockIdx.x, 0, 0);
  if constexpr (PRE2) load_batch(buf1, blockIdx.x, STEP, 0);
  if constexpr (EPI == GV_SWIGLU) exp2_table_fill(exp_tab, tid);

  // ---- the activation row -> LDS (codes, f64 scales)
  if constexpr (PRO == GV_IN_NORM) {
    double sq = 0.0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const double a = v[j].x, b = v[j].y, c = v[j].z, d = v[j].w;
      sq += a * a + b * b + c * c + d * d;
    }
    double ss = wave_sum_d(sq);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    if (wave == 0) {
      double t = lane < WAVES ? red[lane] : 0.0;
      t = wave_sum_d(t);
      if (lane == 0) red[WAVES] = t;
    }
    __syncthreads();
    const double inv_rms = recip_f64(sqrt(red[WAVES] / (double)K + (double)eps));
    // groups of 8 lanes cover one block; a group is entirely inside or outside [0, nvec)
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int c4 = tid + j * TH;
      if (c4 < nvec) {
        float4 o;
        o.x = (float)((double)v[j].x * inv_rms * (double)gm[j].x);
        o.y = (float)((double)v[j].y * inv_rms * (double)gm[j].y);
        o.z = (float)((double)v[j].z * inv_rms * (double)gm[j].z);
        o.w = (float)((double)v[j].w * inv_rms * (double)gm[j].w);
        float dq;
        const uint32_t qv = q8_block_quant4(o, dq);
        reinterpret_cast<uint32_t*>(a_codes)[c4] = qv;
        if ((c4 & 7) == 0) a_d[c4 / 8] = (double)f16_bits_to_f32(f32_to_f16_bits(dq));
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < QW; ++j)
      if (tid + j * TH < nvec) reinterpret_cast<uint32_t*>(a_codes)[tid + j * TH] = xw[j];
#pragma unroll
    for (int j = 0; j < QS; ++j)
      if (tid + j * TH < KB) a_d[tid + j * TH] = (double)f16_bits_to_f32(xsw[j]);
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
#pragma unroll
    for (int ib = 0; ib < RPW; ib += RS) {
      if (ib || grp != (int)blockIdx.x) {  // uniform; the first pass's batches went out before the prologue
        load_batch(buf0, grp, 0, ib);
        if constexpr (PRE2) load_batch(buf1, grp, STEP, ib);
      }
      if constexpr (!PRE2) load_batch(buf1, grp, STEP, ib);
#pragma unroll 1
      for (int c0 = 0;; c0 += 2 * STEP) {
        step(buf0, c0, acc + ib);
        if (c0 + STEP >= nchunk) break;  // uniform
        load_batch(buf0, grp, c0 + 2 * STEP, ib);
        step(buf1, c0 + STEP, acc + ib);
        if (c0 + 2 * STEP >= nchunk) break;
        load_batch(buf1, grp, c0 + 3 * STEP, ib);
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
  if (g.k % QK || g.k <= 0 || lds > 64 * 1024 || (norm && g.k > GV_NORM_K) || g.k > GV_MAX_K ||
      (int64_t)g.n * g.k >= ((int64_t)1 << 31))
    return set_error(MI_ERR_UNSUPPORTED, "gemv: K %d (multiple of 32, LDS %zu bytes, <= %d, <= %d with the norm)", g.k,
                     lds, GV_MAX_K, GV_NORM_K);
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

// ---------------------------------------------------------------- single-query attention
constexpr int AD_THREADS = 512;  // 8 waves
constexpr int AD_KEYS = 64;      // keys of a sub-chunk: 8 lanes per key in the score step
constexpr int AD_HB = 4;         // query heads of a head block

// The query heads of KV head g share every K and V row they read, so a workgroup takes one KV head's
// block of up to AD_HB query heads (GP, the block size rounded up to a power of two; heads past the
// group get a zero query and are never written) over one range of keys, in sub-chunks of 64 keys:
//   scores   lanes 8 * kk + pp share key kk, lane pp reading 16 bytes at offset 128 * i + 16 * pp of
//            the row (every K load instruction reads 8 whole 128-byte lines); each lane converts its
//            slice of the key once and forms the partial dot products of the GP heads (queries,
//            scaled by 1/sqrt(hd) in f64, from LDS); exchange-and-add steps over the 8 lanes, each
//            halving the heads a lane carries while GP allows, leave the full scores in LDS;
//   softmax  wave w keeps head w's running max and sum (f64), lane <-> key;
//   weights  thread (d, kp) accumulates dim d of every head over key part kp, V read as dwords
//            (64 consecutive dims of a row per instruction); the parts are summed in order at the end.
// K and V of a sub-chunk are requested together, before any of its arithmetic.  Workgroup (g, hb, r)
// writes part[(h * n_range + r) * (HD + 2)] = m, l, o[HD] (f64) for its heads h: m the range's
// largest score, l = sum e^(s - m), o = sum e^(s - m) v.  Ranges past pos write nothing.
//
// With `fin` (the decode step), q is the token's Q|K|V row (bias added, one rounding) and the
// per-head steps run here, with the arithmetic of the prefill's Q|K|V epilogue: per-head RMSNorm in
// f64 (when q_norm / k_norm are given), one rounding to f32; NeoX RoPE of the pair (i, i + hd/2) in
// f64 at pos, one rounding.  Waves 0..GP-1 prepare the queries; in the range holding pos, wave 4
// prepares the new K row and wave 5 takes the V row, both kept in LDS and used in place of what the
// region held at row pos, and the head block 0 workgroup stores them there.  Without `fin`, q holds
// finished queries and the regions already hold row pos.
template <int HD, int GP>
__global__ void __launch_bounds__(AD_THREADS) k_attn_decode(const float* __restrict__ q,
                                                            float* __restrict__ k_region,
                                                            float* __restrict__ v_region,
                                                            const int32_t* __restrict__ pos_dev, int n_head,
                                                            int n_head_kv, int keys_per_range,
                                                            double* __restrict__ part, int fin,
                                                            const double2* __restrict__ rope,
                                                            const float* __restrict__ q_norm,
                                                            const float* __restrict__ k_norm, float eps) {
  constexpr int NI = HD / 32;              // K float4s per lane and key (8 lanes x NI x 16 B = one row)
  constexpr int KP = AD_THREADS / HD;      // key parts of the weighted sum: 4 (HD 128), 8 (HD 64)
  constexpr int KPP = AD_KEYS / KP;        // keys per part: 16 (HD 128), 8 (HD 64)
  constexpr int LG = GP == 8 ? 3 : GP == 4 ? 2 : GP == 2 ? 1 : 0;  // halving steps
  __shared__ double qs[GP][HD];
  __shared__ double sc[GP][AD_KEYS];  // scores, then weights, of the sub-chunk
  __shared__ double rs[GP];           // each head's rescale factor for the sub-chunk
  __shared__ double etab[64];
  __shared__ double red[KP - 1][GP][HD];
  __shared__ float knew[HD], vnew[HD];  // the new K and V rows (fin, range holding pos)
  constexpr int HALF = HD / 2;
  static_assert(HALF <= 64, "one RoPE pair per lane");
  const int G = n_head / n_head_kv, n_hb = (G + AD_HB - 1) / AD_HB;
  const int g = blockIdx.x / n_hb, hb = blockIdx.x % n_hb, r = blockIdx.y, n_range = gridDim.y;
  const int h0 = g * G + hb * AD_HB, nh = min(GP, G - hb * AD_HB);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_kv = n_head_kv * HD;
  const int pos = *pos_dev, n_keys = pos + 1;
  const int j0 = r * keys_per_range, j1 = min(j0 + keys_per_range, n_keys);
  if (j0 >= j1) return;  // uniform for the workgroup
  const bool has_pos = fin && j1 == n_keys;  // this range holds key pos, the new row
  const int kk = tid >> 3, pp = tid & 7;  // scores: key kk of the sub-chunk, dim slice pp
  const int d = tid % HD, kp = tid / HD;  // weighted sum: dim d over the keys of part kp
  // 32-bit element offsets from the uniform region bases (n_ctx * n_kv < 2^31 is checked by the host)
  const uint32_t k_off = (uint32_t)(g * HD + 4 * pp), v_off = (uint32_t)(g * HD + d);
  float4 kv4[NI];
  float vv[KPP];
  auto load = [&](int t0, int nk) {
    const uint32_t kr = (uint32_t)(t0 + min(kk, nk - 1)) * (uint32_t)n_kv + k_off;
#pragma unroll
    for (int i = 0; i < NI; ++i) kv4[i] = *reinterpret_cast<const float4*>(k_region + kr + 32 * i);
    // keys past the sub-chunk's end re-read its last key (their weights are 0)
#pragma unroll
    for (int j = 0; j < KPP; ++j) vv[j] = v_region[(uint32_t)(t0 + min(kp * KPP + j, nk - 1)) * (uint32_t)n_kv + v_off];
  };
  double m_w = -1e300, l_w = 0.0;  // wave w: head w's running max and sum
  double o[GP];
#pragma unroll
  for (int hh = 0; hh < GP; ++hh) o[hh] = 0.0;
  // the queries (and, with fin, the new K and V rows), while the first sub-chunk's loads are in flight
  auto prep = [&]() {
    if (tid < 64) exp2_table_fill(etab, tid);
    const double scale = 1.0 / sqrt((double)HD);
    if (!fin) {
      for (int i = tid; i < GP * HD; i += AD_THREADS) {
        const int hh = i / HD;
        qs[hh][i % HD] = hh < nh ? (double)q[(int64_t)(h0 + hh) * HD + i % HD] * scale : 0.0;
      }
    } else if (wave < GP || (has_pos && wave == 4)) {  // a query head, or the new K row
      const bool isq = wave < GP;
      const bool live = isq ? wave < nh : true;  // uniform
      const bool on = lane < HALF;
      const float* src = isq ? q + (int64_t)(h0 + wave) * HD : q + n_head * HD + g * HD;
      const float* gam = isq ? q_norm : k_norm;
      float a = on && live ? src[lane] : 0.0f, bb = on && live ? src[lane + HALF] : 0.0f;
      if (gam) {  // per-head RMSNorm in f64, one rounding
        const double ss = wave_sum_d((double)a * (double)a + (double)bb * (double)bb);
        const double ir = recip_f64(sqrt(ss / (double)HD + (double)eps));
        if (on) {
          a = (float)((double)a * ir * (double)gam[lane]);
          bb = (float)((double)bb * ir * (double)gam[lane + HALF]);
        }
      }
      if (on) {
        const double2 cs = rope[(int64_t)pos * HALF + lane];
        const float ra = (float)((double)a * cs.x - (double)bb * cs.y);
        const float rb = (float)((double)a * cs.y + (double)bb * cs.x);
        if (isq) {
          qs[wave][lane] = live ? (double)ra * scale : 0.0;
          qs[wave][lane + HALF] = live ? (double)rb * scale : 0.0;
        } else {
          knew[lane] = ra;
          knew[lane + HALF] = rb;
          if (hb == 0) {
            float* dst = k_region + (int64_t)pos * n_kv + g * HD;
            dst[lane] = ra;
            dst[lane + HALF] = rb;
          }
        }
      }
    } else if (has_pos && wave == 5) {  // the new V row
      for (int i = lane; i < HD; i += 64) {
        const float vr = q[(int64_t)(n_head + n_head_kv) * HD + g * HD + i];
        vnew[i] = vr;
        if (hb == 0) v_region[(int64_t)pos * n_kv + g * HD + i] = vr;
      }
    }
  };
  // one sub-chunk of 64 keys, its K and V in kv4 / vv
  auto sub_chunk = [&](int t0, int nk) {
    // ---- scores
    double kd[4 * NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      kd[4 * i] = kv4[i].x;
      kd[4 * i + 1] = kv4[i].y;
      kd[4 * i + 2] = kv4[i].z;
      kd[4 * i + 3] = kv4[i].w;
    }
    const int kpos = pos - t0;  // row pos within the sub-chunk (when 0 <= kpos < nk)
    // the new K row, from LDS, for row pos and the rows past the sub-chunk's end (which re-read row
    // pos and are masked below)
    if (has_pos && kk >= kpos) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float4 kn = *reinterpret_cast<const float4*>(&knew[32 * i + 4 * pp]);
        kd[4 * i] = kn.x;
        kd[4 * i + 1] = kn.y;
        kd[4 * i + 2] = kn.z;
        kd[4 * i + 3] = kn.w;
      }
    }
    // two heads at a time: their query slices are read from LDS just before use (the compiler
    // barrier keeps it from hoisting every head's reads, which would need 4 * NI * GP registers)
    constexpr int HS = GP < 2 ? GP : 2;
    double ps[GP];
#pragma unroll
    for (int h2 = 0; h2 < GP; h2 += HS) {
      asm volatile("" ::: "memory");
      double a0[HS], a1[HS];
#pragma unroll
      for (int e = 0; e < HS; ++e) a0[e] = a1[e] = 0.0;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
#pragma unroll
        for (int e = 0; e < HS; ++e) {
          const double2 q01 = *reinterpret_cast<const double2*>(&qs[h2 + e][32 * i + 4 * pp]);
          const double2 q23 = *reinterpret_cast<const double2*>(&qs[h2 + e][32 * i + 4 * pp + 2]);
          a0[e] = fma(q01.x, kd[4 * i], a0[e]);
          a1[e] = fma(q01.y, kd[4 * i + 1], a1[e]);
          a0[e] = fma(q23.x, kd[4 * i + 2], a0[e]);
          a1[e] = fma(q23.y, kd[4 * i + 3], a1[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < HS; ++e) ps[h2 + e] = a0[e] + a1[e];
    }
    // over the 8 lanes of the key, partners lane 7 - pp (bit 2 of pp flips), pp ^ 2 (bit 1), pp ^ 1
    // (bit 0): while a lane carries more than one head, each step keeps half of them (the half the
    // partner does not keep) and adds the partner's sums of that half; then the steps just add
    if constexpr (GP >= 2) {
      const bool hi = pp & 4;
#pragma unroll
      for (int j = 0; j < GP / 2; ++j)
        ps[j] = (hi ? ps[j + GP / 2] : ps[j]) + dpp_f64<DPP_HALF_MIRROR>(hi ? ps[j] : ps[j + GP / 2]);
    } else {
      ps[0] += dpp_f64<DPP_HALF_MIRROR>(ps[0]);
    }
    if constexpr (GP >= 4) {
      const bool hi = pp & 2;
#pragma unroll
      for (int j = 0; j < GP / 4; ++j)
        ps[j] = (hi ? ps[j + GP / 4] : ps[j]) + dpp_f64<DPP_XOR2>(hi ? ps[j] : ps[j + GP / 4]);
    } else {
      ps[0] += dpp_f64<DPP_XOR2>(ps[0]);
    }
    if constexpr (GP >= 8) {
      const bool hi = pp & 1;
      ps[0] = (hi ? ps[1] : ps[0]) + dpp_f64<DPP_XOR1>(hi ? ps[0] : ps[1]);
    } else {
      ps[0] += dpp_f64<DPP_XOR1>(ps[0]);
    }
    // lane pp now holds the score of head pp >> (3 - LG); one lane of each head writes it
    if ((pp & ((8 >> LG) - 1)) == 0) sc[pp >> (3 - LG)][kk] = kk < nk ? ps[0] : -1e300;
    __syncthreads();
    // ---- softmax: wave w, head w
    if (wave < GP) {
      const double s = sc[wave][lane];
      const double m_new = fmax(m_w, wave_reduce_f64<true>(s));
      const double p = lane < nk ? exp_f64(s - m_new, etab) : 0.0;
      const double resc = exp_f64(m_w - m_new, etab);  // 0 for the first sub-chunk (m_w = -1e300)
      l_w = l_w * resc + wave_reduce_f64<false>(p);
      m_w = m_new;
      sc[wave][lane] = p;
      if (lane == 0) rs[wave] = resc;
    }
    __syncthreads();
    // ---- weighted sum
    if (has_pos) {  // the new V row, from LDS (row pos and the rows past the end, weight 0, that re-read it)
#pragma unroll
      for (int j = 0; j < KPP; ++j)
        if (kp * KPP + j >= kpos) vv[j] = vnew[d];
    }
#pragma unroll
    for (int hh = 0; hh < GP; ++hh) o[hh] *= rs[hh];
#pragma unroll
    for (int j = 0; j < KPP; j += 2) {
      if (j % 4 == 0) asm volatile("" ::: "memory");  // weights read 4 keys at a time (registers)
      const double v0 = vv[j], v1 = vv[j + 1];
#pragma unroll
      for (int hh = 0; hh < GP; ++hh) {
        const double2 pk = *reinterpret_cast<const double2*>(&sc[hh][kp * KPP + j]);
        o[hh] = fma(pk.x, v0, o[hh]);
        o[hh] = fma(pk.y, v1, o[hh]);
      }
    }
  };
  load(j0, min(AD_KEYS, j1 - j0));
  prep();
  __syncthreads();
  sub_chunk(j0, min(AD_KEYS, j1 - j0));
  for (int t0 = j0 + AD_KEYS; t0 < j1; t0 += AD_KEYS) {
    load(t0, min(AD_KEYS, j1 - t0));
    __syncthreads();  // sc and rs of the previous sub-chunk consumed
    sub_chunk(t0, min(AD_KEYS, j1 - t0));
  }
  // ---- the key parts, summed in order; m and l from the head's wave
  if (kp > 0) {
#pragma unroll
    for (int hh = 0; hh < GP; ++hh) red[kp - 1][hh][d] = o[hh];
  }
  if (wave < nh && lane == 0) {
    double* out = part + ((int64_t)(h0 + wave) * n_range + r) * (HD + 2);
    out[0] = m_w;
    out[1] = l_w;
  }
  __syncthreads();
  if (kp == 0) {
#pragma unroll
    for (int hh = 0; hh < GP; ++hh) {
      if (hh < nh) {
        double od = o[hh];
#pragma unroll
        for (int k = 0; k < KP - 1; ++k) od += red[k][hh][d];
        part[((int64_t)(h0 + hh) * n_range + r) * (HD + 2) + 2 + d] = od;
      }
    }
  }
}

// Merge head h's n_ne ranges, normalize, round to f32 and Q8_0: workgroup h, thread t takes dims
// 4 * dq .. 4 * dq + 3 (dq = t % (HD / 4)) over the ranges rs, rs + RSETS, ... (rs = t / (HD / 4)),
// every one of its partial rows requested at once; wave 0 meanwhile forms the weights e^(m_r - m)
// (one range per lane).  The range sets are then added in order through LDS, and the first HD / 4
// lanes quantize the row (8 lanes per Q8_0 block).
constexpr int AM_THREADS = 256;

template <int HD>
__global__ void __launch_bounds__(AM_THREADS) k_attn_merge(const double* __restrict__ part, int n_range,
                                                           int keys_per_range, const int32_t* __restrict__ pos_dev,
                                                           int8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  constexpr int DQN = HD / 4;                   // dim quads
  constexpr int RSETS = AM_THREADS / DQN;       // range sets: 8 (HD 128), 16 (HD 64)
  constexpr int RPS = AD_MAX_RANGES / RSETS;    // ranges per set at most
  __shared__ double exp_tab[64];
  __shared__ double fw[AD_MAX_RANGES];          // e^(m_r - m)
  __shared__ double l_sh;
  __shared__ double4 red[RSETS - 1][DQN];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int dq = tid % DQN, rs = tid / DQN;
  const int n_ne = (*pos_dev + keys_per_range) / keys_per_range;  // ranges holding keys 0..pos
  const double* ph = part + (int64_t)h * n_range * (HD + 2);
  double2 po[RPS][2];
#pragma unroll
  for (int i = 0; i < RPS; ++i) {
    const int r = min(rs + RSETS * i, n_ne - 1);  // ranges past n_ne re-read the last one (unused)
    const double2* src = reinterpret_cast<const double2*>(ph + r * (HD + 2) + 2) + 2 * dq;
    po[i][0] = src[0];
    po[i][1] = src[1];
  }
  exp2_table_fill(exp_tab, tid);
  __syncthreads();
  if (tid < 64) {
    double mr = -1e300, lr = 0.0;
    if (lane < n_ne) {  // one range per lane (n_ne <= AD_MAX_RANGES <= 64)
      mr = ph[lane * (HD + 2)];
      lr = ph[lane * (HD + 2) + 1];
    }
    const double m = wave_max_d(mr);
    const double f = lane < n_ne ? exp_f64(mr - m, exp_tab) : 0.0;
    fw[lane] = f;
    const double l = wave_sum_d(lr * f);
    if (lane == 0) l_sh = l;
  }
  __syncthreads();
  double o[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int i = 0; i < RPS; ++i) {
    const int r = rs + RSETS * i;
    if (r < n_ne) {
      const double f = fw[r];
      o[0] = fma(po[i][0].x, f, o[0]);
      o[1] = fma(po[i][0].y, f, o[1]);
      o[2] = fma(po[i][1].x, f, o[2]);
      o[3] = fma(po[i][1].y, f, o[3]);
    }
  }
  if (rs > 0) red[rs - 1][dq] = make_double4(o[0], o[1], o[2], o[3]);
  __syncthreads();
  if (tid < 64) {  // wave 0: lanes 0..DQN-1 hold the row (whole groups of 8 lanes per block)
    if (rs == 0) {
#pragma unroll
      for (int k = 0; k < RSETS - 1; ++k) {
        const double4 v = red[k][dq];
        o[0] += v.x;
        o[1] += v.y;
        o[2] += v.z;
        o[3] += v.w;
      }
    }
    const double inv = recip_f64(l_sh);
    if (lane < DQN) {
      float4 v;
      v.x = (float)(o[0] * inv);
      v.y = (float)(o[1] * inv);
      v.z = (float)(o[2] * inv);
      v.w = (float)(o[3] * inv);
      float d;
      const uint32_t qv = q8_block_quant4(v, d);
      reinterpret_cast<uint32_t*>(codes + h * HD)[lane] = qv;
      if ((lane & 7) == 0) scales[h * (HD / QK) + lane / 8] = f32_to_f16_bits(d);
    }
  }
}

int launch_attn_merge(const double* part, int n_ctx, const int32_t* pos_dev, int n_head, int head_dim, int8_t* codes,
                      uint16_t* scales, hipStream_t s) {
  int kpr = 0;
  const int n_range = attn_decode_ranges(n_ctx, &kpr);
  if (head_dim == 64)
    hipLaunchKernelGGL(k_attn_merge<64>, dim3(n_head), dim3(AM_THREADS), 0, s, part, n_range, kpr, pos_dev, codes,
                       scales);
  else if (head_dim == 128)
    hipLaunchKernelGGL(k_attn_merge<128>, dim3(n_head), dim3(AM_THREADS), 0, s, part, n_range, kpr, pos_dev, codes,
                       scales);
  else
    return set_error(MI_ERR_UNSUPPORTED, "attention merge: head_dim %d", head_dim);
  MI_LAUNCH_CHECK("k_attn_merge");
  return MI_OK;
}

int attn_decode_ranges(int n_ctx, int* keys_per_range) {
  int kpr = AD_KEYS;  // one sub-chunk per workgroup up to 64 ranges, then longer ranges
  while ((n_ctx + kpr - 1) / kpr > AD_MAX_RANGES) kpr *= 2;
  *keys_per_range = kpr;
  return (n_ctx + kpr - 1) / kpr;
}

template <int HD>
static void launch_attn_decode_hd(int gp, dim3 grid, hipStream_t s, const float* q, float* k_region, float* v_region,
                                  const int32_t* pos_dev, int n_head, int n_head_kv, int kpr, double* part,
                                  int fin, const double2* rope, const float* q_norm, const float* k_norm,
                                  float eps) {
  auto k = gp == 4 ? k_attn_decode<HD, 4> : gp == 2 ? k_attn_decode<HD, 2> : k_attn_decode<HD, 1>;
  hipLaunchKernelGGL(k, grid, dim3(AD_THREADS), 0, s, q, k_region, v_region, pos_dev, n_head, n_head_kv, kpr, part,
                     fin, rope, q_norm, k_norm, eps);
}

int launch_attn_decode(const float* q, float* k_region, float* v_region, const int32_t* pos_dev, int n_ctx,
                       int n_head, int n_head_kv, int head_dim, double* part, const AttnFinish* fin, hipStream_t s) {
  int kpr = 0;
  const int n_range = attn_decode_ranges(n_ctx, &kpr);
  const int G = n_head / n_head_kv, n_hb = (G + AD_HB - 1) / AD_HB;
  int gp = 1;  // the head block, rounded up to a power of two
  while (gp < G && gp < AD_HB) gp *= 2;
  const dim3 grid(n_head_kv * n_hb, n_range);
  const double2* rope = fin ? reinterpret_cast<const double2*>(fin->rope) : nullptr;
  const float* qn = fin ? fin->q_norm : nullptr;
  const float* kn = fin ? fin->k_norm : nullptr;
  const float eps = fin ? fin->eps : 0.0f;
  if (head_dim == 64)
    launch_attn_decode_hd<64>(gp, grid, s, q, k_region, v_region, pos_dev, n_head, n_head_kv, kpr, part, fin != nullptr,
                              rope, qn, kn, eps);
  else if (head_dim == 128)
    launch_attn_decode_hd<128>(gp, grid, s, q, k_region, v_region, pos_dev, n_head, n_head_kv, kpr, part,
                               fin != nullptr, rope, qn, kn, eps);
  else
    return set_error(MI_ERR_UNSUPPORTED, "attention decode: head_dim %d", head_dim);
  MI_LAUNCH_CHECK("k_attn_decode");
  return MI_OK;
}

}  // namespace mi
