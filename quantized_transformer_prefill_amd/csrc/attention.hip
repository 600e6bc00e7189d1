// Causal grouped-query attention over a layer's f32 KV regions, flash style, in f64.
//
// o[t][h] = sum_{j <= pos[t]} softmax_j(q[t][h] . k[j][g] / sqrt(hd)) v[j][g],  g = h / (nh/nkv).
// Token t sees region rows 0..=pos[t] (positions are data, read per element), after this call's
// KV store for the layer.  The node's result must round to the same f32 as the exact value, so
// scores, softmax and the weighted sum run in f64 on v_mfma_f64_16x16x4f64; the online-softmax
// bookkeeping (running max, running sum, rescale) is f64 on the VALU.
//
// Work split: a group of NW waves serves 16 query tokens x 1 head.  The key tiles (16 rows each,
// from row 0 to the largest position among the 16 queries) are dealt round-robin to the waves,
// so every wave sees early and late tiles alike.  For head_dim 64 a workgroup holds two groups,
// for query tiles x and (last - x), which balances the causal work across workgroups and SIMDs.  Each wave keeps its own running max,
// sum and output; at the end wave 0 merges the partial states in f64 through LDS in a fixed order
// (o = sum_w O_w 2^(m_w - m) / sum_w l_w 2^(m_w - m)), after two barriers.  The next tile's K and
// V are loaded while the current tile computes.
//
// Softmax in base 2: scores carry the factor log2(e)/sqrt(hd), so the weights are 2^(s - m) (the
// same softmax; one f64 rounding of the factor).  Every VALU instruction here costs the SIMD as
// much as it would alone (the f64 MFMA does not run beside it), so the bookkeeping is kept small:
//  * the running max is raised lazily: a query's reference m moves only when a score exceeds it
//    by more than LAZY_MAX (softmax is invariant to the reference, and 2^(s - m) <= 2^LAZY_MAX is
//    harmless in f64), so most tiles need neither the cross-lane max nor the rescale of O;
//  * the running sum is kept per lane (each lane sums its own keys) and reduced once at the end;
//  * the causal mask is applied only on tiles that some query of the 16 does not fully see.
//
// MFMA 16x16x4 f64 lane layout: A lane l -> (m = l%16, k = l/16), B lane l -> (k = l/16, n =
// l%16), D register i lane l -> (m = 4i + l/16, n = l%16).
//  * scores S^T = K . Q^T  (m = key, n = query, k = head dims): the order of the dims in the
//    contraction is free, so lane slot g = l/16 owns the contiguous dims [g*hd/4, (g+1)*hd/4) and
//    MFMA s uses dim g*hd/4 + s: K is read from the region as float4s, Q (f64, stored in LDS
//    once per workgroup) as pairs for MFMAs s, s+1.  Two accumulators (even/odd s) keep the MFMA
//    dependency chain short.
//  * lane l then holds the scores of query l%16 against keys 4i + l/16 (i = 0..3); the max over
//    a query's keys reduces over the 4 registers and the lanes l^16, l^32.
//  * O^T += V^T . P^T  (m = output dim, n = query, k = key): MFMA c takes key slot s = l/16 as key
//    4c + s, which is exactly register c of the lane's P; the output dim of row m in dim block b is
//    m*(hd/16) + b, so V reads and O stores are contiguous per lane.
#include "common.h"

namespace mi {

typedef double v4d __attribute__((ext_vector_type(4)));

constexpr double LAZY_MAX = 24.0;  // base-2 units

// 2^y for y <= LAZY_MAX; -inf and NaN (a masked score against a reference still at -inf) give 0.
// y = k/64 + r with |r| <= 1/128 (exact); 2^(k/64) from the table `tab` (2^(j/64), j < 64) and an
// exponent shift; 2^r by its degree-5 Taylor polynomial in r ln2 (truncation below 4e-17).
__device__ __forceinline__ double exp2_att(double y, const double* tab) {
  y = fmax(y, -1100.0);
  const double kf = rint(y * 64.0);
  const double r = fma(kf, -1.0 / 64.0, y);
  const double p = fma(fma(fma(fma(fma(0x1.5d87fe78a6731p-10, r, 0x1.3b2ab6fba4e77p-7), r, 0x1.c6b08d704a0c0p-5), r,
                                   0x1.ebfbdff82c58fp-3), r, 0x1.62e42fefa39efp-1), r, 1.0);
  const int k = (int)kf;
  return ldexp(tab[k & 63] * p, k >> 6);
}

// The regions may come from a tile table in memory, where the compiler cannot tell that they are
// global memory: loads through address-space-1 pointers are global loads, not flat ones.
typedef float f4v __attribute__((ext_vector_type(4)));
typedef const float __attribute__((address_space(1))) gfloat;
typedef const f4v __attribute__((address_space(1))) gfloat4;

// One key tile, in two halves with their own registers: the K half is consumed by the score
// MFMAs and the V half by the PV MFMAs, so each half of the next tile is requested as soon as its
// registers are free (one tile of registers, each load a phase ahead of its use).
template <int HD>
struct KHalf {
  f4v k[HD / 16];             // K row (key0 + l%16), dims slot*HD/4 .. +HD/4
};
template <int HD>
struct VHalf {
  f4v v[4][HD / 64];          // V rows key0 + 4c + slot, dims (l%16)*HD/16 .. +HD/16
};

// Rows are clamped to max_pos (the largest position of the call or of the sequence, a row this
// call wrote), so every load is in bounds (row * kv_embd < 2^31, checked by the callers); rows past a query's position are masked later: their
// scores are replaced by -inf, and their V values (which may be anything) are zeroed on the tile
// that straddles the largest position of the 16 queries (mask_v).
template <int HD>
__device__ __forceinline__ void load_k(KHalf<HD>& t, gfloat* kbase, int kv_embd, int key0, int max_pos, int qi,
                                       int slot) {
  constexpr int Q4 = HD / 4;
  gfloat* kp = kbase + (uint32_t)(min(key0 + qi, max_pos) * kv_embd + slot * Q4);
#pragma unroll
  for (int s = 0; s < Q4 / 4; ++s) t.k[s] = *(gfloat4*)(kp + 4 * s);
}

template <int HD>
__device__ __forceinline__ void load_v(VHalf<HD>& t, gfloat* vbase, int kv_embd, int key0, int max_pos, int qi,
                                       int slot) {
  constexpr int NB = HD / 16;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    gfloat* vp = vbase + (uint32_t)(min(key0 + 4 * c + slot, max_pos) * kv_embd + qi * NB);
#pragma unroll
    for (int b = 0; b < NB / 4; ++b) t.v[c][b] = *(gfloat4*)(vp + 4 * b);
  }
}

template <int HD>
__device__ __forceinline__ void mask_v(VHalf<HD>& t, int key0, int pmax, int slot) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (key0 + 4 * c + slot > pmax)
#pragma unroll
      for (int b = 0; b < HD / 64; ++b) t.v[c][b] = f4v{0.f, 0.f, 0.f, 0.f};
}

__device__ __forceinline__ double f4get(const f4v& v, int e) { return (double)v[e]; }

// head_dim 128: at least two waves per SIMD (two workgroups per CU), which keeps the working set in
// 256 registers per lane, with no accumulator copies through AGPRs
template <int HD, int NW, int NG>
__global__ void __launch_bounds__(64 * NW * NG, (HD > 64 ? 2 : 1)) k_attention(const float* __restrict__ q, int64_t ld_q,
                                                       const float* __restrict__ k_region,
                                                       const float* __restrict__ v_region,
                                                       const int32_t* __restrict__ pos, int n_tokens,
                                                       const int32_t* __restrict__ max_pos_p, int max_pos_v,
                                                       int n_head, int n_head_kv, float* __restrict__ out,
                                                       int64_t ld_out, int8_t* __restrict__ q_codes,
                                                       uint16_t* __restrict__ q_scales,
                                                       const AttnSlotTile* __restrict__ tiles, int n_tiles) {
  constexpr int Q4 = HD / 4;    // dims per lane slot (scores) = MFMAs per score tile
  constexpr int NB = HD / 16;   // output dim blocks
  __shared__ double exp_tab[64];
  __shared__ double sh_m[NG][NW][64], sh_l[NG][NW][64];
  // one buffer for the query pairs (during the key loop) and then, after a barrier, the partial
  // outputs of waves 1..NW-1 for the merge
  constexpr int Q_BYTES = NG * 4 * (Q4 / 2) * 16 * (int)sizeof(double2);
  constexpr int O_BYTES = NG * (NW - 1) * NB * 4 * 64 * (int)sizeof(double);
  __shared__ __attribute__((aligned(16))) char sh_u[Q_BYTES > O_BYTES ? Q_BYTES : O_BYTES];
  double2* const sh_q = reinterpret_cast<double2*>(sh_u);
  double* const sh_o = reinterpret_cast<double*>(sh_u);
  // wave and group are uniform in a wave (scalar registers: the tile descriptor is a scalar load)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) % NW),
            grp = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) / NW);
  const int qi = lane & 15, slot = lane >> 4;
  exp2_table_fill(exp_tab, threadIdx.x);
  const int h = blockIdx.y;
  const int g = h / (n_head / n_head_kv);
  const int kv_embd = n_head_kv * HD;
  // query tile of this group: with two groups, workgroup x serves tiles x and nqt-1-x, so that
  // every workgroup (and every SIMD: waves w and w+NW share one) gets about the same number of
  // key tiles under the causal mask; the middle workgroup of an odd count has one group.
  // With a tile table (several sequences in one call) a query tile is up to 16 rows of one
  // sequence, with that sequence's regions and largest position.
  const int nqt = tiles ? n_tiles : (n_tokens + 15) / 16;
  // (one group: the tiles in decreasing order, the heaviest first, so the last workgroups are short)
  const int qt = (NG == 1 || grp == 1) ? nqt - 1 - blockIdx.x : blockIdx.x;
  const bool gactive = grp == 0 || qt != (int)blockIdx.x;
  int t0 = qt * 16, tcount = min(16, n_tokens - qt * 16), max_pos = max_pos_p ? *max_pos_p : max_pos_v;
  const float* k_reg = k_region;
  const float* v_reg = v_region;
  if (tiles) {
    const AttnSlotTile d = tiles[qt];
    t0 = d.t0;
    tcount = d.count;
    k_reg = d.k_region;
    v_reg = d.v_region;
    max_pos = d.max_pos;
  }
  const int t = t0 + qi;
  const bool valid = gactive && qi < tcount;
  const int p = valid ? pos[t] : 0;
  int pmax = p, pmin = valid ? p : 0x7fffffff;
  for (int o = 1; o < 16; o <<= 1) {
    pmax = max(pmax, __shfl_xor(pmax, o));
    pmin = min(pmin, __shfl_xor(pmin, o));
  }

  // query fragment: dims slot*Q4 + s, f64, pre-multiplied by the score factor, in LDS (per group
  // 8 KB at head_dim 64, 16 KB at 128, laid out [slot][s/2][query][s%2] so that the 16 lanes of a
  // slot read 256 contiguous bytes), read as a pair at each pair of score MFMAs.  LDS reads do not
  // stall the f64 MFMA the way VALU instructions do, and the registers stay free for the tiles.
  const double scale = 0x1.71547652b82fep+0 / sqrt((double)HD);  // log2(e) / sqrt(hd)
  if (wave == 0) {  // one wave per group writes the group's 16 queries
    const float* qp = q + (int64_t)(valid ? t : 0) * ld_q + (int64_t)h * HD + slot * Q4;
    f4v qf[Q4 / 4];
#pragma unroll
    for (int s = 0; s < Q4 / 4; ++s) qf[s] = *reinterpret_cast<const f4v*>(qp + 4 * s);
#pragma unroll
    for (int s = 0; s < Q4; s += 2)
      sh_q[((grp * 4 + slot) * (Q4 / 2) + s / 2) * 16 + qi] =
          double2{(double)qf[s / 4][s % 4] * scale, (double)qf[(s + 1) / 4][(s + 1) % 4] * scale};
  }
  const double2* sq = sh_q + (grp * 4 + slot) * (Q4 / 2) * 16 + qi;  // this lane's query pairs, stride 16

  v4d acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = v4d{0.0, 0.0, 0.0, 0.0};
  double m_run = -INFINITY, l_run = 0.0;   // l_run: this lane's keys only

  gfloat* kbase = (gfloat*)k_reg + (int64_t)g * HD;
  gfloat* vbase = (gfloat*)v_reg + (int64_t)g * HD;
  const int ntiles = gactive ? pmax / 16 + 1 : 0;

  // Tiles wave, wave + NW, ... of the 16 queries' keys.  Per tile: scores from the K half; the
  // next tile's K half requested; online softmax; O += V^T P^T from the V half; the next tile's
  // V half requested.  The first tile is requested before the positions arrive.
  KHalf<HD> kt;
  VHalf<HD> vt;
  load_k<HD>(kt, kbase, kv_embd, wave * 16, max_pos, qi, slot);
  load_v<HD>(vt, vbase, kv_embd, wave * 16, max_pos, qi, slot);
  __syncthreads();  // exp_tab, query pairs
  for (int tile = wave; tile < ntiles; tile += NW) {
    const int key0 = tile * 16;
    const bool more = tile + NW < ntiles;
    // the query pairs are read from LDS in the loop (not hoisted into registers)
    asm volatile("" ::: "memory");
    v4d sc0 = {0.0, 0.0, 0.0, 0.0}, sc1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < Q4; s += 2) {
      const double2 qq = sq[(s / 2) * 16];
      sc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(f4get(kt.k[s / 4], s % 4), qq.x, sc0, 0, 0, 0);
      sc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(f4get(kt.k[(s + 1) / 4], (s + 1) % 4), qq.y, sc1, 0, 0, 0);
    }
    if (more) load_k<HD>(kt, kbase, kv_embd, key0 + 16 * NW, max_pos, qi, slot);
    // ---- online softmax for query l%16 over keys key0 + 4i + slot
    const bool full = key0 + 15 <= pmin;  // every query of the 16 sees every key of the tile
    double sv[4];
    double tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = sc0[i] + sc1[i];
      if (!full && key0 + 4 * i + slot > p) sv[i] = -INFINITY;
      tmax = fmax(tmax, sv[i]);
    }
    if (__any(tmax > m_run + LAZY_MAX)) {
      tmax = fmax(tmax, __shfl_xor(tmax, 16));
      tmax = fmax(tmax, __shfl_xor(tmax, 32));
      if (tmax > m_run) {  // the same decision on the 4 lanes of a query
        // a query whose keys so far were all masked has m = -inf and nothing to rescale
        const double corr = (m_run == -INFINITY) ? 0.0 : exp2_att(m_run - tmax, exp_tab);
        l_run *= corr;
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] *= corr;
        m_run = tmax;
      }
    }
    double pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = exp2_att(sv[i] - m_run, exp_tab);  // 0 for a masked key
      l_run += pv[i];
    }
    if (key0 + 15 > pmax) mask_v<HD>(vt, key0, pmax, slot);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(f4get(vt.v[c][b / 4], b % 4), pv[c], acc[b], 0, 0, 0);
    if (more) load_v<HD>(vt, vbase, kv_embd, key0 + 16 * NW, max_pos, qi, slot);
  }

  // ---- merge: the query's sum over its 4 lanes; then wave 0 adds the waves' partial states,
  // each scaled to the common reference max (f64, waves in order 0..NW-1)
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  sh_m[grp][wave][lane] = m_run;
  sh_l[grp][wave][lane] = l_run;
  __syncthreads();  // every key loop is done: the query pairs are dead, their LDS takes the outputs
  if (wave > 0) {
    double* dst = sh_o + (grp * (NW - 1) + wave - 1) * (NB * 4 * 64) + lane;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(b * 4 + i) * 64] = acc[b][i];
  }
  __syncthreads();
  if (wave == 0) {
    double m_all = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) m_all = fmax(m_all, sh_m[grp][w][lane]);
    double f[NW];
    double l_all = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const double mw = sh_m[grp][w][lane];
      f[w] = (mw == -INFINITY) ? 0.0 : exp2_att(mw - m_all, exp_tab);
      l_all += sh_l[grp][w][lane] * f[w];
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      asm volatile("" ::: "memory");  // one dim block's partials in flight at a time (registers)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        double o = acc[b][i] * f[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) o = fma(sh_o[(grp * (NW - 1) + w - 1) * (NB * 4 * 64) + (b * 4 + i) * 64 + lane], f[w], o);
        acc[b][i] = o;
      }
    }
    const double inv = recip_f64(l_all);
    // lane holds dims (4i + slot)*NB + b of query l%16 (i = 0..3, b = 0..NB-1)
    float o[4][NB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int b = 0; b < NB; ++b) o[i][b] = (float)(acc[b][i] * inv);
    if (!q_codes) {
      if (valid) {
        float* op = out + (int64_t)t * ld_out + (int64_t)h * HD;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float* dst = op + (4 * i + slot) * NB;
#pragma unroll
          for (int b = 0; b < NB; b += 4) *reinterpret_cast<float4*>(dst + b) = make_float4(o[i][b], o[i][b + 1], o[i][b + 2], o[i][b + 3]);
        }
      }
    } else {
      // Q8_0 of the output row: block kb of the head covers dims 32kb..32kb+31, i.e. the registers
      // i with i*NB/8 == kb of the query's 4 lanes (slots) -- 8 values per lane
      constexpr int IPB = 8 / NB;  // registers i per block
      const int64_t nq = (int64_t)n_head * HD;
#pragma unroll
      for (int kb = 0; kb < HD / 32; ++kb) {
        float m = 0.0f;
#pragma unroll
        for (int ii = 0; ii < IPB; ++ii)
#pragma unroll
          for (int b = 0; b < NB; ++b) m = fmaxf(m, fabsf(o[kb * IPB + ii][b]));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        const float d = div127_f32(m);
        const float id = (d != 0.0f) ? recip_f32(d) : 0.0f;
        if (valid) {
          int8_t* cp = q_codes + (int64_t)t * nq + (int64_t)h * HD;
#pragma unroll
          for (int ii = 0; ii < IPB; ++ii) {
            const int i = kb * IPB + ii;
#pragma unroll
            for (int b = 0; b < NB; b += 4) {
              const uint32_t w4 = (uint32_t)(uint8_t)q8_code(o[i][b], id) |
                                  ((uint32_t)(uint8_t)q8_code(o[i][b + 1], id) << 8) |
                                  ((uint32_t)(uint8_t)q8_code(o[i][b + 2], id) << 16) |
                                  ((uint32_t)(uint8_t)q8_code(o[i][b + 3], id) << 24);
              *reinterpret_cast<uint32_t*>(cp + (4 * i + slot) * NB + b) = w4;
            }
          }
          if (slot == 0) q_scales[(int64_t)t * (nq / QK) + (int64_t)h * (HD / QK) + kb] = f32_to_f16_bits(d);
        }
      }
    }
  }
}

int launch_attention(const float* q, int64_t ld_q, const float* k_region, const float* v_region,
                     const int32_t* pos, int n_tokens, const int32_t* max_pos_dev, int max_pos, int n_head, int n_head_kv,
                     int head_dim, float* out, int64_t ld_out, hipStream_t s, int8_t* q_codes,
                     uint16_t* q_scales, const AttnSlotTile* tiles, int n_tiles) {
  if (n_tokens == 0 || (tiles && n_tiles == 0)) return MI_OK;
  const int nqt = tiles ? n_tiles : (n_tokens + 15) / 16;
  if (head_dim == 64)
    hipLaunchKernelGGL((k_attention<64, 4, 2>), dim3((nqt + 1) / 2, n_head), dim3(64 * 4 * 2), 0, s, q, ld_q, k_region,
                       v_region, pos, n_tokens, max_pos_dev, max_pos, n_head, n_head_kv, out, ld_out, q_codes, q_scales,
                       tiles, n_tiles);
  else if (head_dim == 128)
    hipLaunchKernelGGL((k_attention<128, 4, 1>), dim3(nqt, n_head), dim3(64 * 4), 0, s, q, ld_q, k_region, v_region,
                       pos, n_tokens, max_pos_dev, max_pos, n_head, n_head_kv, out, ld_out, q_codes, q_scales, tiles,
                       n_tiles);
  else
    return set_error(MI_ERR_UNSUPPORTED, "attention: head_dim %d (supported: 64, 128)", head_dim);
  MI_LAUNCH_CHECK("k_attention");
  return MI_OK;
}

}  // namespace mi
