// Causal grouped-query attention over a layer's f32 KV regions, flash style, in f64.
//
// o[t][h] = sum_{j <= pos[t]} softmax_j(q[t][h] . k[j][g] / sqrt(hd)) v[j][g],  g = h / (nh/nkv).
// Token t sees region rows 0..=pos[t] (positions are data, read per element), after this call's
// KV store for the layer.  The node's result must round to the same f32 as the exact value, so
// scores, softmax and the weighted sum run in f64 on v_mfma_f64_16x16x4f64; the online-softmax
// bookkeeping (running max, running sum, rescale) is f64 on the VALU.
//
// Work split: a workgroup of 4 waves serves 16 query tokens x 1 head.  The key tiles (16 rows
// each, from row 0 to the largest position among the 16 queries) are dealt round-robin to the 4
// waves, so every wave sees early and late tiles alike.  Each wave keeps its own running max,
// sum and output; at the end the four partial states are merged in f64 through LDS
// (o = sum_w O_w e^(m_w - m) / sum_w l_w e^(m_w - m)).  The next tile's K and V are loaded while
// the current tile computes.
//
// MFMA 16x16x4 f64 lane layout: A lane l -> (m = l%16, k = l/16), B lane l -> (k = l/16, n =
// l%16), D register i lane l -> (m = 4i + l/16, n = l%16).
//  * scores S^T = K . Q^T  (m = key, n = query, k = head dims): the order of the dims in the
//    contraction is free, so lane slot g = l/16 owns the contiguous dims [g*hd/4, (g+1)*hd/4) and
//    MFMA s uses dim g*hd/4 + s: K and Q are read as float4s.  Two accumulators (even/odd s) keep
//    the MFMA dependency chain short.
//  * lane l then holds the scores of query l%16 against keys 4i + l/16 (i = 0..3); row max and
//    row sum reduce over the 4 registers and the lanes l^16, l^32.
//  * O^T += V^T . P^T  (m = output dim, n = query, k = key): MFMA c takes key slot s = l/16 as key
//    4c + s, which is exactly register c of the lane's P; the output dim of row m in dim block b is
//    m*(hd/16) + b, so V reads and O stores are contiguous per lane.
#include "common.h"

namespace mi {

typedef double v4d __attribute__((ext_vector_type(4)));

constexpr int AT_WAVES = 4;

template <int HD>
struct AttnTile {
  float4 k[HD / 16];          // K row (key0 + l%16), dims slot*HD/4 .. +HD/4
  float4 v[4][HD / 64];       // V rows key0 + 4c + slot, dims (l%16)*HD/16 .. +HD/16
};

template <int HD>
__device__ __forceinline__ void load_tile(AttnTile<HD>& t, const float* kbase, const float* vbase, int kv_embd,
                                          int key0, int pmax, int qi, int slot) {
  constexpr int Q4 = HD / 4, NB = HD / 16;
  const int krow = key0 + qi;
  const bool kok = krow <= pmax;
  const float* kp = kbase + (int64_t)(kok ? krow : 0) * kv_embd + slot * Q4;
#pragma unroll
  for (int s = 0; s < Q4 / 4; ++s)
    t.k[s] = kok ? *reinterpret_cast<const float4*>(kp + 4 * s) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int vrow = key0 + 4 * c + slot;
    const bool vok = vrow <= pmax;
    const float* vp = vbase + (int64_t)(vok ? vrow : 0) * kv_embd + qi * NB;
#pragma unroll
    for (int b = 0; b < NB / 4; ++b)
      t.v[c][b] = vok ? *reinterpret_cast<const float4*>(vp + 4 * b) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

__device__ __forceinline__ double f4get(const float4& v, int e) {
  return e == 0 ? (double)v.x : e == 1 ? (double)v.y : e == 2 ? (double)v.z : (double)v.w;
}

template <int HD>
__global__ void __launch_bounds__(64 * AT_WAVES) k_attention(const float* __restrict__ q, int64_t ld_q,
                                                             const float* __restrict__ k_region,
                                                             const float* __restrict__ v_region,
                                                             const int32_t* __restrict__ pos, int n_tokens,
                                                             int n_head, int n_head_kv, float* __restrict__ out,
                                                             int64_t ld_out) {
  constexpr int Q4 = HD / 4;    // dims per lane slot (scores) = MFMAs per score tile
  constexpr int NB = HD / 16;   // output dim blocks
  __shared__ double sh_m[AT_WAVES][64], sh_l[AT_WAVES][64];
  __shared__ double sh_o[AT_WAVES - 1][NB * 4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qi = lane & 15, slot = lane >> 4;
  const int h = blockIdx.y;
  const int g = h / (n_head / n_head_kv);
  const int kv_embd = n_head_kv * HD;
  const int t = blockIdx.x * 16 + qi;
  const bool valid = t < n_tokens;
  const int p = valid ? pos[t] : 0;
  int pmax = p;
  for (int o = 1; o < 16; o <<= 1) pmax = max(pmax, __shfl_xor(pmax, o));

  // query fragment: dims slot*Q4 + s, pre-scaled by 1/sqrt(hd) in f64
  const double scale = 1.0 / sqrt((double)HD);
  double qf[Q4];
  {
    const float* qp = q + (int64_t)(valid ? t : 0) * ld_q + (int64_t)h * HD + slot * Q4;
#pragma unroll
    for (int s = 0; s < Q4; s += 4) {
      const float4 v = *reinterpret_cast<const float4*>(qp + s);
      qf[s] = (double)v.x * scale;
      qf[s + 1] = (double)v.y * scale;
      qf[s + 2] = (double)v.z * scale;
      qf[s + 3] = (double)v.w * scale;
    }
  }

  v4d acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = v4d{0.0, 0.0, 0.0, 0.0};
  double m_run = -INFINITY, l_run = 0.0;

  const float* kbase = k_region + (int64_t)g * HD;
  const float* vbase = v_region + (int64_t)g * HD;
  const int ntiles = pmax / 16 + 1;
  AttnTile<HD> cur, nxt;
  int tile = wave;
  if (tile < ntiles) load_tile<HD>(cur, kbase, vbase, kv_embd, tile * 16, pmax, qi, slot);
  for (; tile < ntiles; tile += AT_WAVES) {
    const int key0 = tile * 16;
    if (tile + AT_WAVES < ntiles) load_tile<HD>(nxt, kbase, vbase, kv_embd, key0 + 16 * AT_WAVES, pmax, qi, slot);
    // ---- scores
    v4d sc0 = {0.0, 0.0, 0.0, 0.0}, sc1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < Q4; s += 2) {
      sc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(f4get(cur.k[s / 4], s % 4), qf[s], sc0, 0, 0, 0);
      sc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(f4get(cur.k[(s + 1) / 4], (s + 1) % 4), qf[s + 1], sc1, 0, 0, 0);
    }
    // ---- online softmax for query l%16 over keys key0 + 4i + slot
    double sv[4];
    double tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = key0 + 4 * i + slot;
      sv[i] = (key <= p) ? sc0[i] + sc1[i] : -INFINITY;
      tmax = fmax(tmax, sv[i]);
    }
    tmax = fmax(tmax, __shfl_xor(tmax, 16));
    tmax = fmax(tmax, __shfl_xor(tmax, 32));
    const double m_new = fmax(m_run, tmax);
    // a wave whose tiles so far are all masked for this query keeps m = -inf and p = 0
    const double corr = (m_run == -INFINITY) ? 0.0 : exp(m_run - m_new);
    double pv[4], psum = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = (sv[i] == -INFINITY) ? 0.0 : exp(sv[i] - m_new);
      psum += pv[i];
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] *= corr;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(f4get(cur.v[c][b / 4], b % 4), pv[c], acc[b], 0, 0, 0);
    cur = nxt;
  }

  // ---- merge the four waves' partial softmax states (f64, fixed order)
  sh_m[wave][lane] = m_run;
  sh_l[wave][lane] = l_run;
  if (wave > 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) sh_o[wave - 1][b * 4 + i][lane] = acc[b][i];
  }
  __syncthreads();
  if (wave == 0) {
    double mw[AT_WAVES], m_all = -INFINITY;
#pragma unroll
    for (int w = 0; w < AT_WAVES; ++w) {
      mw[w] = sh_m[w][lane];
      m_all = fmax(m_all, mw[w]);
    }
    double fw[AT_WAVES], l_all = 0.0;
#pragma unroll
    for (int w = 0; w < AT_WAVES; ++w) {
      fw[w] = (mw[w] == -INFINITY) ? 0.0 : exp(mw[w] - m_all);
      l_all += sh_l[w][lane] * fw[w];
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        double o = acc[b][i] * fw[0];
#pragma unroll
        for (int w = 1; w < AT_WAVES; ++w) o += sh_o[w - 1][b * 4 + i][lane] * fw[w];
        acc[b][i] = o;
      }
    if (valid) {
      float* op = out + (int64_t)t * ld_out + (int64_t)h * HD;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float* dst = op + (4 * i + slot) * NB;  // dims (4i + slot)*NB + b
#pragma unroll
        for (int b = 0; b < NB; b += 4) {
          float4 o;
          o.x = (float)(acc[b][i] / l_all);
          o.y = (float)(acc[b + 1][i] / l_all);
          o.z = (float)(acc[b + 2][i] / l_all);
          o.w = (float)(acc[b + 3][i] / l_all);
          *reinterpret_cast<float4*>(dst + b) = o;
        }
      }
    }
  }
}

int launch_attention(const float* q, int64_t ld_q, const float* k_region, const float* v_region,
                     const int32_t* pos, int n_tokens, int max_pos, int n_head, int n_head_kv,
                     int head_dim, float* out, int64_t ld_out, hipStream_t s) {
  (void)max_pos;
  if (n_tokens == 0) return MI_OK;
  dim3 grid((n_tokens + 15) / 16, n_head);
  if (head_dim == 64)
    hipLaunchKernelGGL(k_attention<64>, grid, dim3(64 * AT_WAVES), 0, s, q, ld_q, k_region, v_region, pos, n_tokens,
                       n_head, n_head_kv, out, ld_out);
  else if (head_dim == 128)
    hipLaunchKernelGGL(k_attention<128>, grid, dim3(64 * AT_WAVES), 0, s, q, ld_q, k_region, v_region, pos, n_tokens,
                       n_head, n_head_kv, out, ld_out);
  else
    return set_error(MI_ERR_UNSUPPORTED, "attention: head_dim %d (supported: 64, 128)", head_dim);
  MI_LAUNCH_CHECK("k_attention");
  return MI_OK;
}

}  // namespace mi
