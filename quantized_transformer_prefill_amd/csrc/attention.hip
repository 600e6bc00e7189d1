// Causal grouped-query attention over a layer's f32 KV regions, flash style, in f64.
//
// o[t][h] = sum_{j <= pos[t]} softmax_j(q[t][h] . k[j][g] / sqrt(hd)) v[j][g],  g = h / (nh/nkv).
// Token t sees region rows 0..=pos[t] (positions are data, read per element), after this call's
// KV store for the layer.  The node's result must round to the same f32 as the exact value, so
// scores, softmax and the weighted sum run in f64 on v_mfma_f64_16x16x4f64; the online-softmax
// bookkeeping (running max, running sum, rescale) is f64 on the VALU.
//
// One wave = 16 query tokens x 1 head, sweeping key tiles of 16 rows from row 0 to the largest
// position among its queries.  MFMA 16x16x4 f64 lane layout: A lane l -> (m = l%16, k = l/16),
// B lane l -> (k = l/16, n = l%16), D register i lane l -> (m = 4i + l/16, n = l%16).
//  * scores S^T = K . Q^T  (m = key, n = query, k = head dims): the contraction order over dims
//    is free, so lane slot g = l/16 owns the contiguous dims [g*hd/4, (g+1)*hd/4) and MFMA s uses
//    dim g*hd/4 + s: every lane reads its K and Q dims as float4s.
//  * lane l then holds the scores of query l%16 against keys 4i + l/16 (i = 0..3); row max and
//    row sum reduce over the 4 registers and the lanes l^16, l^32.
//  * O^T += V^T . P^T  (m = output dim, n = query, k = key): MFMA c takes key slot s = l/16 as
//    key 4c + s, which is exactly register c of the lane's P; the output dim of row m in dim
//    block b is m*(hd/16) + b so V reads and O stores are contiguous per lane.
#include "common.h"

namespace mi {

typedef double v4d __attribute__((ext_vector_type(4)));

template <int HD>
__global__ void __launch_bounds__(64) k_attention(const float* __restrict__ q, int64_t ld_q,
                                                  const float* __restrict__ k_region,
                                                  const float* __restrict__ v_region,
                                                  const int32_t* __restrict__ pos, int n_tokens, int n_head,
                                                  int n_head_kv, float* __restrict__ out, int64_t ld_out) {
  constexpr int Q4 = HD / 4;    // dims per lane slot (scores) = MFMAs per score tile
  constexpr int NB = HD / 16;   // output dim blocks
  const int lane = threadIdx.x;
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
  for (int key0 = 0; key0 <= pmax; key0 += 16) {
    // ---- scores: A = K rows key0 + l%16, dims slot*Q4 + s
    const int krow = key0 + qi;
    const bool kok = krow <= pmax;
    double kf[Q4];
    {
      const float* kp = kbase + (int64_t)(kok ? krow : 0) * kv_embd + slot * Q4;
#pragma unroll
      for (int s = 0; s < Q4; s += 4) {
        const float4 v = kok ? *reinterpret_cast<const float4*>(kp + s) : make_float4(0.f, 0.f, 0.f, 0.f);
        kf[s] = v.x;
        kf[s + 1] = v.y;
        kf[s + 2] = v.z;
        kf[s + 3] = v.w;
      }
    }
    v4d sc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < Q4; ++s) sc = __builtin_amdgcn_mfma_f64_16x16x4f64(kf[s], qf[s], sc, 0, 0, 0);

    // ---- V fragments for the 4 key slots: row key0 + 4c + slot, dims (l%16)*NB + b
    double vf[4][NB];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int vrow = key0 + 4 * c + slot;
      const bool vok = vrow <= pmax;
      const float* vp = vbase + (int64_t)(vok ? vrow : 0) * kv_embd + qi * NB;
#pragma unroll
      for (int b = 0; b < NB; b += 4) {
        const float4 v = vok ? *reinterpret_cast<const float4*>(vp + b) : make_float4(0.f, 0.f, 0.f, 0.f);
        vf[c][b] = v.x;
        vf[c][b + 1] = v.y;
        vf[c][b + 2] = v.z;
        vf[c][b + 3] = v.w;
      }
    }

    // ---- online softmax for query l%16 over keys key0 + 4i + slot
    double sv[4];
    double tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = key0 + 4 * i + slot;
      sv[i] = (key <= p) ? sc[i] : -INFINITY;
      tmax = fmax(tmax, sv[i]);
    }
    tmax = fmax(tmax, __shfl_xor(tmax, 16));
    tmax = fmax(tmax, __shfl_xor(tmax, 32));
    const double m_new = fmax(m_run, tmax);
    const double corr = exp(m_run - m_new);
    double pv[4], psum = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = exp(sv[i] - m_new);
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
      for (int b = 0; b < NB; ++b) acc[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(vf[c][b], pv[c], acc[b], 0, 0, 0);
  }

  if (valid) {
    float* op = out + (int64_t)t * ld_out + (int64_t)h * HD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mrow = 4 * i + slot;  // dims mrow*NB + b
      float* dst = op + mrow * NB;
#pragma unroll
      for (int b = 0; b < NB; b += 4) {
        float4 o;
        o.x = (float)(acc[b][i] / l_run);
        o.y = (float)(acc[b + 1][i] / l_run);
        o.z = (float)(acc[b + 2][i] / l_run);
        o.w = (float)(acc[b + 3][i] / l_run);
        *reinterpret_cast<float4*>(dst + b) = o;
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
    hipLaunchKernelGGL(k_attention<64>, grid, dim3(64), 0, s, q, ld_q, k_region, v_region, pos, n_tokens, n_head,
                       n_head_kv, out, ld_out);
  else if (head_dim == 128)
    hipLaunchKernelGGL(k_attention<128>, grid, dim3(64), 0, s, q, ld_q, k_region, v_region, pos, n_tokens, n_head,
                       n_head_kv, out, ld_out);
  else
    return set_error(MI_ERR_UNSUPPORTED, "attention: head_dim %d (supported: 64, 128)", head_dim);
  MI_LAUNCH_CHECK("k_attention");
  return MI_OK;
}

}  // namespace mi
