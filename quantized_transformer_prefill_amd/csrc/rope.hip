// NeoX RoPE of Q and K by token position, and the KV store of the rotated K and the
// raw V into row positions[t] of the layer's regions.
//
// The rotation angle table is computed once on the host in f64 (cos and sin of
// p * theta^(-2i/hd)) and read by the kernel, so every token's rotation uses the same
// angles the host math library gives; the rotation itself runs in f64 and rounds once.
#include <cmath>
#include <vector>

#include "common.h"

namespace mi {

__global__ void __launch_bounds__(256) k_rope_kvstore(float* __restrict__ q, int64_t ld_q,
                                                      const float* __restrict__ k, const float* __restrict__ v,
                                                      int64_t ld_kv, const int32_t* __restrict__ pos,
                                                      int n_head, int n_head_kv, int head_dim,
                                                      const double2* __restrict__ table,
                                                      float* __restrict__ k_region, float* __restrict__ v_region) {
  const int t = blockIdx.x;
  const int half = head_dim / 2;
  const int64_t p = pos[t];
  const double2* row = table + p * half;
  float* qt = q + (int64_t)t * ld_q;
  const float* kt = k + (int64_t)t * ld_kv;
  const float* vt = v + (int64_t)t * ld_kv;
  const int kv_embd = n_head_kv * head_dim;
  float* kr = k_region + p * kv_embd;
  float* vr = v_region + p * kv_embd;
  const int nq = n_head * half, nk = n_head_kv * half;
  for (int idx = threadIdx.x; idx < nq + nk; idx += blockDim.x) {
    const bool is_q = idx < nq;
    const int j = is_q ? idx : idx - nq;
    const int h = j / half, i = j - h * half;
    const float* src = is_q ? qt : kt;
    const int64_t o0 = (int64_t)h * head_dim + i, o1 = o0 + half;
    const double a = src[o0], b = src[o1];
    const double2 cs = row[i];
    const float r0 = (float)(a * cs.x - b * cs.y);
    const float r1 = (float)(a * cs.y + b * cs.x);
    if (is_q) {
      qt[o0] = r0;
      qt[o1] = r1;
    } else {
      kr[o0] = r0;
      kr[o1] = r1;
    }
  }
  for (int j = threadIdx.x; j < kv_embd; j += blockDim.x) vr[j] = vt[j];
}

int launch_rope_kvstore(float* q, int64_t ld_q, const float* k, const float* v, int64_t ld_kv,
                        const int32_t* pos, int n_tokens, int n_head, int n_head_kv, int head_dim,
                        const double* table, float* k_region, float* v_region, hipStream_t s) {
  if (n_tokens == 0) return MI_OK;
  hipLaunchKernelGGL(k_rope_kvstore, dim3(n_tokens), dim3(256), 0, s, q, ld_q, k, v, ld_kv, pos, n_head,
                     n_head_kv, head_dim, reinterpret_cast<const double2*>(table), k_region, v_region);
  MI_LAUNCH_CHECK("k_rope_kvstore");
  return MI_OK;
}

}  // namespace mi

extern "C" size_t mi_rope_table_bytes(const mi_hparams* hp, int32_t rows) {
  if (!hp || rows <= 0 || hp->head_dim <= 0) return 0;
  return (size_t)rows * (size_t)(hp->head_dim / 2) * 2 * sizeof(double);
}

extern "C" int mi_rope_table_init(const mi_hparams* hp, int32_t rows, double* table, void* stream) {
  using namespace mi;
  if (!hp || !table || rows <= 0 || hp->head_dim <= 0 || (hp->head_dim & 1))
    return set_error(MI_ERR_INVALID_ARG, "mi_rope_table_init: bad arguments");
  const int hd = hp->head_dim, half = hd / 2;
  std::vector<double> host((size_t)rows * half * 2);
  const double theta = (double)hp->rope_theta;
  std::vector<double> inv(half);
  for (int i = 0; i < half; ++i) inv[i] = std::pow(theta, -2.0 * (double)i / (double)hd);
  for (int p = 0; p < rows; ++p)
    for (int i = 0; i < half; ++i) {
      const double ang = (double)p * inv[i];
      host[((size_t)p * half + i) * 2 + 0] = std::cos(ang);
      host[((size_t)p * half + i) * 2 + 1] = std::sin(ang);
    }
  hipStream_t s = as_stream(stream);
  MI_HIP(hipMemcpyAsync(table, host.data(), host.size() * sizeof(double), hipMemcpyHostToDevice, s));
  MI_HIP(hipStreamSynchronize(s));
  return MI_OK;
}
