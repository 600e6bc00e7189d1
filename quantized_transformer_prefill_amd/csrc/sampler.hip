// Sampler: one next token from last-token logits (the sampler row of the walkthrough index: penalties
// over the last-64 window -> top-k -> top-p -> temperature -> seeded sample).
//
//   penalties   token t seen c_t > 0 times in the window: l = l / repeat if l > 0 else l * repeat,
//               then l - c_t * frequency - presence, in f64 from the f32 logit
//   top-k       the k largest penalized logits, ties by the smaller token id
//   top-p       softmax of the candidates (untempered: temperature comes later in the chain); the
//               shortest prefix whose cumulative probability reaches top_p
//   temperature kept logits / T; T = 0 picks the first candidate
//   sample      u = SplitMix64(seed, step) >> 11 * 2^-53; weights e^(l_i - l_0); the first
//               candidate whose running weight sum exceeds u * total
//
// k_sample_slices: 256 workgroups, one vocabulary slice each (at most 1024 tokens): penalize the
// slice's window tokens, bitonic-sort the slice in LDS by (value desc, id asc), keep its top k.
// k_sample_merge: 16 workgroups, each sorting the survivors of 16 slices (16 k <= 1024), keep k.
// k_sample_pick: one workgroup sorts the 16 x k survivors the same way, then one thread runs the
// top-p / temperature / draw steps in order (k <= 64 values).
#include "common.h"

namespace mi {

constexpr int SP_SLICES = 256;
constexpr int SP_GROUP = 16;        // slices merged per k_sample_merge workgroup
constexpr int SP_MAX_SLICE = 1024;  // elements sorted per workgroup
constexpr int SP_THREADS = 512;     // one compare-exchange per thread per pass

struct SampleParamsDev {
  double repeat, frequency, presence, top_p, temperature;
  int top_k;
};

// a before b: larger value first, then the smaller id
__device__ __forceinline__ bool sp_before(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// bitonic sort of n (a power of two) (value, id) pairs in LDS into sp_before order
__device__ void sp_sort(double* v, int* id, int n) {
  for (int k = 2; k <= n; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int p = i ^ j;
        if (p > i) {
          const bool swap = (i & k) == 0 ? sp_before(v[p], id[p], v[i], id[i]) : sp_before(v[i], id[i], v[p], id[p]);
          if (swap) {
            const double tv = v[i]; v[i] = v[p]; v[p] = tv;
            const int ti = id[i]; id[i] = id[p]; id[p] = ti;
          }
        }
      }
      __syncthreads();
    }
}

// the last (up to) 64 window ids, passed by value as a kernel argument: no host-to-device copy
struct SampleWindow {
  int32_t ids[64];
};

__global__ void __launch_bounds__(SP_THREADS) k_sample_slices(const float* __restrict__ logits, int vocab,
                                                             const SampleWindow win, int n_window,
                                                             SampleParamsDev p, double* __restrict__ cand_v,
                                                             int* __restrict__ cand_id) {
  __shared__ double v[SP_MAX_SLICE];
  __shared__ int id[SP_MAX_SLICE];
  __shared__ int window[64];
  if ((int)threadIdx.x < n_window) window[threadIdx.x] = win.ids[threadIdx.x];
  const int slice = (vocab + SP_SLICES - 1) / SP_SLICES;
  const int lo = blockIdx.x * slice, hi = min(lo + slice, vocab);
  int n = 1;
  while (n < slice) n <<= 1;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int t = lo + i;
    const bool in = i < slice && t < hi;
    v[i] = in ? (double)logits[t] : -INFINITY;
    id[i] = in ? t : 0x7fffffff;
  }
  __syncthreads();
  if ((int)threadIdx.x < n_window) {  // each distinct window token once: at its first occurrence
    const int t = window[threadIdx.x];
    bool first = true;
    int c = 0;
    for (int s = 0; s < n_window; ++s) {
      const int u = window[s];
      c += u == t;
      if (u == t && s < (int)threadIdx.x) first = false;
    }
    if (first && t >= lo && t < hi) {
      double x = v[t - lo];
      x = x > 0.0 ? x / p.repeat : x * p.repeat;
      x = x - (double)c * p.frequency - p.presence;
      v[t - lo] = x;
    }
  }
  __syncthreads();
  sp_sort(v, id, n);
  for (int i = threadIdx.x; i < p.top_k; i += blockDim.x) {
    cand_v[blockIdx.x * p.top_k + i] = i < n ? v[i] : -INFINITY;
    cand_id[blockIdx.x * p.top_k + i] = i < n ? id[i] : 0x7fffffff;
  }
}

// survivors of SP_GROUP slices -> their top k (candidate lists of the slices in order)
__global__ void __launch_bounds__(SP_THREADS) k_sample_merge(const double* __restrict__ in_v,
                                                            const int* __restrict__ in_id, int top_k,
                                                            double* __restrict__ out_v, int* __restrict__ out_id) {
  __shared__ double v[SP_MAX_SLICE];
  __shared__ int id[SP_MAX_SLICE];
  const int m = SP_GROUP * top_k;
  int n = 1;
  while (n < m) n <<= 1;
  const int64_t base = (int64_t)blockIdx.x * m;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    v[i] = i < m ? in_v[base + i] : -INFINITY;
    id[i] = i < m ? in_id[base + i] : 0x7fffffff;
  }
  __syncthreads();
  sp_sort(v, id, n);
  for (int i = threadIdx.x; i < top_k; i += blockDim.x) {
    out_v[blockIdx.x * top_k + i] = v[i];
    out_id[blockIdx.x * top_k + i] = id[i];
  }
}

__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t step) {
  uint64_t z = seed + (step + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void __launch_bounds__(SP_THREADS) k_sample_pick(const double* __restrict__ cand_v,
                                                           const int* __restrict__ cand_id, SampleParamsDev p,
                                                           uint64_t seed, uint64_t step, int32_t* __restrict__ token_out) {
  __shared__ double v[SP_MAX_SLICE];
  __shared__ int id[SP_MAX_SLICE];
  __shared__ double exp_tab[64];
  exp2_table_fill(exp_tab, threadIdx.x);
  const int m = (SP_SLICES / SP_GROUP) * p.top_k;
  int n = 1;
  while (n < m) n <<= 1;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    v[i] = i < m ? cand_v[i] : -INFINITY;
    id[i] = i < m ? cand_id[i] : 0x7fffffff;
  }
  __syncthreads();
  sp_sort(v, id, n);
  if (threadIdx.x != 0) return;
  int k = p.top_k;
  while (k > 1 && id[k - 1] == 0x7fffffff) --k;  // fewer real tokens than k (tiny vocabularies)
  if (p.top_p < 1.0) {  // untempered softmax of the candidates, cumulative in order
    double total = 0.0;
    for (int i = 0; i < k; ++i) total += exp_f64(v[i] - v[0], exp_tab);
    double run = 0.0;
    int keep = k;
    for (int i = 0; i < k; ++i) {
      run += exp_f64(v[i] - v[0], exp_tab) / total;
      if (run >= p.top_p) {
        keep = i + 1;
        break;
      }
    }
    k = keep;
  }
  if (p.temperature == 0.0) {
    *token_out = id[0];
    return;
  }
  const double l0 = v[0] / p.temperature;
  double total = 0.0;
  for (int i = 0; i < k; ++i) total += exp_f64(v[i] / p.temperature - l0, exp_tab);
  const double target = (double)(splitmix64(seed, step) >> 11) * 0x1p-53 * total;
  double run = 0.0;
  int pick = id[k - 1];
  for (int i = 0; i < k; ++i) {
    run += exp_f64(v[i] / p.temperature - l0, exp_tab);
    if (run > target) {
      pick = id[i];
      break;
    }
  }
  *token_out = pick;
}

size_t sampler_workspace_bytes() {
  const size_t first = (size_t)SP_SLICES * MI_SAMPLER_MAX_K, second = (size_t)(SP_SLICES / SP_GROUP) * MI_SAMPLER_MAX_K;
  return (first + second) * (sizeof(double) + sizeof(int)) + 64 * sizeof(int32_t) + 256;
}

int launch_sample(const float* logits, int vocab, const int32_t* window, int n_window, const mi_sampler_params& hp,
                  uint64_t seed, uint64_t step, void* workspace, int32_t* token_out, hipStream_t s) {
  SampleWindow win{};
  for (int i = 0; i < n_window && i < 64; ++i) win.ids[i] = window[i];
  SampleParamsDev p;
  p.repeat = hp.repeat_penalty;
  p.frequency = hp.frequency_penalty;
  p.presence = hp.presence_penalty;
  p.top_p = hp.top_p;
  p.temperature = hp.temperature;
  p.top_k = hp.top_k;
  const size_t first = (size_t)SP_SLICES * MI_SAMPLER_MAX_K, second = (size_t)(SP_SLICES / SP_GROUP) * MI_SAMPLER_MAX_K;
  char* ws = reinterpret_cast<char*>(workspace);
  double* cv = reinterpret_cast<double*>(ws);
  double* cv2 = cv + first;
  int* ci = reinterpret_cast<int*>(cv2 + second);
  int* ci2 = ci + first;
  hipLaunchKernelGGL(k_sample_slices, dim3(SP_SLICES), dim3(SP_THREADS), 0, s, logits, vocab, win, n_window, p,
                     cv, ci);
  MI_LAUNCH_CHECK("k_sample_slices");
  hipLaunchKernelGGL(k_sample_merge, dim3(SP_SLICES / SP_GROUP), dim3(SP_THREADS), 0, s, cv, ci, p.top_k, cv2, ci2);
  MI_LAUNCH_CHECK("k_sample_merge");
  hipLaunchKernelGGL(k_sample_pick, dim3(1), dim3(SP_THREADS), 0, s, cv2, ci2, p, seed, step, token_out);
  MI_LAUNCH_CHECK("k_sample_pick");
  return MI_OK;
}

}  // namespace mi
