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
// Selection: a wave holds a list of 64 (value, id) pairs, one per lane, and sorts it with a bitonic
// network of lane exchanges (no barriers); two sorted lists give the best 64 of both by comparing
// A[i] with B[63 - i] and six more exchange steps; a workgroup of 16 waves merges its 16 lists in a
// tree of 4 steps through LDS.  Every step keeps the total order above, so the kept set and its
// order are those of a full sort.
// k_sample_slices: 256 workgroups, one vocabulary slice each (at most 1024 tokens): penalize the
// slice's window tokens, sort each wave's 64, merge, keep the slice's top k.
// k_sample_merge: 16 workgroups, each merging the top-k lists of 16 slices, keep k.
// k_sample_pick: one workgroup merges the 16 lists; the weights of the top-p and temperature steps
// are computed one per lane, then one thread runs those steps and the draw in order (k <= 64).
#include "common.h"

namespace mi {

constexpr int SP_SLICES = 256;
constexpr int SP_GROUP = 16;        // slices merged per k_sample_merge workgroup
constexpr int SP_MAX_SLICE = 1024;  // elements per slice workgroup
constexpr int SP_THREADS = 1024;    // 16 waves: one 64-entry list per wave

struct SampleParamsDev {
  double repeat, frequency, presence, top_p, temperature;
  int top_k;
};

// a before b: larger value first, then the smaller id
__device__ __forceinline__ bool sp_before(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// compare-exchange with the lane at distance j: keep the better of the two (keep_best) or the worse
__device__ __forceinline__ void sp_cmpx(double& v, int& id, int j, bool keep_best) {
  const double pv = __shfl_xor(v, j, 64);
  const int pid = __shfl_xor(id, j, 64);
  const bool take = keep_best ? sp_before(pv, pid, v, id) : sp_before(v, id, pv, pid);
  if (take) {
    v = pv;
    id = pid;
  }
}

// the wave's 64 pairs (one per lane) into sp_before order, lane 0 first: bitonic network
__device__ __forceinline__ void sp_wave_sort(double& v, int& id, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) sp_cmpx(v, id, j, ((lane & j) == 0) == ((lane & k) == 0));
}

// sorted A (in the lanes) and sorted B (lane l given B[63 - l]) -> the best 64 of both, sorted:
// the better of A[l] and B[63 - l] form a bitonic sequence holding them, which six steps sort
__device__ __forceinline__ void sp_wave_merge(double& v, int& id, double bv, int bid, int lane) {
  if (sp_before(bv, bid, v, id)) {
    v = bv;
    id = bid;
  }
#pragma unroll
  for (int j = 32; j > 0; j >>= 1) sp_cmpx(v, id, j, (lane & j) == 0);
}

// the 16 waves' sorted lists -> wave 0 holds the best 64 of all, sorted.  At step s, waves
// w = s mod 2s publish and waves w = 0 mod 2s merge list w + s; the slots a step writes are never
// the ones the step before read, so one barrier per step suffices.
__device__ __forceinline__ void sp_tree(double& v, int& id, int lane, int wave, double (*sv)[64], int (*sid)[64]) {
#pragma unroll
  for (int s = 1; s < SP_THREADS / 64; s <<= 1) {
    if (wave % (2 * s) == s) {
      sv[wave][lane] = v;
      sid[wave][lane] = id;
    }
    __syncthreads();
    if (wave % (2 * s) == 0) sp_wave_merge(v, id, sv[wave + s][63 - lane], sid[wave + s][63 - lane], lane);
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
  __shared__ double sv[SP_THREADS / 64][64];
  __shared__ int sid[SP_THREADS / 64][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if ((int)threadIdx.x < n_window) window[threadIdx.x] = win.ids[threadIdx.x];
  const int slice = (vocab + SP_SLICES - 1) / SP_SLICES;
  const int lo = blockIdx.x * slice, hi = min(lo + slice, vocab);
  {
    const int i = threadIdx.x;  // slice <= SP_MAX_SLICE = SP_THREADS
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
  double x = v[threadIdx.x];
  int xi = id[threadIdx.x];
  sp_wave_sort(x, xi, lane);
  sp_tree(x, xi, lane, wave, sv, sid);
  if (wave == 0 && lane < p.top_k) {
    cand_v[blockIdx.x * p.top_k + lane] = x;
    cand_id[blockIdx.x * p.top_k + lane] = xi;
  }
}

// survivors of SP_GROUP slices -> their top k (candidate lists of the slices in order; each is
// sorted, so wave w takes list w as it is)
__global__ void __launch_bounds__(SP_THREADS) k_sample_merge(const double* __restrict__ in_v,
                                                            const int* __restrict__ in_id, int top_k,
                                                            double* __restrict__ out_v, int* __restrict__ out_id) {
  static_assert(SP_GROUP == SP_THREADS / 64, "one list per wave");
  __shared__ double sv[SP_THREADS / 64][64];
  __shared__ int sid[SP_THREADS / 64][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t base = ((int64_t)blockIdx.x * SP_GROUP + wave) * top_k;
  double x = lane < top_k ? in_v[base + lane] : -INFINITY;
  int xi = lane < top_k ? in_id[base + lane] : 0x7fffffff;
  sp_tree(x, xi, lane, wave, sv, sid);
  if (wave == 0 && lane < top_k) {
    out_v[blockIdx.x * top_k + lane] = x;
    out_id[blockIdx.x * top_k + lane] = xi;
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
  static_assert(SP_SLICES / SP_GROUP == SP_THREADS / 64, "one list per wave");
  __shared__ double sv[SP_THREADS / 64][64];
  __shared__ int sid[SP_THREADS / 64][64];
  __shared__ double exp_tab[64];
  __shared__ double e_top[64], e_tmp[64];  // e^(v_i - v_0) and e^(v_i / T - v_0 / T)
  exp2_table_fill(exp_tab, threadIdx.x);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double x = lane < p.top_k ? cand_v[wave * p.top_k + lane] : -INFINITY;
  int xi = lane < p.top_k ? cand_id[wave * p.top_k + lane] : 0x7fffffff;
  sp_tree(x, xi, lane, wave, sv, sid);
  if (wave != 0) return;
  // the best 64 in lane order: v, id; each lane computes its weights as the steps below use them
  double* v = sv[0];
  int* id = sid[0];
  v[lane] = x;
  id[lane] = xi;
  const double v0 = __shfl(x, 0, 64);
  e_top[lane] = exp_f64(x - v0, exp_tab);
  if (p.temperature != 0.0) e_tmp[lane] = exp_f64(x / p.temperature - v0 / p.temperature, exp_tab);
  if (lane != 0) return;  // a wave's own LDS writes are complete for its later reads
  int k = p.top_k;
  while (k > 1 && id[k - 1] == 0x7fffffff) --k;  // fewer real tokens than k (tiny vocabularies)
  if (p.top_p < 1.0) {  // untempered softmax of the candidates, cumulative in order
    double total = 0.0;
    for (int i = 0; i < k; ++i) total += e_top[i];
    double run = 0.0;
    int keep = k;
    for (int i = 0; i < k; ++i) {
      run += e_top[i] / total;
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
  double total = 0.0;
  for (int i = 0; i < k; ++i) total += e_tmp[i];
  const double target = (double)(splitmix64(seed, step) >> 11) * 0x1p-53 * total;
  double run = 0.0;
  int pick = id[k - 1];
  for (int i = 0; i < k; ++i) {
    run += e_tmp[i];
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
