// Q8_0 x Q8_0 matmul on int8 MFMA with an exact per-block scale epilogue.
//
// out[m][n] = sum_kb da[m][kb] * dw[n][kb] * I[m][n][kb],  I = sum over the 32 values of the
// block of qa * qw (the matmul node of the Qwen2 layer; activations quantized to Q8_0 on the
// fly, weights stored [out][in]).
//
// * I comes from v_mfma_i32_32x32x32_i8: K = 32 is exactly one Q8_0 block, so every MFMA
//   yields the integer block sums of one block.
// * The scale epilogue is exact.  Only the even rows of each 32x32 MFMA carry data; the odd
//   rows have all-zero A rows, so the accumulator initial value passes through them
//   unchanged.  The initial value is 0x80000000 on even rows and 0x43380000 on odd rows, so
//   each (even, odd) output register pair is directly the f64 number 1.5*2^52 + 2^31 + I.
//   Then t = fma(x, dw, -(1.5*2^52 + 2^31)*dw) is exactly I*dw, and acc = fma(t, da, acc)
//   adds the exact product I*dw*da with a single f64 rounding.  With f64 accumulation the
//   rounded f32 result matches f32(exact sum) except for f64 rounding at ties.
// * The VALU f64 epilogue (2 f64 FMAs per output per block) bounds this kernel, not the
//   MFMA: half-used MFMAs cost nothing extra.
//
// Tiling: 256 threads = 4 waves (2 x 2, or 4 x 1 for the fused SwiGLU at few rows).  Wave tile
// RG x CG MFMAs of 16 real rows x 32 columns: 4 x 2 (workgroup 128 x 128) for large problems of
// >= 1024 rows, 2 x 2 (64 x 128) for other large ones, 1 x 2 (32 x 128, or 64 x 64 with the waves
// stacked 4 x 1) and 1 x 1 (workgroup 32 x 64) for small ones; 1 x 1 tiles of long reductions
// that cannot fill the chip run two groups of 4 waves per workgroup, each over half of the K range,
// their f64 sums added in LDS before the epilogue.  A stage of 4 blocks (128 K values) of codes and f64 scales goes through LDS, double-buffered,
// with the next stage's global loads in flight while the current one computes.  Split-K writes f64 partials that a second kernel
// reduces in a fixed order (deterministic).
#include <mutex>

#include "common.h"
#include "q8_epilogue.h"

namespace mi {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef double v8d __attribute__((ext_vector_type(8)));

constexpr int G_THREADS = 256;
constexpr int G_KS = 4;     // Q8_0 blocks per LDS stage (128 K values)

// Wave tile = RG x CG MFMAs (16 real rows x 32 columns each); workgroup = 2 x 2 waves.
// LDS rows hold the 4 blocks of a stage back to back (128 bytes = 8 chunks of 16).  Chunk c of
// row r sits at position c ^ (r & 7), so the 16-byte fragment reads of 8 consecutive rows at one
// chunk hit 8 different 16-byte bank groups; one extra all-zero row feeds the odd (dummy) MFMA
// rows.
constexpr int G_ROWB = G_KS * QK;  // bytes per LDS row
// Ring depth (stages in LDS) per tile shape.  Two: deeper rings cost more in workgroups per CU (LDS)
// than they gain in latency hiding at the model's shapes (measured for 3 and 4 stages).
constexpr int G_NS_11 = 2, G_NS_12 = 2, G_NS_22 = 2;
__device__ __forceinline__ int swz(int row, int chunk) { return ((chunk ^ (row & 7)) << 4); }

// NS stages live in a ring; every load into it is a global->LDS transfer.
// Scales of a stage, two layouts:
//  * SP (scale pairs; the row length in blocks is even): word [row][p] holds the fp16 scales of
//    blocks 2p (low half) and 2p+1 (high half) of the stage, moved 4 bytes per lane -- one
//    transfer instruction covers 32 rows x 4 blocks;
//  * otherwise word [block][row] holds one fp16 scale in its low half, moved 2 bytes per lane.
// WM: waves along the rows (2: a 2 x 2 arrangement; 4: the waves stacked 4 x 1)
template <int RG, int CG, int NS, bool SP, int WM = 2>
struct GemmTile {
  static constexpr int BM = WM * 16 * RG;         // real activation rows per workgroup
  static constexpr int BN = (4 / WM) * 32 * CG;   // weight rows (output columns) per workgroup
  int8_t a[NS][BM + 1][G_ROWB];   // row BM is all zeros
  int8_t b[NS][BN][G_ROWB];
  uint32_t as[NS][SP ? 2 * BM : G_KS * BM];
  uint32_t bs[NS][SP ? 2 * BN : G_KS * BN];
};

// 16 bytes per lane from gbase + voff into LDS at lds + 16 * lane (global_load_lds_dwordx4: M0
// holds the wave's LDS base; one wait state between writing M0 and the load).  Written as inline
// assembly so that the compiler does not make every later LDS read wait for these loads: they
// target the other LDS buffer, and the kernel waits for them (vmcnt) before its barrier.
// a wave-uniform pointer, held in SGPRs
template <typename P>
__device__ __forceinline__ P* sgpr_ptr(P* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void lds_dma16(void* lds, const int8_t* gbase, uint32_t voff) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  gbase = sgpr_ptr(gbase);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(l), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
// The same for 2 bytes per lane (global_load_lds_ushort): lane l's value lands in the low half of
// the 4-byte word at lds + 4 * lane, the high half is zeroed.
__device__ __forceinline__ void lds_dma2(void* lds, const uint16_t* gbase, uint32_t voff) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  gbase = sgpr_ptr(gbase);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_ushort %1, %2"
               :
               : "s"(l), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
// The same for 4 bytes per lane (global_load_lds_dword): lane l's word lands at lds + 4 * lane.
__device__ __forceinline__ void lds_dma4(void* lds, const uint16_t* gbase, uint32_t voff) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  gbase = sgpr_ptr(gbase);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(l), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
// x, as a value the compiler cannot compute ahead of this point (keeps loop-invariant address
// arithmetic inside the loop instead of in registers)
__device__ __forceinline__ uint32_t opaque_u32(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
// s_waitcnt vmcnt(N), expcnt and lgkmcnt left at their maxima
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// KW: groups of 4 waves that split the workgroup's K range between them and add their f64 sums in
// LDS before the epilogue (2: more waves per output tile when the tiles cannot fill the chip)
template <int RG, int CG, int EPI, bool SPLIT, int NS, bool SP, int WM = 2, int KW = 1>
__global__ void __launch_bounds__(G_THREADS * KW, KW == 2 ? 2 : (WM == 4 ? 4 : (RG == 1 ? 3 : 2)))
k_gemm_q8(const int8_t* __restrict__ a_codes, const uint16_t* __restrict__ a_scales, int M,
          const int8_t* __restrict__ w_codes, const uint16_t* __restrict__ w_scales, int N, int K,
          const float* __restrict__ bias, const float* residual, float* out, int64_t ld_out,
          int8_t* __restrict__ q_codes, uint16_t* __restrict__ q_scales,
          double* __restrict__ partial, int kb_per_split, int xcd_order, QkvEpi qe) {
  using T = GemmTile<RG, CG, NS, SP, WM>;
  constexpr int BM = T::BM, BN = T::BN;
  static_assert(!SP || NS == 2, "scale pairs: one wait for all of a stage's transfers");
  static_assert(KW == 1 || (KW == 2 && EPI == EPI_F32 && WM == 2), "K groups: plain f32 / partial epilogue");
  __shared__ __align__(16) T sm_all[KW];
  __shared__ double exp_tab[EPI == EPI_SWIGLU_Q8 ? 64 : 1];  // 2^(j/64) for the SiLU
  const int tid = threadIdx.x;
  if constexpr (EPI == EPI_SWIGLU_Q8) exp2_table_fill(exp_tab, tid);
  const int lane = tid & 63, wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index held in an SGPR
  const int kgrp = wave_all >> 2, wave = wave_all & 3;  // K group, wave within it
  T& sm = sm_all[kgrp];
  const int wm = wave / (4 / WM), wn = wave % (4 / WM);
  // XCD-aware tile order.  Workgroups are dispatched round-robin over the 8 XCDs, each with its
  // own L2; workgroup L is given tile t so that every XCD owns one contiguous range of tiles, and
  // t walks the row tiles fastest, so the workgroups of an XCD share the weight tiles they read.
  // Applied when the weight matrix exceeds what one XCD's L2 holds (xcd_order != 0).
  const int gx = gridDim.x, gy = gridDim.y;
  const int n_all = gx * gy * gridDim.z;
  const int L = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int xq = n_all >> 3, xr = n_all & 7, xcd = L & 7;
  const int t = xcd_order ? xcd * xq + min(xcd, xr) + (L >> 3)
                          : blockIdx.y + gy * (blockIdx.x + gx * blockIdx.z);
  const int n0 = ((t / gy) % gx) * BN, m0 = (t % gy) * BM;
  const int kz = t / (gx * gy);  // K split
  const int KB = K / QK;
  int kb0 = kz * kb_per_split;
  int kb1 = min(KB, kb0 + kb_per_split);
  // K groups: the first takes the first half of the slice's stages (rounded up), the second the rest
  const int ns_it = KW == 1 ? (kb1 - kb0 + G_KS - 1) / G_KS : ((kb1 - kb0 + G_KS - 1) / G_KS + 1) / 2;
  if constexpr (KW == 2) {
    const int mid = min(kb1, kb0 + ns_it * G_KS);
    if (kgrp == 0) kb1 = mid;
    else kb0 = mid;
  }

  // QKV epilogue of the smallest tile: the positions and (cos, sin) of this thread's RoPE pairs
  // are requested now, so they arrive while the K loop runs
  constexpr int QPRE = (EPI == EPI_QKV && RG == 1 && CG == 1) ? BM * BN / 2 / G_THREADS : 0;
  double2 qcs[QPRE > 0 ? QPRE : 1];
  int64_t qpos[QPRE > 0 ? QPRE : 1];
  if constexpr (QPRE > 0) {
#pragma unroll
    for (int k = 0; k < QPRE; ++k) {
      const int row = m0 + (tid + k * G_THREADS) / (BN / 2);
      qpos[k] = row < M ? qe.pos[row] : 0;
    }
  }
  // bias of this lane's output columns (bit patterns), requested before the K loop
  uint32_t bias_b[CG];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) bias_b[cg] = 0u;
  if (bias) {
#pragma unroll
    for (int cg = 0; cg < CG; ++cg)
      bias_b[cg] = reinterpret_cast<const uint32_t*>(bias)[min(n0 + wn * 32 * CG + cg * 32 + (lane & 31), N - 1)];
  }

  // zero row for the dummy MFMA rows (every ring slot)
  if ((tid & (G_THREADS - 1)) < NS * G_ROWB / 16)
    *reinterpret_cast<v4i*>(&sm.a[(tid & (G_THREADS - 1)) / (G_ROWB / 16)][BM][((tid & (G_THREADS - 1)) % (G_ROWB / 16)) * 16]) =
        v4i{0, 0, 0, 0};

  // ---- codes: global -> LDS directly (global_load_lds_dwordx4).  One wave instruction moves 64
  // chunks of 16 bytes = 8 whole LDS rows; lane l lands at row 8q + (l >> 3), position l & 7,
  // which holds chunk (l & 7) ^ (l >> 3) of that row (the XOR layout above).  Instruction q of
  // wave w covers rows 8(4q + w)..+7.  Rows past M (N) re-read the last valid row: their outputs
  // are never stored.  The per-lane source offsets do not change from stage to stage; the stage's
  // K position goes into the uniform base address.
  constexpr int A_DMA = BM / 32, B_DMA = BN / 32;   // instructions per wave per stage
  const int lchunk = (lane & 7) ^ (lane >> 3);
  // The 4-row-group tile keeps one offset per operand: in a tile without row (column) tail the
  // instructions differ by 32 rows, which go into the uniform base address; a tail tile computes
  // its clamped offsets at each issue (from a value the compiler cannot hoist), so they hold no
  // registers through the K loop.
  constexpr bool LEAN = RG == 4;
  constexpr int A_OFF = LEAN ? 1 : A_DMA, B_OFF = LEAN ? 1 : B_DMA;
  const bool a_full = m0 + BM <= M, b_full = n0 + BN <= N;
  const int a_r0 = m0 + 8 * wave + (lane >> 3), b_r0 = n0 + 8 * wave + (lane >> 3);
  uint32_t a_off[A_OFF], b_off[B_OFF];
#pragma unroll
  for (int q = 0; q < A_OFF; ++q) a_off[q] = (uint32_t)min(a_r0 + 32 * q, M - 1) * (uint32_t)K + lchunk * 16;
#pragma unroll
  for (int q = 0; q < B_OFF; ++q) b_off[q] = (uint32_t)min(b_r0 + 32 * q, N - 1) * (uint32_t)K + lchunk * 16;
  // ---- scales: global -> LDS directly too.
  // SP: 4 bytes per lane; wave w moves the pairs of rows 32w..32w+31 (lane l: row l/2, pair l%2)
  // of A (w < BM/32) and of B (w < BN/32).
  // Otherwise 2 bytes per lane; per stage, wave w moves the A scales of block w (rows 64i + l,
  // l < AS_L, one instruction per 64 rows) and the B-scale elements 64(w + 4i) + l (block
  // (64(w + 4i) + l) / BN, row (64(w + 4i) + l) % BN).
  static_assert(G_KS == 4, "one A-scale block per wave");
  constexpr int AS_L = BM < 64 ? BM : 64;   // lanes per A-scale instruction
  constexpr int AS_I = SP ? 0 : BM / AS_L;  // A-scale instructions per wave: 1 or 2
  constexpr int BS_I = SP ? 0 : BN * G_KS / 256;  // 1 or 2
  constexpr int AP_I = SP ? BM / 32 : 0, BP_I = SP ? BN / 32 : 0;  // waves moving pairs
  static_assert(SP || (AS_L * AS_I == BM && BS_I * 256 == BN * G_KS), "scale transfer shape");
  static_assert(AP_I <= 4 && BP_I <= 4, "one pair instruction per wave and operand");
  constexpr int L_OPS = A_DMA + B_DMA + AS_I + BS_I + (SP ? 2 : 0);  // transfers per wave per stage (at most)
  constexpr int AS_OFF = SP ? 1 : (LEAN ? 1 : AS_I);
  uint32_t as_off[AS_OFF];
  if constexpr (SP) {
    as_off[0] = (uint32_t)min(m0 + 32 * wave + (lane >> 1), M - 1) * (uint32_t)(KB * 2) + 4 * (lane & 1);
  } else {
#pragma unroll
    for (int i = 0; i < AS_OFF; ++i) as_off[i] = (uint32_t)min(m0 + 64 * i + lane, M - 1) * (uint32_t)(KB * 2);
  }
  // row (64(w + 4i) + l) % BN does not depend on i (256 is a multiple of BN)
  static_assert(256 % BN == 0, "B-scale rows");
  const uint32_t bs_off = SP ? (uint32_t)min(n0 + 32 * wave + (lane >> 1), N - 1) * (uint32_t)(KB * 2) + 4 * (lane & 1)
                             : (uint32_t)min(n0 + (64 * wave + lane) % BN, N - 1) * (uint32_t)(KB * 2);
  auto issue = [&](int kbs, int st) {
    // a stage past the end of the slice (K not a multiple of the stage) re-reads its last block
    // for the missing ones; compute() skips them
    const int nbk = min(G_KS, kb1 - kbs);
    const uint32_t fix = nbk < G_KS ? (uint32_t)((min(lchunk, 2 * nbk - 1) - lchunk) * 16) : 0u;
    const int8_t* ga = a_codes + (int64_t)kbs * QK;
    const int8_t* gb = w_codes + (int64_t)kbs * QK;
    const uint16_t* gas = a_scales + kbs + min(wave, nbk - 1);
    if constexpr (LEAN) {
      if (a_full) {
#pragma unroll
        for (int q = 0; q < A_DMA; ++q) lds_dma16(&sm.a[st][8 * (4 * q + wave)][0], ga + (int64_t)32 * q * K, a_off[0] + fix);
#pragma unroll
        for (int i = 0; i < AS_I; ++i)
          if (lane < AS_L) lds_dma2(&sm.as[st][wave * BM + 64 * i], gas + (int64_t)64 * i * KB, as_off[0]);
      } else {
        const int r0 = (int)opaque_u32((uint32_t)a_r0), l0 = (int)opaque_u32((uint32_t)lane);
#pragma unroll
        for (int q = 0; q < A_DMA; ++q)
          lds_dma16(&sm.a[st][8 * (4 * q + wave)][0], ga,
                    (uint32_t)min(r0 + 32 * q, M - 1) * (uint32_t)K + lchunk * 16 + fix);
#pragma unroll
        for (int i = 0; i < AS_I; ++i)
          if (lane < AS_L)
            lds_dma2(&sm.as[st][wave * BM + 64 * i], gas, (uint32_t)min(m0 + 64 * i + l0, M - 1) * (uint32_t)(KB * 2));
      }
      if (b_full) {
#pragma unroll
        for (int q = 0; q < B_DMA; ++q) lds_dma16(&sm.b[st][8 * (4 * q + wave)][0], gb + (int64_t)32 * q * K, b_off[0] + fix);
      } else {
        const int r0 = (int)opaque_u32((uint32_t)b_r0);
#pragma unroll
        for (int q = 0; q < B_DMA; ++q)
          lds_dma16(&sm.b[st][8 * (4 * q + wave)][0], gb,
                    (uint32_t)min(r0 + 32 * q, N - 1) * (uint32_t)K + lchunk * 16 + fix);
      }
    } else {
#pragma unroll
      for (int q = 0; q < A_DMA; ++q) lds_dma16(&sm.a[st][8 * (4 * q + wave)][0], ga, a_off[q] + fix);
#pragma unroll
      for (int q = 0; q < B_DMA; ++q) lds_dma16(&sm.b[st][8 * (4 * q + wave)][0], gb, b_off[q] + fix);
#pragma unroll
      for (int i = 0; i < AS_I; ++i)
        if (lane < AS_L) lds_dma2(&sm.as[st][wave * BM + 64 * i], gas, as_off[i]);
    }
    if constexpr (SP) {
      // a stage shorter than G_KS blocks has 2 (rows hold an even number of blocks, and stages
      // start at multiples of 4): its second pair re-reads the first, which compute() skips
      const uint32_t pfix = (nbk < G_KS && (lane & 1)) ? 4u : 0u;
      if (wave < AP_I) lds_dma4(&sm.as[st][64 * wave], a_scales + kbs, as_off[0] - pfix);
      if (wave < BP_I) lds_dma4(&sm.bs[st][64 * wave], w_scales + kbs, bs_off - pfix);
    } else {
#pragma unroll
      for (int i = 0; i < BS_I; ++i)
        lds_dma2(&sm.bs[st][64 * (wave + 4 * i)], w_scales + kbs + min(64 * (wave + 4 * i) / BN, nbk - 1), bs_off);
    }
  };

  v16i cinit;
#pragma unroll
  for (int i = 0; i < 16; ++i) cinit[i] = (i & 1) ? 0x43380000 : (int)0x80000000;

  double acc[RG][CG][8];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int cg = 0; cg < CG; ++cg)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[rg][cg][j] = 0.0;

  const bool a_lane = (lane & 1) == 0;                   // even MFMA rows carry data
  const int a_rrow = wm * 16 * RG + ((lane & 31) >> 1);   // + rg*16
  const int khalf = lane >> 5;                             // 16-byte half of the block
  const int b_rrow = wn * 32 * CG + (lane & 31);          // + cg*32
  // Activation scales of a stage, two per lane: register p holds, in each 16-lane row, the 8 rows
  // this half-wave's MFMA outputs carry (register pair j <-> real row 4(j>>1) + 2(lane>>5) + (j&1))
  // for blocks 2p (lanes 0-7 of the row) and 2p+1 (lanes 8-15); the accumulate FMA broadcasts
  // lane 8(jb&1) + j of the row, so the scale is read from LDS once per stage, not once per use.
  const int da_lrow = wm * 16 * RG + 4 * ((lane & 7) >> 1) + 2 * (lane >> 5) + (lane & 1);  // + rg*16
  const int da_lblk = (lane & 15) >> 3;

  // one stage of G_KS blocks from LDS buffer st
  auto compute = [&](int st, int nbk) {
    asm volatile("" : "+v"(cinit));  // keep the accumulator initial value resident in VGPRs
    double dav[RG][2];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        dav[rg][p] = SP ? (double)f16_bits_to_f32((uint16_t)(sm.as[st][2 * (da_lrow + rg * 16) + p] >> (16 * da_lblk)))
                        : (double)f16_bits_to_f32((uint16_t)sm.as[st][(2 * p + da_lblk) * BM + da_lrow + rg * 16]);
#pragma unroll
    for (int jb = 0; jb < G_KS; ++jb) {
      if (jb >= nbk) break;  // past the end of the slice
      v4i fa[RG], fb[CG];
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        // odd lanes read the zero row, at a chunk that no real row of their 16-lane group uses in
        // the same pass (the rows of one parity take chunks c ^ 0, 2, 4, 6 of a 64-bank row), so
        // the read is a broadcast without a bank conflict; the 4 x 2 tile keeps chunk c, where the
        // extra selects cost more than the conflicts (measured)
        const int r = a_lane ? a_rrow + rg * 16 : BM;
        const int ch = (a_lane || RG == 4) ? swz(r, 2 * jb + khalf) : (((2 * jb + khalf) ^ 1) << 4);
        fa[rg] = *reinterpret_cast<const v4i*>(&sm.a[st][r][ch]);
      }
#pragma unroll
      for (int cg = 0; cg < CG; ++cg)
        fb[cg] = *reinterpret_cast<const v4i*>(&sm.b[st][b_rrow + cg * 32][swz(b_rrow, 2 * jb + khalf)]);
      // 4-row-group tiles produce and consume the MFMA results one row group at a time (all of
      // them at once would not fit in the registers of two waves per SIMD)
      constexpr int RD = RG == 4 ? 1 : RG;
      v16i d[RG][CG];
#pragma unroll
      for (int rg = 0; rg < RD; ++rg)
#pragma unroll
        for (int cg = 0; cg < CG; ++cg) d[rg][cg] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[rg], fb[cg], cinit, 0, 0, 0);
      double dw[CG], cdw[CG];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        dw[cg] = SP ? (double)f16_bits_to_f32((uint16_t)(sm.bs[st][2 * (b_rrow + cg * 32) + (jb >> 1)] >> (16 * (jb & 1))))
                    : (double)f16_bits_to_f32((uint16_t)sm.bs[st][jb * BN + b_rrow + cg * 32]);
        cdw[cg] = -G_MAGIC * dw[cg];
      }
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int cg = 0; cg < CG; ++cg) {
          if constexpr (RD < RG) {
            if (rg > 0) d[rg][cg] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[rg], fb[cg], cinit, 0, 0, 0);
          }
          // the 8 (even, odd) register pairs are the f64 values 1.5*2^52 + 2^31 + I
          v8d xv = __builtin_bit_cast(v8d, d[rg][cg]);
          double x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = fma(xv[j], dw[cg], cdw[cg]);   // exactly I*dw
          if (jb & 1) fmac8_bcast<1>(acc[rg][cg], x, dav[rg][jb >> 1]);
          else fmac8_bcast<0>(acc[rg][cg], x, dav[rg][jb >> 1]);
        }
    }
  };

  // Stages of G_KS blocks through a ring of NS LDS slots: NS - 1 stages are in flight while one
  // computes.  Slot (s + NS - 1) % NS is refilled right after the barrier that ends stage s - 1.
  const int ns = (kb1 - kb0 + G_KS - 1) / G_KS;
#pragma unroll
  for (int u = 0; u < NS - 1; ++u)
    if (u < ns) issue(kb0 + u * G_KS, u);
  if (ns >= NS - 1) wait_vmcnt<(NS - 2) * L_OPS>();
  else wait_vmcnt<0>();
  __syncthreads();
  if constexpr (QPRE > 0) {  // the positions are in; their (cos, sin) rows arrive during the K loop
    const int half = qe.head_dim / 2;
#pragma unroll
    for (int k = 0; k < QPRE; ++k) {
      const int e = tid + k * G_THREADS;
      const int i = (e % (BN / 2)) % half;
      qcs[k] = reinterpret_cast<const double2*>(qe.rope)[qpos[k] * half + i];
    }
  }
  // (with two K groups the second may have one stage less: it skips its last iteration's work but
  // keeps the barriers)
  for (int s = 0; s < ns_it; ++s) {
    const bool more = s + NS - 1 < ns;
    if (more) issue(kb0 + (s + NS - 1) * G_KS, (s + NS - 1) % NS);
    if (KW == 1 || s < ns) compute(s % NS, min(G_KS, kb1 - kb0 - s * G_KS));
    // stage s + 1 has landed once at most the later stages' transfers are outstanding
    if (more) wait_vmcnt<(NS - 2) * L_OPS>();
    else wait_vmcnt<0>();
    __syncthreads();
  }
  if constexpr (KW == 2) {
    // the second group's sums go through its (now idle) LDS ring to the first group, which adds
    // them to its own in a fixed order and runs the epilogue alone
    constexpr int NACC = RG * CG * 8;
    static_assert(sizeof(T) >= sizeof(double) * NACC * 64 * 4, "K-group sums in LDS");
    double* red = reinterpret_cast<double*>(&sm_all[1]);
    if (kgrp == 1) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int cg = 0; cg < CG; ++cg)
#pragma unroll
          for (int j = 0; j < 8; ++j) red[(wave * NACC + (rg * CG + cg) * 8 + j) * 64 + lane] = acc[rg][cg][j];
    }
    __syncthreads();
    if (kgrp == 1) return;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int cg = 0; cg < CG; ++cg)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[rg][cg][j] += red[(wave * NACC + (rg * CG + cg) * 8 + j) * 64 + lane];
  }

  // ---- epilogue.  Lane holds, for each (rg, cg, j): real row, column.
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) asm volatile("" : "+v"(bias_b[cg]));  // the bias is used from here on
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = m0 + wm * 16 * RG + rg * 16 + 4 * (j >> 1) + 2 * (lane >> 5) + (j & 1);
      if (SPLIT) {
        if (row < M) {
#pragma unroll
          for (int cg = 0; cg < CG; ++cg) {
            const int col = n0 + wn * 32 * CG + cg * 32 + (lane & 31);
            if (col < N) partial[((int64_t)kz * M + row) * N + col] = acc[rg][cg][j];
          }
        }
      } else if (EPI == EPI_F32 || EPI == EPI_QKV) {
        if (EPI == EPI_F32 && row < M) {
#pragma unroll
          for (int cg = 0; cg < CG; ++cg) {
            const int col = n0 + wn * 32 * CG + cg * 32 + (lane & 31);
            if (col < N) {
              double v = acc[rg][cg][j];
              if (bias) v += (double)__uint_as_float(bias_b[cg]);
              float y = (float)v;
              const int64_t o = (int64_t)row * ld_out + col;
              if (residual) y = residual[o] + y;
              out[o] = y;
            }
          }
        }
      }
    }

  if constexpr (EPI == EPI_QKV && !SPLIT) {
    // Stage the tile's outputs (bias added in f64, one rounding to f32) in LDS -- the staging
    // buffers are free after the K loop's last barrier -- so that each RoPE pair (i, i + hd/2) and
    // each head's QK-norm sum meet in one thread.  Tiles hold whole heads (BN % head_dim == 0).
    float* tb = reinterpret_cast<float*>(&sm);
    static_assert(sizeof(T) >= sizeof(float) * BM * BN + sizeof(double) * BM * 4, "QKV staging");
    double* inv_rms = reinterpret_cast<double*>(tb + BM * BN);   // [BM][BN / head_dim]
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row_l = wm * 16 * RG + rg * 16 + 4 * (j >> 1) + 2 * (lane >> 5) + (j & 1);
#pragma unroll
        for (int cg = 0; cg < CG; ++cg) {
          const int col_l = wn * 32 * CG + cg * 32 + (lane & 31);
          double v = acc[rg][cg][j];
          if (bias) v += (double)__uint_as_float(bias_b[cg]);
          tb[row_l * BN + col_l] = (float)v;
        }
      }
    __syncthreads();
    const int hd = qe.head_dim, half = hd / 2, heads = BN / hd;
    if (qe.q_norm) {
      // f64 sum of squares per (row, head) of the Q and K heads: one thread per pair
      for (int gidx = tid; gidx < BM * heads; gidx += G_THREADS) {
        const int row_l = gidx / heads, hh = gidx - row_l * heads;
        const float* xr = tb + row_l * BN + hh * hd;
        double ss = 0.0;
        for (int i = 0; i < hd; ++i) ss += (double)xr[i] * (double)xr[i];
        inv_rms[gidx] = recip_f64(sqrt(ss / (double)hd + (double)qe.eps));
      }
      __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < BM * BN / 2 / G_THREADS; ++k) {
      const int e = tid + k * G_THREADS;
      const int row_l = e / (BN / 2), r2 = e - row_l * (BN / 2);
      const int hh = r2 / half, i = r2 - hh * half;
      const int col0 = hh * hd + i;
      const int row = m0 + row_l, gcol = n0 + col0;
      if (row >= M || gcol >= N) continue;
      float a = tb[row_l * BN + col0], b = tb[row_l * BN + col0 + half];
      int64_t p;
      double2 cs;
      if constexpr (QPRE > 0) {
        p = qpos[k];
        cs = qcs[k];
      } else {
        p = qe.pos[row];
        cs = reinterpret_cast<const double2*>(qe.rope)[p * half + i];
      }
      if (gcol < qe.n_q + qe.n_kv) {
        const bool isq = gcol < qe.n_q;
        if (qe.q_norm) {
          const float* gam = isq ? qe.q_norm : qe.k_norm;
          const double ir = inv_rms[row_l * heads + hh];
          a = (float)((double)a * ir * (double)gam[i]);
          b = (float)((double)b * ir * (double)gam[i + half]);
        }
        const float r0 = (float)((double)a * cs.x - (double)b * cs.y);
        const float r1 = (float)((double)a * cs.y + (double)b * cs.x);
        if (isq) {
          out[(int64_t)row * ld_out + gcol] = r0;
          out[(int64_t)row * ld_out + gcol + half] = r1;
        } else {
          float* kr = (qe.slot_of_row ? qe.k_slots[qe.slot_of_row[row]] : qe.k_region) + p * qe.n_kv + (gcol - qe.n_q);
          kr[0] = r0;
          kr[half] = r1;
        }
      } else {
        float* vr = (qe.slot_of_row ? qe.v_slots[qe.slot_of_row[row]] : qe.v_region) + p * qe.n_kv +
                    (gcol - qe.n_q - qe.n_kv);
        vr[0] = a;
        vr[half] = b;
      }
    }
  }

  if constexpr (EPI == EPI_SWIGLU_Q8 && !SPLIT) {
    // Column group pairs (2p, 2p+1) = 32 gate rows, 32 up rows of the interleaved weight; lane
    // l%32 holds column l%32 of both, so the SwiGLU runs per element in registers.  The results
    // then pass through a wave-private LDS tile (16 rows x 32 columns) so that 8 lanes x 4 values
    // cover one Q8_0 block: the block maximum, scale and reciprocal are computed once per 4
    // values instead of once per value.  The staging buffers are free after the K loop's last
    // barrier, and a wave's own LDS accesses complete in order.
    const int ncols = N / 2;
    constexpr int TS = 36;  // floats per tile row: 144-byte stride spreads the float4 reads
    float* ts = reinterpret_cast<float*>(&sm) + wave * 16 * TS;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int cp = 0; cp < CG / 2; ++cp) {
        const int gcol = n0 + wn * 32 * CG + cp * 64;
        const int scol0 = gcol / 2;  // first SwiGLU column of this 32-wide block
#pragma unroll
        for (int j = 0; j < 8; ++j)
          ts[(4 * (j >> 1) + 2 * (lane >> 5) + (j & 1)) * TS + (lane & 31)] =
              swiglu_f32((float)acc[rg][2 * cp][j], (float)acc[rg][2 * cp + 1][j], exp_tab);
#pragma unroll
        for (int hr = 0; hr < 2; ++hr) {
          const int r = hr * 8 + (lane >> 3), c4 = lane & 7;
          const float4 v = *reinterpret_cast<const float4*>(ts + r * TS + c4 * 4);
          float d;
          const uint32_t q = q8_block_quant4(v, d);
          const int row = m0 + wm * 16 * RG + rg * 16 + r;
          if (row < M && gcol < N) {  // offsets below 2^31: M * N / 2 codes
            *reinterpret_cast<uint32_t*>(q_codes + (uint32_t)(row * ncols + scol0 + c4 * 4)) = q;
            if (c4 == 0) q_scales[(uint32_t)(row * (ncols / QK) + scol0 / QK)] = f32_to_f16_bits(d);
          }
        }
      }
  }
}

// ---- split-K reductions (fixed order over the splits)
__global__ void __launch_bounds__(256) k_splitk_f32(const double* __restrict__ partial, int S, int M, int N,
                                                    const float* __restrict__ bias, const float* residual,
                                                    float* out, int64_t ld_out) {
  const int64_t total = (int64_t)M * N;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / N;
    const int col = (int)(i - row * N);
    double v = 0.0;
    for (int z = 0; z < S; ++z) v += partial[(int64_t)z * total + i];
    if (bias) v += (double)bias[col];
    float y = (float)v;
    const int64_t o = row * ld_out + col;
    if (residual) y = residual[o] + y;
    out[o] = y;
  }
}

__global__ void __launch_bounds__(256) k_splitk_swiglu(const double* __restrict__ partial, int S, int M, int N,
                                                       int8_t* __restrict__ q_codes, uint16_t* __restrict__ q_scales) {
  __shared__ double exp_tab[64];
  exp2_table_fill(exp_tab, threadIdx.x);
  __syncthreads();
  const int ncols = N / 2;
  const int64_t nvec_row = ncols / 4;
  const int64_t total = (int64_t)M * nvec_row;
  const int64_t plane = (int64_t)M * N;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / nvec_row;
    const int c4 = (int)(i - row * nvec_row);
    float s[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int sc = c4 * 4 + e;
      const int gcol = (sc / 32) * 64 + (sc % 32);
      double g = 0.0, u = 0.0;
      for (int z = 0; z < S; ++z) {
        g += partial[z * plane + row * N + gcol];
        u += partial[z * plane + row * N + gcol + 32];
      }
      s[e] = swiglu_f32((float)g, (float)u, exp_tab);
    }
    float d;
    const uint32_t q = q8_block_quant4(make_float4(s[0], s[1], s[2], s[3]), d);
    reinterpret_cast<uint32_t*>(q_codes + row * ncols)[c4] = q;
    if ((c4 & 7) == 0) q_scales[row * (ncols / QK) + c4 / 8] = f32_to_f16_bits(d);
  }
}

// Tile and split choice: aim for at least ~4 waves per CU of independent work; split K only when
// the output tiles alone cannot fill the chip, keeping >= 2 stages (8 blocks) per split.
// Tile shapes: 0 = 1x1 MFMA wave tile (workgroup 32 x 64), 1 = 2x2 (64 x 128), 2 = 1x2 (32 x 128),
// 3 = 4x2 (128 x 128).
struct GemmPlan { int shape; int split; };
constexpr double G_TILE42_REL = 0.89;  // time of a 4x2-tile workgroup / two 2x2-tile workgroups (measured)

// defer: the caller reduces f32-epilogue partials itself (no reduction kernel), which makes a
// split worth it for short reductions too.
static GemmPlan plan_gemm(int m, int n, int k, bool swiglu, bool defer = false) {
  const int KB = k / QK;
  GemmPlan p{1, 1};
  const int tiles_big = ((m + 63) / 64) * ((n + 127) / 128);
  if (swiglu) {
    // gate/up pairs live in column-group pairs: 2x2 or 1x2 (waves 4 x 1); prefer enough workgroups for 2 per CU
    p.shape = tiles_big >= 1024 ? 1 : 2;
  } else if (tiles_big < 512) {
    p.shape = 0;
  }
  // (the SwiGLU's 1 x 2 tiles are 64 x 64 workgroups, the others 32 x 128; see launch_gemm_q8)
  const int tiles = p.shape == 1   ? tiles_big
                    : p.shape == 2 ? (swiglu ? ((m + 63) / 64) * ((n + 63) / 64) : ((m + 31) / 32) * ((n + 127) / 128))
                                   : ((m + 31) / 32) * ((n + 63) / 64);
  // Split K only for long reductions whose output tiles cannot fill the chip, keeping the f64
  // partials (written once, read once) at most 8 MB.
  const int target = 512;
  const size_t max_partial = KB >= 256 ? ((size_t)64 << 20) : ((size_t)8 << 20);
  if (KB >= 256 && tiles_big >= 128 && !swiglu) p.shape = 1;  // long reductions: big tiles, split K
  // blocks per split at least 2 stages (1.5 for deferred partials)
  const int min_kb = defer ? 3 * G_KS / 2 : 2 * G_KS;
  auto split_for = [&](int t) {
    int sp = 1;
    if (KB > (defer ? 16 : 64))
      while (sp < 16 && t * sp < target && KB / (sp * 2) >= min_kb &&
             (size_t)(sp * 2) * m * n * sizeof(double) <= max_partial)
        sp *= 2;
    return sp;
  };
  // 128 x 128 workgroups (4x2 wave tiles) do the same work in fewer transfers and fragment reads
  // per output (measured: 0.89x the time of two 64 x 128 workgroups), but half as many
  // workgroups fill the chip's 512 slots (two per CU) in coarser rounds.  Cost of a plan: rounds
  // of workgroups x area of a workgroup / split.
  const int tiles_huge = ((m + 127) / 128) * ((n + 127) / 128);
  if (p.shape == 1 && m >= 256) {
    const int s22 = split_for(tiles_big), s42 = split_for(tiles_huge);
    const double c22 = (double)((tiles_big * s22 + 511) / 512) / s22;
    const double c42 = (double)((tiles_huge * s42 + 511) / 512) * (2.0 * G_TILE42_REL) / s42;
    if (c42 < c22) p.shape = 3;
  }
  p.split = split_for(p.shape == 1 ? tiles_big : p.shape == 3 ? tiles_huge : tiles);
  return p;
}

size_t gemm_workspace_bytes(int m, int n, int k) {
  const GemmPlan p = plan_gemm(m, n, k, false);
  const GemmPlan q = plan_gemm(m, n, k, true);
  const GemmPlan d = plan_gemm(m, n, k, false, true);
  int s = std::max(std::max(p.split, q.split), d.split);
  return s > 1 ? (size_t)s * m * n * sizeof(double) : 0;
}

template <int RG, int CG, int NS, bool SP, int WM = 2, int KW = 1>
static void launch_tiles(const GemmArgs& g, int split, int kb_per, hipStream_t s) {
  using T = GemmTile<RG, CG, NS, SP, WM>;
  dim3 grid((g.n + T::BN - 1) / T::BN, (g.m + T::BM - 1) / T::BM, split);
  // XCD-aware order once the weights outgrow one XCD's 4 MB L2 several times over
  const int xcd = (int64_t)g.n * g.k > ((int64_t)16 << 20) ? 1 : 0;
  double* partial = reinterpret_cast<double*>(g.workspace);
  if constexpr (KW == 2) {
    if (split > 1)
      hipLaunchKernelGGL((k_gemm_q8<RG, CG, EPI_F32, true, NS, SP, WM, 2>), grid, dim3(2 * G_THREADS), 0, s, g.a_codes,
                         g.a_scales, g.m, g.w_codes, g.w_scales, g.n, g.k, g.bias, g.residual, g.out, g.ld_out,
                         g.q_codes, g.q_scales, partial, kb_per, xcd, g.qkv);
    else
      hipLaunchKernelGGL((k_gemm_q8<RG, CG, EPI_F32, false, NS, SP, WM, 2>), grid, dim3(2 * G_THREADS), 0, s, g.a_codes,
                         g.a_scales, g.m, g.w_codes, g.w_scales, g.n, g.k, g.bias, g.residual, g.out, g.ld_out,
                         g.q_codes, g.q_scales, nullptr, kb_per, xcd, g.qkv);
    return;
  }
  if (split > 1)
    hipLaunchKernelGGL((k_gemm_q8<RG, CG, EPI_F32, true, NS, SP, WM>), grid, dim3(G_THREADS), 0, s, g.a_codes, g.a_scales, g.m,
                       g.w_codes, g.w_scales, g.n, g.k, g.bias, g.residual, g.out, g.ld_out, g.q_codes, g.q_scales,
                       partial, kb_per, xcd, g.qkv);
  else if (g.qkv.pos)
    hipLaunchKernelGGL((k_gemm_q8<RG, CG, EPI_QKV, false, NS, SP, WM>), grid, dim3(G_THREADS), 0, s, g.a_codes, g.a_scales, g.m,
                       g.w_codes, g.w_scales, g.n, g.k, g.bias, g.residual, g.out, g.ld_out, g.q_codes, g.q_scales,
                       nullptr, kb_per, xcd, g.qkv);
  else if (g.q_codes) {
    if constexpr (CG >= 2)
      hipLaunchKernelGGL((k_gemm_q8<RG, CG, EPI_SWIGLU_Q8, false, NS, SP, WM>), grid, dim3(G_THREADS), 0, s, g.a_codes,
                         g.a_scales, g.m, g.w_codes, g.w_scales, g.n, g.k, g.bias, g.residual, g.out, g.ld_out,
                         g.q_codes, g.q_scales, nullptr, kb_per, xcd, g.qkv);
  } else
    hipLaunchKernelGGL((k_gemm_q8<RG, CG, EPI_F32, false, NS, SP, WM>), grid, dim3(G_THREADS), 0, s, g.a_codes, g.a_scales, g.m,
                       g.w_codes, g.w_scales, g.n, g.k, g.bias, g.residual, g.out, g.ld_out, g.q_codes, g.q_scales,
                       nullptr, kb_per, xcd, g.qkv);
}

int launch_gemm_q8(const GemmArgs& g, hipStream_t s) {
  if (g.m == 0) return MI_OK;
  const int KB = g.k / QK;
  GemmPlan p = plan_gemm(g.m, g.n, g.k, g.q_codes != nullptr,
                         g.split_out && !g.q_codes && !g.bias && !g.qkv.pos);
  if (g.split_k > 0) p.split = g.split_k;
  if (g.qkv.pos) {  // whole heads per tile, no split
    p.split = 1;
    if (g.qkv.head_dim > 64 && p.shape == 0) p.shape = 2;
    const int bn = p.shape == 0 ? 64 : 128;
    if (g.qkv.head_dim <= 0 || bn % g.qkv.head_dim || (g.qkv.head_dim & 1))
      return set_error(MI_ERR_UNSUPPORTED, "gemm: QKV epilogue needs head_dim dividing %d (got %d)", bn,
                       g.qkv.head_dim);
  }
  int split = std::min(p.split, KB);
  const size_t need = split > 1 ? (size_t)split * g.m * g.n * sizeof(double) : 0;
  if (need > g.workspace_bytes || (need && !g.workspace)) split = 1;
  // splits cover whole stages where possible
  int kb_per = (KB + split - 1) / split;
  kb_per = ((kb_per + G_KS - 1) / G_KS) * G_KS;
  split = (KB + kb_per - 1) / kb_per;
  // scale pairs: rows of an even number of blocks, scale planes 4-byte aligned
  const bool sp = KB % 2 == 0 && ((uintptr_t)g.a_scales & 3) == 0 && ((uintptr_t)g.w_scales & 3) == 0;
  // The fused SwiGLU on 1 x 2 wave tiles stacks its waves 4 x 1 (64 x 64 workgroups: 35 KB of LDS and
  // 126 registers, four workgroups per CU instead of three; measured 30.2 -> 28.8 us at 512 x 9728 x
  // 896); the Q|K|V matmul keeps 32 x 128 (whole heads of 128 per tile).
  const bool tall = p.shape == 2 && g.q_codes;
  // Plain f32 (or partial) outputs on 1 x 1 tiles too few to give every CU two workgroups, with at
  // least 8 stages per slice: two K groups of 4 waves per workgroup, which double the waves working
  // on the chip's few tiles (measured: 512 x 896 x 4864 22.2 -> 21.0 us, 0.5B forward -0.7%; with 4
  // to 7 stages per slice no gain or slower).
  const int wgs = ((g.m + 31) / 32) * ((g.n + 63) / 64) * split;
  const bool kgroups = p.shape == 0 && !g.qkv.pos && !g.q_codes && wgs <= 512 && kb_per >= 8 * G_KS;
  if (sp && p.shape != 3) {  // (the 4x2 tile: more spills with pairs, measured no faster)
    if (p.shape == 1) launch_tiles<2, 2, G_NS_22, true>(g, split, kb_per, s);
    else if (tall) launch_tiles<1, 2, G_NS_12, true, 4>(g, split, kb_per, s);
    else if (p.shape == 2) launch_tiles<1, 2, G_NS_12, true>(g, split, kb_per, s);
    else if (kgroups) launch_tiles<1, 1, G_NS_11, true, 2, 2>(g, split, kb_per, s);
    else launch_tiles<1, 1, G_NS_11, true>(g, split, kb_per, s);
  } else {
    if (p.shape == 3) launch_tiles<4, 2, G_NS_22, false>(g, split, kb_per, s);
    else if (p.shape == 1) launch_tiles<2, 2, G_NS_22, false>(g, split, kb_per, s);
    else if (tall) launch_tiles<1, 2, G_NS_12, false, 4>(g, split, kb_per, s);
    else if (p.shape == 2) launch_tiles<1, 2, G_NS_12, false>(g, split, kb_per, s);
    else if (kgroups) launch_tiles<1, 1, G_NS_11, false, 2, 2>(g, split, kb_per, s);
    else launch_tiles<1, 1, G_NS_11, false>(g, split, kb_per, s);
  }
  MI_LAUNCH_CHECK("k_gemm_q8");
  const bool defer = g.split_out && !g.q_codes && !g.bias && split > 1;  // the consumer reduces the partials
  if (g.split_out) *g.split_out = defer ? split : 1;
  if (split == 1 || defer) return MI_OK;
  double* partial = reinterpret_cast<double*>(g.workspace);
  if (g.q_codes) {
    const int64_t total = (int64_t)g.m * (g.n / 2 / 4);
    const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
    hipLaunchKernelGGL(k_splitk_swiglu, dim3((unsigned)blocks), dim3(256), 0, s, partial, split, g.m, g.n,
                       g.q_codes, g.q_scales);
  } else {
    const int64_t total = (int64_t)g.m * g.n;
    const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
    hipLaunchKernelGGL(k_splitk_f32, dim3((unsigned)blocks), dim3(256), 0, s, partial, split, g.m, g.n, g.bias,
                       g.residual, g.out, g.ld_out);
  }
  MI_LAUNCH_CHECK("k_splitk_reduce");
  return MI_OK;
}

// ---------------------------------------------------------------- static scratch
// Split-K partials of the matmul variant that allocates nothing (mi_gemm_q8_0_static): one array per
// GPU for the life of the process.  Host code never passes `scratch` itself to a kernel (on the host
// that name is only a stand-in); it looks up the device address once per device and uses that.
__device__ __align__(256) char scratch[MI_STATIC_SCRATCH_BYTES];

int static_scratch(void** ptr) {
  constexpr int MAX_DEV = 64;
  static std::mutex mu;
  static void* addr[MAX_DEV] = {};
  int dev = 0;
  MI_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEV) return set_error(MI_ERR_UNSUPPORTED, "static scratch: device %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    MI_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return set_error(MI_ERR_HIP, "static scratch: no device address");
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return MI_OK;
}

// ---------------------------------------------------------------- last-row lm_head
// logits[v] = f32( sum_kb dx[kb] * dw[v][kb] * sum_32 qx * qw ), one row of activations.
// HBM-bound: every weight byte is read once.  One wave per two weight rows at a time; a lane
// takes 16-byte chunks (half a block), sdot4 gives the integer half-block sums, lane pairs
// combine to the block sum, and the exact f64 epilogue accumulates per lane.
constexpr int LM_MAXC = 4;  // 16-byte activation chunks held per lane (K <= 4096)

__global__ void __launch_bounds__(256) k_lm_head(const int8_t* __restrict__ xq, const uint16_t* __restrict__ xs,
                                                 int K, const int8_t* __restrict__ w_codes,
                                                 const uint16_t* __restrict__ w_scales, int rows,
                                                 float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const int nchunk = K / 16;
  const int KB = K / QK;
  v4i xc[LM_MAXC];
  double xd[LM_MAXC];
#pragma unroll
  for (int c = 0; c < LM_MAXC; ++c) {
    const int ch = lane + 64 * c;
    xc[c] = ch < nchunk ? *reinterpret_cast<const v4i*>(xq + ch * 16) : v4i{0, 0, 0, 0};
    xd[c] = ch < nchunk ? (double)f16_bits_to_f32(xs[ch / 2]) : 0.0;
  }
  // two rows per wave and iteration (r and r + nwaves), both rows' loads issued before either's
  // arithmetic: twice the bytes in flight per wave
  for (int64_t r = wave; r < rows; r += 2 * nwaves) {
    const int64_t r2 = r + nwaves;
    const bool two = r2 < rows;  // uniform in the wave
    const int8_t* wr = w_codes + r * K;
    const uint16_t* wsr = w_scales + r * KB;
    const int8_t* wr2 = w_codes + (two ? r2 : r) * K;
    const uint16_t* wsr2 = w_scales + (two ? r2 : r) * KB;
    v4i wv[LM_MAXC], wv2[LM_MAXC];
    uint16_t sb[LM_MAXC], sb2[LM_MAXC];
#pragma unroll
    for (int c = 0; c < LM_MAXC; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nchunk) {
        wv[c] = *reinterpret_cast<const v4i*>(wr + ch * 16);
        wv2[c] = *reinterpret_cast<const v4i*>(wr2 + ch * 16);
        sb[c] = wsr[ch / 2];
        sb2[c] = wsr2[ch / 2];
      }
    }
    double acc = 0.0, acc2 = 0.0;
#pragma unroll
    for (int c = 0; c < LM_MAXC; ++c) {
      const int ch = lane + 64 * c;
      int isum = 0, isum2 = 0;
      double dw = 0.0, dw2 = 0.0;
      if (ch < nchunk) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          isum = __builtin_amdgcn_sdot4(xc[c][e], wv[c][e], isum, false);
          isum2 = __builtin_amdgcn_sdot4(xc[c][e], wv2[c][e], isum2, false);
        }
        dw = (double)f16_bits_to_f32(sb[c]);
        dw2 = (double)f16_bits_to_f32(sb2[c]);
      }
      isum += __shfl_xor(isum, 1);  // both lanes of the pair now hold the block sum
      isum2 += __shfl_xor(isum2, 1);
      if ((lane & 1) == 0 && ch < nchunk) {
        acc = fma((double)isum * dw, xd[c], acc);
        acc2 = fma((double)isum2 * dw2, xd[c], acc2);
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      acc += __shfl_xor(acc, o);
      acc2 += __shfl_xor(acc2, o);
    }
    if (lane == 0) {
      logits[r] = (float)acc;
      if (two) logits[r2] = (float)acc2;
    }
  }
}

int launch_lm_head(const int8_t* xq, const uint16_t* xs, int cols, const int8_t* w_codes,
                   const uint16_t* w_scales, int rows, float* logits, hipStream_t s) {
  if (cols > 64 * 16 * LM_MAXC) return set_error(MI_ERR_UNSUPPORTED, "lm_head: cols %d > %d", cols, 64 * 16 * LM_MAXC);
  const int blocks = 256 * 8;
  hipLaunchKernelGGL(k_lm_head, dim3(blocks), dim3(256), 0, s, xq, xs, cols, w_codes, w_scales, rows, logits);
  MI_LAUNCH_CHECK("k_lm_head");
  return MI_OK;
}

}  // namespace mi
