// The exact per-block scale epilogue of the Q8_0 matmul, shared by the matmul kernels and the rate
// probes that bound them.
//
// v_mfma_i32_32x32x32_i8 yields the integer sum I of one Q8_0 block (K = 32) per output.  With the
// odd MFMA rows fed all-zero activations and the accumulator started at 0x80000000 (even rows) and
// 0x43380000 (odd rows), each (even, odd) register pair of the result is the f64 number
// G_MAGIC + I, G_MAGIC = 1.5*2^52 + 2^31.  Then
//   t   = fma(G_MAGIC + I, dw, -G_MAGIC * dw) = I * dw          (exact: 19 + 11 significant bits)
//   acc = fma(t, da, acc)                                        (one f64 rounding)
// adds I * dw * da to the f64 accumulator: two f64 FMAs per output and block, no conversion.
#pragma once

#include "common.h"

namespace mi {

constexpr double G_MAGIC = 0x1.8p+52 + 0x1p+31;  // 1.5*2^52 + 2^31, exact

// acc[j] += bcast(da, lane 8*HALF + j of each 16-lane row) * x[j] for j = 0..7: v_fmac_f64 with a
// DPP row_newbcast source (the one DPP form of the f64 ALU).  da comes from an LDS load; the
// leading s_nop gives the two wait states a DPP source needs after any VALU write of it.
template <int HALF>
__device__ __forceinline__ void fmac8_bcast(double (&acc)[8], const double (&x)[8], double da) {
  if constexpr (HALF == 0)
    asm("s_nop 1\n\t"
        "v_fmac_f64_dpp %0, %8, %9 row_newbcast:0\n\t"
        "v_fmac_f64_dpp %1, %8, %10 row_newbcast:1\n\t"
        "v_fmac_f64_dpp %2, %8, %11 row_newbcast:2\n\t"
        "v_fmac_f64_dpp %3, %8, %12 row_newbcast:3\n\t"
        "v_fmac_f64_dpp %4, %8, %13 row_newbcast:4\n\t"
        "v_fmac_f64_dpp %5, %8, %14 row_newbcast:5\n\t"
        "v_fmac_f64_dpp %6, %8, %15 row_newbcast:6\n\t"
        "v_fmac_f64_dpp %7, %8, %16 row_newbcast:7"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]), "+v"(acc[6]),
          "+v"(acc[7])
        : "v"(da), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]));
  else
    asm("s_nop 1\n\t"
        "v_fmac_f64_dpp %0, %8, %9 row_newbcast:8\n\t"
        "v_fmac_f64_dpp %1, %8, %10 row_newbcast:9\n\t"
        "v_fmac_f64_dpp %2, %8, %11 row_newbcast:10\n\t"
        "v_fmac_f64_dpp %3, %8, %12 row_newbcast:11\n\t"
        "v_fmac_f64_dpp %4, %8, %13 row_newbcast:12\n\t"
        "v_fmac_f64_dpp %5, %8, %14 row_newbcast:13\n\t"
        "v_fmac_f64_dpp %6, %8, %15 row_newbcast:14\n\t"
        "v_fmac_f64_dpp %7, %8, %16 row_newbcast:15"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]), "+v"(acc[6]),
          "+v"(acc[7])
        : "v"(da), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]));
}

}  // namespace mi
