/*
 * mi_probes.h - rate probes of the gfx950 Q8_0 prefill library (libmi_probes.so): measurement only,
 * not part of the prefill path.
 *
 * Each probe is one kernel of n_workgroups x 256 threads that loops `iters` times (the matmul-loop
 * probes: `iters` stages of 4 Q8_0 blocks) over an
 * instruction mix with its operands in registers (no memory traffic) and writes one f64 per thread
 * to `out` so that the work is kept.  The probes bound the Q8_0 x Q8_0 matmul of mi_prefill.h, whose
 * scale epilogue (the walkthrough index, stage 10: quantized weights times activations quantized on
 * the fly) runs in exact f64 arithmetic: the caller times the launch and divides `*work` by the time.
 *   MI_PROBE_F64_FMA         f64 FMAs of the vector ALU (8 independent chains per lane); work = FMAs
 *   MI_PROBE_MFMA_I8         v_mfma_i32_32x32x32_i8 back to back (4 chains per wave); work = int8 ops
 *   MI_PROBE_LOOP_EXACT_1X2  the matmul's block loop with the exact f64 epilogue, 1 x 2 MFMA wave tile;
 *                            work = algorithmic int8 ops (16 real rows per MFMA)
 *   MI_PROBE_LOOP_EXACT_4X2  the same for the 4 x 2 wave tile of large matmuls
 *   MI_PROBE_LOOP_F32_2X2    the block loop with an f32 epilogue (all 32 rows real), 2 x 2 wave tile
 * out: device, n_workgroups * 256 doubles.  Enqueued on `stream`.  MI_ERR_INVALID_ARG on bad
 * arguments.  Status codes are those of mi_prefill.h.
 */
#ifndef MI_PROBES_H
#define MI_PROBES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MI_PROBE_F64_FMA = 0,
  MI_PROBE_MFMA_I8 = 1,
  MI_PROBE_LOOP_EXACT_1X2 = 2,
  MI_PROBE_LOOP_EXACT_4X2 = 3,
  MI_PROBE_LOOP_F32_2X2 = 4
};

int mi_probe_run(int32_t probe, int32_t n_workgroups, int32_t iters, double* out, double* work, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MI_PROBES_H */
