/*
 * cem_probe.h - measurement probe of the MI355X (gfx950) CEM library, built as
 * its own shared library (libcem_probe.so) so that the plan library carries
 * none of it.  The benchmark reads the matrix cores' sustained ceiling next to
 * the dense projections' throughput.  Status codes are those of cem_jepa.h.
 */
#ifndef CEM_PROBE_H
#define CEM_PROBE_H

#include "cem_jepa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Measurement of the matrix cores' sustained ceiling on the current device:
 * `launches` back-to-back launches (the first half untimed) of a kernel in
 * which every wave issues only v_mfma_f32_32x32x16_bf16 on register-resident
 * operands (one 4-wave workgroup per CU, no memory traffic).  With
 * random_operands = 1 the operand bits are pseudo-random, as real activations
 * and weights are; with 0 they are constant.  Returns the sustained dense bf16
 * TFLOP/s and the shader clock (MHz) the timed launches ran at.  Synchronous;
 * allocates and frees a small device buffer; about 6 ms per launch on MI355X.
 * The dense projections' throughput is reported against the published peak
 * and read next to this figure: under full MFMA load with changing operand
 * bits the part lowers its clock to stay within its power limit.
 * Errors: CEM_E_ARG for a null pointer, random_operands outside {0, 1} or
 * launches outside [2, 10000] (nothing is launched); CEM_E_HIP if a HIP call
 * fails (the small device buffer is freed). */
cem_status cem_mfma_ceiling(int32_t random_operands, int32_t launches, double* tflops,
                            double* mhz);

#ifdef __cplusplus
}
#endif
#endif /* CEM_PROBE_H */
