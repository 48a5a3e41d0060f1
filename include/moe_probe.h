/* Measurement probe, exported by libmoe_probe.so (a library of its own, not
 * part of the MoE forward path).
 *
 * The expert GEMM's roofline is quoted against the datasheet's dense bf16
 * matrix peak (2.5 PFLOP/s).  This probe measures what the matrix cores
 * sustain on this part when nothing but the GEMM's inner-loop mix runs:
 * one wavefront per SIMD, bf16 MFMAs 32x32x16 with fp32 accumulation, A
 * fragments re-read from LDS, no global memory traffic.  bench.py
 * --mfma-probe times it with HIP events; bench.py --hbm-probe times the
 * streaming read, write and copy probes below.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <hip/hip_runtime.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launch the probe once on `stream`: `grid` workgroups of 256 threads (one
 * per CU at most: each takes 160 KB of LDS), `iters` iterations of 64 MFMAs
 * per wavefront.  random_data != 0 fills the operands with random bf16
 * numbers (random sign and mantissa, magnitude in [0.5, 1)), otherwise with
 * small values repeating every 8 words.  `out` is caller-owned device memory
 * of grid * 256 floats (one sum per thread, written so that no work is
 * optimised away).  Returns 0, 1 for invalid arguments (nothing launched),
 * 2 for a launch error.  Asynchronous. */
int moe_probe_mfma(float* out, int grid, int iters, int random_data, hipStream_t stream);

/* Floating-point operations of one moe_probe_mfma launch with these sizes. */
double moe_probe_mfma_flop(int grid, int iters);

/* HBM bandwidth probes (the memory side of the rooflines): one launch on
 * `stream` over `bytes` (a multiple of 16) of device memory, each thread
 * moving 16-byte chunks in a grid-stride loop over `grid` workgroups of 256:
 *   mode 0  read only: every chunk of src is loaded (non-temporally) and
 *           folded into one word per thread, written to out[grid * 256]
 *   mode 1  write only: every chunk of dst is stored (non-temporally)
 *   mode 2  copy: src chunks stored to dst
 * Returns 0, 1 for invalid arguments (nothing launched), 2 for a launch
 * error.  Asynchronous. */
int moe_probe_hbm(int mode, const void* src, void* dst, size_t bytes, unsigned* out, int grid,
                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
