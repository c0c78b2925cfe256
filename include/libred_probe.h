/*
 * libred_probe.h -- measurement probes and device facts.
 *
 * The simulator page ("simt_lab.py -- a numpy-simulated GPU", section 6,
 * estimate_time) bounds a kernel's time below by its memory traffic over the
 * device's bandwidth. These probes measure the two figures that bound needs
 * on real hardware: what a plain copy of known size reads and writes (to
 * scale hardware byte counters), and how fast a read-only stream runs.
 * Conventions are those of libred.h.
 */
#ifndef LIBRED_PROBE_H_
#define LIBRED_PROBE_H_

#include "libred.h"

#ifdef __cplusplus
extern "C" {
#endif

/* y[i] = x[i] for i < n. x and y must be 16-byte aligned and must not
 * overlap. */
red_status red_probe_copy_f32(const float *x, float *y, size_t n, hipStream_t stream);

/* Reads every 32-bit word of x[0..n) once, with the launch shape and kernel
 * structure of red_sum_f32, and stores their xor at *sink: the reduction's
 * load path with one integer op per element instead of the float64 adds.
 * x and sink must be 4-byte aligned and must not overlap. */
red_status red_probe_read_f32(const float *x, size_t n, unsigned int *sink, hipStream_t stream);

/*
 * LDS bank probe, after the reduction lesson's demo 1 (how many rounds one
 * warp's shared-memory read takes for a given stride), for a 64-lane wave:
 * one wave fills LDS word i with i (64 * 65 words), then each lane l reads
 * word (l * stride) mod 4160 -- or word l / 2 when stride == -1 -- `iters`
 * times, and the sum of everything read is added to *sink (which the caller
 * zeroes). Stride 0 is a broadcast. The bank-conflict counters of this
 * kernel, per stride, give the hardware's bank geometry. stride outside
 * [-1, 2^20], iters outside [0, 2^24] or a NULL sink is RED_ERR_INVALID_ARG.
 */
red_status red_probe_lds_stride(int stride, int iters, unsigned int *sink, hipStream_t stream);

/*
 * The wave-level combine of the production kernels, alone: for each w <
 * nwaves, out[w] = the reduction of in[64w .. 64w + 63] by one 64-lane wave
 * with the library's DPP sequence (quad_perm [1,0,3,2] and [2,3,0,1],
 * row_half_mirror, row_mirror, row_bcast:15 into rows 1 and 3, row_bcast:31
 * into rows 2 and 3, then lane 63). op 0: in/out are double, summed; op 1:
 * int64_t, summed; op 2: float, max (strictly-greater rule). The pairing
 * order is fixed, so a float64 result is reproducible bit for bit. op outside
 * 0..2, nwaves outside 1..2^20, NULL or misaligned pointers, or overlap is
 * RED_ERR_INVALID_ARG.
 */
red_status red_probe_wave_reduce(int op, const void *in, size_t nwaves, void *out, hipStream_t stream);

/*
 * The register shuffle of ablation rung 5, alone, with the semantics of the
 * simulator page "simt_lab.py" (section 4, Block.shfl_down): one 64-lane
 * wave; out[l] = in[l + offset] when l + offset < 64, else in[l]. in and out
 * hold 64 floats. offset outside 0..64 or NULL pointers is
 * RED_ERR_INVALID_ARG.
 */
red_status red_probe_shfl_down_f32(const float *in, int offset, float *out, hipStream_t stream);

/* Facts about the current device: compute-unit count and architecture name
 * (e.g. "gfx950:sramecc+:xnack-"), copied into arch[0..arch_len). */
red_status red_device_info(int *cu_count, char *arch, size_t arch_len);

#ifdef __cplusplus
}
#endif

#endif /* LIBRED_PROBE_H_ */
