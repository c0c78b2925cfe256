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

/*
 * Launch shape of the load-only read probe: `block` threads per block (64,
 * 256 or 1024), `blocks_per_cu` blocks per compute unit (1..32), `unroll`
 * 16-byte loads in flight per lane (4, 8, 16 or 32; with 1024-thread blocks
 * at most 16, and at most 8 with layouts 2 and 3), `nontemporal` (0 or 1:
 * the streaming hint on the loads), `layout` (0 grid-stride, 1 wave tiles of
 * 64 * unroll vectors, 2 wave tiles with the next tile's loads in flight
 * while the current one is folded, 3 as 2 with each XCD's blocks (block b
 * runs on XCD b mod 8) reading one contiguous eighth of the tiles).
 */
typedef struct red_read_shape {
    int block;
    int blocks_per_cu;
    int unroll;
    int nontemporal;
    int layout;
} red_read_shape;

/* The read probe's default shape: the fastest found by its launch-shape
 * sweep on a 1 GiB buffer of this device. */
void red_default_read_shape(red_read_shape *shape);

/*
 * Load-only read probe: reads each 16-byte vector of x[0 .. bytes) once with
 * the given launch shape (NULL = the default) and xors every 32-bit word
 * into *sink (which the caller sets first; xor is order-free, so the result
 * is exact whatever the shape). Its time gives how fast this device can
 * stream a buffer, the measured counterpart of the memory bound of the
 * simulator page ("simt_lab.py", section 6, estimate_time). x must be
 * 16-byte aligned and bytes a multiple of 16; an unsupported shape, a NULL
 * or misaligned pointer, or overlap is RED_ERR_INVALID_ARG.
 */
red_status red_probe_read_ceiling(const void *x, size_t bytes, const red_read_shape *shape,
                                  unsigned int *sink, hipStream_t stream);

/* The copy probe's default shape (see red_probe_copy_ceiling). */
void red_default_copy_shape(red_read_shape *shape);

/*
 * Copy ceiling: y = x over `bytes` (a multiple of 16; x and y 16-byte
 * aligned and not overlapping), read and written as 16-byte vectors by
 * single-wave blocks streaming wave tiles with the next tile's loads in
 * flight, the load-only probe's fastest layout. A shape (NULL = the
 * default) must have block 64 and layout 2; it chooses blocks per compute
 * unit (1..32), loads per lane per tile (4, 8 or 16) and whether loads and
 * stores are non-temporal. Its time bounds what a reduction whose output is
 * as large as its input (rows of one float) can reach. Errors as for
 * red_probe_read_ceiling.
 */
red_status red_probe_copy_ceiling(const void *x, void *y, size_t bytes, const red_read_shape *shape,
                                  hipStream_t stream);

/*
 * Test probe for the poison check of the simulator page ("simt.py", section
 * 3, shared memory filled with NaN so that unwritten values show): sets every
 * block-partial slot of the workspace of (current device, stream) -- creating
 * the workspace first if the stream has none -- and every word of the
 * stream's column scratch, if it has any, to the 32-bit `word`, with an
 * ordinary store kernel on `stream`. The completion counter is left alone.
 * A later call on the stream must overwrite every partial it reads, so its
 * result does not change. Returns RED_ERR_CAPTURE, enqueuing nothing, while
 * the stream is being captured.
 */
red_status red_probe_fill_workspace(unsigned int word, hipStream_t stream);

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
