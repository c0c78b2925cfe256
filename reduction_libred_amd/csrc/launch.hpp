// launch.hpp -- internal interface between the C ABI (libred.cpp) and the
// kernel translation units. Every launcher enqueues on `stream` and returns
// the hipError_t of the launch (hipGetLastError right after it).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace libred {

// MI355X: 8 XCDs of 32 CUs, each with its own L2; the workgroups of a launch
// are dealt to them in turn (workgroup b to XCD b mod 8).
constexpr int kXcds = 8;

// Launch shape of the single-value kernels: `block` threads per block, at
// most `blocks_per_cu` blocks per compute unit, `unroll` independent 16-byte
// loads in flight per lane per loop trip, `nontemporal` marks the streaming
// loads non-temporal, `layout` 0 = grid-stride, 1 = wave tiles, `prefetch`
// (wave tiles only) issues the next tile before folding the current one,
// `combine` 0 = last block combines, 1 = a second one-block launch does.
enum { kGridStride = 0, kWaveTiles = 1 };
enum { kCombineTicket = 0, kCombineTwoPass = 1 };

struct FlatPolicy {
    int block;
    int blocks_per_cu;
    int unroll;
    int nontemporal;
    int layout;
    int prefetch;
    int combine;
};

// Launch shape of the row kernels: `block` threads (one row per 64-lane
// wave at a time), `unroll` loads in flight per lane, `max_blocks` caps the
// grid (rows beyond it are taken in a wave-uniform grid-stride loop), `split`
// 0 = split few long rows across blocks automatically, 1 = never, 2 = always.
struct RowsPolicy {
    int block;
    int unroll;
    int nontemporal;
    int max_blocks;
    int split;
    int prefetch;
    int short_rows;
    int cover;
    int defer;
    int lines;
    int xcd;
    int max_fold;
};

// How one row call launches: `grid` blocks of the one-wave-per-row kernel,
// or, when split_gx > 0, rows * split_gx single-wave blocks writing partials
// (acc_t, at most kMaxSplitPartials of them) into `partials`.
struct RowsLaunch {
    int grid;
    unsigned int split_gx;
    void* partials;
    int packed_log2l;   // with packed_v > 0: the packed-row kernel, 2^packed_log2l lanes per row,
    int packed_v;       //   up to packed_v units per lane per row,
    int packed_scalar;  //   units of one element (1) or of one 16-byte vector (0)
    int staged_u;       // > 0: the LDS-staged kernel, tiles of staged_rows rows (at most
    unsigned int staged_rows;  //   256 * staged_u elements), 2^staged_log2s lanes per row
    int staged_log2s;
    int cover;          // one wave per row: read each row through its aligned cover
    int staged_vread;   // the LDS-staged kernel reads 16-byte vectors (rows of whole vectors)
    unsigned int staged_hold;  // > 0: the LDS-staged kernel holds this many results per wave in
                               //   dynamic LDS and stores them after the wave's last tile
    int staged_spread;  // the LDS-staged kernel's element reads start at a different element
                        //   in each row of a pass (rows at a stride of a multiple of 16)
    int narrow;         // the register kernel for narrow rows (rows_narrow.hip), `grid` waves:
                        //   1 = results stored as each tile is folded, 2 = held in LDS and
                        //   stored in bursts
    int xmap;           // grid-stride row kernels: the blocks of each XCD take consecutive
                        //   block indices (used when the grid is a multiple of kXcds)
    int staged_fmax;    // maxima in the LDS-staged kernel fold with a hardware max
};

// Narrow rows: a contiguous, 16-byte aligned matrix of rows of 1 to
// kNarrowMaxCols floats, each lane folding whole rows (op 0 = sum, 1 = max),
// `grid` single-wave blocks, tiles of at least kNarrowTileLoads 16-byte loads
// per lane. rows_narrow_tile_rows(cols) rows make one tile (0 for another
// width).
constexpr int kNarrowTileLoads = 8;
constexpr size_t kNarrowMaxCols = 32;
size_t rows_narrow_tile_rows(size_t cols);
// Static LDS bytes of one narrow block (0 for another width); with hold,
// the block keeps its results in LDS and stores them in bursts.
size_t rows_narrow_lds_bytes(size_t cols, bool hold);
hipError_t launch_rows_narrow(int op, const float* x, size_t rows, size_t cols, float* out, int grid, bool nt,
                              bool hold, hipStream_t stream);
constexpr size_t kMaxSplitPartials = 32768;

// Library-owned scratch of one (device, stream): a completion counter that
// is zero between calls, and room for `max_partials` block partials of up to
// kMaxPartialBytes each.
constexpr size_t kMaxPartialBytes = 32;
struct Workspace {
    unsigned int* ticket;
    void* partials;
    size_t max_partials;
};

// Launch shape of the column kernels: `unroll` rows in flight per lane,
// `nontemporal`, `target_waves` (rows are cut into chunks until about this
// many single-wave blocks run), `vec` 0 = four columns per lane when the
// layout allows it (16-byte aligned, cols and ld multiples of 4), 1 = one,
// 4 = four when allowed.
struct ColsPolicy {
    int unroll;
    int nontemporal;
    int target_waves;
    int vec;
    int width;
    int prefetch;
    int fold;
    int order;
    int xcd;
};

// How one column call launches: ncb column blocks of ngroups*vec*width
// columns times nchunks row phases (phase k takes every nchunks-th group of
// rows, starting at group k; ngroups == 64, or a divisor of 64 for a narrow
// matrix whose wave then covers 64 / ngroups rows per load); with
// nchunks > 1, partials (nchunks * cols acc_t) live in `partials`.
struct ColsLaunch {
    size_t ncb;
    size_t nchunks;
    int vec;
    int width;
    unsigned int ngroups;
    void* partials;
    // fold_m > 1 or rot > 0: the launch runs on a view of a contiguous
    // matrix, fold_m consecutive rows as one view row of fold_m * real_cols
    // columns starting rot (0-31) elements into the matrix, so that view rows
    // start 16-byte aligned. View column c' holds real column
    // (c' + rot) % real_cols. Pass 2 adds, per real column, the partials of
    // its fold_m view columns, then its elements among the tail_elems after
    // the view (from `tail`) and among the rot before it (from `head`).
    int fold_m;
    size_t real_cols;
    size_t tail_elems;
    const void* tail;
    unsigned int rot;
    const void* head;
    // With vec 4: the rows need not start 16-byte aligned (cols, ld and x
    // arbitrary); each lane loads the aligned vector its four columns start
    // in and takes the next one from the next lane. A block then owns cspan
    // columns: 4 * (64 * width - 1) with one column group per lane, or
    // 4 * (ngroups - 1) for packed rows whose last group is a spare that only
    // lends its vector (4 * ngroups when no row's last group reaches past its
    // vector).
    int shift;
    size_t cspan;
    // Rows of a phase: 0 = every nchunks-th group from group k (a launch
    // reads one band of the matrix at a time); 1 = the same rows, block b
    // starting at its (b mod n)-th of n groups and wrapping around to the
    // first; 2 = one run of consecutive rows per phase.
    int order;
    // 1: the blocks on each XCD take all column blocks of consecutive phases
    // (nchunks a multiple of kXcds); 0: column block b mod ncb, phase b / ncb.
    int xmap;
    // 1: maxima fold with the hardware max (see cols_partial_kernel's FMAX),
    // where the launch shape has that variant.
    int col_fmax;
};

bool flat_policy_supported(const FlatPolicy& p);
bool cols_policy_supported(const ColsPolicy& p);
bool rows_policy_supported(const RowsPolicy& p);

// Single-value reductions with `grid` blocks (1 <= grid <= ws.max_partials).
hipError_t launch_sum_f32(const float* x, size_t n, float* out, int grid, const FlatPolicy& p,
                          const Workspace& ws, hipStream_t stream);
hipError_t launch_sum_i32_i64(const int32_t* x, size_t n, int64_t* out, int grid,
                              const FlatPolicy& p, const Workspace& ws, hipStream_t stream);
hipError_t launch_max_f32(const float* x, size_t n, float* out, int grid, const FlatPolicy& p,
                          const Workspace& ws, hipStream_t stream);
hipError_t launch_min_f32(const float* x, size_t n, float* out, int grid, const FlatPolicy& p,
                          const Workspace& ws, hipStream_t stream);
hipError_t launch_argmax_f32(const float* x, size_t n, int64_t* out, int grid, const FlatPolicy& p,
                             const Workspace& ws, hipStream_t stream);
hipError_t launch_argmin_f32(const float* x, size_t n, int64_t* out, int grid, const FlatPolicy& p,
                             const Workspace& ws, hipStream_t stream);
hipError_t launch_sum_bf16(const uint16_t* x, size_t n, float* out, int grid, const FlatPolicy& p,
                           const Workspace& ws, hipStream_t stream);
hipError_t launch_sum_f16(const uint16_t* x, size_t n, float* out, int grid, const FlatPolicy& p,
                          const Workspace& ws, hipStream_t stream);
hipError_t launch_sum_f64(const double* x, size_t n, double* out, int grid, const FlatPolicy& p,
                          const Workspace& ws, hipStream_t stream);
// Fused: out3[0] = sum, out3[1] = max, out3[2] = sum of |x|.
hipError_t launch_sum_max_f32(const float* x, size_t n, float* out3, int grid, const FlatPolicy& p,
                              const Workspace& ws, hipStream_t stream);

// Steps 1-5 of the float32 sum only: one float64 partial per block into
// partials[0..grid), whatever p.combine says.
hipError_t launch_sum_f32_partials(const float* x, size_t n, double* partials, int grid,
                                   const FlatPolicy& p, hipStream_t stream);

// Zero `words` 32-bit words at p (used once, when a workspace is created).
hipError_t launch_zero_words(unsigned int* p, size_t words, hipStream_t stream);
// Set `words` 32-bit words at p to `value` (test probe: poisons scratch).
hipError_t launch_fill_words(unsigned int* p, size_t words, unsigned int value, hipStream_t stream);

// Row reductions (rows >= 1, rows starting ld >= cols elements apart).
hipError_t launch_rows_sum_f32(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                               const RowsLaunch& L, const RowsPolicy& p, hipStream_t stream);
hipError_t launch_rows_max_f32(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                               const RowsLaunch& L, const RowsPolicy& p, hipStream_t stream);

// Column reductions: out[c] over r < rows of x[r * ld + c], c < cols (>= 1).
hipError_t launch_cols_sum_f32(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                               const ColsLaunch& L, const ColsPolicy& p, hipStream_t stream);
hipError_t launch_cols_max_f32(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                               const ColsLaunch& L, const ColsPolicy& p, hipStream_t stream);

// Ablation ladder: rung 1..5 writes one float partial per block of
// kRungBlock threads into `partials`.
constexpr int kRungBlock = 256;
size_t rung_elems_per_block(int rung);
hipError_t launch_rung(int rung, const float* x, size_t n, float* partials, size_t nblocks,
                       hipStream_t stream);

// LDS bank probe: one wave reads LDS word (lane * stride) mod kLdsProbeWords
// (stride -1: lane / 2) `iters` times; *sink = the sum of all values read.
constexpr int kLdsProbeWords = 64 * 65;
hipError_t launch_lds_stride(int stride, int iters, unsigned int* sink, hipStream_t stream);

// Cross-lane primitives alone: op 0 = float64 sum, 1 = int64 sum, 2 = f32
// max over each group of 64 inputs; and one 64-lane shuffle-down.
hipError_t launch_wave_reduce_probe(int op, const void* in, size_t nwaves, void* out, hipStream_t stream);
hipError_t launch_shfl_down_probe(const float* in, int offset, float* out, hipStream_t stream);

// Load-only read probe: `block` threads, `blocks_per_cu` blocks per compute
// unit, `unroll` 16-byte loads in flight per lane, `nontemporal`, `layout`
// 0 = grid-stride, 1 = wave tiles, 2 = wave tiles with the next tile in
// flight. *sink ^= the xor of every 32-bit word of x[0 .. 16 * nvec).
struct ReadShape {
    int block;
    int blocks_per_cu;
    int unroll;
    int nontemporal;
    int layout;
};
bool read_shape_supported(const ReadShape& s);
hipError_t launch_read_probe(const void* x, size_t nvec, unsigned int* sink, int grid, const ReadShape& s,
                             hipStream_t stream);
// Copy ceiling: y[0 .. nvec) = x[0 .. nvec) in 16-byte vectors, wave tiles
// with the next tile in flight (block 64, layout 2, unroll 4 / 8 / 16).
bool copy_shape_supported(const ReadShape& s);
hipError_t launch_copy_probe(const void* x, void* y, size_t nvec, int grid, const ReadShape& s, hipStream_t stream);

// Probes: a plain copy y = x with 16-byte accesses and a scalar tail, and
// the single-value kernel with an xor fold (*out = xor of all words), which
// reads like the reductions but does one ALU op per element.
hipError_t launch_copy_f32(const float* x, float* y, size_t n, int grid, hipStream_t stream);
hipError_t launch_xor_u32(const uint32_t* x, size_t n, uint32_t* out, int grid, const FlatPolicy& p,
                          const Workspace& ws, hipStream_t stream);

}  // namespace libred
