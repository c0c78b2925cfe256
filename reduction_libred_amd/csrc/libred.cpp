// libred.cpp -- the C ABI of libred: argument checks, device facts, the
// per-(device, stream) workspace, launch shapes, and the calls into the
// kernel translation units. Host code, apart from the one device array of
// the allocation-free sum below.
#include <stdint.h>
#include <string.h>

#include <map>
#include <mutex>
#include <numeric>
#include <utility>
#include <vector>

#include "dispatch_table.hpp"
#include "launch.hpp"
#include "libred.h"
#include "libred_ablate.h"
#include "libred_probe.h"

using libred::FlatPolicy;
using libred::RowsPolicy;
using libred::Workspace;

// The block partials of red_sum_f32_noalloc, which allocates nothing: a
// fixed device array instead of a workspace. Every device the library runs
// on holds its own copy until the process ends. In host code `scratch`
// names only a host-side stand-in, never device memory; host code uses the
// device address that hipGetSymbolAddress gives for the current device
// (noalloc_scratch below), and passes that to the kernels.
constexpr size_t kNoAllocMaxPartials = 4096;  // float64 partials: 32 KiB
static __device__ __align__(256) double scratch[kNoAllocMaxPartials];

namespace {

thread_local int g_last_hip = 0;

red_status fail(hipError_t e, red_status code) {
    g_last_hip = (int)e;
    return code;
}

struct DeviceInfo {
    int cu_count;
    size_t lds_per_cu;     // bytes of LDS per compute unit
    size_t lds_per_block;  // bytes of LDS one block may use
    char arch[64];
};

// Workspace layout: the completion counter alone in the first 256 bytes,
// then room for kMaxPartials partials of up to kMaxPartialBytes each. The
// grid never exceeds kMaxPartials blocks.
constexpr size_t kTicketBytes = 256;
constexpr size_t kMaxPartials = 8192;
constexpr size_t kWorkspaceBytes = kTicketBytes + kMaxPartials * libred::kMaxPartialBytes;

std::mutex g_mu;
std::map<int, DeviceInfo> g_devices;
std::map<std::pair<int, hipStream_t>, Workspace> g_workspaces;
std::map<int, double*> g_noalloc_scratch;  // device -> its copy of `scratch`

// Per-(device, stream) scratch for column partials, grown on demand up to
// kColsScratchMax bytes (starting at 1 MiB and at least doubling each time,
// so growth is rare). A buffer that is outgrown is kept, not freed, until the
// process exits: a graph captured earlier may still write to it.
struct Scratch {
    void* ptr;
    size_t bytes;
};
std::map<std::pair<int, hipStream_t>, Scratch> g_scratch;
std::vector<void*> g_retired_scratch;
// Workspaces replaced by red_stream_new_workspace: kept, like outgrown
// scratch, because graphs captured earlier may still use them.
std::vector<Workspace> g_retired_workspaces;
constexpr size_t kColsScratchMax = (size_t)64 << 20;

// Default launch shapes, chosen by measurement on MI355X (256 CUs, 8 TB/s):
// single-wave blocks streaming 8 KiB tiles with the next tile in flight and
// a second one-block launch for the combine. Arrays of 2^20 to 2^24
// elements prefer fewer, larger blocks; tiny arrays fewer blocks.
// Up to kTinyMax elements one 1024-thread block reads everything and stores
// the result itself, with no second launch: in a graph of calls on a
// cache-resident array, 2^12 / 2^14 / 2^15 floats took 2.0 / 2.2 / 2.6 us
// against 3.2 / 3.4 / 3.5 us for the small shape's two launches (2^16: 4.5
// against 3.5 us).
constexpr FlatPolicy kFlatTiny = {1024, 1, 8, 1, libred::kWaveTiles, 1, libred::kCombineTwoPass};
constexpr size_t kTinyMax = (size_t)1 << 15;  // elements: one block of 1024 x 8 loads of 4
constexpr FlatPolicy kFlatSmall = {64, 1, 8, 1, libred::kWaveTiles, 1, libred::kCombineTwoPass};
constexpr FlatPolicy kFlatMid = {256, 1, 8, 1, libred::kWaveTiles, 1, libred::kCombineTwoPass};
constexpr FlatPolicy kFlatCached = {1024, 1, 4, 1, libred::kWaveTiles, 1, libred::kCombineTwoPass};
constexpr FlatPolicy kFlatLarge = {64, 2, 8, 1, libred::kWaveTiles, 1, libred::kCombineTwoPass};
// Up to 2^20 elements the small shape, then 256-thread blocks up to 2^23. In
// graphs of calls on one array / on rotating copies, medians of three rounds,
// int32 sums: 2^20 small 3.7 / 4.6 us against 4.1 / 4.6 for 256 x 8 loads;
// 2^21 4.6 / 5.6 against 4.2 / 5.1; 3 x 2^20 5.9 / 6.5 against 5.2 / 5.9;
// 2^22 7.0 / 7.4 against 5.6 / 6.2; 6 x 2^20 8.9 / 9.3 against 6.4 / 7.6
// (float32 alike); at 2^23 the cached shape ties it (7.1-7.3 / 8.4-8.6).
constexpr size_t kSmallMax = (size_t)1 << 20;   // elements
constexpr size_t kMidMax = (size_t)1 << 23;     // elements
// Up to 2^24 elements the cached shape; above, the large one. In graphs of
// calls (one array, or rotating copies that evict each other), int32 and
// float32 sums: 2^24 cached 11.2-11.5 / 13.6-13.9 us against 11.8-12.7 /
// 13.0-14.0 large; 2^25 22.1-22.7 / 24.1-24.6 against 20.6-21.6 / 22.4-23.0;
// 2^26 41.2-43.1 / 44.8-45.4 against 38.6-39.7 / 41.3-42.2.
constexpr size_t kCachedMax = (size_t)1 << 24;  // elements
constexpr RowsPolicy kDefaultRows = {64, 8, 1, 1024, 0, 0, 0, 0, 0, 0};
using libred::table::kSplitMinCols;
using libred::table::kSplitRowsBelow;
using libred::table::kSplitTargetWaves;

// The fused sum/max/sum-of-magnitudes pass folds three accumulators per
// element (two of them float64) and keeps four waves per CU on large arrays:
// with the common shape's two, its sustained launches slowed from 148 to
// 165 us within a few dozen back-to-back calls, while this shape held
// 146 us.
constexpr FlatPolicy kFusedLarge = {256, 1, 4, 1, libred::kWaveTiles, 1, libred::kCombineTwoPass};

// The allocation-free sum reads only partials its own first launch wrote,
// which holds for the two-launch combine of every default shape (the
// counter of the single-launch combine would have to start at zero).
static_assert(kFlatTiny.combine == libred::kCombineTwoPass && kFlatSmall.combine == libred::kCombineTwoPass &&
                  kFlatMid.combine == libred::kCombineTwoPass && kFlatCached.combine == libred::kCombineTwoPass &&
                  kFlatLarge.combine == libred::kCombineTwoPass,
              "red_sum_f32_noalloc relies on the two-launch combine");

FlatPolicy default_flat(size_t n) {
    if (n <= kTinyMax) return kFlatTiny;
    if (n <= kSmallMax) return kFlatSmall;
    if (n <= kMidMax) return kFlatMid;
    if (n <= kCachedMax) return kFlatCached;
    return kFlatLarge;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t abytes, const void* b, size_t bbytes) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return abytes && bbytes && a0 < b0 + bbytes && b0 < a0 + abytes;
}

red_status current_device(int* dev_out, DeviceInfo* info_out) {
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count <= 0) return fail(e == hipSuccess ? hipErrorNoDevice : e, RED_ERR_NO_DEVICE);
    int dev = -1;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(e, RED_ERR_NO_DEVICE);
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_devices.find(dev);
    if (it == g_devices.end()) {
        DeviceInfo di;
        memset(&di, 0, sizeof(di));
        e = hipDeviceGetAttribute(&di.cu_count, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return fail(e, RED_ERR_HIP);
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return fail(e, RED_ERR_HIP);
        strncpy(di.arch, prop.gcnArchName, sizeof(di.arch) - 1);
        di.lds_per_cu = prop.maxSharedMemoryPerMultiProcessor;
        di.lds_per_block = prop.sharedMemPerBlock;
        if (di.cu_count <= 0) return fail(hipErrorInvalidDevice, RED_ERR_NO_DEVICE);
        it = g_devices.emplace(dev, di).first;
    }
    *dev_out = dev;
    *info_out = it->second;
    return RED_OK;
}

// Allocating while `stream` is being captured into a graph would break the
// capture (or put a fill kernel into the graph), so a call that needs a new
// or larger buffer then fails before touching the stream.
red_status refuse_if_capturing(hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return fail(e, RED_ERR_HIP);
    return cs == hipStreamCaptureStatusNone ? RED_OK : RED_ERR_CAPTURE;
}

// hipMalloc with this thread in relaxed capture mode. Another stream may be
// being captured in global mode (PyTorch's default) while this call runs on a
// stream that is not; an allocation is then harmless to that capture, but in
// global mode the runtime would refuse it and could invalidate the capture.
// The caller has already checked that its own stream is not capturing.
hipError_t malloc_outside_capture(void** p, size_t bytes) {
    hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
    hipError_t e = hipThreadExchangeStreamCaptureMode(&mode);
    if (e != hipSuccess) return e;
    e = hipMalloc(p, bytes);
    hipStreamCaptureMode back = mode;
    const hipError_t e2 = hipThreadExchangeStreamCaptureMode(&back);
    return e != hipSuccess ? e : e2;
}

// A new workspace for (dev, stream), zeroed on the stream; not yet recorded.
red_status new_workspace(hipStream_t stream, Workspace* ws) {
    void* p = nullptr;
    hipError_t e = malloc_outside_capture(&p, kWorkspaceBytes);
    if (e != hipSuccess || p == nullptr) return fail(e, RED_ERR_ALLOC);
    // Zeroed by a kernel on the caller's stream, so the counter is 0 before
    // the first reduction on this stream runs.
    e = libred::launch_zero_words(static_cast<unsigned int*>(p), kWorkspaceBytes / 4, stream);
    if (e != hipSuccess) {
        (void)hipFree(p);
        return fail(e, RED_ERR_HIP);
    }
    ws->ticket = static_cast<unsigned int*>(p);
    ws->partials = static_cast<char*>(p) + kTicketBytes;
    ws->max_partials = kMaxPartials;
    return RED_OK;
}

red_status get_workspace(int dev, hipStream_t stream, Workspace* ws) {
    std::lock_guard<std::mutex> lock(g_mu);
    const auto key = std::make_pair(dev, stream);
    auto it = g_workspaces.find(key);
    if (it != g_workspaces.end()) {
        *ws = it->second;
        return RED_OK;
    }
    const red_status cap = refuse_if_capturing(stream);
    if (cap != RED_OK) return cap;
    Workspace w;
    const red_status st = new_workspace(stream, &w);
    if (st != RED_OK) return st;
    g_workspaces.emplace(key, w);
    *ws = w;
    return RED_OK;
}

// Device address of `scratch` on device `dev`, which must be current: looked
// up once per device, then cached. No allocation.
red_status noalloc_scratch(int dev, double** out) {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_noalloc_scratch.find(dev);
    if (it == g_noalloc_scratch.end()) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) return fail(e == hipSuccess ? hipErrorInvalidSymbol : e, RED_ERR_HIP);
        it = g_noalloc_scratch.emplace(dev, static_cast<double*>(ptr)).first;
    }
    *out = it->second;
    return RED_OK;
}

red_status get_scratch(int dev, hipStream_t stream, size_t bytes, void** out) {
    std::lock_guard<std::mutex> lock(g_mu);
    Scratch& sc = g_scratch[std::make_pair(dev, stream)];
    if (sc.ptr != nullptr && sc.bytes >= bytes) {
        *out = sc.ptr;
        return RED_OK;
    }
    const red_status cap = refuse_if_capturing(stream);
    if (cap != RED_OK) return cap;
    size_t nb = bytes < ((size_t)1 << 20) ? ((size_t)1 << 20) : bytes;
    if (sc.ptr != nullptr && nb < 2 * sc.bytes) nb = 2 * sc.bytes;
    if (nb > kColsScratchMax && bytes <= kColsScratchMax) nb = kColsScratchMax;
    void* p = nullptr;
    const hipError_t e = malloc_outside_capture(&p, nb);
    if (e != hipSuccess || p == nullptr) return fail(e, RED_ERR_ALLOC);
    if (sc.ptr != nullptr) g_retired_scratch.push_back(sc.ptr);
    sc.ptr = p;
    sc.bytes = nb;
    *out = p;
    return RED_OK;
}

// Column defaults, from a sweep over five 1 GiB shapes (65536 x 4096,
// 16K x 16K, 1M x 256, 256K x 1024, 256 x 1M): 512 waves with two groups of
// 8 rows in flight each are best on average. Short-wide matrices (more than
// 1024 blocks of 256 columns) instead read 4 KiB of a row per wave and
// 2 rows at a time, without prefetch (256 x 1M: 5.9 -> 7.1 TB/s).
constexpr libred::ColsPolicy kDefaultCols = {8, 1, 512, 0, 1, 1, 0, 0};

// The read probe's default shape: the fastest of its sweep on a 1 GiB buffer.
constexpr red_read_shape kDefaultReadShape = {64, 2, 8, 1, 2};
// The copy probe's default shape (single-wave blocks, next tile in flight).
constexpr red_read_shape kDefaultCopyShape = {64, 2, 8, 1, 2};
constexpr libred::ColsPolicy kWideCols = {2, 1, 1024, 0, 4, 0, 0, 0};
// Columns read one element per lane (rows not 16-byte aligned, or cols or ld
// not a multiple of 4) with at least 64 of them: two loads per row per lane,
// 2048 waves (a sweep over 4097, 1001, 257 and 65 columns: 2.3-2.8 ->
// 3.4-5.3 TB/s against the vector default).
constexpr libred::ColsPolicy kScalarCols = {8, 1, 2048, 0, 2, 0, 0, 0};
// Columns read four per lane from rows that do not start 16-byte aligned
// (the shifted form), the best of a sweep of launch shapes over 1 GiB
// matrices at odd ld. Rows that take 64 lanes: 4 rows in flight twice over,
// 2 KiB of a row per wave, 1024 waves (9 shapes over 255-16000 columns).
// Packed rows: 8 rows in flight twice over, 2048 waves (6 shapes over 5-200
// columns). Against one column per lane (kScalarCols): 256-8192 columns
// 5.1-5.6 -> 5.4-6.5 TB/s with the XCD grouping, 5-200 columns 3.2-4.9 ->
// 4.5-6.3.
static_assert(libred::table::kXcdGroupMinPhases >= (size_t)libred::kXcds, "a whole number of phases per XCD");
constexpr libred::ColsPolicy kShiftWideCols = {4, 1, 1024, 0, 2, 1, 0, 0};
constexpr libred::ColsPolicy kShiftNarrowCols = {8, 1, 2048, 0, 1, 1, 0, 0};
// Folded views whose default launch leaves too few row phases to group the
// blocks per XCD (kFoldFewPhasesMaxBlocks): 4 rows in flight, 1024 waves.
constexpr libred::ColsPolicy kFoldPhasesCols = {4, 1, 1024, 0, 1, 1, 0, 0};
// Unfolded rows of more than kUnfoldedWideAboveCols columns (up to the
// short-wide limit): 4 rows in flight, 2 KiB of a row per wave, 1024 waves.
constexpr libred::ColsPolicy kUnfoldedWideCols = {4, 1, 1024, 0, 2, 0, 0, 0};

libred::ColsPolicy to_cols(const red_cols_policy* p) {
    if (!p) return kDefaultCols;
    libred::ColsPolicy c = {p->unroll, p->nontemporal, p->target_waves, p->vec, p->width, p->prefetch, p->fold,
                            p->order,  p->xcd};
    return c;
}

FlatPolicy default_fused(size_t n) { return n <= kCachedMax ? default_flat(n) : kFusedLarge; }

FlatPolicy to_flat(const red_flat_policy* p, size_t n, bool fused = false) {
    if (!p) return fused ? default_fused(n) : default_flat(n);
    FlatPolicy f = {p->block,  p->blocks_per_cu, p->unroll,  p->nontemporal,
                    p->layout, p->prefetch,      p->combine};
    return f;
}

// The row defaults follow the row length (a sweep over 1 GiB matrices with
// rows of 1024, 4096, 16384 and 65536 floats): rows of at least 16384 floats
// take 16 loads per lane and 512 waves; rows under 2048 floats take a tile
// no longer than the row (at most 4 loads per lane) and 2048 waves, so that
// the per-row wave reduce is spread over more waves; the rest keep
// kDefaultRows.
RowsPolicy default_rows(size_t cols) {
    RowsPolicy p = kDefaultRows;
    const size_t nvec = cols / 4;
    namespace T = libred::table;
    if (cols >= T::kRowsLongFromCols) {
        p.unroll = T::kRowsLongUnroll;
        p.max_blocks = T::kRowsLongWaves;
    } else if (cols < T::kRowsShortBelowCols) {
        const size_t u = nvec / 64;
        p.unroll = u >= 4 ? 4 : (u >= 2 ? 2 : 1);
        p.max_blocks = T::kRowsShortWaves;
    } else if (nvec < 1024 && nvec % 512 != 0 && nvec % 512 <= T::kPartialTileMaxVectors) {
        // Rows of 1-1.75 tiles of 8 loads per lane: the partial tile costs a
        // round trip of its own, better hidden by 4-load tiles on 2048 waves
        // (2052: 4.9 -> 6.4, 2560: 5.6 -> 7.1, 3072: 6.2 -> 6.9, 3584: 6.7 ->
        // 7.0 TB/s; at 4000 floats, a 95% full second tile, 3% slower).
        p.unroll = 4;
        p.max_blocks = T::kRowsShortWaves;
    }
    return p;
}

RowsPolicy to_rows(const red_rows_policy* p, size_t cols) {
    if (!p) return default_rows(cols);
    RowsPolicy r = {p->block,      p->unroll, p->nontemporal, p->max_blocks, p->split,
                    p->prefetch,   p->short_rows, p->cover,   p->defer,      p->lines, p->xcd, p->max_fold};
    return r;
}

// Blocks for n elements: enough for one unrolled loop trip per thread, at
// most blocks_per_cu per CU and at most kMaxPartials.
size_t flat_grid_for(size_t n, const FlatPolicy& p, int cu_count) {
    const size_t per_block = (size_t)p.block * (size_t)p.unroll * 4;
    size_t want = (n + per_block - 1) / per_block;
    if (want < 1) want = 1;
    size_t cap = (size_t)p.blocks_per_cu * (size_t)cu_count;
    if (cap > kMaxPartials) cap = kMaxPartials;
    return want < cap ? want : cap;
}

template <class In, class Out, class Launch>
red_status flat_call(const In* x, size_t n, Out* out, const red_flat_policy* pol, hipStream_t stream,
                     Launch launch, size_t out_count = 1, bool fused = false) {
    if (n > RED_MAX_N || (n > 0 && x == nullptr) || out == nullptr) return RED_ERR_INVALID_ARG;
    if (!aligned(x, sizeof(In)) || !aligned(out, sizeof(Out))) return RED_ERR_INVALID_ARG;
    if (overlap(x, n * sizeof(In), out, out_count * sizeof(Out))) return RED_ERR_INVALID_ARG;
    const FlatPolicy p = to_flat(pol, n, fused);
    if (!libred::flat_policy_supported(p)) return RED_ERR_INVALID_ARG;
    int dev;
    DeviceInfo info;
    red_status st = current_device(&dev, &info);
    if (st != RED_OK) return st;
    Workspace ws;
    st = get_workspace(dev, stream, &ws);
    if (st != RED_OK) return st;
    const int grid = (int)flat_grid_for(n, p, info.cu_count);
    const hipError_t e = launch(x, n, out, grid, p, ws, stream);
    if (e != hipSuccess) return fail(e, RED_ERR_HIP);
    return RED_OK;
}

template <class Launch>
red_status rows_call(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                     const red_rows_policy* pol, hipStream_t stream, Launch launch) {
    if (ld < cols || rows > RED_MAX_N || cols > RED_MAX_N || ld > RED_MAX_N) return RED_ERR_INVALID_ARG;
    // Elements spanned: (rows - 1) * ld + cols.
    if (rows > 1 && ld != 0 && rows - 1 > (RED_MAX_N - cols) / ld) return RED_ERR_INVALID_ARG;
    const size_t span = rows == 0 ? 0 : (rows - 1) * ld + cols;
    if (span > RED_MAX_N) return RED_ERR_INVALID_ARG;
    RowsPolicy p = to_rows(pol, cols);
    if (!libred::rows_policy_supported(p)) return RED_ERR_INVALID_ARG;
    if (cols < 16) p.prefetch = 0;  // the streaming kernel takes rows of at least 16 elements
    if (rows == 0) return RED_OK;
    if ((span > 0 && x == nullptr) || out == nullptr) return RED_ERR_INVALID_ARG;
    if (!aligned(x, sizeof(float)) || !aligned(out, sizeof(float))) return RED_ERR_INVALID_ARG;
    if (overlap(x, span * sizeof(float), out, rows * sizeof(float))) return RED_ERR_INVALID_ARG;
    int dev;
    DeviceInfo info;
    red_status st = current_device(&dev, &info);
    if (st != RED_OK) return st;
    namespace T = libred::table;

    libred::RowsLaunch L = {0, 0, nullptr, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    // Grid-stride kernels with the blocks of each XCD on consecutive rows
    // (RowsLaunch::xmap): the grid rounded up to a multiple of kXcds, so a
    // wave keeps its number of rows or gets one fewer.
    const bool whole_lines = aligned(x, T::kRowLineBytes) && (rows == 1 || ld * sizeof(float) % T::kRowLineBytes == 0);
    const bool group_default = !whole_lines && cols >= T::kGroupRowsMinCols && cols < T::kGroupRowsMaxCols;
    const int chunk = p.xcd >= 2 ? p.xcd : (p.xcd == 0 && group_default) ? T::kGroupRowsChunk : 0;
    auto group = [&]() {
        if (chunk <= 0) return;
        const size_t per = (size_t)libred::kXcds * (size_t)chunk;
        if ((size_t)L.grid < per) return;
        L.grid = (int)(((size_t)L.grid + per - 1) / per * per);
        L.xmap = chunk;
    };
    // Rows of fewer than 1024 floats go to the LDS-staged kernel (short_rows
    // 0), or do so with 2^(short_rows - 3) lanes per row (short_rows 3-9),
    // when the rows are contiguous or their gaps hold at most a quarter of a
    // row's elements, or at most kStagedGapMaxFloats for rows of
    // kStagedGapMinCols to kStagedGapMaxCols floats (the tiles read the gaps
    // along), the matrix spans at
    // least 8 elements, and a tile fits 4096 floats. A contiguous, 16-byte
    // aligned matrix ("dense") is tiled in 16-byte aligned spans of rows;
    // other matrices in spans that start anywhere.
    const size_t step = rows == 1 ? cols : ld;  // elements from one row to the next
    const bool dense = step == cols && aligned(x, 16);
    const size_t fold = cols % 4 == 0 ? 1 : cols % 2 == 0 ? 2 : 4;  // rows per 16-byte aligned span
    const size_t span_all = (rows - 1) * step + cols;
    // (Strided rows of 512 floats and more stay with the packed or
    // one-wave-per-row kernels: 512 floats at a stride of 516 ran 6% slower
    // staged.)
    // Rows of 1 to 32 floats of a contiguous, 16-byte aligned matrix: the
    // narrow kernel, each lane reducing the whole rows of its own 16-byte
    // vectors (through LDS when they span several) and storing its results
    // side by side (short_rows 17).
    // The default for rows of up to 32 floats, on the measured number of
    // waves for the width (the table).
    // Each wave holds its results in LDS and stores them in bursts where
    // the table says so (defer 0), always (defer 2) or never (defer 1); by
    // default on the table's waves for the width, no more than the CUs hold
    // at once with that LDS.
    const bool narrow_default = p.short_rows == 0 && cols <= T::kNarrowDefaultMaxCols;
    if (dense && libred::rows_narrow_tile_rows(cols) > 0 && (p.short_rows == 17 || narrow_default)) {
        const size_t steps = rows / libred::rows_narrow_tile_rows(cols);
        const bool hold = (p.defer == 2 || (p.defer == 0 && T::kNarrowHold[cols])) &&
                          libred::rows_narrow_lds_bytes(cols, true) <= info.lds_per_block;
        size_t cap = pol != nullptr ? (size_t)p.max_blocks
                     : hold         ? (size_t)T::kNarrowHoldWaves
                                    : (size_t)T::kNarrowWaves[cols];
        if (pol == nullptr && hold) {
            const size_t lds = libred::rows_narrow_lds_bytes(cols, true);
            const size_t resident = (size_t)info.cu_count * (info.lds_per_cu / lds);
            if (cap > resident && resident > 0) cap = resident;
        }
        L.narrow = hold ? 2 : 1;
        L.grid = (int)(steps == 0 ? 1 : steps < cap ? steps : cap);
        const hipError_t e = launch(x, rows, cols, ld, out, L, p, stream);
        if (e != hipSuccess) return fail(e, RED_ERR_HIP);
        return RED_OK;
    }
    if (p.short_rows == 17) p.short_rows = 0;  // where the register kernel does not apply: the default
    const bool staged_ok =
        cols > 0 && (dense ? rows * cols >= 4 && fold * cols <= T::kStagedMaxTileFloats
                           : span_all >= 8 &&
                                 ((step - cols) * 4 <= cols ||
                                  (cols >= T::kStagedGapMinCols && cols <= T::kStagedGapMaxCols &&
                                   step - cols <= T::kStagedGapMaxFloats)) &&
                                 cols + 3 <= T::kStagedMaxTileFloats &&
                                 (step == cols || cols < T::kStagedStridedBelowCols));
    const bool staged_default = p.short_rows == 0 && cols < T::kStagedBelowCols;
    if (staged_ok && (staged_default || p.short_rows >= 3)) {
        const size_t span_floats = dense ? fold * cols : cols + 3;  // one aligned span of rows
        const size_t base_u = span_floats <= T::kTileFloats4 ? 4 : span_floats <= T::kTileFloats8 ? 8 : 16;
        // x's offset in elements from the 16-byte boundary before it.
        const size_t sh = ((uintptr_t)x % 16) / sizeof(float);
        // Rows of whole vectors that start 16-byte aligned, the condition for
        // reading them from LDS a vector at a time.
        const bool vec_rows = cols % 4 == 0 && sh == 0 && step % 4 == 0;
        size_t max_blocks = (size_t)p.max_blocks;
        const bool vread_default = vec_rows && cols <= T::kVectorReadMaxCols;
        // Rows per tile: dense, a whole number of aligned spans in 256 * u
        // elements; otherwise as many rows as fit with room for a span that
        // starts 3 elements into its first vector.
        // Whole-line tiles (lines 1): for a contiguous, 16-byte aligned
        // matrix, R a multiple of 32, so that a tile's rows span whole 128-byte
        // lines of input (R * cols floats) and of output (R floats) when x and
        // out are 128-byte aligned; a line shared by two tiles is otherwise
        // read, or written in part, by two waves.
        // By default (lines 0) for contiguous, aligned rows of fewer than 32
        // floats, whose results are too many to hold to the end of the wave:
        // 1 GiB, 3 floats 4.7 -> 5.4, 5-15 and 17 floats 5.0-5.4 -> 5.7-5.9,
        // 24 floats 5.3 -> 5.8 TB/s of input and output (widths 4, 8, 16 and
        // 32 had whole-line tiles already).
        const bool whole_lines = dense && (p.lines == 1 || (p.lines == 0 && cols < T::kWholeLinesBelowCols));
        auto tile_rows = [&](size_t u) {
            if (!dense) return (256 * u - 3 - cols) / step + 1;
            if (whole_lines && (256 * u) / (32 * cols) >= 1) return (256 * u) / (32 * cols) * 32;
            return (256 * u) / (fold * cols) * fold;
        };
        // Lanes per row first: the tile size below depends on them.
        bool lanes_by_tile = false;
        if (p.short_rows >= 10) {  // vector reads (rows of whole vectors), 2^(short_rows - 10) lanes
            L.staged_log2s = p.short_rows - 10;
            L.staged_vread = vec_rows ? 1 : 0;
        } else if (p.short_rows >= 3) {
            L.staged_log2s = p.short_rows - 3;
        } else if (vread_default) {
            // Rows of up to 16 whole vectors: 16-byte reads from LDS, one lane
            // per 2 vectors of the row (per 4 from 16 vectors). Element reads
            // at a stride of cols words put the rows of a pass on the same
            // LDS banks (8-32 floats: 5.1-5.5 -> 5.4-5.9 TB/s).
            const size_t v = cols / 4, per = v >= 16 ? 4 : 2;
            int lg = 0;
            while (((size_t)2 << lg) <= v / per) ++lg;
            L.staged_log2s = lg;
            L.staged_vread = 1;
        } else if (pol == nullptr && cols >= T::kLanesFourFromCols && cols < T::kLanesByTileFromCols &&
                   cols % T::kLanesWholeVecEvenCols != 0 && tile_rows(16) >= T::kLanesFourMinRows &&
                   (tile_rows(16) < T::kLanesFourMaxRows ||
                    (tile_rows(16) == T::kLanesFourMaxRows && cols < T::kLanesFourMaxRowsBelowCols))) {
            // Rows of 257-511 floats whose 4096-float tile holds 10-12 rows:
            // 4 lanes per row reduce them in one pass (cols / 24 lanes took
            // two, the second a quarter to a half full).
            L.staged_log2s = 2;
        } else if (pol == nullptr && cols >= T::kLanesByTileFromCols && cols <= T::kWholeWaveAboveCols) {
            // Rows of 513-1023 floats: lanes per row by the rows R that a
            // 4096-float tile holds, so that few of a tile's row slots go
            // unused and the passes are few.
            const size_t r16 = tile_rows(16);
            const int lg = r16 >= 7   ? 4
                           : r16 == 6 ? (cols < T::kLanesSixRowsWideFromCols ? 3 : 5)
                           : r16 == 5 ? 3
                           : r16 == 4 ? (cols < T::kLanesFourRowsWideFromCols ? 4 : 5)
                                      : 5;
            L.staged_log2s = lg;
            lanes_by_tile = true;
        } else {
            // Lanes per row: the largest power of two up to cols / 8 below
            // 32 floats (1024-float tiles), cols / 24 from there, or cols / 16
            // for rows of whole vectors from 128 floats (4096-float tiles);
            // longer rows take the whole wave.
            const size_t per = cols < T::kLanesNarrowBelowCols ? T::kLanesDivNarrow
                               : (cols % 4 == 0 && cols >= T::kLanesWholeVecFromCols &&
                                  cols % T::kLanesWholeVecEvenCols == 0) ? T::kLanesDivWholeVec
                                                                          : T::kLanesDivOther;
            int lg = 0;
            while (lg < 6 && ((size_t)2 << lg) <= cols / per) ++lg;
            L.staged_log2s = cols > T::kWholeWaveAboveCols ? 6 : lg;
        }
        // Tile size: 16-byte vectors per lane (4, 8 or 16, at least base_u
        // so that a tile holds one aligned span of rows).
        const size_t pass = (size_t)64 >> L.staged_log2s;  // rows reduced at a time
        auto pass_use = [&](size_t u) {  // share of the passes' row slots that hold a row
            const size_t r = tile_rows(u);
            return r == 0 ? 0.0 : (double)r / (double)(pass * ((r + pass - 1) / pass));
        };
        size_t u = base_u;
        if (pol == nullptr && whole_lines && cols >= T::kWholeLinesWideTileFromCols &&
            cols < T::kWholeLinesBelowCols && (cols & (cols - 1)) != 0 && base_u <= 8) {
            // Whole-line tiles of rows of 5-31 floats that are not a power of
            // two: 8 loads per lane on 2048 waves came within 3% of the best
            // of nine shapes at each width measured (5-15, 17, 24 floats);
            // 3 floats and the powers of two ran 1-3% faster with 4.
            u = 8;
        } else if (pol == nullptr && vread_default && cols >= T::kVectorReadBigTileFromCols) {
            // Rows of 11-16 whole vectors (measured on 1 GiB, sums): 4096-float
            // tiles on 1024 waves for 44-60 floats (48: 5.9 -> 6.3, 60: 5.4 ->
            // 6.4 TB/s), 2048-float tiles on 1024 waves for 64 floats (6.5 ->
            // 6.8 TB/s); narrower rows keep 1024-float tiles on 2048 waves.
            u = cols == 64 ? 8 : 16;
            max_blocks = T::kStagedBigTileWaves;
        } else if (pol == nullptr && !vread_default && cols >= T::kElementTileRuleMinCols &&
                   cols <= T::kElementTileRuleMaxCols) {
            // Rows of 33 to 512 floats read element by element: the largest
            // tile whose passes are within 2% as full as the fullest, on 1024
            // waves for 4096-float tiles and 2048 below (over 54 widths of
            // 33-512 floats on 1 GiB, 97.3% of the best of four shapes on
            // geometric mean, against 95.8% for 4096-float tiles throughout).
            double best = 0.0;
            for (size_t c : {(size_t)16, (size_t)8, (size_t)4})
                if (c >= base_u && pass_use(c) > best + T::kPassUseSlack) {
                    best = pass_use(c);
                    u = c;
                }
            max_blocks = u == 16 ? T::kStagedBigTileWaves : T::kStagedWaves;
            // A tile that takes more than one pass, the last at most a quarter
            // full, yields to the largest smaller one that takes one pass or
            // fills its last better (on 2048 waves), for rows of
            // kThinPassFromCols to 512 floats.
            auto thin_last_pass = [&](size_t c) {
                const size_t r = tile_rows(c);
                if (r == 0) return false;
                const size_t n = (r + pass - 1) / pass, last = r - (n - 1) * pass;
                return n > 1 && last * T::kThinPassDivisor <= pass;
            };
            if (cols >= T::kThinPassFromCols && cols < T::kLanesByTileFromCols && thin_last_pass(u)) {
                for (size_t c : {(size_t)8, (size_t)4})
                    if (c < u && c >= base_u && tile_rows(c) > 0 && !thin_last_pass(c)) {
                        u = c;
                        max_blocks = T::kStagedWaves;
                        break;
                    }
            }
            // Rows of 513-1023 floats whose 4096-float tile holds fewer floats
            // of rows than kStagedSparseTileFloats (odd widths to 583: four
            // rows): 2048 waves.
            if (lanes_by_tile && u == 16 && tile_rows(16) * step < T::kStagedSparseTileFloats)
                max_blocks = T::kStagedWaves;
            // Rows of 33-39 floats: when 4096-float tiles leave no room to
            // hold the results in LDS but 2048-float tiles on 1024 waves do,
            // and their passes are within 5% as full, take those (1 GiB: sums
            // 5.5 -> 5.5-6.4, maxima 5.5-5.6 -> 5.7-6.0 TB/s; at 41-43 floats
            // the maxima ran 8% slower).
            auto holds = [&](size_t c, size_t mb) {
                const size_t r = tile_rows(c), tl = (rows + r - 1) / r;
                const size_t g = tl < mb ? tl : mb;
                const size_t need = 64 * c * 16 + (tl + g - 1) / g * r * sizeof(float);
                return need <= info.lds_per_cu / ((g + info.cu_count - 1) / info.cu_count) &&
                       need <= info.lds_per_block;
            };
            if (u == 16 && p.defer != 1 && cols < T::kHoldSmallTileBelowCols && base_u <= 8 &&
                !holds(16, T::kStagedBigTileWaves) && holds(8, T::kStagedBigTileWaves) &&
                pass_use(8) >= pass_use(16) - T::kHoldSmallTileSlack) {
                u = 8;
                max_blocks = T::kStagedBigTileWaves;
            }
        }
        L.staged_u = (int)u;
        // An explicit policy may ask for larger tiles (unroll 8 or 16).
        if (pol != nullptr && p.unroll > L.staged_u) L.staged_u = p.unroll >= 16 ? 16 : 8;
        L.staged_rows = (unsigned int)tile_rows((size_t)L.staged_u);
        // Element reads: LDS serves each 32-lane half of a wave from 32
        // banks of 4 bytes. When 16 or more rows of a half start on the same
        // bank ((pass / 2) * gcd(step, 32) / 32 of them), their lanes read
        // the same banks at every step; then each row's lanes start at a
        // different element (32 floats at an unaligned x 2.3 -> 5.7, 64
        // floats 4.0 -> 5.6 TB/s; at 8 such rows and fewer, the wrapping
        // index cost 7-30%).
        const size_t low = step & (~step + 1), bank_gcd = low < 32 ? low : 32;
        L.staged_spread = !L.staged_vread && (pass / 2) * bank_gcd >= 16 * 32 ? 1 : 0;
        const size_t tiles = (rows + L.staged_rows - 1) / L.staged_rows;
        L.grid = (int)(tiles < max_blocks ? tiles : max_blocks);
        group();
        // Maxima fold with a hardware max (max_fold 2), or where the table
        // says so (max_fold 0); the row sums ignore this.
        L.staged_fmax = p.max_fold == 2 || (p.max_fold == 0 && cols < T::kStagedMaxFmaxBelowCols) ? 1 : 0;
        // A wave's results are held in LDS and stored after its last tile
        // (defer 0) when they fit beside its staging tile in one wave's share
        // of a CU's LDS (the grid's waves spread evenly over the CUs) and in
        // one block's limit.
        // Rows of 960 floats and more are left out: with a row or two per
        // tile, holding measured 1-10% slower there (and 5-20% faster on
        // narrower rows).
        if (p.defer != 1 && cols < T::kHoldBelowCols) {
            const size_t results = (tiles + L.grid - 1) / L.grid * L.staged_rows;
            const size_t waves_per_cu = ((size_t)L.grid + info.cu_count - 1) / info.cu_count;
            const size_t stage = (size_t)64 * L.staged_u * 16;  // 64 lanes x staged_u 16-byte vectors
            const size_t need = stage + results * sizeof(float);
            if (need <= info.lds_per_cu / waves_per_cu && need <= info.lds_per_block)
                L.staged_hold = (unsigned int)results;
        }
        const hipError_t e = launch(x, rows, cols, ld, out, L, p, stream);
        if (e != hipSuccess) return fail(e, RED_ERR_HIP);
        return RED_OK;
    }
    // Rows of at most 512 floats go to the packed-row kernel unless the
    // policy turns that off (short_rows 1): 16-byte units when every row
    // starts 16-byte aligned and holds whole vectors (segments of up to 16
    // lanes), else single elements (segments of up to 64 lanes).
    if (p.short_rows != 1 && cols > 0 && cols <= T::kPackedMaxCols) {
        const bool vec = aligned(x, 16) && cols % 4 == 0 && ld % 4 == 0;
        const size_t units = vec ? cols / 4 : cols;
        const int max_lg = vec ? 4 : 6;
        int lg = 0;
        while ((1u << lg) < units && lg < max_lg) ++lg;  // lanes per row: pow2ceil(units), capped
        const size_t lanes = (size_t)1 << lg;
        const size_t per_lane = (units + lanes - 1) / lanes;
        L.packed_log2l = lg;
        L.packed_v = per_lane <= 1 ? 1 : per_lane <= 2 ? 2 : per_lane <= 4 ? 4 : 8;
        L.packed_scalar = vec ? 0 : 1;
        const size_t groups = (rows + (64 / lanes) - 1) / (64 / lanes);
        const size_t per_trip_groups = (size_t)(vec ? 16 : 32) / (size_t)L.packed_v;
        const size_t waves = (groups + per_trip_groups - 1) / per_trip_groups;
        L.grid = (int)(waves < (size_t)p.max_blocks ? waves : (size_t)p.max_blocks);
        group();
        const hipError_t e = launch(x, rows, cols, ld, out, L, p, stream);
        if (e != hipSuccess) return fail(e, RED_ERR_HIP);
        return RED_OK;
    }
    const size_t tile_elems = (size_t)64 * (size_t)p.unroll * 4;
    const size_t tiles_per_row = cols / tile_elems;
    const bool want_split =
        p.split == 2 || (p.split == 0 && rows < kSplitRowsBelow && cols >= kSplitMinCols);
    if (want_split && tiles_per_row >= 2) {
        size_t gx = (kSplitTargetWaves + rows - 1) / rows;
        if (gx > tiles_per_row) gx = tiles_per_row;
        if (gx > libred::kMaxSplitPartials / rows) gx = libred::kMaxSplitPartials / rows;
        if (gx >= 2) {
            Workspace ws;
            st = get_workspace(dev, stream, &ws);
            if (st != RED_OK) return st;
            L.split_gx = (unsigned int)gx;
            L.partials = ws.partials;
        }
    }
    if (L.split_gx == 0) {
        // One wave per row. Rows that do not all start 16-byte aligned are
        // read through their aligned covers (cover 0), or always (cover 2),
        // or never (cover 1); the covered kernel takes rows of at least 16
        // elements. Its defaults by row length come from a sweep over
        // unaligned rows of 1025 to 50257 floats.
        const bool misaligned = !aligned(x, 16) || (rows > 1 && ld % 4 != 0);
        // Aligned rows whose last round of loads would be at most half a
        // tile take the covered kernel's shape too (see kCoverLastRoundMax).
        const size_t nvec = cols / 4, tile_vecs = (size_t)64 * p.unroll;
        const bool thin_last = pol == nullptr && cols < T::kRowsLongFromCols && nvec % tile_vecs != 0 &&
                               (double)(nvec % tile_vecs) <= T::kCoverLastRoundMax * (double)tile_vecs;
        L.cover = cols >= 16 && (p.cover == 2 || (p.cover == 0 && (misaligned || thin_last))) ? 1 : 0;
        if (L.cover && pol == nullptr) {
            // A wave folds its rows one after another, so below 16384 floats
            // more waves hide more of each row's memory latency: 8 loads per
            // lane on up to 32768 waves ran 4-21% faster over 1025-8193
            // floats than 4096 or 2048 waves (2049: 5.8 -> 6.8, 2500: 5.5 ->
            // 6.6 TB/s) and within 2% at 1700, 3001 and 6001; longer rows
            // keep 1024 waves (50257 floats: 6% slower with more).
            p.unroll = T::kCoverUnroll;
            p.max_blocks = cols < T::kRowsLongFromCols ? T::kCoverWavesBelowLong : T::kCoverWavesLong;
        }
        // Every wave gets the same number of rows, give or take one: with
        // per = ceil(rows / (max_blocks waves)), ceil(rows / per) waves, so
        // no few waves are left with an extra round of rows. (Filling the
        // cap exactly, or going past it to even out the rounds, measured
        // slower: 8388 x 32001 and 5341 x 50257 ran 6-7% slower with the
        // larger grids.)
        const size_t W = (size_t)p.block / 64;
        size_t target = (size_t)p.max_blocks * W;
        if (target > rows) target = rows;
        const size_t per = (rows + target - 1) / target;  // rows per wave
        const size_t waves = (rows + per - 1) / per;
        L.grid = (int)((waves + W - 1) / W);
        group();
    }
    const hipError_t e = launch(x, rows, cols, ld, out, L, p, stream);
    if (e != hipSuccess) return fail(e, RED_ERR_HIP);
    return RED_OK;
}

// Fraction of a column kernel's lanes that read data when the (view) rows
// hold `groups` 16-byte column groups: below 64 groups a wave packs
// 64 / groups rows per load; from 64 up each block takes 64 groups, the last
// block of a row only what is left.
double cols_lane_use(size_t groups) {
    if (groups < 64) return (double)(groups * (64 / groups)) / 64.0;
    return (double)groups / (double)(64 * ((groups + 63) / 64));
}

// Rows per view row for a contiguous matrix (1 = no fold). m is a multiple
// of m0 = 4 / gcd(cols, 4) and at most rows:
// - a width of at least 256 that is not a multiple of 32 (nor 2 mod 4) takes
//   32 when that leaves at least 1024 view rows;
// - another width of at least 256 that is not a multiple of 4 takes the
//   largest up to 16;
// - a width of 32 to 255 (a multiple of 4 only if its own rows leave 5% of
//   the lanes idle) takes the smallest multiple of 32 / gcd(cols, 32) with
//   512 groups of four columns in a view row, at most 64;
// - a width under 32 takes the smallest multiple of 32 / gcd(cols, 32) up
//   to 32 (16 for multiples of 4) that keeps 84% of the lanes busy, unless
//   the m below already keeps 99%;
// - otherwise the m up to 16 whose view uses the most lanes, the smallest
//   on a tie;
// - a width that is a multiple of 4 is folded only when that uses at least
//   5% more lanes than the matrix itself (65 groups of four columns, say,
//   leave a second block per row phase with one group).
size_t fold_rows(size_t rows, size_t cols) {
    namespace T = libred::table;
    const size_t m0 = cols % 4 == 0 ? 1 : cols % 2 == 0 ? 2 : 4;
    // m_line rows span whole 128-byte lines. A wave reads 1 KiB of a row per
    // load; when rows do not start on a line, the line at each boundary is
    // fetched by the two waves (on different XCDs) that read either side of
    // it: 6.3% more HBM bytes with 16-row views of odd widths, 11-14% at 3,
    // 7, 17 and 100 columns (FETCH_SIZE).
    const size_t m_line = 32 / std::gcd(cols, (size_t)32);
    if (cols >= T::kFoldWideFromCols && cols % 32 != 0 && m_line != 16 && rows / 32 >= T::kFold32MinViewRows &&
        cols * 32 <= RED_MAX_N) {
        // 32 rows per view row (a multiple of m_line): odd widths of 257 to
        // 4097 ran 7-17% faster than with 16 rows (1025: 5.8 -> 6.3, 2049:
        // 5.9 -> 6.9 TB/s), multiples of 4 from 300 to 6000 0-15% faster
        // than unfolded. Widths of 2 mod 4 keep 16 rows, which already
        // span whole lines (32 measured up to 8% slower there).
        return 32;
    }
    if (m0 > 1 && cols >= T::kFoldWideFromCols) {
        // Over 1023 to 65537 columns, 16 rows ran 3-24% faster than 4 rows,
        // which already use 98% of the lanes.
        size_t m = T::kFold16Rows;
        while (m > rows || cols * m > RED_MAX_N) m -= m0;
        return m < m0 ? 1 : m;
    }
    if (cols >= T::kFoldMidFromCols && cols < T::kFoldWideFromCols &&
        (m0 > 1 || cols_lane_use(cols / 4) < T::kFoldMidLaneUse)) {
        // Widths of 32 to 255 (multiples of 4 only when their own rows leave
        // lanes idle) take the smallest m whose view rows hold 512 groups of
        // four columns (8 KiB) and span whole lines, at most 64: over 33 to
        // 132 columns 512 groups matched the best measured m within 1-4%
        // (33: 5.6 -> 6.7 TB/s, 65: 5.5 -> 6.8, 68: 6.0 -> 6.7 against the
        // choice by lane use below, whose 4-16 rows already keep most lanes
        // busy).
        size_t m = (T::kFoldViewFloats + cols - 1) / cols;
        m = (m + m_line - 1) / m_line * m_line;
        if (m > T::kFoldMaxRows) m = T::kFoldMaxRows;
        while (m > rows || cols * m > RED_MAX_N) m -= m0;
        return m < m0 ? 1 : m;
    }
    size_t best = 1;
    double best_use = -1.0;
    for (size_t m = m0; m <= 16 && m <= rows && cols * m <= RED_MAX_N; m += m0) {
        const double use = cols_lane_use(m * cols / 4);
        if (use > best_use + 1e-9) best_use = use, best = m;  // the smallest m on a tie
    }
    if (cols < T::kFoldMidFromCols && best_use < T::kFoldNarrowEnough) {
        // Below 32 columns, a view whose rows span whole lines wins when it
        // keeps 84% of the lanes busy (23: 5.7 -> 6.3, 28: 6.1 -> 6.5, 31:
        // 6.1 -> 6.8 TB/s; 7, 14, 21, 27, 29 3-5% faster); with fewer lanes
        // busy it lost up to 27%, and 64 rows lost 2% at 17 and 19 columns.
        // Multiples of 4 look no further than 16 rows (24 columns kept its
        // own rows best).
        const size_t top = m0 == 1 ? 16 : 32;
        for (size_t m = m_line; m <= top && m <= rows && cols * m <= RED_MAX_N; m += m_line)
            if (cols_lane_use(m * cols / 4) >= T::kFoldNarrowLaneUse) return m;
    }
    if (m0 == 1 && best_use < cols_lane_use(cols / 4) + T::kFoldGain) return 1;
    return best;
}

template <class Launch>
red_status cols_call(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                     const red_cols_policy* pol, hipStream_t stream, Launch launch) {
    if (ld < cols || rows > RED_MAX_N || cols > RED_MAX_N || ld > RED_MAX_N) return RED_ERR_INVALID_ARG;
    if (rows > 1 && ld != 0 && rows - 1 > (RED_MAX_N - cols) / ld) return RED_ERR_INVALID_ARG;
    const size_t span = rows == 0 ? 0 : (rows - 1) * ld + cols;
    libred::ColsPolicy p = to_cols(pol);
    if (!libred::cols_policy_supported(p)) return RED_ERR_INVALID_ARG;
    if (cols == 0) return RED_OK;
    if ((span > 0 && x == nullptr) || out == nullptr) return RED_ERR_INVALID_ARG;
    if (!aligned(x, sizeof(float)) || !aligned(out, sizeof(float))) return RED_ERR_INVALID_ARG;
    if (overlap(x, span * sizeof(float), out, cols * sizeof(float))) return RED_ERR_INVALID_ARG;
    int dev;
    DeviceInfo info;
    red_status st = current_device(&dev, &info);
    if (st != RED_OK) return st;

    libred::ColsLaunch L;
    L.fold_m = 1;
    L.real_cols = cols;
    L.tail_elems = 0;
    L.tail = nullptr;
    L.rot = 0;
    L.head = nullptr;
    L.order = 0;
    L.shift = 0;
    L.xmap = 0;
    L.col_fmax = 0;
    // A contiguous matrix may be viewed with m consecutive rows as one row
    // of m * cols columns (see fold_rows): for a width that is not a
    // multiple of 4 this makes every view row start 16-byte aligned, so four
    // columns go per lane; for any width it can leave fewer lanes idle.
    // When x is not 16-byte aligned the view starts rot = 1-31 elements into
    // the matrix, at the next 128-byte boundary (m * cols is a multiple of 4,
    // so every view row starts 16-byte aligned, and on a line when m * cols
    // is a multiple of 32: 4096 columns at x + 4 bytes ran at 6.3 TB/s from
    // the next 16-byte boundary). Column membership depends only on
    // an element's position mod cols, so view column c' holds real column
    // (c' + rot) mod cols. Pass 2 adds each real column's m view columns,
    // then its elements after the last whole view row and before the view.
    const size_t cols_real = cols;
    if (p.vec != 1 && p.fold != 1 && (ld == cols || rows == 1) && rows > 0) {
        size_t m = fold_rows(rows, cols);
        if (p.fold > 1) {  // the policy's m, made a multiple of 4 / gcd(cols, 4) that fits the rows
            const size_t m0 = cols % 4 == 0 ? 1 : cols % 2 == 0 ? 2 : 4;
            m = ((size_t)p.fold + m0 - 1) / m0 * m0;
            while (m > rows || cols * m > RED_MAX_N) m -= m0;
            if (m < m0) m = 1;
        }
        const size_t rot = (uintptr_t)x % 16 == 0 ? 0 : (128 - (uintptr_t)x % 128) % 128 / sizeof(float);
        const size_t W = cols_real * m;  // view columns
        const size_t total = rows * cols_real;
        const size_t vrows = total >= rot ? (total - rot) / W : 0;
        if ((m > 1 || rot > 0) && W % 4 == 0 && vrows >= 1) {
            L.fold_m = (int)m;
            L.rot = (unsigned int)rot;
            L.head = x;
            x += rot;
            rows = vrows;
            cols = W;
            ld = W;
            L.tail = x + vrows * W;
            L.tail_elems = total - rot - vrows * W;
        }
    }
    const bool vec_ok = aligned(x, 16) && cols % 4 == 0 && ld % 4 == 0;
    L.vec = (p.vec != 1 && vec_ok) ? 4 : 1;
    // Rows that do not start 16-byte aligned (or widths that are not a
    // multiple of 4) still read four columns per lane: a lane loads the
    // aligned vector its columns start in and takes the next from the next
    // lane.
    if (p.vec != 1 && !vec_ok && cols >= 4) {
        L.vec = 4;
        L.shift = 1;
    }
    const bool short_wide = pol == nullptr && L.vec == 4 && !L.shift && cols / 256 > libred::table::kWideColBlocks;
    if (short_wide) p = kWideCols;
    // Rows that are not a whole number of 128-byte lines (and not a folded
    // view) also read best 4 KiB at a time, 2 rows in flight: 1020, 1500,
    // 3000 and 6000 columns ran 8-12% faster than with the default shape.
    if (pol == nullptr && L.vec == 4 && L.fold_m == 1 && cols % 32 != 0 && cols >= libred::table::kFoldWideFromCols)
        p = kWideCols;
    // Whether a launch shape q would have its blocks grouped per XCD below
    // (at xcd 0), for rows of 64 groups of four columns per block (8 rows
    // per phase at least; the scratch cap on the phases, far above the
    // phases these shapes reach, is left out).
    auto grouped_with = [&](const libred::ColsPolicy& q) {
        const size_t pitch_b = ld * sizeof(float);
        if (pitch_b == 0 || (pitch_b & (pitch_b - 1)) == 0) return false;
        const size_t ncb_q = (cols + 256 * (size_t)q.width - 1) / (256 * (size_t)q.width);
        size_t ph = ((size_t)q.target_waves + ncb_q - 1) / ncb_q;
        const size_t by_rows = (rows + 7) / 8;
        if (ph > by_rows) ph = by_rows;
        const size_t dn = ph / libred::kXcds * libred::kXcds;
        return dn >= libred::table::kXcdGroupMinPhases &&
               (double)dn >= libred::table::kXcdGroupKeepPhases * (double)ph;
    };
    const bool unfolded_wide = pol == nullptr && L.vec == 4 && !L.shift && L.fold_m == 1 &&
                               cols > libred::table::kUnfoldedWideAboveCols &&
                               cols / 256 <= libred::table::kWideColBlocks &&
                               ((ld * sizeof(float)) & (ld * sizeof(float) - 1)) != 0 &&
                               (grouped_with(kUnfoldedWideCols) || !grouped_with(p));
    if (unfolded_wide) p = kUnfoldedWideCols;
    // Narrow matrix: if the column groups divide a wave, pack several rows
    // into each load.
    // With shift, a packed row's last group reaches into the vector after
    // its own when its first column can sit at position s of its vector
    // with s + (its columns) > 4; then one more lane per row (a spare) loads
    // that vector. The position is fixed by x when ld is a multiple of 4,
    // else it runs through 0-3.
    const size_t groups = L.shift ? (cols + 3) / 4 : cols / (size_t)L.vec;
    size_t spare = 0;
    if (L.shift) {
        const size_t last = cols - 4 * (groups - 1);  // columns of the last group, 1-4
        const size_t smax = ld % 4 == 0 ? (uintptr_t)x % 16 / sizeof(float) : 3;
        spare = last + smax > 4 ? 1 : 0;
    }
    L.ngroups = 64;
    if (groups + spare < 64) L.ngroups = (unsigned int)(groups + spare);
    if (pol == nullptr && L.vec == 1 && L.ngroups == 64) p = kScalarCols;
    if (pol == nullptr && L.fold_m > 1 && L.vec == 4 && !L.shift && L.ngroups == 64 &&
        (cols + 255) / 256 <= libred::table::kFoldFewPhasesMaxBlocks &&
        ((ld * sizeof(float)) & (ld * sizeof(float) - 1)) != 0 && !grouped_with(kDefaultCols))
        p = kFoldPhasesCols;
    if (pol == nullptr && L.shift) p = L.ngroups == 64 ? kShiftWideCols : kShiftNarrowCols;
    // Maxima of folded views of fewer than kColsFmaxBelowCols real columns
    // and of short-wide matrices fold with the hardware max.
    if (pol == nullptr && L.vec == 4 && !L.shift &&
        ((L.fold_m > 1 && L.real_cols < libred::table::kColsFmaxBelowCols) || short_wide))
        L.col_fmax = 1;
    L.width = L.ngroups == 64 ? p.width : 1;
    if (!L.shift)
        L.cspan = (size_t)L.ngroups * L.vec * L.width;
    else if (L.ngroups == 64)
        L.cspan = 4 * (64 * (size_t)L.width - 1);
    else
        L.cspan = 4 * (L.ngroups - spare);
    L.ncb = (cols + L.cspan - 1) / L.cspan;
    size_t nchunks = 1;
    if (rows > 0) {
        nchunks = ((size_t)p.target_waves + L.ncb - 1) / L.ncb;
        const size_t by_rows = (rows + 8 * (64 / L.ngroups) - 1) / (8 * (64 / L.ngroups));  // >= 8 loads per lane
        if (nchunks > by_rows) nchunks = by_rows;
        const size_t by_scratch = kColsScratchMax / (cols * 8);
        if (nchunks > by_scratch) nchunks = by_scratch;
        if (nchunks < 1) nchunks = 1;
    }
    // The short-wide shape keeps its grid within kShortWideMaxWaves
    // single-wave blocks (row phases rounded down, not up), with the
    // prefetch on where that leaves kShortWidePrefetchMaxWaves or fewer.
    if (short_wide && L.ncb <= (size_t)libred::table::kShortWideMaxWaves &&
        L.ncb * nchunks > (size_t)libred::table::kShortWideMaxWaves)
        nchunks = (size_t)libred::table::kShortWideMaxWaves / L.ncb;
    if (short_wide && L.ncb * nchunks <= (size_t)libred::table::kShortWidePrefetchMaxWaves) p.prefetch = 1;
    // The unfolded-wide shape does the same with few phases of many blocks,
    // but only where the rounded grid keeps kUnfoldedRoundMinWaves blocks or
    // leaves at most kShortWidePrefetchMaxWaves (then with the prefetch).
    if (unfolded_wide && L.ncb >= libred::table::kUnfoldedRoundMinBlocks &&
        L.ncb <= (size_t)libred::table::kShortWideMaxWaves &&
        L.ncb * nchunks > (size_t)libred::table::kShortWideMaxWaves) {
        const size_t down = (size_t)libred::table::kShortWideMaxWaves / L.ncb;
        if (L.ncb * down >= libred::table::kUnfoldedRoundMinWaves) {
            nchunks = down;
        } else if (L.ncb * down <= (size_t)libred::table::kShortWidePrefetchMaxWaves) {
            nchunks = down;
            p.prefetch = 1;
        }
    }
    // Blocks grouped per XCD (see ColsLaunch::xmap and
    // kXcdGroupMinPhases): a whole number of phases per XCD, rounded down
    // (kXcdGroupKeepPhases).
    const size_t pitch = ld * sizeof(float);
    const bool pow2_pitch = pitch != 0 && (pitch & (pitch - 1)) == 0;
    const size_t down = nchunks / libred::kXcds * libred::kXcds;
    const bool keeps = (double)down >= libred::table::kXcdGroupKeepPhases * (double)nchunks;
    if (p.xcd == 2) {
        L.xmap = 1;  // the kernel deals any grid
    } else if (p.xcd == 0 && !pow2_pitch && keeps && down >= libred::table::kXcdGroupMinPhases) {
        nchunks = down;
        L.xmap = 1;
    }
    L.nchunks = nchunks;
    // Row order: rotated starts at pitches the memory channels alias on
    // (see kRotateRowsPitchFactorA); runs of rows where a load covers rows
    // that do not span whole lines (see kLineBytes); else one band at a time.
    const size_t load_rows = 64 / L.ngroups;  // rows per wave load
    if (p.order > 0)
        L.order = p.order - 1;
    else if (rows > 1 && (ld % libred::table::kRotateRowsPitchFactorA == 0 ||
                          ld % libred::table::kRotateRowsPitchFactorB == 0))
        L.order = (L.fold_m == 1 && L.rot == 0) ? 2 : 1;  // runs unfolded, rotated through views
    else if (rows > 1 && L.ngroups < 64 && load_rows * ld * sizeof(float) % libred::table::kLineBytes != 0)
        L.order = 2;
    else
        L.order = 0;
    L.partials = nullptr;
    if (nchunks > 1 || L.fold_m > 1 || L.rot > 0) {
        st = get_scratch(dev, stream, nchunks * cols * 8, &L.partials);
        if (st != RED_OK) return st;
    }
    const hipError_t e = launch(x, rows, cols, ld, out, L, p, stream);
    if (e != hipSuccess) return fail(e, RED_ERR_HIP);
    return RED_OK;
}

}  // namespace

extern "C" {

red_status red_sum_f32(const float* x, size_t n, float* out, hipStream_t stream) {
    return flat_call(x, n, out, nullptr, stream, libred::launch_sum_f32);
}

red_status red_sum_i32_i64(const int32_t* x, size_t n, int64_t* out, hipStream_t stream) {
    return flat_call(x, n, out, nullptr, stream, libred::launch_sum_i32_i64);
}

red_status red_sum_f32_noalloc(const float* x, size_t n, float* out, hipStream_t stream) {
    if (n > RED_MAX_N || (n > 0 && x == nullptr) || out == nullptr) return RED_ERR_INVALID_ARG;
    if (!aligned(x, sizeof(float)) || !aligned(out, sizeof(float))) return RED_ERR_INVALID_ARG;
    if (overlap(x, n * sizeof(float), out, sizeof(float))) return RED_ERR_INVALID_ARG;
    const FlatPolicy p = default_flat(n);
    int dev;
    DeviceInfo info;
    red_status st = current_device(&dev, &info);
    if (st != RED_OK) return st;
    const size_t grid = flat_grid_for(n, p, info.cu_count);
    if (grid > kNoAllocMaxPartials) return RED_ERR_SCRATCH;
    double* ptr = nullptr;
    st = noalloc_scratch(dev, &ptr);
    if (st != RED_OK) return st;
    Workspace ws;
    ws.ticket = nullptr;  // the two-launch combine never touches a counter
    ws.partials = ptr;
    ws.max_partials = kNoAllocMaxPartials;
    const hipError_t e = libred::launch_sum_f32(x, n, out, (int)grid, p, ws, stream);
    if (e != hipSuccess) return fail(e, RED_ERR_HIP);
    return RED_OK;
}

red_status red_max_f32(const float* x, size_t n, float* out, hipStream_t stream) {
    return flat_call(x, n, out, nullptr, stream, libred::launch_max_f32);
}

red_status red_sum_max_f32(const float* x, size_t n, float* out3, hipStream_t stream) {
    return flat_call(x, n, out3, nullptr, stream, libred::launch_sum_max_f32, 3, true);
}

red_status red_min_f32(const float* x, size_t n, float* out, hipStream_t stream) {
    return flat_call(x, n, out, nullptr, stream, libred::launch_min_f32);
}

red_status red_argmax_f32(const float* x, size_t n, int64_t* out, hipStream_t stream) {
    return flat_call(x, n, out, nullptr, stream, libred::launch_argmax_f32);
}

red_status red_argmin_f32(const float* x, size_t n, int64_t* out, hipStream_t stream) {
    return flat_call(x, n, out, nullptr, stream, libred::launch_argmin_f32);
}

red_status red_sum_bf16_f32(const uint16_t* x, size_t n, float* out, hipStream_t stream) {
    return flat_call(x, n, out, nullptr, stream, libred::launch_sum_bf16);
}

red_status red_sum_f16_f32(const uint16_t* x, size_t n, float* out, hipStream_t stream) {
    return flat_call(x, n, out, nullptr, stream, libred::launch_sum_f16);
}

red_status red_sum_f64(const double* x, size_t n, double* out, hipStream_t stream) {
    return flat_call(x, n, out, nullptr, stream, libred::launch_sum_f64);
}

red_status red_rows_sum_f32(const float* x, size_t rows, size_t cols, float* out, hipStream_t stream) {
    return rows_call(x, rows, cols, cols, out, nullptr, stream, libred::launch_rows_sum_f32);
}

red_status red_rows_max_f32(const float* x, size_t rows, size_t cols, float* out, hipStream_t stream) {
    return rows_call(x, rows, cols, cols, out, nullptr, stream, libred::launch_rows_max_f32);
}

red_status red_rows_sum_f32_ld(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                               hipStream_t stream) {
    return rows_call(x, rows, cols, ld, out, nullptr, stream, libred::launch_rows_sum_f32);
}

red_status red_rows_max_f32_ld(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                               hipStream_t stream) {
    return rows_call(x, rows, cols, ld, out, nullptr, stream, libred::launch_rows_max_f32);
}

red_status red_cols_sum_f32(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                            hipStream_t stream) {
    return cols_call(x, rows, cols, ld, out, nullptr, stream, libred::launch_cols_sum_f32);
}

red_status red_cols_max_f32(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                            hipStream_t stream) {
    return cols_call(x, rows, cols, ld, out, nullptr, stream, libred::launch_cols_max_f32);
}

red_status red_stream_new_workspace(hipStream_t stream) {
    int dev;
    DeviceInfo info;
    red_status st = current_device(&dev, &info);
    if (st != RED_OK) return st;
    std::lock_guard<std::mutex> lock(g_mu);
    st = refuse_if_capturing(stream);
    if (st != RED_OK) return st;
    Workspace w;
    st = new_workspace(stream, &w);
    if (st != RED_OK) return st;
    const auto key = std::make_pair(dev, stream);
    auto it = g_workspaces.find(key);
    if (it != g_workspaces.end()) {
        g_retired_workspaces.push_back(it->second);
        it->second = w;
    } else {
        g_workspaces.emplace(key, w);
    }
    // The column scratch starts over too: the next column call on the stream
    // allocates its own (a capture on the stream must warm it up first).
    auto sc = g_scratch.find(key);
    if (sc != g_scratch.end()) {
        if (sc->second.ptr != nullptr) g_retired_scratch.push_back(sc->second.ptr);
        g_scratch.erase(sc);
    }
    return RED_OK;
}

const char* red_status_string(red_status status) {
    switch (status) {
        case RED_OK: return "RED_OK";
        case RED_ERR_INVALID_ARG: return "RED_ERR_INVALID_ARG: bad pointer, length, shape or alignment";
        case RED_ERR_NO_DEVICE: return "RED_ERR_NO_DEVICE: no usable HIP device";
        case RED_ERR_HIP: return "RED_ERR_HIP: a HIP call or kernel launch failed";
        case RED_ERR_ALLOC: return "RED_ERR_ALLOC: workspace allocation failed";
        case RED_ERR_CAPTURE:
            return "RED_ERR_CAPTURE: the stream is being captured and its workspace is missing or too small";
        case RED_ERR_SCRATCH:
            return "RED_ERR_SCRATCH: the call needs more block partials than the fixed scratch array holds";
    }
    return "unknown red_status";
}

int red_last_hip_error(void) { return g_last_hip; }

const char* red_version(void) { return "libred 0.1.0 gfx950"; }

// ---------------------------------------------------------------- ablation

size_t red_ablate_num_partials(int rung, size_t n) {
    if (rung < 1 || rung > 5) return 0;
    const size_t epb = libred::rung_elems_per_block(rung);
    return (n + epb - 1) / epb;
}

red_status red_ablate_sum_f32(int rung, const float* x, size_t n, float* partials, size_t partials_cap,
                              float* out, hipStream_t stream) {
    if (rung == 6) return red_sum_f32(x, n, out, stream);
    if (rung < 1 || rung > 5) return RED_ERR_INVALID_ARG;
    if (n == 0 || n > ((size_t)1 << 31) || x == nullptr || partials == nullptr) return RED_ERR_INVALID_ARG;
    if (!aligned(x, 4) || !aligned(partials, 4) || !aligned(out, 4)) return RED_ERR_INVALID_ARG;
    const size_t np = red_ablate_num_partials(rung, n);
    if (partials_cap < np) return RED_ERR_INVALID_ARG;
    if (overlap(x, n * 4, partials, np * 4) || overlap(x, n * 4, out, out ? 4 : 0) ||
        overlap(partials, np * 4, out, out ? 4 : 0))
        return RED_ERR_INVALID_ARG;
    int dev;
    DeviceInfo info;
    const red_status st = current_device(&dev, &info);
    if (st != RED_OK) return st;
    const hipError_t e = libred::launch_rung(rung, x, n, partials, np, stream);
    if (e != hipSuccess) return fail(e, RED_ERR_HIP);
    if (out == nullptr) return RED_OK;
    // The partials are float32 values; their float64 sum, rounded once, is
    // exactly what red_sum_f32 computes over them.
    return red_sum_f32(partials, np, out, stream);
}

void red_default_flat_policy(size_t n, red_flat_policy* p) {
    if (!p) return;
    const FlatPolicy d = default_flat(n);
    p->block = d.block;
    p->blocks_per_cu = d.blocks_per_cu;
    p->unroll = d.unroll;
    p->nontemporal = d.nontemporal;
    p->layout = d.layout;
    p->prefetch = d.prefetch;
    p->combine = d.combine;
}

void red_default_rows_policy(red_rows_policy* p) {
    if (!p) return;
    p->block = kDefaultRows.block;
    p->unroll = kDefaultRows.unroll;
    p->nontemporal = kDefaultRows.nontemporal;
    p->max_blocks = kDefaultRows.max_blocks;
    p->split = kDefaultRows.split;
    p->prefetch = kDefaultRows.prefetch;
    p->short_rows = kDefaultRows.short_rows;
    p->cover = kDefaultRows.cover;
    p->defer = kDefaultRows.defer;
    p->lines = kDefaultRows.lines;
    p->xcd = kDefaultRows.xcd;
    p->max_fold = kDefaultRows.max_fold;
}

size_t red_flat_grid(size_t n, const red_flat_policy* pol) {
    const FlatPolicy p = to_flat(pol, n);
    if (!libred::flat_policy_supported(p)) return 0;
    int dev;
    DeviceInfo info;
    if (current_device(&dev, &info) != RED_OK) return 0;
    return flat_grid_for(n, p, info.cu_count);
}

red_status red_sum_f32_partials(const float* x, size_t n, double* partials, size_t partials_cap,
                                const red_flat_policy* pol, size_t* count, hipStream_t stream) {
    if (n > RED_MAX_N || (n > 0 && x == nullptr) || partials == nullptr || count == nullptr)
        return RED_ERR_INVALID_ARG;
    if (!aligned(x, sizeof(float)) || !aligned(partials, sizeof(double))) return RED_ERR_INVALID_ARG;
    const FlatPolicy p = to_flat(pol, n);
    if (!libred::flat_policy_supported(p)) return RED_ERR_INVALID_ARG;
    int dev;
    DeviceInfo info;
    const red_status st = current_device(&dev, &info);
    if (st != RED_OK) return st;
    const size_t grid = flat_grid_for(n, p, info.cu_count);
    if (partials_cap < grid || overlap(x, n * sizeof(float), partials, grid * sizeof(double)))
        return RED_ERR_INVALID_ARG;
    *count = grid;
    const hipError_t e = libred::launch_sum_f32_partials(x, n, partials, (int)grid, p, stream);
    if (e != hipSuccess) return fail(e, RED_ERR_HIP);
    return RED_OK;
}

red_status red_sum_f32_with(const float* x, size_t n, float* out, const red_flat_policy* p,
                            hipStream_t stream) {
    if (!p) return RED_ERR_INVALID_ARG;
    return flat_call(x, n, out, p, stream, libred::launch_sum_f32);
}

red_status red_sum_i32_i64_with(const int32_t* x, size_t n, int64_t* out, const red_flat_policy* p,
                                hipStream_t stream) {
    if (!p) return RED_ERR_INVALID_ARG;
    return flat_call(x, n, out, p, stream, libred::launch_sum_i32_i64);
}

red_status red_flat_with(int op, const void* x, size_t n, void* out, const red_flat_policy* p,
                         hipStream_t stream) {
    if (!p) return RED_ERR_INVALID_ARG;
    switch (op) {
        case RED_OP_SUM_F32:
            return flat_call(static_cast<const float*>(x), n, static_cast<float*>(out), p, stream,
                             libred::launch_sum_f32);
        case RED_OP_SUM_I32_I64:
            return flat_call(static_cast<const int32_t*>(x), n, static_cast<int64_t*>(out), p, stream,
                             libred::launch_sum_i32_i64);
        case RED_OP_MAX_F32:
            return flat_call(static_cast<const float*>(x), n, static_cast<float*>(out), p, stream,
                             libred::launch_max_f32);
        case RED_OP_MIN_F32:
            return flat_call(static_cast<const float*>(x), n, static_cast<float*>(out), p, stream,
                             libred::launch_min_f32);
        case RED_OP_ARGMAX_F32:
            return flat_call(static_cast<const float*>(x), n, static_cast<int64_t*>(out), p, stream,
                             libred::launch_argmax_f32);
        case RED_OP_ARGMIN_F32:
            return flat_call(static_cast<const float*>(x), n, static_cast<int64_t*>(out), p, stream,
                             libred::launch_argmin_f32);
        case RED_OP_SUM_BF16_F32:
            return flat_call(static_cast<const uint16_t*>(x), n, static_cast<float*>(out), p, stream,
                             libred::launch_sum_bf16);
        case RED_OP_SUM_F16_F32:
            return flat_call(static_cast<const uint16_t*>(x), n, static_cast<float*>(out), p, stream,
                             libred::launch_sum_f16);
        case RED_OP_SUM_F64:
            return flat_call(static_cast<const double*>(x), n, static_cast<double*>(out), p, stream,
                             libred::launch_sum_f64);
        case RED_OP_SUM_MAX_F32:
            return flat_call(static_cast<const float*>(x), n, static_cast<float*>(out), p, stream,
                             libred::launch_sum_max_f32, 3, true);
        default:
            return RED_ERR_INVALID_ARG;
    }
}

red_status red_sum_max_f32_with(const float* x, size_t n, float* out3, const red_flat_policy* p,
                                hipStream_t stream) {
    if (!p) return RED_ERR_INVALID_ARG;
    return flat_call(x, n, out3, p, stream, libred::launch_sum_max_f32, 3);
}

red_status red_max_f32_with(const float* x, size_t n, float* out, const red_flat_policy* p,
                            hipStream_t stream) {
    if (!p) return RED_ERR_INVALID_ARG;
    return flat_call(x, n, out, p, stream, libred::launch_max_f32);
}

red_status red_rows_sum_f32_with(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                                 const red_rows_policy* p, hipStream_t stream) {
    if (!p) return RED_ERR_INVALID_ARG;
    return rows_call(x, rows, cols, ld, out, p, stream, libred::launch_rows_sum_f32);
}

red_status red_rows_max_f32_with(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                                 const red_rows_policy* p, hipStream_t stream) {
    if (!p) return RED_ERR_INVALID_ARG;
    return rows_call(x, rows, cols, ld, out, p, stream, libred::launch_rows_max_f32);
}

void red_default_cols_policy(red_cols_policy* p) {
    if (!p) return;
    p->unroll = kDefaultCols.unroll;
    p->nontemporal = kDefaultCols.nontemporal;
    p->target_waves = kDefaultCols.target_waves;
    p->vec = kDefaultCols.vec;
    p->width = kDefaultCols.width;
    p->prefetch = kDefaultCols.prefetch;
    p->fold = kDefaultCols.fold;
    p->order = kDefaultCols.order;
    p->xcd = kDefaultCols.xcd;
}

red_status red_cols_sum_f32_with(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                                 const red_cols_policy* p, hipStream_t stream) {
    if (!p) return RED_ERR_INVALID_ARG;
    return cols_call(x, rows, cols, ld, out, p, stream, libred::launch_cols_sum_f32);
}

red_status red_cols_max_f32_with(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                                 const red_cols_policy* p, hipStream_t stream) {
    if (!p) return RED_ERR_INVALID_ARG;
    return cols_call(x, rows, cols, ld, out, p, stream, libred::launch_cols_max_f32);
}

// ---------------------------------------------------------------- probes

red_status red_probe_copy_f32(const float* x, float* y, size_t n, hipStream_t stream) {
    if (n > RED_MAX_N || (n > 0 && (x == nullptr || y == nullptr))) return RED_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(y, 16) || overlap(x, n * 4, y, n * 4)) return RED_ERR_INVALID_ARG;
    int dev;
    DeviceInfo info;
    const red_status st = current_device(&dev, &info);
    if (st != RED_OK) return st;
    if (n == 0) return RED_OK;
    size_t grid = (n / 4 + 255) / 256;
    const size_t cap = (size_t)8 * info.cu_count;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    const hipError_t e = libred::launch_copy_f32(x, y, n, (int)grid, stream);
    if (e != hipSuccess) return fail(e, RED_ERR_HIP);
    return RED_OK;
}

red_status red_probe_read_f32(const float* x, size_t n, unsigned int* sink, hipStream_t stream) {
    return flat_call(reinterpret_cast<const uint32_t*>(x), n, reinterpret_cast<uint32_t*>(sink), nullptr,
                     stream, libred::launch_xor_u32);
}

void red_default_read_shape(red_read_shape* s) {
    if (!s) return;
    *s = kDefaultReadShape;
}

red_status red_probe_read_ceiling(const void* x, size_t bytes, const red_read_shape* shape, unsigned int* sink,
                                  hipStream_t stream) {
    if (bytes > RED_MAX_N * 4 || bytes % 16 != 0 || (bytes > 0 && x == nullptr) || sink == nullptr)
        return RED_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(sink, 4) || overlap(x, bytes, sink, 4)) return RED_ERR_INVALID_ARG;
    const red_read_shape& r = shape ? *shape : kDefaultReadShape;
    const libred::ReadShape rs = {r.block, r.blocks_per_cu, r.unroll, r.nontemporal, r.layout};
    if (!libred::read_shape_supported(rs)) return RED_ERR_INVALID_ARG;
    int dev;
    DeviceInfo info;
    const red_status st = current_device(&dev, &info);
    if (st != RED_OK) return st;
    if (bytes == 0) return RED_OK;
    const int grid = rs.blocks_per_cu * info.cu_count;
    const hipError_t e = libred::launch_read_probe(x, bytes / 16, sink, grid, rs, stream);
    if (e != hipSuccess) return fail(e, RED_ERR_HIP);
    return RED_OK;
}

void red_default_copy_shape(red_read_shape* s) {
    if (!s) return;
    *s = kDefaultCopyShape;
}

red_status red_probe_copy_ceiling(const void* x, void* y, size_t bytes, const red_read_shape* shape,
                                  hipStream_t stream) {
    if (bytes > RED_MAX_N * 4 || bytes % 16 != 0 || (bytes > 0 && (x == nullptr || y == nullptr)))
        return RED_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(y, 16) || overlap(x, bytes, y, bytes)) return RED_ERR_INVALID_ARG;
    const red_read_shape& r = shape ? *shape : kDefaultCopyShape;
    const libred::ReadShape rs = {r.block, r.blocks_per_cu, r.unroll, r.nontemporal, r.layout};
    if (!libred::copy_shape_supported(rs)) return RED_ERR_INVALID_ARG;
    int dev;
    DeviceInfo info;
    const red_status st = current_device(&dev, &info);
    if (st != RED_OK) return st;
    if (bytes == 0) return RED_OK;
    const hipError_t e = libred::launch_copy_probe(x, y, bytes / 16, rs.blocks_per_cu * info.cu_count, rs, stream);
    if (e != hipSuccess) return fail(e, RED_ERR_HIP);
    return RED_OK;
}

red_status red_probe_fill_workspace(unsigned int word, hipStream_t stream) {
    int dev;
    DeviceInfo info;
    red_status st = current_device(&dev, &info);
    if (st != RED_OK) return st;
    Workspace ws;
    st = get_workspace(dev, stream, &ws);
    if (st != RED_OK) return st;
    std::lock_guard<std::mutex> lock(g_mu);
    st = refuse_if_capturing(stream);
    if (st != RED_OK) return st;
    // The partial slots only: the counter line stays zero.
    hipError_t e = libred::launch_fill_words(static_cast<unsigned int*>(ws.partials),
                                             kMaxPartials * libred::kMaxPartialBytes / 4, word, stream);
    if (e != hipSuccess) return fail(e, RED_ERR_HIP);
    auto sc = g_scratch.find(std::make_pair(dev, stream));
    if (sc != g_scratch.end() && sc->second.ptr != nullptr) {
        e = libred::launch_fill_words(static_cast<unsigned int*>(sc->second.ptr), sc->second.bytes / 4, word,
                                      stream);
        if (e != hipSuccess) return fail(e, RED_ERR_HIP);
    }
    return RED_OK;
}

red_status red_probe_lds_stride(int stride, int iters, unsigned int* sink, hipStream_t stream) {
    if (stride < -1 || stride > 1 << 20 || iters < 0 || iters > 1 << 24 || sink == nullptr ||
        !aligned(sink, 4))
        return RED_ERR_INVALID_ARG;
    int dev;
    DeviceInfo info;
    const red_status st = current_device(&dev, &info);
    if (st != RED_OK) return st;
    const hipError_t e = libred::launch_lds_stride(stride, iters, sink, stream);
    if (e != hipSuccess) return fail(e, RED_ERR_HIP);
    return RED_OK;
}

red_status red_probe_wave_reduce(int op, const void* in, size_t nwaves, void* out, hipStream_t stream) {
    const size_t esize = op == 2 ? 4 : 8;
    if (op < 0 || op > 2 || nwaves == 0 || nwaves > (1u << 20) || in == nullptr || out == nullptr)
        return RED_ERR_INVALID_ARG;
    if (!aligned(in, esize) || !aligned(out, esize) || overlap(in, nwaves * 64 * esize, out, nwaves * esize))
        return RED_ERR_INVALID_ARG;
    int dev;
    DeviceInfo info;
    const red_status st = current_device(&dev, &info);
    if (st != RED_OK) return st;
    const hipError_t e = libred::launch_wave_reduce_probe(op, in, nwaves, out, stream);
    if (e != hipSuccess) return fail(e, RED_ERR_HIP);
    return RED_OK;
}

red_status red_probe_shfl_down_f32(const float* in, int offset, float* out, hipStream_t stream) {
    if (in == nullptr || out == nullptr || offset < 0 || offset > 64 || !aligned(in, 4) || !aligned(out, 4) ||
        overlap(in, 256, out, 256))
        return RED_ERR_INVALID_ARG;
    int dev;
    DeviceInfo info;
    const red_status st = current_device(&dev, &info);
    if (st != RED_OK) return st;
    const hipError_t e = libred::launch_shfl_down_probe(in, offset, out, stream);
    if (e != hipSuccess) return fail(e, RED_ERR_HIP);
    return RED_OK;
}

red_status red_device_info(int* cu_count, char* arch, size_t arch_len) {
    if (cu_count == nullptr) return RED_ERR_INVALID_ARG;
    int dev;
    DeviceInfo info;
    const red_status st = current_device(&dev, &info);
    if (st != RED_OK) return st;
    *cu_count = info.cu_count;
    if (arch && arch_len) {
        strncpy(arch, info.arch, arch_len - 1);
        arch[arch_len - 1] = '\0';
    }
    return RED_OK;
}

}  // extern "C"
