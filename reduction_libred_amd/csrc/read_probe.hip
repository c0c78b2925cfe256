// read_probe.hip -- a load-only streaming kernel that measures how fast this
// device reads HBM, the achievable counterpart of the simulator page's memory
// bound ("simt_lab.py", section 6, estimate_time: time = bytes / bandwidth),
// and a copy kernel of the same layout that measures reads and writes
// together.
//
// Each lane issues 16-byte loads and folds every 32-bit word into one xor
// (one VALU op per word, far below what the loads take), so the result is
// checkable and no load can be dropped. The launch shape is free: block
// size, blocks per compute unit, loads in flight per lane, the non-temporal
// hint, and the access layout, so that a sweep can find the fastest way this
// device streams a buffer. Section 7 of the same page (latency_hiding)
// sizes the bytes in flight that need: bandwidth per CU times latency.
//
// Layouts:
//   0 grid-stride: thread i of the grid reads vectors i, i + G*T, ...
//     (UNROLL per loop trip), a wave-wide load covering 1 KiB;
//   1 wave tiles: the buffer is cut into tiles of 64 * UNROLL vectors; wave
//     w reads tiles w, w + nwaves, ... whole;
//   2 wave tiles with the next tile's loads issued before the current tile
//     is folded (two register buffers);
//   3 as 2, but each XCD reads one contiguous eighth of the tiles: blocks
//     are dispatched to the eight XCDs round robin (block b on XCD b mod 8),
//     so the blocks b = x mod 8 take tiles [x T / 8, (x + 1) T / 8) of the T
//     tiles, their waves round robin.
#include "device_common.hpp"
#include "launch.hpp"

namespace libred {

namespace {

__device__ __forceinline__ uint32_t xor4(u32x4 v) { return (v.x ^ v.y) ^ (v.z ^ v.w); }

template <int UNROLL, bool NT>
__device__ __forceinline__ void read_tile(u32x4 (&v)[UNROLL], const u32x4* __restrict__ p) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = load_vec<NT>(p + u * kWave);
}

template <int UNROLL>
__device__ __forceinline__ uint32_t fold_tile_xor(const u32x4 (&v)[UNROLL]) {
    uint32_t a = 0;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) a ^= xor4(v[u]);
    return a;
}

template <int BLOCK, int UNROLL, bool NT, int LAYOUT>
__global__ __launch_bounds__(BLOCK) void read_probe_kernel(const u32x4* __restrict__ xv, size_t nvec,
                                                           unsigned int* __restrict__ sink) {
    uint32_t acc = 0;
    const int lane = threadIdx.x % kWave;
    if constexpr (LAYOUT == 0) {
        const size_t stride = (size_t)gridDim.x * BLOCK;
        size_t i = (size_t)blockIdx.x * BLOCK + threadIdx.x;
        for (; i + (size_t)(UNROLL - 1) * stride < nvec; i += (size_t)UNROLL * stride) {
            u32x4 v[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) v[u] = load_vec<NT>(xv + i + (size_t)u * stride);
            acc ^= fold_tile_xor<UNROLL>(v);
        }
        for (; i < nvec; i += stride) acc ^= xor4(load_vec<NT>(xv + i));
    } else {
        constexpr int W = BLOCK / kWave;
        constexpr size_t TILE = (size_t)kWave * UNROLL;
        const size_t wave = (size_t)__builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
        const size_t nwaves = (size_t)gridDim.x * W;
        const size_t ntiles = nvec / TILE;
        size_t t = (size_t)blockIdx.x * W + wave;
        // Tiles t, t + step, ... below t1.
        size_t t1 = ntiles, step = nwaves;
        if constexpr (LAYOUT == 3) {
            const size_t G = gridDim.x, xcd = blockIdx.x % 8;
            const size_t xblocks = (G + 7 - xcd) / 8;  // blocks on this XCD
            t = xcd * ntiles / 8 + (blockIdx.x / 8) * W + wave;
            t1 = (xcd + 1) * ntiles / 8;
            step = xblocks * W;
        }
        if constexpr (LAYOUT == 1) {
            for (; t < t1; t += step) {
                u32x4 v[UNROLL];
                read_tile<UNROLL, NT>(v, xv + t * TILE + lane);
                acc ^= fold_tile_xor<UNROLL>(v);
            }
        } else if (t < t1) {
            u32x4 a[UNROLL], b[UNROLL];
            read_tile<UNROLL, NT>(a, xv + t * TILE + lane);
            while (true) {
                if (t + step >= t1) {
                    acc ^= fold_tile_xor<UNROLL>(a);
                    break;
                }
                read_tile<UNROLL, NT>(b, xv + (t + step) * TILE + lane);
                acc ^= fold_tile_xor<UNROLL>(a);
                t += step;
                if (t + step >= t1) {
                    acc ^= fold_tile_xor<UNROLL>(b);
                    break;
                }
                read_tile<UNROLL, NT>(a, xv + (t + step) * TILE + lane);
                acc ^= fold_tile_xor<UNROLL>(b);
                t += step;
            }
        }
        // Vectors after the last whole tile.
        const size_t w = (size_t)blockIdx.x * W + wave;
        for (size_t i = ntiles * TILE + w * kWave + lane; i < nvec; i += nwaves * kWave)
            acc ^= xor4(load_vec<NT>(xv + i));
    }
    // Xor across the wave, then one atomic per wave (xor is order-free).
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, kWave);
    if (lane == 0) atomicXor(sink, acc);
}

// Shapes whose registers fit without spilling: 1024-thread blocks (four
// waves per SIMD, 128 VGPRs each) take at most 16 loads per lane, 8 with the
// second register buffer.
template <int BLOCK, int UNROLL, int LAYOUT>
constexpr bool rp_fits() {
    return BLOCK < 1024 || (LAYOUT >= 2 ? UNROLL <= 8 : UNROLL <= 16);
}

template <int BLOCK, int UNROLL, int LAYOUT>
hipError_t launch_rp(const u32x4* xv, size_t nvec, unsigned int* sink, int grid, bool nt, hipStream_t stream) {
    if constexpr (!rp_fits<BLOCK, UNROLL, LAYOUT>()) {
        return hipErrorInvalidValue;
    } else {
        if (nt)
            hipLaunchKernelGGL((read_probe_kernel<BLOCK, UNROLL, true, LAYOUT>), dim3(grid), dim3(BLOCK), 0,
                               stream, xv, nvec, sink);
        else
            hipLaunchKernelGGL((read_probe_kernel<BLOCK, UNROLL, false, LAYOUT>), dim3(grid), dim3(BLOCK), 0,
                               stream, xv, nvec, sink);
        return hipGetLastError();
    }
}

template <int BLOCK, int LAYOUT>
hipError_t launch_rp_u(const u32x4* xv, size_t nvec, unsigned int* sink, int grid, const ReadShape& s,
                       hipStream_t stream) {
    switch (s.unroll) {
        case 4: return launch_rp<BLOCK, 4, LAYOUT>(xv, nvec, sink, grid, s.nontemporal != 0, stream);
        case 8: return launch_rp<BLOCK, 8, LAYOUT>(xv, nvec, sink, grid, s.nontemporal != 0, stream);
        case 16: return launch_rp<BLOCK, 16, LAYOUT>(xv, nvec, sink, grid, s.nontemporal != 0, stream);
        case 32: return launch_rp<BLOCK, 32, LAYOUT>(xv, nvec, sink, grid, s.nontemporal != 0, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int BLOCK>
hipError_t launch_rp_b(const u32x4* xv, size_t nvec, unsigned int* sink, int grid, const ReadShape& s,
                       hipStream_t stream) {
    switch (s.layout) {
        case 0: return launch_rp_u<BLOCK, 0>(xv, nvec, sink, grid, s, stream);
        case 1: return launch_rp_u<BLOCK, 1>(xv, nvec, sink, grid, s, stream);
        case 2: return launch_rp_u<BLOCK, 2>(xv, nvec, sink, grid, s, stream);
        case 3: return launch_rp_u<BLOCK, 3>(xv, nvec, sink, grid, s, stream);
        default: return hipErrorInvalidValue;
    }
}

// Copy ceiling: y = x with the read probe's fastest layout (single-wave
// blocks, wave tiles of UNROLL 16-byte loads per lane, the next tile's loads
// in flight while the current one is stored). NT marks both the loads and
// the stores non-temporal.
template <int UNROLL, bool NT>
__global__ __launch_bounds__(kWave) void copy_probe_kernel(const u32x4* __restrict__ xv, u32x4* __restrict__ yv,
                                                           size_t nvec) {
    constexpr size_t TILE = (size_t)kWave * UNROLL;
    const int lane = threadIdx.x;
    const size_t G = gridDim.x;
    const size_t ntiles = nvec / TILE;
    auto load = [&](u32x4 (&v)[UNROLL], size_t t) { read_tile<UNROLL, NT>(v, xv + t * TILE + lane); };
    auto store = [&](const u32x4 (&v)[UNROLL], size_t t) {
        u32x4* __restrict__ p = yv + t * TILE + lane;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            if constexpr (NT)
                __builtin_nontemporal_store(v[u], p + u * kWave);
            else
                p[u * kWave] = v[u];
        }
    };
    size_t t = blockIdx.x;
    if (t < ntiles) {
        size_t n = (ntiles - t + G - 1) / G;
        u32x4 a[UNROLL], b[UNROLL];
        load(a, t);
        for (; n > 2; n -= 2, t += 2 * G) {
            load(b, t + G);
            store(a, t);
            load(a, t + 2 * G);
            store(b, t + G);
        }
        if (n == 2) {
            load(b, t + G);
            store(a, t);
            store(b, t + G);
        } else {
            store(a, t);
        }
    }
    // Vectors after the last whole tile.
    for (size_t i = ntiles * TILE + (size_t)blockIdx.x * kWave + lane; i < nvec; i += G * kWave) yv[i] = xv[i];
}

template <int UNROLL>
hipError_t launch_cp(const u32x4* xv, u32x4* yv, size_t nvec, int grid, bool nt, hipStream_t stream) {
    if (nt)
        hipLaunchKernelGGL((copy_probe_kernel<UNROLL, true>), dim3(grid), dim3(kWave), 0, stream, xv, yv, nvec);
    else
        hipLaunchKernelGGL((copy_probe_kernel<UNROLL, false>), dim3(grid), dim3(kWave), 0, stream, xv, yv, nvec);
    return hipGetLastError();
}

}  // namespace

bool copy_shape_supported(const ReadShape& s) {
    return s.block == 64 && s.layout == 2 && (s.unroll == 4 || s.unroll == 8 || s.unroll == 16) &&
           s.blocks_per_cu >= 1 && s.blocks_per_cu <= 32 && (s.nontemporal == 0 || s.nontemporal == 1);
}

hipError_t launch_copy_probe(const void* x, void* y, size_t nvec, int grid, const ReadShape& s, hipStream_t stream) {
    const u32x4* xv = static_cast<const u32x4*>(x);
    u32x4* yv = static_cast<u32x4*>(y);
    const bool nt = s.nontemporal != 0;
    switch (s.unroll) {
        case 4: return launch_cp<4>(xv, yv, nvec, grid, nt, stream);
        case 8: return launch_cp<8>(xv, yv, nvec, grid, nt, stream);
        case 16: return launch_cp<16>(xv, yv, nvec, grid, nt, stream);
        default: return hipErrorInvalidValue;
    }
}

bool read_shape_supported(const ReadShape& s) {
    const bool block = s.block == 64 || s.block == 256 || s.block == 1024;
    const bool unroll = s.unroll == 4 || s.unroll == 8 || s.unroll == 16 || s.unroll == 32;
    const bool fits = s.block < 1024 || (s.layout >= 2 ? s.unroll <= 8 : s.unroll <= 16);
    return block && unroll && fits && s.layout >= 0 && s.layout <= 3 && s.blocks_per_cu >= 1 &&
           s.blocks_per_cu <= 32 && (s.nontemporal == 0 || s.nontemporal == 1);
}

hipError_t launch_read_probe(const void* x, size_t nvec, unsigned int* sink, int grid, const ReadShape& s,
                             hipStream_t stream) {
    const u32x4* xv = static_cast<const u32x4*>(x);
    switch (s.block) {
        case 64: return launch_rp_b<64>(xv, nvec, sink, grid, s, stream);
        case 256: return launch_rp_b<256>(xv, nvec, sink, grid, s, stream);
        case 1024: return launch_rp_b<1024>(xv, nvec, sink, grid, s, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace libred
