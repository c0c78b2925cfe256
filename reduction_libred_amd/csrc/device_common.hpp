// device_common.hpp -- reduction operators, 16-byte loads and the wave64 /
// block combine steps shared by the libred kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace libred {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Reduction operators. Each names its element type, the 16-byte vector of four
// elements, the accumulator type, the output type, the identity, how an
// element enters the accumulator, the binary combine and the final rounding.
// ---------------------------------------------------------------------------

// Float32 sum, accumulated in float64 from the first addition: the f32 input
// widens exactly, and only the final store rounds to float.
struct SumF32 {
    using elem_t = float;
    using vec_t = f32x4;
    using acc_t = double;
    using out_t = float;
    static __device__ __forceinline__ acc_t identity() { return 0.0; }
    static __device__ __forceinline__ acc_t lift(elem_t v) { return (double)v; }
    static __device__ __forceinline__ acc_t combine(acc_t a, acc_t b) { return a + b; }
    static __device__ __forceinline__ out_t finish(acc_t a) { return (float)a; }
};

// Int32 sum into int64: every element is sign-extended before it is added.
struct SumI32 {
    using elem_t = int32_t;
    using vec_t = i32x4;
    using acc_t = int64_t;
    using out_t = int64_t;
    static __device__ __forceinline__ acc_t identity() { return 0; }
    static __device__ __forceinline__ acc_t lift(elem_t v) { return (int64_t)v; }
    static __device__ __forceinline__ acc_t combine(acc_t a, acc_t b) {
        // Wrap-around (two's complement) addition without signed overflow.
        return (int64_t)((uint64_t)a + (uint64_t)b);
    }
    static __device__ __forceinline__ out_t finish(acc_t a) { return a; }
};

// Float32 max: the running value b is replaced by a only if a > b, so a NaN
// never enters and the identity -inf survives an all-NaN input.
struct MaxF32 {
    using elem_t = float;
    using vec_t = f32x4;
    using acc_t = float;
    using out_t = float;
    static __device__ __forceinline__ acc_t identity() { return -__builtin_inff(); }
    static __device__ __forceinline__ acc_t lift(elem_t v) { return v; }
    static __device__ __forceinline__ acc_t combine(acc_t a, acc_t b) { return (b > a) ? b : a; }
    static __device__ __forceinline__ out_t finish(acc_t a) { return a; }
};

// Fused float32 sum, max and sum of magnitudes in one pass: a float64 sum
// and a float64 sum of |x| (each rounded once at the end) and the max under
// the strictly-greater rule. NaN and infinities follow IEEE arithmetic in the
// two sums.
struct SumMaxAbs {
    double s;
    double a;
    float m;
    float pad;
};
struct SumMaxAbsOut {
    float s;
    float m;
    float a;
};
struct SumMaxAbsF32 {
    using elem_t = float;
    using vec_t = f32x4;
    using acc_t = SumMaxAbs;
    using out_t = SumMaxAbsOut;
    static __device__ __forceinline__ acc_t identity() { return {0.0, 0.0, -__builtin_inff(), 0.0f}; }
    static __device__ __forceinline__ acc_t lift(elem_t v) {
        const double d = (double)v;
        return {d, __builtin_fabs(d), v, 0.0f};
    }
    static __device__ __forceinline__ acc_t combine(acc_t x, acc_t y) {
        return {x.s + y.s, x.a + y.a, (y.m > x.m) ? y.m : x.m, 0.0f};
    }
    static __device__ __forceinline__ out_t finish(acc_t x) { return {(float)x.s, x.m, (float)x.a}; }
};

// Read probe: xor of every 32-bit word. One cheap ALU op per element, so a
// kernel built on it measures the load path alone.
struct XorU32 {
    using elem_t = uint32_t;
    using vec_t = uint32_t __attribute__((ext_vector_type(4)));
    using acc_t = uint32_t;
    using out_t = uint32_t;
    static __device__ __forceinline__ acc_t identity() { return 0u; }
    static __device__ __forceinline__ acc_t lift(elem_t v) { return v; }
    static __device__ __forceinline__ acc_t combine(acc_t a, acc_t b) { return a ^ b; }
    static __device__ __forceinline__ out_t finish(acc_t a) { return a; }
};

// ---------------------------------------------------------------------------
// Loads
// ---------------------------------------------------------------------------
template <bool NT, class V>
__device__ __forceinline__ V load_vec(const V* p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);  // streaming hint: do not keep in cache
    else
        return *p;
}

template <class Op>
__device__ __forceinline__ void accumulate4(typename Op::acc_t (&acc)[4], typename Op::vec_t v) {
    acc[0] = Op::combine(acc[0], Op::lift(v.x));
    acc[1] = Op::combine(acc[1], Op::lift(v.y));
    acc[2] = Op::combine(acc[2], Op::lift(v.z));
    acc[3] = Op::combine(acc[3], Op::lift(v.w));
}

// ---------------------------------------------------------------------------
// Wave reduce 64 -> 1 with DPP cross-lane moves.
//
// Six combine steps, each pairing a lane with one chosen by a DPP pattern:
//   quad_perm [1,0,3,2] and [2,3,0,1]: every lane of a quad holds its quad's total
//   row_half_mirror: every lane of an 8-lane half row holds the half row's total
//   row_mirror:      every lane of a 16-lane row holds the row's total
//   row_bcast:15 into rows 1 and 3: those rows hold rows 0+1 and 2+3
//   row_bcast:31 into rows 2 and 3: row 3 holds the wave total
// Lanes a masked step does not write receive the identity, so combining
// leaves them unchanged. The total is read from lane 63. The pairing order is
// fixed, so the result is deterministic. All 64 lanes must be active.
// ---------------------------------------------------------------------------
// Cross-lane moves act on 32-bit words: a 64-bit value is moved as its two
// halves, a struct word by word. (The compiler builtins convert a non-int
// argument or result by value, which would truncate a double, so every value
// is bit-cast.)
template <class T>
struct Words {
    static_assert(sizeof(T) % 4 == 0, "values must be whole 32-bit words");
    static constexpr int n = sizeof(T) / 4;
    int w[n];
};

template <int CTRL, int ROW_MASK, class T>
__device__ __forceinline__ T dpp_move(T old, T src) {
    Words<T> o = __builtin_bit_cast(Words<T>, old);
    Words<T> s = __builtin_bit_cast(Words<T>, src);
#pragma unroll
    for (int k = 0; k < Words<T>::n; ++k)
        s.w[k] = __builtin_amdgcn_update_dpp(o.w[k], s.w[k], CTRL, ROW_MASK, 0xF, false);
    return __builtin_bit_cast(T, s);
}

template <class T>
__device__ __forceinline__ T read_lane(T v, int lane) {
    Words<T> s = __builtin_bit_cast(Words<T>, v);
#pragma unroll
    for (int k = 0; k < Words<T>::n; ++k) s.w[k] = __builtin_amdgcn_readlane(s.w[k], lane);
    return __builtin_bit_cast(T, s);
}

template <class Op>
__device__ __forceinline__ typename Op::acc_t wave_reduce(typename Op::acc_t v) {
    using T = typename Op::acc_t;
    const T id = Op::identity();
    v = Op::combine(v, dpp_move<0xB1, 0xF>(id, v));   // quad_perm:[1,0,3,2]
    v = Op::combine(v, dpp_move<0x4E, 0xF>(id, v));   // quad_perm:[2,3,0,1]
    v = Op::combine(v, dpp_move<0x141, 0xF>(id, v));  // row_half_mirror
    v = Op::combine(v, dpp_move<0x140, 0xF>(id, v));  // row_mirror
    v = Op::combine(v, dpp_move<0x142, 0xA>(id, v));  // row_bcast:15 -> rows 1, 3
    v = Op::combine(v, dpp_move<0x143, 0xC>(id, v));  // row_bcast:31 -> rows 2, 3
    return read_lane(v, 63);
}

// ---------------------------------------------------------------------------
// Block reduce: wave totals go to LDS (one word per wave, consecutive, so no
// bank conflicts), one barrier, then wave 0 reduces them. The result is valid
// in wave 0. `lds` needs BLOCK / 64 entries. A caller that reuses `lds` must
// put a barrier between the previous read of it and this call.
// ---------------------------------------------------------------------------
template <class Op, int BLOCK>
__device__ __forceinline__ typename Op::acc_t block_reduce(typename Op::acc_t v,
                                                           typename Op::acc_t* lds) {
    constexpr int W = BLOCK / kWave;
    v = wave_reduce<Op>(v);
    if constexpr (W == 1) {
        return v;
    } else {
        const int lane = threadIdx.x % kWave;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
        if (lane == 0) lds[wave] = v;
        __syncthreads();
        if (wave == 0) {
            v = lane < W ? lds[lane] : Op::identity();
            v = wave_reduce<Op>(v);
        }
        return v;
    }
}

// Head length for a 16-byte aligned vector body: the number of elements of
// size `esize` before the first 16-byte boundary at or after p, capped at n.
__device__ __forceinline__ size_t head_elems(const void* p, size_t esize, size_t n) {
    const size_t mis = (size_t)(uintptr_t)p & 15u;
    const size_t h = mis ? (16u - mis) / esize : 0;
    return h < n ? h : n;
}

}  // namespace libred
