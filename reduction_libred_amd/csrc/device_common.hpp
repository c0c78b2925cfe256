// device_common.hpp -- reduction operators, 16-byte loads and the wave64 /
// block combine steps shared by the libred kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace libred {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

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

template <bool NT, class V>
__device__ __forceinline__ void store_vec(V* p, V v) {
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);  // streaming hint: do not keep in cache
    else
        *p = v;
}

// ---------------------------------------------------------------------------
// Reduction operators. Each names its element type, the 16-byte vector and
// how many elements it holds (kPerVec), the accumulator type, the output type,
// the identity, how element number i enters the accumulator (lift), the
// binary combine and the final rounding (finish). An operator may also
// bring its own streaming fold of a vector (fold) or of a whole tile
// (kTileFold: fold_tile), and a step that completes its accumulators after
// the stream (kResolve: resolve).
// ---------------------------------------------------------------------------

// Float32 sum, accumulated in float64 from the first addition: the f32 input
// widens exactly, and only the final store rounds to float.
struct SumF32 {
    using elem_t = float;
    using vec_t = f32x4;
    using acc_t = double;
    using out_t = float;
    static constexpr int kPerVec = 4;
    static __device__ __forceinline__ acc_t identity() { return 0.0; }
    static __device__ __forceinline__ acc_t lift(elem_t v, size_t) { return (double)v; }
    static __device__ __forceinline__ acc_t combine(acc_t a, acc_t b) { return a + b; }
    static __device__ __forceinline__ out_t finish(acc_t a) { return (float)a; }
};

// Int32 sum into int64: every element is sign-extended before it is added.
struct SumI32 {
    using elem_t = int32_t;
    using vec_t = i32x4;
    using acc_t = int64_t;
    using out_t = int64_t;
    static constexpr int kPerVec = 4;
    static __device__ __forceinline__ acc_t identity() { return 0; }
    static __device__ __forceinline__ acc_t lift(elem_t v, size_t) { return (int64_t)v; }
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
    static constexpr int kPerVec = 4;
    static __device__ __forceinline__ acc_t identity() { return -__builtin_inff(); }
    static __device__ __forceinline__ acc_t lift(elem_t v, size_t) { return v; }
    static __device__ __forceinline__ acc_t combine(acc_t a, acc_t b) { return (b > a) ? b : a; }
    static __device__ __forceinline__ out_t finish(acc_t a) { return a; }
};

// Fold the kPerVec elements of one 16-byte vector, the first of which is
// element number i0, into four accumulators (element k into acc[k % 4]), or
// with the operator's own fold when it has one. Callers hand each thread's
// vectors over in increasing index order.
template <class Op, class = void>
struct HasFold : std::false_type {};
template <class Op>
struct HasFold<Op, std::void_t<decltype(&Op::fold)>> : std::true_type {};

template <class Op, class = void>
struct HasTileFold : std::false_type {};
template <class Op>
struct HasTileFold<Op, std::void_t<decltype(Op::kTileFold)>> : std::true_type {};
template <class Op, class = void>
struct HasResolve : std::false_type {};
template <class Op>
struct HasResolve<Op, std::void_t<decltype(Op::kResolve)>> : std::true_type {};

template <class Op>
__device__ __forceinline__ void fold_vec(typename Op::acc_t (&acc)[4], typename Op::vec_t v, size_t i0) {
    if constexpr (HasFold<Op>::value) {
        Op::fold(acc, v, i0);
    } else {
#pragma unroll
        for (int k = 0; k < Op::kPerVec; ++k) acc[k & 3] = Op::combine(acc[k & 3], Op::lift(v[k], i0 + k));
    }
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
