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

// ---------------------------------------------------------------------------
// Reduction operators. Each names its element type, the 16-byte vector and
// how many elements it holds (kPerVec), the accumulator type, the output type,
// the identity, how element number i enters the accumulator (lift), the
// binary combine and the final rounding (finish). An operator may also
// bring its own streaming fold of a vector (fold) or of a whole tile
// (kTileFold: fold_tile, then resolve after the stream).
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

// Float32 min: the mirror of MaxF32 (strictly smaller wins, from +inf).
struct MinF32 {
    using elem_t = float;
    using vec_t = f32x4;
    using acc_t = float;
    using out_t = float;
    static constexpr int kPerVec = 4;
    static __device__ __forceinline__ acc_t identity() { return __builtin_inff(); }
    static __device__ __forceinline__ acc_t lift(elem_t v, size_t) { return v; }
    static __device__ __forceinline__ acc_t combine(acc_t a, acc_t b) { return (b < a) ? b : a; }
    static __device__ __forceinline__ out_t finish(acc_t a) { return a; }
};

// Index of the max (MAX) or min of float32 values: the lowest index of the
// extreme among non-NaN elements, -1 if there is none. A candidate is a
// (value, index) pair; index -1, with value NaN, is "none". The full combine
// is a total order on candidates (better value, then lower index), so any
// grouping of the elements gives the same answer.
//
// Streaming. Each thread meets its elements in increasing index order, and a
// later candidate replaces an earlier one only when it is strictly better, so
// the first occurrence of a thread's extreme is what survives:
//  - a whole tile of UNROLL vectors is reduced to its extreme value alone
//    (fmaxf / fminf, which skip NaN), and acc[3] keeps the best tile value
//    with the tile's first element index (fold_tile);
//  - after the stream, resolve() reads that one tile again and finds its
//    first element equal to the kept value, making acc[3] exact;
//  - vectors outside whole tiles find their exact index at once (fold, into
//    acc[0]).
// The streaming loop thus costs about two vector operations per element and
// never selects a 64-bit index per element; the second read is one tile per
// thread.
struct ArgExt {
    float v;
    int32_t unused;
    int64_t idx;
};
template <bool MAX>
struct ArgExtF32 {
    using elem_t = float;
    using vec_t = f32x4;
    using acc_t = ArgExt;
    using out_t = int64_t;
    static constexpr int kPerVec = 4;
    static constexpr bool kTileFold = true;
    static __device__ __forceinline__ bool better(float a, float b) { return MAX ? (a > b) : (a < b); }
    // The extreme of two values; a NaN operand is ignored (NaN only if both are).
    static __device__ __forceinline__ float ext(float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); }
    static __device__ __forceinline__ float ext4(vec_t v) { return ext(ext(v[0], v[1]), ext(v[2], v[3])); }
    // Does extreme e (NaN: no number) replace the running value m (NaN: none)?
    static __device__ __forceinline__ bool replaces(float e, float m) {
        return (MAX ? !(e <= m) : !(e >= m)) & (e == e);
    }
    static __device__ __forceinline__ acc_t identity() { return {__builtin_nanf(""), 0, -1}; }
    static __device__ __forceinline__ acc_t lift(elem_t v, size_t i) {
        return (v != v) ? identity() : acc_t{v, 0, (int64_t)i};
    }
    static __device__ __forceinline__ acc_t combine(acc_t a, acc_t b) {
        if (b.idx < 0) return a;
        if (a.idx < 0) return b;
        return (better(b.v, a.v) || (b.v == a.v && b.idx < a.idx)) ? b : a;
    }
    static __device__ __forceinline__ out_t finish(acc_t a) { return a.idx; }

    // One vector whose first element is number i0, into acc[0].
    static __device__ __forceinline__ void fold(acc_t (&acc)[4], vec_t v, size_t i0) {
        const float e = ext4(v);
        int pos = 3;
        pos = v[2] == e ? 2 : pos;
        pos = v[1] == e ? 1 : pos;
        pos = v[0] == e ? 0 : pos;
        const bool take = replaces(e, acc[0].v);
        acc[0].v = take ? e : acc[0].v;
        acc[0].idx = take ? (int64_t)(i0 + pos) : acc[0].idx;
    }

    // A tile: vector u starts at element i0 + u * 64 * kPerVec. Into acc[3].
    template <int UNROLL>
    static __device__ __forceinline__ void fold_tile(acc_t (&acc)[4], const vec_t (&v)[UNROLL], size_t i0) {
        float e = ext4(v[0]);
#pragma unroll
        for (int u = 1; u < UNROLL; ++u) e = ext(e, ext4(v[u]));
        const bool take = replaces(e, acc[3].v);
        acc[3].v = take ? e : acc[3].v;
        acc[3].idx = take ? (int64_t)i0 : acc[3].idx;
    }

    // Turn acc[3]'s tile into the index of its first element equal to the
    // kept value, re-reading the tile from x (the start of the whole array).
    // The value was produced by ext() from one of those elements, so the
    // match compares ext(e, e), the form in which ext saw e.
    template <int UNROLL, bool NT>
    static __device__ __forceinline__ void resolve(acc_t (&acc)[4], const elem_t* __restrict__ x) {
        acc_t& a = acc[3];
        if (a.idx < 0) return;
        const vec_t* __restrict__ p = reinterpret_cast<const vec_t*>(x + a.idx);
        vec_t v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = load_vec<NT>(p + u * kWave);
        int pos = 0;
#pragma unroll
        for (int u = UNROLL - 1; u >= 0; --u)
#pragma unroll
            for (int k = 3; k >= 0; --k) pos = ext(v[u][k], v[u][k]) == a.v ? u * kWave * kPerVec + k : pos;
        a.idx += pos;
    }
};
using ArgMaxF32 = ArgExtF32<true>;
using ArgMinF32 = ArgExtF32<false>;

// Sums of 16-bit floats given as bit patterns, widened exactly to float and
// then to float64; eight elements per 16-byte vector.
struct SumBF16 {
    using elem_t = uint16_t;
    using vec_t = u16x8;
    using acc_t = double;
    using out_t = float;
    static constexpr int kPerVec = 8;
    static __device__ __forceinline__ acc_t identity() { return 0.0; }
    static __device__ __forceinline__ acc_t lift(elem_t v, size_t) {
        return (double)__builtin_bit_cast(float, (uint32_t)v << 16);  // bfloat16 = float's upper half
    }
    static __device__ __forceinline__ acc_t combine(acc_t a, acc_t b) { return a + b; }
    static __device__ __forceinline__ out_t finish(acc_t a) { return (float)a; }
};
struct SumF16 {
    using elem_t = uint16_t;
    using vec_t = u16x8;
    using acc_t = double;
    using out_t = float;
    static constexpr int kPerVec = 8;
    static __device__ __forceinline__ acc_t identity() { return 0.0; }
    static __device__ __forceinline__ acc_t lift(elem_t v, size_t) {
        return (double)(float)__builtin_bit_cast(_Float16, v);
    }
    static __device__ __forceinline__ acc_t combine(acc_t a, acc_t b) { return a + b; }
    static __device__ __forceinline__ out_t finish(acc_t a) { return (float)a; }
};

// Float64 sum in float64; two elements per 16-byte vector.
struct SumF64 {
    using elem_t = double;
    using vec_t = f64x2;
    using acc_t = double;
    using out_t = double;
    static constexpr int kPerVec = 2;
    static __device__ __forceinline__ acc_t identity() { return 0.0; }
    static __device__ __forceinline__ acc_t lift(elem_t v, size_t) { return v; }
    static __device__ __forceinline__ acc_t combine(acc_t a, acc_t b) { return a + b; }
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
    static constexpr int kPerVec = 4;
    static __device__ __forceinline__ acc_t identity() { return {0.0, 0.0, -__builtin_inff(), 0.0f}; }
    static __device__ __forceinline__ acc_t lift(elem_t v, size_t) {
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
    using vec_t = u32x4;
    using acc_t = uint32_t;
    using out_t = uint32_t;
    static constexpr int kPerVec = 4;
    static __device__ __forceinline__ acc_t identity() { return 0u; }
    static __device__ __forceinline__ acc_t lift(elem_t v, size_t) { return v; }
    static __device__ __forceinline__ acc_t combine(acc_t a, acc_t b) { return a ^ b; }
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
