// ops_ext.hpp -- the reduction operators beyond float32 sum, int32 sum and
// float32 max: min, argmax / argmin, 16-bit float sums, float64 sum, the fused
// sum / max / sum of magnitudes, and the xor used by the read-bandwidth probe.
// Each has the members the kernels expect of an operator (see
// device_common.hpp).
#pragma once

#include "device_common.hpp"

namespace libred {

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
//  - a whole tile of UNROLL vectors is reduced to its extreme value and the
//    first of its vectors that holds it (fmaxf / fminf, which skip NaN), and
//    acc[3] keeps the best tile value with that vector's first element index
//    (fold_tile);
//  - after the stream, resolve() reads that one vector again and finds its
//    first element equal to the kept value, making acc[3] exact;
//  - vectors outside whole tiles find their exact index at once (fold, into
//    acc[0]).
// The streaming loop thus costs about two and a half vector operations per
// element and never selects a 64-bit index per element; the second read is
// one 16-byte vector per thread.
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
    static constexpr bool kResolve = true;
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

    // A tile: vector u starts at element i0 + u * 64 * kPerVec. Into acc[3],
    // which keeps the first element number of the first vector of the tile
    // that holds the tile's extreme.
    template <int UNROLL>
    static __device__ __forceinline__ void fold_tile(acc_t (&acc)[4], const vec_t (&v)[UNROLL], size_t i0) {
        float vm[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) vm[u] = ext4(v[u]);
        float e = vm[0];
#pragma unroll
        for (int u = 1; u < UNROLL; ++u) e = ext(e, vm[u]);
        int first = UNROLL - 1;
#pragma unroll
        for (int u = UNROLL - 2; u >= 0; --u) first = vm[u] == e ? u : first;
        const bool take = replaces(e, acc[3].v);
        acc[3].v = take ? e : acc[3].v;
        acc[3].idx = take ? (int64_t)(i0 + (size_t)first * kWave * kPerVec) : acc[3].idx;
    }

    // Turn acc[3]'s vector into the index of its first element equal to the
    // kept value, re-reading that one vector from x (the start of the whole
    // array). The value was produced by ext() from one of those elements, so
    // the match compares ext(e, e), the form in which ext saw e.
    template <int UNROLL, bool NT>
    static __device__ __forceinline__ void resolve(acc_t (&acc)[4], const elem_t* __restrict__ x) {
        acc_t& a = acc[3];
        if (a.idx < 0) return;
        const vec_t v = load_vec<NT>(reinterpret_cast<const vec_t*>(x + a.idx));
        int pos = 3;
#pragma unroll
        for (int k = 2; k >= 0; --k) pos = ext(v[k], v[k]) == a.v ? k : pos;
        a.idx += pos;
    }
};
using ArgMaxF32 = ArgExtF32<true>;
using ArgMinF32 = ArgExtF32<false>;

// Sums of 16-bit floats given as bit patterns, widened exactly to float;
// eight elements per 16-byte vector.
struct SumBF16 {
    using elem_t = uint16_t;
    using vec_t = u16x8;
    using acc_t = double;
    using out_t = float;
    static constexpr int kPerVec = 8;
    static __device__ __forceinline__ float widen(elem_t v) {
        return __builtin_bit_cast(float, (uint32_t)v << 16);  // bfloat16 = float's upper half
    }
    static __device__ __forceinline__ acc_t identity() { return 0.0; }
    static __device__ __forceinline__ acc_t lift(elem_t v, size_t) { return (double)widen(v); }
    static __device__ __forceinline__ acc_t combine(acc_t a, acc_t b) { return a + b; }
    static __device__ __forceinline__ out_t finish(acc_t a) { return (float)a; }
    // The eight values of a vector are added in float32 as a balanced tree,
    // each first scaled by 1/8. The scaling is exact for every bfloat16 (its
    // eight significant bits stay above float32's smallest subnormal, 2^-149,
    // and float32 subnormals are kept), and it keeps the tree from
    // overflowing: eight values of at most FLT_MAX / 8 cannot sum past
    // FLT_MAX. Three roundings at most on any path, each within 2^-24 of the
    // magnitudes added; the vector total is scaled back by 8 in float64
    // (exactly). Infinities and NaN propagate as in IEEE arithmetic.
    static __device__ __forceinline__ float tree8(vec_t v) {
        constexpr float s = 0.125f;
        const float s01 = __builtin_fmaf(widen(v[0]), s, widen(v[1]) * s);
        const float s23 = __builtin_fmaf(widen(v[2]), s, widen(v[3]) * s);
        const float s45 = __builtin_fmaf(widen(v[4]), s, widen(v[5]) * s);
        const float s67 = __builtin_fmaf(widen(v[6]), s, widen(v[7]) * s);
        return (s01 + s23) + (s45 + s67);
    }
    static __device__ __forceinline__ void fold(acc_t (&acc)[4], vec_t v, size_t) {
        acc[0] = __builtin_fma(8.0, (double)tree8(v), acc[0]);
    }
    static constexpr bool kTileFold = true;
    template <int UNROLL>
    static __device__ __forceinline__ void fold_tile(acc_t (&acc)[4], const vec_t (&v)[UNROLL], size_t) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc[u & 3] = __builtin_fma(8.0, (double)tree8(v[u]), acc[u & 3]);
    }
};
// IEEE half: the eight values of a vector are first added in float32 as a
// balanced tree (three roundings on any path, each at most 2^-24 of the
// magnitudes it adds; no overflow, since eight halves stay below 2^19), and
// each vector's float32 total then enters a float64 accumulator. This halves
// the vector work per element against widening every value to float64.
struct SumF16 {
    using elem_t = uint16_t;
    using vec_t = u16x8;
    using acc_t = double;
    using out_t = float;
    static constexpr int kPerVec = 8;
    static __device__ __forceinline__ float widen(elem_t v) { return (float)__builtin_bit_cast(_Float16, v); }
    static __device__ __forceinline__ acc_t identity() { return 0.0; }
    static __device__ __forceinline__ acc_t lift(elem_t v, size_t) { return (double)widen(v); }
    static __device__ __forceinline__ acc_t combine(acc_t a, acc_t b) { return a + b; }
    static __device__ __forceinline__ out_t finish(acc_t a) { return (float)a; }
    static __device__ __forceinline__ float sum8(vec_t v) {
        const float s01 = widen(v[0]) + widen(v[1]), s23 = widen(v[2]) + widen(v[3]);
        const float s45 = widen(v[4]) + widen(v[5]), s67 = widen(v[6]) + widen(v[7]);
        return (s01 + s23) + (s45 + s67);
    }
    static __device__ __forceinline__ void fold(acc_t (&acc)[4], vec_t v, size_t) { acc[0] += (double)sum8(v); }
    // A tile's vectors rotate over the four accumulators, so the float64
    // additions of one tile form four independent chains.
    static constexpr bool kTileFold = true;
    template <int UNROLL>
    static __device__ __forceinline__ void fold_tile(acc_t (&acc)[4], const vec_t (&v)[UNROLL], size_t) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc[u & 3] += (double)sum8(v[u]);
    }
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

}  // namespace libred
