// Device helpers shared by the cross-entropy kernels (gfx950 only).
//
// The online log-sum-exp state of a set of logits is the pair (m, s): m is the
// largest logit seen and s = sum_j exp(z_j - m).  Ineshin, "A fused linear
// cross-entropy forward kernel for Apple GPUs", section 1, gives the update for a
// new block with maximum m_t: m' = max(m, m_t), s' = s * exp(m - m') +
// sum_j exp(z_j - m').  Merging two partial states is the same update with the
// second state's sum rescaled by exp(m_2 - m').
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ce {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// exp and log through the hardware base-2 units (v_exp_f32 = 2^x, v_log_f32 = log2 x).
// The argument is always a difference (z - m) formed before scaling by log2(e): the
// gap between two large logits is exact in that difference and would be lost in
// z * log2(e) - m * log2(e).
__device__ __forceinline__ float exp_e(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
// log s is rounded on its own (the multiply is not fused into whatever consumes it), so
// a stored log s is exactly the value the loss was assembled from, and two equal sums
// give two equal logs wherever they are used.
__device__ __forceinline__ float log_e(float x) {
#pragma clang fp contract(off)
    return __builtin_amdgcn_logf(x) * kLn2;
}

// Exponent shift S for gradients written in bfloat16.  bfloat16 shares float32's exponent
// range, so its subnormals [2^-133, 2^-126) lie below the smallest normal float32, where
// v_exp_f32 returns 0.  A bf16 gradient g p is therefore formed as (g 2^-S) (2^S p): the
// shift goes into the exponent's constant, the factor into g, and the product rounds once,
// into float32's subnormal range where it must.  With e = floor(log2 |g|) and a further
// factor of up to 2^7 on p when extra = 8, every product of at least 2^-134 (half the
// smallest bf16 subnormal) needs p >= 2^(-135 - e - extra), which 2^S p keeps normal when
// S = e + 9 + extra; g 2^-S is then about 2^(-9 - extra) and exact.  S is clamped to
// [0, 120]: at 0 the needed p are normal already, and at 120 the scaled values (times 2^7)
// stay below float32's overflow, which covers every |g| < 2^(111 - extra).  Other output
// types use S = 0, which leaves their arithmetic bit for bit as without it.
template <typename T>
__device__ __forceinline__ int out_shift(float g, int extra = 0) {
    if constexpr (__is_same(T, __bf16)) {
        // frexp's exponent is floor(log2 |g|) + 1; zero, infinities and NaN give 0, and any
        // shift serves them
        const int s = __builtin_amdgcn_frexp_expf(g) + 8 + extra;
        return s < 0 ? 0 : (s > 120 ? 120 : s);
    } else {
        return 0;
    }
}

// Reference point for rescaling.  A state that has seen only -inf (or nothing) has
// m = -inf and s = 0; rescaling against -inf would form exp(-inf - -inf) = NaN, so it
// rescales against 0 instead, which leaves s = 0 and keeps the state an identity.
__device__ __forceinline__ float ref_point(float m) { return m == kNegInf ? 0.0f : m; }

struct MS {
    float m;
    float s;
};

__device__ __forceinline__ MS ms_empty() { return MS{kNegInf, 0.0f}; }

// Merge two states.  Symmetric in its arguments bit for bit (the two products are
// rounded separately before the add: no fused multiply-add), so lanes exchanging
// states agree exactly.
__device__ __forceinline__ MS ms_merge(MS a, MS b) {
#pragma clang fp contract(off)
    float m = fmaxf(a.m, b.m);
    float r = ref_point(m);
    float pa = __fmul_rn(a.s, exp_e(a.m - r));
    float pb = __fmul_rn(b.s, exp_e(b.m - r));
    return MS{m, pa + pb};
}

// Fold N logits into a state: one rescale of the running sum per call.
template <int N>
__device__ __forceinline__ void ms_add(MS& st, const float (&v)[N]) {
    float t = v[0];
#pragma unroll
    for (int k = 1; k < N; ++k) t = fmaxf(t, v[k]);
    float m = fmaxf(st.m, t);
    float r = ref_point(m);
    float part[N];
#pragma unroll
    for (int k = 0; k < N; ++k) part[k] = exp_e(v[k] - r);
    // pairwise sum of the new terms
#pragma unroll
    for (int w = 1; w < N; w *= 2)
#pragma unroll
        for (int k = 0; k + w < N; k += 2 * w) part[k] += part[k + w];
    st.s = __fmul_rn(st.s, exp_e(st.m - r)) + part[0];
    st.m = m;
}

__device__ __forceinline__ void ms_add1(MS& st, float v) {
    float vv[1] = {v};
    ms_add<1>(st, vv);
}

// Butterfly merge across groups of G consecutive lanes (G a power of two <= 64).
// Every lane of a group ends with the same state.
template <int G>
__device__ __forceinline__ MS ms_group_reduce(MS st) {
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) {
        MS o{__shfl_xor(st.m, off, G), __shfl_xor(st.s, off, G)};
        st = ms_merge(st, o);
    }
    return st;
}

// ---- element types --------------------------------------------------------------

// 16-byte vectors: 4 x fp32, 8 x fp16 or 8 x bf16.
struct alignas(16) U4 {
    uint32_t w[4];
};

template <typename T> struct Elem;

template <> struct Elem<float> {
    static constexpr int kVec = 4;
    __device__ static __forceinline__ void unpack(const U4& u, float (&f)[4]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) f[k] = __uint_as_float(u.w[k]);
    }
    __device__ static __forceinline__ float load1(const float* p) { return *p; }
    __device__ static __forceinline__ U4 pack(const float (&f)[4]) {
        U4 u;
#pragma unroll
        for (int k = 0; k < 4; ++k) u.w[k] = __float_as_uint(f[k]);
        return u;
    }
    __device__ static __forceinline__ void store1(float* p, float v) { *p = v; }
};

template <> struct Elem<_Float16> {
    static constexpr int kVec = 8;
    __device__ static __forceinline__ float half(uint32_t bits) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
    }
    __device__ static __forceinline__ void unpack(const U4& u, float (&f)[8]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = half(u.w[k] & 0xffffu);
            f[2 * k + 1] = half(u.w[k] >> 16);
        }
    }
    __device__ static __forceinline__ float load1(const _Float16* p) { return (float)*p; }
    // float -> binary16, round to nearest even (v_cvt_f16_f32); subnormals are kept.
    __device__ static __forceinline__ uint32_t bits(float v) {
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
    }
    __device__ static __forceinline__ U4 pack(const float (&f)[8]) {
        U4 u;
#pragma unroll
        for (int k = 0; k < 4; ++k) u.w[k] = bits(f[2 * k]) | (bits(f[2 * k + 1]) << 16);
        return u;
    }
    __device__ static __forceinline__ void store1(_Float16* p, float v) { *p = (_Float16)v; }
};

template <> struct Elem<__bf16> {
    static constexpr int kVec = 8;
    __device__ static __forceinline__ void unpack(const U4& u, float (&f)[8]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = __uint_as_float(u.w[k] << 16);
            f[2 * k + 1] = __uint_as_float(u.w[k] & 0xffff0000u);
        }
    }
    __device__ static __forceinline__ float load1(const __bf16* p) {
        return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, *p) << 16);
    }
    // float pair -> packed bfloat16 pair, round to nearest even: one v_cvt_pk_bf16_f32.
    __device__ static __forceinline__ uint32_t bits2(float lo, float hi) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, b2));
    }
    __device__ static __forceinline__ U4 pack(const float (&f)[8]) {
        U4 u;
#pragma unroll
        for (int k = 0; k < 4; ++k) u.w[k] = bits2(f[2 * k], f[2 * k + 1]);
        return u;
    }
    __device__ static __forceinline__ void store1(__bf16* p, float v) { *p = (__bf16)v; }
};

// ---- row addressing -----------------------------------------------------------

// Strided view in elements; `uniform` means row r starts at r * row_stride (a single
// batch, or batch_stride == rows_per_batch * row_stride), which skips the division.
struct RowLayout {
    int64_t rows_per_batch;
    int64_t row_stride;
    int64_t batch_stride;
    int32_t uniform;
};

__device__ __forceinline__ int64_t row_offset(int64_t r, const RowLayout& L) {
    if (L.uniform) return r * L.row_stride;
    int64_t b = r / L.rows_per_batch;
    return b * L.batch_stride + (r - b * L.rows_per_batch) * L.row_stride;
}

// Split a row of V elements starting at `p` into a scalar head (up to the first
// 16-byte boundary), whole 16-byte vectors, and a scalar tail.
template <typename T>
struct RowSplit {
    int64_t head;   // elements before the first vector
    int64_t nvec;   // whole vectors
    int64_t tail0;  // first tail element = head + nvec * kVec
    __device__ __forceinline__ RowSplit(const T* p, int64_t V) {
        constexpr int kVec = Elem<T>::kVec;
        int64_t h = (int64_t)(((16u - ((uint32_t)(uintptr_t)p & 15u)) & 15u) / sizeof(T));
        head = h < V ? h : V;
        nvec = (V - head) / kVec;
        tail0 = head + nvec * kVec;
    }
    // k-th scalar element (0 <= k < head + V - tail0)
    __device__ __forceinline__ int64_t scalar_index(int64_t k) const {
        return k < head ? k : tail0 + (k - head);
    }
    __device__ __forceinline__ int64_t n_scalar(int64_t V) const { return head + (V - tail0); }
};

// 16-byte load with the non-temporal hint: every logit is read once per call (the
// forward and the VJP each stream the whole batch, which is larger than the caches),
// so the lines are not worth keeping.  Stores stay ordinary; marking them
// non-temporal measured slower.
__device__ __forceinline__ U4 load_u4_stream(const void* p) {
    const U4* q = reinterpret_cast<const U4*>(p);
    U4 u;
#pragma unroll
    for (int k = 0; k < 4; ++k) u.w[k] = __builtin_nontemporal_load(&q->w[k]);
    return u;
}

// Plain 16-byte load, for a pass whose lines are read again soon after (the one-pass
// forward and VJP reads each row twice).
__device__ __forceinline__ U4 load_u4(const void* p) { return *reinterpret_cast<const U4*>(p); }

__device__ __forceinline__ void store_u4(void* p, const U4& u) {
    *reinterpret_cast<U4*>(p) = u;
}

}  // namespace ce
