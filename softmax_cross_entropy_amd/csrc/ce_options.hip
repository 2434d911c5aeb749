// Cross-entropy options for gfx950: label smoothing, probability targets, ignore_index
// and the sum / mean reductions.
//
// MLX PR #4188 "Shift by the max in cross_entropy", Proposed changes: the loss takes
// class-index or probability targets and a label smoothing whose term subtracts the
// mean logit, with three reductions; the max shift serves every path.  Written with
// target weights w_j, the loss of a row is -sum_j w_j log p_j, where
//   class index y:    w = (1 - eps) onehot(y) + eps / V
//   probabilities t:  w = (1 - eps) t + eps / V.
// With log p_j = (z_j - m) - log s this is W log s - A, where W = sum_j w_j and
// A = sum_j w_j (z_j - m) <= 0, so the loss is a sum of two non-negative terms.  For an
// index target W = 1 and A = (1 - eps)(z_y - m) + (eps / V) C with C = sum_j (z_j - m):
//   loss = (1 - eps) ((m - z_y) + log s) + eps (log s - C / V),
// the plain loss blended with log-sum-exp minus the mean logit.  The gradient of
// sum_i g_i loss_i is g_i (W_i p_ij - w_ij).
//
// One pass per row keeps, per lane, the online pair (m, s) and (a, w): a is the
// weighted sum of (z_j - m) against the running max m and w the sum of the weights;
// when the max rises from m to m', a gains w (m - m').  A weight of 0 adds nothing,
// even at z_j = -inf (0 log 0 = 0).
//
// Layouts as in the other kernels: G lanes per row (G <= 64) or one workgroup per row
// with one exchange of states through LDS slots that alternate between two buffers.
// The VJP is elementwise and cuts long rows into chunks of 256 * kChunkU vectors.
#include <hip/hip_runtime.h>

#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace ce {
namespace {

constexpr int kBlock = 256;

__device__ __forceinline__ bool target_in(int32_t y, int64_t V) { return y >= 0 && (int64_t)y < V; }

struct OState {
    float m, s;  // online log-sum-exp pair
    float a;     // sum_j w_j (z_j - m)
    float w;     // sum_j w_j
};

__device__ __forceinline__ OState os_empty() { return OState{kNegInf, 0.f, 0.f, 0.f}; }

// a's correction when the running max rises from st.m to m (nothing to correct while
// st.m is -inf: every term so far was then 0 or -inf already).
__device__ __forceinline__ float a_shift(const OState& st, float m) {
    return st.m > kNegInf ? __fmul_rn(st.w, st.m - m) : 0.f;
}

// Folds N logits z with weights wt (kWeighted) or weight 1 each (otherwise).
template <bool kWeighted, int N>
__device__ __forceinline__ void os_add(OState& st, const float (&z)[N], const float (&wt)[N]) {
    float t = z[0];
#pragma unroll
    for (int k = 1; k < N; ++k) t = fmaxf(t, z[k]);
    const float m = fmaxf(st.m, t);
    const float r = ref_point(m);
    float s = 0.f, a = 0.f, w = 0.f;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        s += exp_e(z[k] - r);
        if constexpr (kWeighted) {
            w += wt[k];
            a += wt[k] != 0.f ? wt[k] * (z[k] - r) : 0.f;
        } else {
            a += z[k] - r;
        }
    }
    if constexpr (!kWeighted) w = (float)N;
    st.s = __fmul_rn(st.s, exp_e(st.m - r)) + s;
    st.a = (st.a + a_shift(st, m)) + a;
    st.w = st.w + w;
    st.m = m;
}

// Merge of two states, symmetric bit for bit.
__device__ __forceinline__ OState os_merge(const OState& x, const OState& y) {
#pragma clang fp contract(off)
    const MS ms = ms_merge(MS{x.m, x.s}, MS{y.m, y.s});
    const float ax = x.a + a_shift(x, ms.m);
    const float ay = y.a + a_shift(y, ms.m);
    return OState{ms.m, ms.s, ax + ay, x.w + y.w};
}

template <int G>
__device__ __forceinline__ OState os_group_reduce(OState st) {
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) {
        OState o{__shfl_xor(st.m, off, G), __shfl_xor(st.s, off, G), __shfl_xor(st.a, off, G),
                 __shfl_xor(st.w, off, G)};
        st = os_merge(st, o);
    }
    return st;
}

// ---- forward --------------------------------------------------------------------

struct OFwdArgs {
    const void* z;
    RowLayout zl;
    const void* t;  // probability targets (kProbs)
    RowLayout tl;
    const int32_t* y;  // class-index targets (otherwise)
    int64_t n_rows;
    int64_t V;
    float keep;   // 1 - eps
    float eps;    // eps
    float eps_v;  // eps / V
    float inv_v;  // 1 / V
    float* loss;
    float2* lse;
    float* wsum;  // kProbs: W per row
};

template <bool kProbs>
__device__ __forceinline__ void ofwd_store(const OFwdArgs& a, int64_t r, const OState& st, float zy, bool ok) {
    const float ls = log_e(st.s);
    float loss;
    if constexpr (kProbs) {
        loss = st.w * ls - st.a;
        a.wsum[r] = st.w;
    } else {
        const float base = (st.m - zy) + ls;
        loss = ok ? a.keep * base + a.eps * (ls - st.a * a.inv_v) : __builtin_nanf("");
    }
    a.loss[r] = loss;
    a.lse[r] = make_float2(st.m, ls);
}

// This lane's share of one row: 16-byte vectors lane, lane + G, ... in groups of U, then
// the scalar head and tail.  With probability targets the target row is read alongside
// when both rows share a 16-byte phase, element by element otherwise.
template <typename T, int G, int U, bool kProbs>
__device__ __forceinline__ void ostream_row(const OFwdArgs& a, const T* zrow, const T* trow, int lane, OState& st) {
    constexpr int kVec = Elem<T>::kVec;
    const int64_t V = a.V;
    const bool vec_ok = !kProbs || ((((uintptr_t)zrow) ^ ((uintptr_t)trow)) & 15u) == 0;
    if (vec_ok) {
        RowSplit<T> sp(zrow, V);
        const char* zb = reinterpret_cast<const char*>(zrow + sp.head);
        const char* tb = kProbs ? reinterpret_cast<const char*>(trow + sp.head) : nullptr;
        int64_t j = lane;
        for (; j + (int64_t)(U - 1) * G < sp.nvec; j += (int64_t)U * G) {
            U4 bz[U], bt[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                bz[u] = load_u4_stream(zb + (j + (int64_t)u * G) * 16);
                if constexpr (kProbs) bt[u] = load_u4_stream(tb + (j + (int64_t)u * G) * 16);
            }
            float fz[U * kVec], fw[U * kVec];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float tz[kVec], tt[kVec];
                Elem<T>::unpack(bz[u], tz);
                if constexpr (kProbs) Elem<T>::unpack(bt[u], tt);
#pragma unroll
                for (int k = 0; k < kVec; ++k) {
                    fz[u * kVec + k] = tz[k];
                    fw[u * kVec + k] = kProbs ? __builtin_fmaf(a.keep, tt[k], a.eps_v) : 1.f;
                }
            }
            os_add<kProbs, U * kVec>(st, fz, fw);
        }
        for (; j < sp.nvec; j += G) {
            float fz[kVec], fw[kVec], tt[kVec];
            Elem<T>::unpack(load_u4_stream(zb + j * 16), fz);
            if constexpr (kProbs) Elem<T>::unpack(load_u4_stream(tb + j * 16), tt);
#pragma unroll
            for (int k = 0; k < kVec; ++k) fw[k] = kProbs ? __builtin_fmaf(a.keep, tt[k], a.eps_v) : 1.f;
            os_add<kProbs, kVec>(st, fz, fw);
        }
        const int64_t ns = sp.n_scalar(V);
        for (int64_t k = lane; k < ns; k += G) {
            const int64_t i = sp.scalar_index(k);
            const float fz[1] = {Elem<T>::load1(zrow + i)};
            const float fw[1] = {kProbs ? __builtin_fmaf(a.keep, Elem<T>::load1(trow + i), a.eps_v) : 1.f};
            os_add<kProbs, 1>(st, fz, fw);
        }
    } else {
        for (int64_t i = lane; i < V; i += G) {
            const float fz[1] = {Elem<T>::load1(zrow + i)};
            const float fw[1] = {__builtin_fmaf(a.keep, Elem<T>::load1(trow + i), a.eps_v)};
            os_add<true, 1>(st, fz, fw);
        }
    }
}

template <typename T, bool kProbs>
__device__ __forceinline__ void orow_ptrs(const OFwdArgs& a, int64_t r, const T*& z, const T*& t) {
    z = static_cast<const T*>(a.z) + row_offset(r, a.zl);
    t = kProbs ? static_cast<const T*>(a.t) + row_offset(r, a.tl) : nullptr;
}

template <typename T, int G, int U, bool kProbs>
__global__ __launch_bounds__(kBlock) void ceo_fwd_lanes(OFwdArgs a) {
    constexpr int kRowsPerBlock = kBlock / G;
    const int lane = threadIdx.x % G;
    const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
    for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / G; r < a.n_rows; r += stride) {
        const T *z, *t;
        orow_ptrs<T, kProbs>(a, r, z, t);
        bool ok = true;
        float zy = 0.f;
        if constexpr (!kProbs) {
            const int32_t y = a.y[r];
            ok = target_in(y, a.V);
            if (lane == 0 && ok) zy = Elem<T>::load1(z + y);
        }
        OState st = os_empty();
        ostream_row<T, G, U, kProbs>(a, z, t, lane, st);
        st = os_group_reduce<G>(st);
        if (lane == 0) ofwd_store<kProbs>(a, r, st, zy, ok);
    }
}

template <typename T, int NW, int U, bool kProbs>
__global__ __launch_bounds__(64 * NW, 8) void ceo_fwd_rowwg(OFwdArgs a) {
    constexpr int G = 64 * NW;
    // One state per wave, exchanged once per row; the slots alternate between two
    // buffers from row to row so that no slot is written again before wave 0 has read
    // it (the next row's barrier holds back a wave that runs ahead).
    __shared__ OState slots[2][NW];
    const int tid = threadIdx.x;
    const int wave = tid / 64;
    const int lane = tid % 64;
    int parity = 0;
    for (int64_t r = blockIdx.x; r < a.n_rows; r += gridDim.x, parity ^= 1) {
        const T *z, *t;
        orow_ptrs<T, kProbs>(a, r, z, t);
        bool ok = true;
        float zy = 0.f;
        if constexpr (!kProbs) {
            const int32_t y = a.y[r];
            ok = target_in(y, a.V);
            if (tid == 0 && ok) zy = Elem<T>::load1(z + y);
        }
        OState st = os_empty();
        ostream_row<T, G, U, kProbs>(a, z, t, tid, st);
        st = os_group_reduce<64>(st);
        if (lane == 0) slots[parity][wave] = st;
        __syncthreads();
        if (wave == 0) {
            OState v = lane < NW ? slots[parity][lane] : os_empty();
            v = os_group_reduce<NW>(v);
            if (lane == 0) ofwd_store<kProbs>(a, r, v, zy, ok);
        }
    }
}

// ---- reduction of the per-row losses ---------------------------------------------

// Stage 1: partial sums over fixed blocks of rows, in float64, in a fixed order; a single
// block writes the result itself.  With ignore_index it also writes loss 0 for the
// ignored rows and leaves them out of the count.
struct RedArgs {
    float* loss;
    const int32_t* y;  // NULL: every row counts
    int64_t n_rows;
    int64_t rows_per_part;
    int32_t ignore_index;
    int32_t has_ignore;
    int32_t reduce;  // 0: only the ignore_index fix-up
    double* part_sum;
    int64_t* part_cnt;
    // one part covers every row: write the result here directly
    int32_t single;
    int32_t mean;
    float* total;
    int64_t* count;
};

__device__ __forceinline__ void write_total(double s, int64_t c, int32_t mean, float* total, int64_t* count) {
    total[0] = (float)(mean ? s / (double)c : s);
    count[0] = c;
}

__global__ __launch_bounds__(kBlock) void ceo_reduce_parts(RedArgs a) {
    __shared__ double ssum[kBlock];
    __shared__ int64_t scnt[kBlock];
    const int64_t r0 = (int64_t)blockIdx.x * a.rows_per_part;
    const int64_t r1 = r0 + a.rows_per_part < a.n_rows ? r0 + a.rows_per_part : a.n_rows;
    double sum = 0.0;
    int64_t cnt = 0;
    for (int64_t r = r0 + threadIdx.x; r < r1; r += kBlock) {
        const bool ignored = a.has_ignore && a.y[r] == a.ignore_index;
        if (ignored) {
            a.loss[r] = 0.f;
        } else {
            sum += (double)a.loss[r];
            ++cnt;
        }
    }
    if (!a.reduce) return;
    ssum[threadIdx.x] = sum;
    scnt[threadIdx.x] = cnt;
    __syncthreads();
    for (int w = kBlock / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
            ssum[threadIdx.x] += ssum[threadIdx.x + w];
            scnt[threadIdx.x] += scnt[threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        if (a.single) {
            write_total(ssum[0], scnt[0], a.mean, a.total, a.count);
        } else {
            a.part_sum[blockIdx.x] = ssum[0];
            a.part_cnt[blockIdx.x] = scnt[0];
        }
    }
}

// Stage 2: one workgroup folds the partials in a fixed order; 'mean' divides by the
// count (0 / 0 = NaN when no row counts).
__global__ __launch_bounds__(kBlock) void ceo_reduce_final(const double* part_sum, const int64_t* part_cnt,
                                                           int64_t n_parts, int32_t mean, float* total,
                                                           int64_t* count) {
    __shared__ double ssum[kBlock];
    __shared__ int64_t scnt[kBlock];
    double sum = 0.0;
    int64_t cnt = 0;
    for (int64_t i = threadIdx.x; i < n_parts; i += kBlock) {
        sum += part_sum[i];
        cnt += part_cnt[i];
    }
    ssum[threadIdx.x] = sum;
    scnt[threadIdx.x] = cnt;
    __syncthreads();
    for (int w = kBlock / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
            ssum[threadIdx.x] += ssum[threadIdx.x + w];
            scnt[threadIdx.x] += scnt[threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) write_total(ssum[0], scnt[0], mean, total, count);
}

// ---- VJP --------------------------------------------------------------------------

struct OVjpArgs {
    const void* z;
    RowLayout zl;
    const void* t;
    RowLayout tl;
    const int32_t* y;
    const float2* lse;
    const float* wsum;
    const float* g;
    const int64_t* count;
    int64_t n_rows;
    int64_t V;
    int32_t reduction;  // 0 none (g per row), 1 sum, 2 mean (g[0] for every row)
    int32_t ignore_index;
    int32_t has_ignore;
    float keep;   // 1 - eps
    float eps_v;  // eps / V
    void* d;
    RowLayout dl;
};

struct ORow {
    float m;    // row max, NaN for an invalid index target
    float c;    // S - log s * log2(e), S the output type's exponent shift (out_shift)
    float g;    // coefficient of p times 2^-S: g (index targets) or g W (probability targets)
    float gk;   // g (1 - eps) (probability targets)
    float ge;   // g eps / V, 0 when eps is 0
    float cy;   // target weight ((1 - eps) + eps / V) 2^S (index targets)
    int32_t y;
    int32_t zero;  // ignored row: the gradient is 0 whatever the logits hold
};

// The upstream gradient shared by every row of a reduced loss: g, or g / count for a
// mean (formed once per thread, not per work item).
__device__ __forceinline__ float shared_upstream(const OVjpArgs& a) {
    if (a.reduction == 0) return 0.f;
    if (a.reduction == 1) return a.g[0];
    return (float)((double)a.g[0] / (double)a.count[0]);
}

// The row's constants.  oprob returns 2^S p, so every product with p takes g 2^-S, and
// every term that p is compared with on its own scale (the target weight) takes 2^S.
template <typename T, bool kProbs>
__device__ __forceinline__ ORow load_orow(const OVjpArgs& a, int64_t r, float gs) {
    ORow o;
    const float2 l = a.lse[r];
    const float g = a.reduction == 0 ? a.g[r] : gs;
    // eps = 0 leaves g p - 0 = g p, bit for bit, even for an infinite g
    o.ge = a.eps_v == 0.f ? 0.f : g * a.eps_v;
    o.gk = g * a.keep;
    o.zero = 0;
    o.y = -1;
    float gp = g;
    if constexpr (kProbs) {
        o.m = l.x;
        gp = g * a.wsum[r];
    } else {
        o.y = a.y[r];
        o.zero = a.has_ignore && o.y == a.ignore_index;
        o.m = target_in(o.y, a.V) ? l.x : __builtin_nanf("");
    }
    const int S = out_shift<T>(gp);
    o.c = (float)S - l.y * kLog2e;
    o.g = __builtin_ldexpf(gp, -S);
    o.cy = __builtin_ldexpf(a.keep + a.eps_v, S);
    return o;
}

// 2^S p: the softmax probability of z on the row's exponent shift.
__device__ __forceinline__ float oprob(float z, const ORow& o) {
    return __builtin_amdgcn_exp2f(__builtin_fmaf(z - o.m, kLog2e, o.c));
}

// Gradient of one element, with g folded into the per-row constants: index targets
// g p - g eps / V off the target; probability targets g W p - (g (1 - eps) t + g eps / V).
// Ignored rows never come here: their work items store zeros without reading the logits.
template <bool kProbs>
__device__ __forceinline__ float ograd(float z, float t, const ORow& o) {
    const float p = oprob(z, o);
    if constexpr (kProbs)
        return __builtin_fmaf(o.g, p, -__builtin_fmaf(o.gk, t, o.ge));
    else
        return __builtin_fmaf(o.g, p, -o.ge);
}

// One 16-byte vector of gradients.  Index targets: the one lane whose vector holds the
// target stores that element again with the target weight, g (p - ((1 - eps) + eps / V));
// same lane, same address.  The target logit is picked from registers by a bitwise
// select chain: an indexed read of the vector would make the compiler stage every
// vector through LDS.
template <typename T, bool kProbs>
__device__ __forceinline__ void ovec(const U4& bz, const U4& bt, const ORow& o, int64_t first,
                                     char* dst, T* drow) {
    constexpr int kVec = Elem<T>::kVec;
    float fz[kVec], ft[kVec], out[kVec];
    Elem<T>::unpack(bz, fz);
    if constexpr (kProbs) Elem<T>::unpack(bt, ft);
#pragma unroll
    for (int k = 0; k < kVec; ++k) out[k] = ograd<kProbs>(fz[k], kProbs ? ft[k] : 0.f, o);
    store_u4(dst, Elem<T>::pack(out));
    if constexpr (!kProbs) {
        const int64_t rel = (int64_t)o.y - first;
        if ((uint64_t)rel < (uint64_t)kVec) {
            const uint32_t r = (uint32_t)rel;
            uint32_t bits = 0;
#pragma unroll
            for (int k = 0; k < kVec; ++k) bits |= (r == (uint32_t)k ? 0xffffffffu : 0u) & __float_as_uint(fz[k]);
            const float zy = __uint_as_float(bits);
            Elem<T>::store1(drow + o.y, o.g * (oprob(zy, o) - o.cy));
        }
    }
}

template <typename T, bool kProbs>
__device__ __forceinline__ void oscalar(const T* z, const T* t, T* d, int64_t i, const ORow& o) {
    const float zi = Elem<T>::load1(z + i);
    float v;
    if constexpr (kProbs) {
        v = ograd<true>(zi, Elem<T>::load1(t + i), o);
    } else {
        v = ograd<false>(zi, 0.f, o);
        if (i == (int64_t)o.y) v = o.g * (oprob(zi, o) - o.cy);
    }
    Elem<T>::store1(d + i, v);
}

// Zeros over elements [e0, e1) of an ignored row's gradient, in 16-byte stores where
// the row allows, by threads tid, tid + nthr, ...
template <typename T>
__device__ __forceinline__ void ozero(T* d, int64_t e0, int64_t e1, int tid, int nthr) {
    if (e0 >= e1) return;
    RowSplit<T> sp(d + e0, e1 - e0);
    char* vb = reinterpret_cast<char*>(d + e0 + sp.head);
    const U4 zero{};
    for (int64_t j = tid; j < sp.nvec; j += nthr) store_u4(vb + j * 16, zero);
    const int64_t ns = sp.n_scalar(e1 - e0);
    for (int64_t k = tid; k < ns; k += nthr) Elem<T>::store1(d + e0 + sp.scalar_index(k), 0.f);
}

template <typename T, bool kProbs>
__device__ __forceinline__ bool ophases(const T* z, const T* t, const T* d) {
    const uintptr_t az = (uintptr_t)z, ad = (uintptr_t)d;
    bool ok = ((az ^ ad) & 15u) == 0;
    if constexpr (kProbs) ok = ok && ((az ^ (uintptr_t)t) & 15u) == 0;
    return ok;
}

template <typename T, int G, int U, bool kProbs>
__global__ __launch_bounds__(G > kBlock ? G : kBlock) void ceo_vjp_lanes(OVjpArgs a) {
    constexpr int kVec = Elem<T>::kVec;
    constexpr int kThreads = G > kBlock ? G : kBlock;
    constexpr int kRowsPerBlock = kThreads / G;
    const int lane = threadIdx.x % G;
    const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
    const float gs = shared_upstream(a);
    for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / G; r < a.n_rows; r += stride) {
        const T* z = static_cast<const T*>(a.z) + row_offset(r, a.zl);
        const T* t = kProbs ? static_cast<const T*>(a.t) + row_offset(r, a.tl) : nullptr;
        T* d = static_cast<T*>(a.d) + row_offset(r, a.dl);
        const ORow o = load_orow<T, kProbs>(a, r, gs);
        if (o.zero) {
            ozero(d, 0, a.V, lane, G);
        } else if (ophases<T, kProbs>(z, t, d)) {
            RowSplit<T> sp(z, a.V);
            const char* zb = reinterpret_cast<const char*>(z + sp.head);
            const char* tb = kProbs ? reinterpret_cast<const char*>(t + sp.head) : nullptr;
            char* db = reinterpret_cast<char*>(d + sp.head);
            int64_t j = lane;
            for (; j + (int64_t)(U - 1) * G < sp.nvec; j += (int64_t)U * G) {
                U4 bz[U], bt[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    bz[u] = load_u4_stream(zb + (j + (int64_t)u * G) * 16);
                    if constexpr (kProbs) bt[u] = load_u4_stream(tb + (j + (int64_t)u * G) * 16);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t v = j + (int64_t)u * G;
                    ovec<T, kProbs>(bz[u], bt[u], o, sp.head + v * kVec, db + v * 16, d);
                }
            }
            for (; j < sp.nvec; j += G) {
                U4 bt{};
                if constexpr (kProbs) bt = load_u4_stream(tb + j * 16);
                ovec<T, kProbs>(load_u4_stream(zb + j * 16), bt, o, sp.head + j * kVec, db + j * 16, d);
            }
            const int64_t ns = sp.n_scalar(a.V);
            for (int64_t k = lane; k < ns; k += G) oscalar<T, kProbs>(z, t, d, sp.scalar_index(k), o);
        } else {
            for (int64_t i = lane; i < a.V; i += G) oscalar<T, kProbs>(z, t, d, i, o);
        }
    }
}

template <typename T, int U, bool kProbs>
__global__ __launch_bounds__(kBlock) void ceo_vjp_chunks(OVjpArgs a, int64_t chunks_per_row) {
    constexpr int kVec = Elem<T>::kVec;
    constexpr int64_t kChunkVec = (int64_t)kBlock * U;
    const int tid = threadIdx.x;
    const int64_t items = a.n_rows * chunks_per_row;
    const float gs = shared_upstream(a);
    for (int64_t w = blockIdx.x; w < items; w += gridDim.x) {
        const int64_t r = w / chunks_per_row;
        const int64_t c = w - r * chunks_per_row;
        const T* z = static_cast<const T*>(a.z) + row_offset(r, a.zl);
        const T* t = kProbs ? static_cast<const T*>(a.t) + row_offset(r, a.tl) : nullptr;
        T* d = static_cast<T*>(a.d) + row_offset(r, a.dl);
        const ORow o = load_orow<T, kProbs>(a, r, gs);
        if (o.zero) {
            // the same element ranges as the path for rows in different 16-byte phases
            const int64_t e0 = c * kChunkVec * kVec;
            ozero(d, e0, e0 + kChunkVec * kVec < a.V ? e0 + kChunkVec * kVec : a.V, tid, kBlock);
        } else if (ophases<T, kProbs>(z, t, d)) {
            RowSplit<T> sp(z, a.V);
            const char* zb = reinterpret_cast<const char*>(z + sp.head);
            const char* tb = kProbs ? reinterpret_cast<const char*>(t + sp.head) : nullptr;
            char* db = reinterpret_cast<char*>(d + sp.head);
            const int64_t v0 = c * kChunkVec + tid;
            if (c * kChunkVec + kChunkVec <= sp.nvec) {
                U4 bz[U], bt[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    bz[u] = load_u4_stream(zb + (v0 + (int64_t)u * kBlock) * 16);
                    if constexpr (kProbs) bt[u] = load_u4_stream(tb + (v0 + (int64_t)u * kBlock) * 16);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t v = v0 + (int64_t)u * kBlock;
                    ovec<T, kProbs>(bz[u], bt[u], o, sp.head + v * kVec, db + v * 16, d);
                }
            } else {
                for (int64_t j = v0; j < sp.nvec; j += kBlock) {
                    U4 bt{};
                    if constexpr (kProbs) bt = load_u4_stream(tb + j * 16);
                    ovec<T, kProbs>(load_u4_stream(zb + j * 16), bt, o, sp.head + j * kVec, db + j * 16, d);
                }
            }
            if (c == 0) {
                const int64_t ns = sp.n_scalar(a.V);
                for (int64_t k = tid; k < ns; k += kBlock) oscalar<T, kProbs>(z, t, d, sp.scalar_index(k), o);
            }
        } else {
            const int64_t e0 = c * kChunkVec * kVec;
            const int64_t e1 = e0 + kChunkVec * kVec < a.V ? e0 + kChunkVec * kVec : a.V;
            for (int64_t i = e0 + tid; i < e1; i += kBlock) oscalar<T, kProbs>(z, t, d, i, o);
        }
    }
}

// ---- dispatch -----------------------------------------------------------------------

RowLayout olayout(const HostLayout& h) { return RowLayout{h.rows_per_batch, h.row_stride, h.batch_stride, h.uniform}; }

template <typename T, bool kProbs>
hipError_t ofwd_typed(const OptFwdCall& c) {
    const float V = (float)c.V;
    OFwdArgs a{c.z,       olayout(c.zl), c.t,  olayout(c.tl),     c.y,    c.n_rows, c.V,
               1.f - c.eps, c.eps,       c.eps / V, 1.f / V, c.loss, reinterpret_cast<float2*>(c.lse), c.wsum};
    const dim3 grid((unsigned)c.plan.blocks);
    // 16 elements folded per rescale for one row, 8 of each row for two: the extra
    // (a, w) state leaves no room for wider groups within 64 VGPRs
    constexpr int kU = kProbs ? (Elem<T>::kVec == 8 ? 1 : 2) : (Elem<T>::kVec == 8 ? 2 : 4);
    constexpr int kUs = kProbs ? 1 : 2;  // narrower groups for few lanes
    switch (c.plan.lanes) {
        case 1: hipLaunchKernelGGL((ceo_fwd_lanes<T, 1, kUs, kProbs>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 2: hipLaunchKernelGGL((ceo_fwd_lanes<T, 2, kUs, kProbs>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 4: hipLaunchKernelGGL((ceo_fwd_lanes<T, 4, kUs, kProbs>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 8: hipLaunchKernelGGL((ceo_fwd_lanes<T, 8, kU, kProbs>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 16: hipLaunchKernelGGL((ceo_fwd_lanes<T, 16, kU, kProbs>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 32: hipLaunchKernelGGL((ceo_fwd_lanes<T, 32, kU, kProbs>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 64: hipLaunchKernelGGL((ceo_fwd_lanes<T, 64, kU, kProbs>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 128: hipLaunchKernelGGL((ceo_fwd_rowwg<T, 2, kU, kProbs>), grid, dim3(128), 0, c.stream, a); break;
        case 256: hipLaunchKernelGGL((ceo_fwd_rowwg<T, 4, kU, kProbs>), grid, dim3(256), 0, c.stream, a); break;
        case 512: hipLaunchKernelGGL((ceo_fwd_rowwg<T, 8, kU, kProbs>), grid, dim3(512), 0, c.stream, a); break;
        case 1024: hipLaunchKernelGGL((ceo_fwd_rowwg<T, 16, kU, kProbs>), grid, dim3(1024), 0, c.stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, bool kProbs>
hipError_t ovjp_typed(const OptVjpCall& c) {
    OVjpArgs a{c.z,      olayout(c.zl), c.t,          olayout(c.tl),  c.y,         reinterpret_cast<const float2*>(c.lse),
               c.wsum,   c.g,           c.count,      c.n_rows,       c.V,         c.reduction,
               c.ignore_index, c.has_ignore, 1.f - c.eps, c.eps / (float)c.V, c.d, olayout(c.dl)};
    const dim3 grid((unsigned)c.plan.blocks);
    if (c.plan.chunks > 0) {
        hipLaunchKernelGGL((ceo_vjp_chunks<T, kChunkU, kProbs>), grid, dim3(kBlock), 0, c.stream, a, c.plan.chunks);
        return hipGetLastError();
    }
    constexpr int kU = 2;
    switch (c.plan.lanes) {
        case 1: hipLaunchKernelGGL((ceo_vjp_lanes<T, 1, 1, kProbs>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 2: hipLaunchKernelGGL((ceo_vjp_lanes<T, 2, 1, kProbs>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 4: hipLaunchKernelGGL((ceo_vjp_lanes<T, 4, 1, kProbs>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 8: hipLaunchKernelGGL((ceo_vjp_lanes<T, 8, kU, kProbs>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 16: hipLaunchKernelGGL((ceo_vjp_lanes<T, 16, kU, kProbs>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 32: hipLaunchKernelGGL((ceo_vjp_lanes<T, 32, kU, kProbs>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 64: hipLaunchKernelGGL((ceo_vjp_lanes<T, 64, kU, kProbs>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 128: hipLaunchKernelGGL((ceo_vjp_lanes<T, 128, kU, kProbs>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 256: hipLaunchKernelGGL((ceo_vjp_lanes<T, 256, kU, kProbs>), grid, dim3(256), 0, c.stream, a); break;
        case 512: hipLaunchKernelGGL((ceo_vjp_lanes<T, 512, kU, kProbs>), grid, dim3(512), 0, c.stream, a); break;
        case 1024: hipLaunchKernelGGL((ceo_vjp_lanes<T, 1024, kU, kProbs>), grid, dim3(1024), 0, c.stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool kProbs>
hipError_t ofwd_dt(const OptFwdCall& c) {
    switch (c.dt) {
        case Dt::F32: return ofwd_typed<float, kProbs>(c);
        case Dt::F16: return ofwd_typed<_Float16, kProbs>(c);
        case Dt::BF16: return ofwd_typed<__bf16, kProbs>(c);
    }
    return hipErrorInvalidValue;
}

template <bool kProbs>
hipError_t ovjp_dt(const OptVjpCall& c) {
    switch (c.dt) {
        case Dt::F32: return ovjp_typed<float, kProbs>(c);
        case Dt::F16: return ovjp_typed<_Float16, kProbs>(c);
        case Dt::BF16: return ovjp_typed<__bf16, kProbs>(c);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_opt_forward(const OptFwdCall& c) { return c.t ? ofwd_dt<true>(c) : ofwd_dt<false>(c); }

hipError_t launch_opt_vjp(const OptVjpCall& c) { return c.t ? ovjp_dt<true>(c) : ovjp_dt<false>(c); }

// Reduction partials of ce_forward_ex_noalloc, for callers that cannot allocate device
// memory: one fixed array per GPU, held for the life of the process.  Its size is the
// reduction's whole need at any n_rows (at most kReduceMaxParts partial sums and
// counts).  In host code `scratch` names a host-side stand-in, not device memory: host
// code uses only the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kReduceWorkspaceBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t reduce_scratch(void** ptr, size_t* bytes) {
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev)) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        // the device is current: this is its own copy of the array
        void* p = nullptr;
        if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = sizeof(scratch);
    return hipSuccess;
}

int64_t reduce_parts(int64_t n_rows) {
    if (n_rows <= 0) return 0;
    int64_t parts = (n_rows + kReduceRowsMin - 1) / kReduceRowsMin;
    return parts < kReduceMaxParts ? parts : kReduceMaxParts;
}

hipError_t launch_loss_reduce(const ReduceCall& c) {
    const int64_t parts = reduce_parts(c.n_rows);
    double* part_sum = static_cast<double*>(c.workspace);
    int64_t* part_cnt = reinterpret_cast<int64_t*>(part_sum + kReduceMaxParts);
    const bool reduce = c.reduction != 0;
    const bool single = reduce && parts == 1;
    if (parts > 0 && (reduce || c.has_ignore)) {
        RedArgs a{c.loss,    c.y,         c.n_rows, (c.n_rows + parts - 1) / parts, c.ignore_index, c.has_ignore ? 1 : 0,
                  reduce ? 1 : 0, part_sum, part_cnt, single ? 1 : 0, c.reduction == 2 ? 1 : 0, c.total, c.count};
        hipLaunchKernelGGL(ceo_reduce_parts, dim3((unsigned)parts), dim3(kBlock), 0, c.stream, a);
        if (hipError_t e = hipGetLastError()) return e;
    }
    if (reduce && !single) {
        hipLaunchKernelGGL(ceo_reduce_final, dim3(1), dim3(kBlock), 0, c.stream, part_sum, part_cnt, parts,
                           c.reduction == 2 ? 1 : 0, c.total, c.count);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace ce
