// Row-wise Jensen-Shannon divergence of a student row q and a teacher row p, and its
// gradient with respect to q, for gfx950.
//
// "One barrier short", first section and section "The fix": mlx-lm fuses the
// Jensen-Shannon divergence the way it fuses the KL one, and at a logit scale of 20
// its loss overflowed until a stable softplus was used.  With P = softmax(p),
// Q = softmax(q) and M = (P + Q) / 2,
//   js = 1/2 sum_j P_j (log P_j - log M_j) + 1/2 sum_j Q_j (log Q_j - log M_j),
//   d js / d q_k = Q_k (h_k - H),  h_k = (log Q_k - log M_k) / 2,  H = sum_j Q_j h_j.
// With d = log P - log Q, log M = log Q + softplus(d) - ln 2, so
//   log P - log M = ln 2 - softplus(-d),   log Q - log M = ln 2 - softplus(d),
// and softplus(x) = max(x, 0) + log(1 + e^-|x|) never overflows: e^-|x| <= 1.  The
// kernels work in base 2 (u = log2 of a probability, sp2 = softplus in bits), which is
// what the hardware exp2 / log2 units compute, and scale by ln 2 once per row.
//
// The terms need both row normalisers, so the forward reads each row twice: pass 1 keeps
// the online (m, s) pairs of q and p, the lanes of a row agree on them (butterfly, and
// for one workgroup per row one exchange through LDS), pass 2 sums the two halves, and a
// second exchange through a separate LDS array combines them.  Every wave passes the
// row's second barrier only after all waves have read the first array, and wave 0 reads
// the second array before it reaches the next row's first barrier, so no slot is written
// again before it has been read ("One barrier short", The fix).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace ce {
namespace {

constexpr int kBlock = 256;

struct JSStats {
    MS q, p;
};

__device__ __forceinline__ JSStats js_empty() { return JSStats{ms_empty(), ms_empty()}; }

__device__ __forceinline__ JSStats js_merge(const JSStats& a, const JSStats& b) {
    return JSStats{ms_merge(a.q, b.q), ms_merge(a.p, b.p)};
}

template <int G>
__device__ __forceinline__ JSStats js_stats_reduce(JSStats st) {
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) {
        JSStats o{MS{__shfl_xor(st.q.m, off, G), __shfl_xor(st.q.s, off, G)},
                  MS{__shfl_xor(st.p.m, off, G), __shfl_xor(st.p.s, off, G)}};
        st = js_merge(st, o);
    }
    return st;
}

template <int G>
__device__ __forceinline__ float2 sum2_reduce(float2 v) {
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) {
        v.x += __shfl_xor(v.x, off, G);
        v.y += __shfl_xor(v.y, off, G);
    }
    return v;
}

// Per-row constants: u(z) = (z - m) log2 e - log2 s is log2 of the probability.
struct JSRow {
    float mq, lq2;  // student max, log2 s_q
    float mp, lp2;  // teacher max, log2 s_p
};

__device__ __forceinline__ float log2_of(float s) {
#pragma clang fp contract(off)
    return log_e(s) * kLog2e;  // log s rounded as stored, then in bits
}

__device__ __forceinline__ JSRow js_row(const JSStats& st) {
    return JSRow{st.q.m, log2_of(st.q.s), st.p.m, log2_of(st.p.s)};
}

// softplus in bits: sp2(x) = max(x, 0) + log2(1 + 2^-|x|).
struct SP2 {
    float pos, neg;  // sp2(d) and sp2(-d)
};

__device__ __forceinline__ SP2 softplus2_pair(float d) {
    const float l = __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(-__builtin_fabsf(d)));
    return SP2{fmaxf(d, 0.f) + l, fmaxf(-d, 0.f) + l};
}

// Pass-2 terms of one element, in bits: P (1 - sp2(-d)) and Q (1 - sp2(d)); a zero
// probability contributes nothing (0 log 0 = 0).
__device__ __forceinline__ void js_terms(float q, float p, const JSRow& r, float2& acc) {
    const float uq = __builtin_fmaf(q - r.mq, kLog2e, -r.lq2);
    const float up = __builtin_fmaf(p - r.mp, kLog2e, -r.lp2);
    const SP2 sp = softplus2_pair(up - uq);
    const float P = __builtin_amdgcn_exp2f(up), Q = __builtin_amdgcn_exp2f(uq);
    acc.x += P > 0.f ? P * (1.f - sp.neg) : 0.f;
    acc.y += Q > 0.f ? Q * (1.f - sp.pos) : 0.f;
}

struct JSFwdArgs {
    const void* q;
    RowLayout ql;
    const void* p;
    RowLayout pl;
    int64_t n_rows;
    int64_t V;
    float* js;
    float2* lse_q;
    float2* lse_p;
    float* hq;
};

__device__ __forceinline__ void js_store(const JSFwdArgs& a, int64_t r, const JSStats& st, float2 acc) {
    const bool ok = st.q.m != kNegInf && st.p.m != kNegInf;
    const float H = 0.5f * kLn2 * acc.y;
    a.js[r] = ok ? 0.5f * kLn2 * (acc.x + acc.y) : __builtin_nanf("");
    a.hq[r] = ok ? H : __builtin_nanf("");
    a.lse_q[r] = make_float2(st.q.m, log_e(st.q.s));
    a.lse_p[r] = make_float2(st.p.m, log_e(st.p.s));
}

// Streams this lane's share of both rows through `fn(float q, float p)`: 16-byte vectors
// lane, lane + G, ... in groups of U when q and p share a 16-byte phase, element by
// element otherwise.
template <typename T, int G, int U, typename Fn>
__device__ __forceinline__ void js_stream(const T* qrow, const T* prow, int64_t V, int lane, Fn&& fn) {
    constexpr int kVec = Elem<T>::kVec;
    if (((((uintptr_t)qrow) ^ ((uintptr_t)prow)) & 15u) == 0) {
        RowSplit<T> sp(qrow, V);
        const char* qb = reinterpret_cast<const char*>(qrow + sp.head);
        const char* pb = reinterpret_cast<const char*>(prow + sp.head);
        int64_t j = lane;
        for (; j + (int64_t)(U - 1) * G < sp.nvec; j += (int64_t)U * G) {
            U4 bq[U], bp[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                bq[u] = load_u4_stream(qb + (j + (int64_t)u * G) * 16);
                bp[u] = load_u4_stream(pb + (j + (int64_t)u * G) * 16);
            }
            float fq[U * kVec], fp[U * kVec];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float tq[kVec], tp[kVec];
                Elem<T>::unpack(bq[u], tq);
                Elem<T>::unpack(bp[u], tp);
#pragma unroll
                for (int k = 0; k < kVec; ++k) {
                    fq[u * kVec + k] = tq[k];
                    fp[u * kVec + k] = tp[k];
                }
            }
            fn(fq, fp);
        }
        for (; j < sp.nvec; j += G) {
            float fq[kVec], fp[kVec];
            Elem<T>::unpack(load_u4_stream(qb + j * 16), fq);
            Elem<T>::unpack(load_u4_stream(pb + j * 16), fp);
            fn(fq, fp);
        }
        const int64_t ns = sp.n_scalar(V);
        for (int64_t k = lane; k < ns; k += G) {
            const int64_t i = sp.scalar_index(k);
            const float fq[1] = {Elem<T>::load1(qrow + i)}, fp[1] = {Elem<T>::load1(prow + i)};
            fn(fq, fp);
        }
    } else {
        for (int64_t i = lane; i < V; i += G) {
            const float fq[1] = {Elem<T>::load1(qrow + i)}, fp[1] = {Elem<T>::load1(prow + i)};
            fn(fq, fp);
        }
    }
}

template <typename T, int G, int U>
__device__ __forceinline__ JSStats js_pass1(const T* q, const T* p, int64_t V, int lane) {
    JSStats st = js_empty();
    js_stream<T, G, U>(q, p, V, lane, [&](const auto& fq, const auto& fp) {
        ms_add(st.q, fq);
        ms_add(st.p, fp);
    });
    return st;
}

template <typename T, int G, int U>
__device__ __forceinline__ float2 js_pass2(const T* q, const T* p, int64_t V, int lane, const JSRow& rw) {
    float2 acc = make_float2(0.f, 0.f);
    js_stream<T, G, U>(q, p, V, lane, [&](const auto& fq, const auto& fp) {
        constexpr int N = sizeof(fq) / sizeof(float);
#pragma unroll
        for (int k = 0; k < N; ++k) js_terms(fq[k], fp[k], rw, acc);
    });
    return acc;
}

template <typename T, int G, int U>
__global__ __launch_bounds__(kBlock) void js_fwd_lanes(JSFwdArgs a) {
    constexpr int kRowsPerBlock = kBlock / G;
    const int lane = threadIdx.x % G;
    const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
    for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / G; r < a.n_rows; r += stride) {
        const T* q = static_cast<const T*>(a.q) + row_offset(r, a.ql);
        const T* p = static_cast<const T*>(a.p) + row_offset(r, a.pl);
        const JSStats st = js_stats_reduce<G>(js_pass1<T, G, U>(q, p, a.V, lane));
        const float2 acc = sum2_reduce<G>(js_pass2<T, G, U>(q, p, a.V, lane, js_row(st)));
        if (lane == 0) js_store(a, r, st, acc);
    }
}

template <typename T, int NW, int U>
__global__ __launch_bounds__(64 * NW, 8) void js_fwd_rowwg(JSFwdArgs a) {
    constexpr int G = 64 * NW;
    __shared__ JSStats stat_slots[NW];
    __shared__ float2 sum_slots[NW];
    const int tid = threadIdx.x;
    const int wave = tid / 64;
    const int lane = tid % 64;
    for (int64_t r = blockIdx.x; r < a.n_rows; r += gridDim.x) {
        const T* q = static_cast<const T*>(a.q) + row_offset(r, a.ql);
        const T* p = static_cast<const T*>(a.p) + row_offset(r, a.pl);
        JSStats st = js_stats_reduce<64>(js_pass1<T, G, U>(q, p, a.V, tid));
        if (lane == 0) stat_slots[wave] = st;
        __syncthreads();
        // every wave folds all slots in the same order, so all agree bit for bit
        st = stat_slots[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) st = js_merge(st, stat_slots[w]);
        float2 acc = sum2_reduce<64>(js_pass2<T, G, U>(q, p, a.V, tid, js_row(st)));
        if (lane == 0) sum_slots[wave] = acc;
        __syncthreads();
        if (tid == 0) {
            float2 t = sum_slots[0];
            for (int w = 1; w < NW; ++w) {
                t.x += sum_slots[w].x;
                t.y += sum_slots[w].y;
            }
            js_store(a, r, st, t);
        }
    }
}

// ---- VJP --------------------------------------------------------------------------

struct JSVjpArgs {
    const void* q;
    RowLayout ql;
    const void* p;
    RowLayout pl;
    const float2* lse_q;
    const float2* lse_p;
    const float* hq;
    const float* g;
    int64_t n_rows;
    int64_t V;
    void* dq;
    RowLayout dl;
};

struct JSGrad {
    JSRow r;
    float H2;  // H in bits
    float gl;  // g ln 2 (times 2^-S)
};

// The row's constants on the output type's exponent shift S (out_shift, with room for the
// factor h2 - H2, below 2^7 in size wherever 2^S Q is nonzero): both log2-probabilities
// carry + S, so Q comes out times 2^S while their difference d keeps its value, and g ln 2
// is taken times 2^-S.
template <typename T>
__device__ __forceinline__ JSGrad js_grad_row(const JSVjpArgs& a, int64_t r) {
    const float2 lq = a.lse_q[r], lp = a.lse_p[r];
    const float gl = a.g[r] * kLn2;
    const int S = out_shift<T>(gl, 8);
    return JSGrad{JSRow{lq.x, lq.y * kLog2e - (float)S, lp.x, lp.y * kLog2e - (float)S}, a.hq[r] * kLog2e,
                  __builtin_ldexpf(gl, -S)};
}

// g Q (h - H) = g ln 2 Q (h2 - H2), h2 = (1 - sp2(d)) / 2 in bits; 0 where Q = 0.  uq and up
// are the log2-probabilities plus S, so Q here is 2^S Q.
__device__ __forceinline__ float js_grad(float q, float p, const JSGrad& w) {
    const float uq = __builtin_fmaf(q - w.r.mq, kLog2e, -w.r.lq2);
    const float up = __builtin_fmaf(p - w.r.mp, kLog2e, -w.r.lp2);
    const SP2 sp = softplus2_pair(up - uq);
    const float Q = __builtin_amdgcn_exp2f(uq);
    const float h2 = 0.5f * (1.f - sp.pos);
    return Q > 0.f ? w.gl * (Q * (h2 - w.H2)) : (Q == 0.f ? 0.f : Q);
}

template <typename T>
__device__ __forceinline__ void js_vec(const U4& bq, const U4& bp, const JSGrad& w, char* dst) {
    constexpr int kVec = Elem<T>::kVec;
    float fq[kVec], fp[kVec], o[kVec];
    Elem<T>::unpack(bq, fq);
    Elem<T>::unpack(bp, fp);
#pragma unroll
    for (int k = 0; k < kVec; ++k) o[k] = js_grad(fq[k], fp[k], w);
    store_u4(dst, Elem<T>::pack(o));
}

template <typename T>
__device__ __forceinline__ bool js_phases(const T* q, const T* p, const T* d) {
    const uintptr_t aq = (uintptr_t)q;
    return ((aq ^ (uintptr_t)p) & 15u) == 0 && ((aq ^ (uintptr_t)d) & 15u) == 0;
}

template <typename T, int G, int U>
__global__ __launch_bounds__(G > kBlock ? G : kBlock) void js_vjp_lanes(JSVjpArgs a) {
    constexpr int kThreads = G > kBlock ? G : kBlock;
    constexpr int kRowsPerBlock = kThreads / G;
    const int lane = threadIdx.x % G;
    const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
    for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / G; r < a.n_rows; r += stride) {
        const T* q = static_cast<const T*>(a.q) + row_offset(r, a.ql);
        const T* p = static_cast<const T*>(a.p) + row_offset(r, a.pl);
        T* d = static_cast<T*>(a.dq) + row_offset(r, a.dl);
        const JSGrad w = js_grad_row<T>(a, r);
        if (js_phases(q, p, d)) {
            RowSplit<T> sp(q, a.V);
            const char* qb = reinterpret_cast<const char*>(q + sp.head);
            const char* pb = reinterpret_cast<const char*>(p + sp.head);
            char* db = reinterpret_cast<char*>(d + sp.head);
            int64_t j = lane;
            for (; j + (int64_t)(U - 1) * G < sp.nvec; j += (int64_t)U * G) {
                U4 bq[U], bp[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    bq[u] = load_u4_stream(qb + (j + (int64_t)u * G) * 16);
                    bp[u] = load_u4_stream(pb + (j + (int64_t)u * G) * 16);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) js_vec<T>(bq[u], bp[u], w, db + (j + (int64_t)u * G) * 16);
            }
            for (; j < sp.nvec; j += G) js_vec<T>(load_u4_stream(qb + j * 16), load_u4_stream(pb + j * 16), w, db + j * 16);
            const int64_t ns = sp.n_scalar(a.V);
            for (int64_t k = lane; k < ns; k += G) {
                const int64_t i = sp.scalar_index(k);
                Elem<T>::store1(d + i, js_grad(Elem<T>::load1(q + i), Elem<T>::load1(p + i), w));
            }
        } else {
            for (int64_t i = lane; i < a.V; i += G)
                Elem<T>::store1(d + i, js_grad(Elem<T>::load1(q + i), Elem<T>::load1(p + i), w));
        }
    }
}

template <typename T, int U>
__global__ __launch_bounds__(kBlock) void js_vjp_chunks(JSVjpArgs a, int64_t chunks_per_row) {
    constexpr int kVec = Elem<T>::kVec;
    constexpr int64_t kChunkVec = (int64_t)kBlock * U;
    const int tid = threadIdx.x;
    const int64_t items = a.n_rows * chunks_per_row;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int64_t r = it / chunks_per_row;
        const int64_t c = it - r * chunks_per_row;
        const T* q = static_cast<const T*>(a.q) + row_offset(r, a.ql);
        const T* p = static_cast<const T*>(a.p) + row_offset(r, a.pl);
        T* d = static_cast<T*>(a.dq) + row_offset(r, a.dl);
        const JSGrad w = js_grad_row<T>(a, r);
        if (js_phases(q, p, d)) {
            RowSplit<T> sp(q, a.V);
            const char* qb = reinterpret_cast<const char*>(q + sp.head);
            const char* pb = reinterpret_cast<const char*>(p + sp.head);
            char* db = reinterpret_cast<char*>(d + sp.head);
            const int64_t v0 = c * kChunkVec + tid;
            if (c * kChunkVec + kChunkVec <= sp.nvec) {
                U4 bq[U], bp[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    bq[u] = load_u4_stream(qb + (v0 + (int64_t)u * kBlock) * 16);
                    bp[u] = load_u4_stream(pb + (v0 + (int64_t)u * kBlock) * 16);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) js_vec<T>(bq[u], bp[u], w, db + (v0 + (int64_t)u * kBlock) * 16);
            } else {
                for (int64_t j = v0; j < sp.nvec; j += kBlock)
                    js_vec<T>(load_u4_stream(qb + j * 16), load_u4_stream(pb + j * 16), w, db + j * 16);
            }
            if (c == 0) {
                const int64_t ns = sp.n_scalar(a.V);
                for (int64_t k = tid; k < ns; k += kBlock) {
                    const int64_t i = sp.scalar_index(k);
                    Elem<T>::store1(d + i, js_grad(Elem<T>::load1(q + i), Elem<T>::load1(p + i), w));
                }
            }
        } else {
            const int64_t e0 = c * kChunkVec * kVec;
            const int64_t e1 = e0 + kChunkVec * kVec < a.V ? e0 + kChunkVec * kVec : a.V;
            for (int64_t i = e0 + tid; i < e1; i += kBlock)
                Elem<T>::store1(d + i, js_grad(Elem<T>::load1(q + i), Elem<T>::load1(p + i), w));
        }
    }
}

// ---- dispatch -----------------------------------------------------------------------

RowLayout js_layout(const HostLayout& h) { return RowLayout{h.rows_per_batch, h.row_stride, h.batch_stride, h.uniform}; }

template <typename T>
hipError_t js_fwd_typed(const JSFwdCall& c) {
    JSFwdArgs a{c.q,    js_layout(c.ql), c.p, js_layout(c.pl), c.n_rows, c.V, c.js, reinterpret_cast<float2*>(c.lse_q),
                reinterpret_cast<float2*>(c.lse_p), c.hq};
    const dim3 grid((unsigned)c.plan.blocks);
    constexpr int kU = Elem<T>::kVec == 8 ? 1 : 2;  // 8 elements of each row per step
    switch (c.plan.lanes) {
        case 1: hipLaunchKernelGGL((js_fwd_lanes<T, 1, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 2: hipLaunchKernelGGL((js_fwd_lanes<T, 2, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 4: hipLaunchKernelGGL((js_fwd_lanes<T, 4, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 8: hipLaunchKernelGGL((js_fwd_lanes<T, 8, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 16: hipLaunchKernelGGL((js_fwd_lanes<T, 16, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 32: hipLaunchKernelGGL((js_fwd_lanes<T, 32, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 64: hipLaunchKernelGGL((js_fwd_lanes<T, 64, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 128: hipLaunchKernelGGL((js_fwd_rowwg<T, 2, kU>), grid, dim3(128), 0, c.stream, a); break;
        case 256: hipLaunchKernelGGL((js_fwd_rowwg<T, 4, kU>), grid, dim3(256), 0, c.stream, a); break;
        case 512: hipLaunchKernelGGL((js_fwd_rowwg<T, 8, kU>), grid, dim3(512), 0, c.stream, a); break;
        case 1024: hipLaunchKernelGGL((js_fwd_rowwg<T, 16, kU>), grid, dim3(1024), 0, c.stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t js_vjp_typed(const JSVjpCall& c) {
    JSVjpArgs a{c.q,     js_layout(c.ql), c.p,      js_layout(c.pl), reinterpret_cast<const float2*>(c.lse_q),
                reinterpret_cast<const float2*>(c.lse_p), c.hq, c.g, c.n_rows, c.V, c.dq, js_layout(c.dl)};
    const dim3 grid((unsigned)c.plan.blocks);
    if (c.plan.chunks > 0) {
        hipLaunchKernelGGL((js_vjp_chunks<T, kChunkU>), grid, dim3(kBlock), 0, c.stream, a, c.plan.chunks);
        return hipGetLastError();
    }
    constexpr int kU = Elem<T>::kVec == 8 ? 1 : 2;
    switch (c.plan.lanes) {
        case 1: hipLaunchKernelGGL((js_vjp_lanes<T, 1, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 2: hipLaunchKernelGGL((js_vjp_lanes<T, 2, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 4: hipLaunchKernelGGL((js_vjp_lanes<T, 4, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 8: hipLaunchKernelGGL((js_vjp_lanes<T, 8, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 16: hipLaunchKernelGGL((js_vjp_lanes<T, 16, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 32: hipLaunchKernelGGL((js_vjp_lanes<T, 32, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 64: hipLaunchKernelGGL((js_vjp_lanes<T, 64, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 128: hipLaunchKernelGGL((js_vjp_lanes<T, 128, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 256: hipLaunchKernelGGL((js_vjp_lanes<T, 256, kU>), grid, dim3(256), 0, c.stream, a); break;
        case 512: hipLaunchKernelGGL((js_vjp_lanes<T, 512, kU>), grid, dim3(512), 0, c.stream, a); break;
        case 1024: hipLaunchKernelGGL((js_vjp_lanes<T, 1024, kU>), grid, dim3(1024), 0, c.stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_js_forward(const JSFwdCall& c) {
    switch (c.dt) {
        case Dt::F32: return js_fwd_typed<float>(c);
        case Dt::F16: return js_fwd_typed<_Float16>(c);
        case Dt::BF16: return js_fwd_typed<__bf16>(c);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_js_vjp(const JSVjpCall& c) {
    switch (c.dt) {
        case Dt::F32: return js_vjp_typed<float>(c);
        case Dt::F16: return js_vjp_typed<_Float16>(c);
        case Dt::BF16: return js_vjp_typed<__bf16>(c);
    }
    return hipErrorInvalidValue;
}

}  // namespace ce
