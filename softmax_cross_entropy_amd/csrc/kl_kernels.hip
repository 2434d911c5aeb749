// Row-wise KL divergence of a teacher row p from a student row q, and its gradient
// with respect to q, for gfx950.
//
// "One barrier short", section "Run it yourself": with lq, lp the log-softmaxes of
// the student and teacher logits, kl = sum_j exp(lp_j) (lp_j - lq_j), and the gradient
// of sum_i g_i kl_i with respect to q_i is g_i (softmax(q_i) - softmax(p_i)).  The
// page's section "Sixty-four floats" describes the fused kernel: one threadgroup per
// row keeps two online log-sum-exps, one per distribution, and combines them across
// SIMD groups through shared memory (where the shipped version reused one scratch
// array for two exchanges without a barrier between them).
//
// One pass per row keeps, per lane, the online pair (m_q, s_q) of the student, the
// pair (m_p, s_p) of the teacher and
//   t = sum_j exp(p_j - m_p) ((p_j - m_p) - (q_j - m_q)),
// each logit taken against its own row's running maximum and t rescaled with s_p.
// Since sum_j softmax(p)_j = 1,
//   kl = t / s_p - log s_p + log s_q,
// so neither log-softmax is ever materialised.  Every term of t is a difference of
// logits of one row, so t / s_p stays of the size of the rows' spread whatever offset
// either row carries: a sum over the raw differences p_j - q_j would carry the offset
// gap m_p - m_q and cancel it against the maxima at the end, losing the result in
// float32 once that gap reaches 1e4.  When a maximum moves, the terms already in t
// shift by the move: t' = c (t + s_p ((m_p - m_p') - (m_q - m_q'))), c = exp(m_p - m_p').
// A teacher entry whose weight exp(p_j - m_p) is 0 (p_j = -inf) contributes nothing
// to t (0 log 0 = 0).
//
// Row layouts as in the cross-entropy kernels: G lanes per row (G <= 64, 64 / G rows
// per wavefront) or one workgroup of 64 * NW threads per row, whose waves exchange
// their states once through LDS slots that alternate between two buffers from row to
// row (the page's fix: no scratch slot is written again before it has been read).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace ce {
namespace {

constexpr int kBlock = 256;

struct KLState {
    float mq, sq;  // student: running max and sum exp(q - mq)
    float mp, sp;  // teacher: running max and sum exp(p - mp)
    float t;       // sum exp(p - mp) ((p - mp) - (q - mq)), rescaled with sp
};

__device__ __forceinline__ KLState kl_empty() { return KLState{kNegInf, 0.f, kNegInf, 0.f, 0.f}; }

// The terms already in t, taken against the reference points (rq, rp), moved to the
// reference points (nq, np): each term gains (rp - np) - (rq - nq), and the teacher
// weights scale by c = exp(rp - np).  Reference points are ref_point of the maxima, so
// an empty state (s_p = 0, t = 0) moves to any point without forming -inf - -inf.
__device__ __forceinline__ float kl_shift_t(float t, float sp, float rq, float rp, float nq, float np_,
                                            float c) {
#pragma clang fp contract(off)
    return __fmul_rn(t + __fmul_rn(sp, (rp - np_) - (rq - nq)), c);
}

// Folds N pairs (q_k, p_k) into the state with one rescale per distribution.
template <int N>
__device__ __forceinline__ void kl_add(KLState& st, const float (&q)[N], const float (&p)[N]) {
    float tq = q[0], tp = p[0];
#pragma unroll
    for (int k = 1; k < N; ++k) {
        tq = fmaxf(tq, q[k]);
        tp = fmaxf(tp, p[k]);
    }
    const float mq = fmaxf(st.mq, tq), mp = fmaxf(st.mp, tp);
    const float rq = ref_point(mq), rp = ref_point(mp);
    float sq = 0.f, sp = 0.f, t = 0.f;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const float dq = q[k] - rq;
        sq += exp_e(dq);
        const float dp = p[k] - rp;
        const float w = exp_e(dp);
        sp += w;
        t += w > 0.f ? w * (dp - dq) : 0.f;
    }
    const float cp = exp_e(st.mp - rp);
    st.t = kl_shift_t(st.t, st.sp, ref_point(st.mq), ref_point(st.mp), rq, rp, cp) + t;
    st.sq = __fmul_rn(st.sq, exp_e(st.mq - rq)) + sq;
    st.sp = __fmul_rn(st.sp, cp) + sp;
    st.mq = mq;
    st.mp = mp;
}

// Merge of two states; symmetric bit for bit (each product is rounded on its own: no
// fused multiply-add).
__device__ __forceinline__ KLState kl_merge(const KLState& a, const KLState& b) {
#pragma clang fp contract(off)
    KLState o;
    const MS q = ms_merge(MS{a.mq, a.sq}, MS{b.mq, b.sq});
    o.mq = q.m;
    o.sq = q.s;
    o.mp = fmaxf(a.mp, b.mp);
    const float rq = ref_point(o.mq), rp = ref_point(o.mp);
    const float ca = exp_e(a.mp - rp), cb = exp_e(b.mp - rp);
    o.sp = __fmul_rn(a.sp, ca) + __fmul_rn(b.sp, cb);
    o.t = kl_shift_t(a.t, a.sp, ref_point(a.mq), ref_point(a.mp), rq, rp, ca) +
          kl_shift_t(b.t, b.sp, ref_point(b.mq), ref_point(b.mp), rq, rp, cb);
    return o;
}

template <int G>
__device__ __forceinline__ KLState kl_group_reduce(KLState st) {
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) {
        KLState o{__shfl_xor(st.mq, off, G), __shfl_xor(st.sq, off, G), __shfl_xor(st.mp, off, G),
                  __shfl_xor(st.sp, off, G), __shfl_xor(st.t, off, G)};
        st = kl_merge(st, o);
    }
    return st;
}

struct KLFwdArgs {
    const void* q;
    RowLayout ql;
    const void* p;
    RowLayout pl;
    int64_t n_rows;
    int64_t V;
    float* kl;
    float2* lse_q;
    float2* lse_p;
};

__device__ __forceinline__ void kl_store(const KLFwdArgs& a, int64_t r, const KLState& st) {
    const float lsq = log_e(st.sq), lsp = log_e(st.sp);
    a.kl[r] = st.t / st.sp + (lsq - lsp);
    a.lse_q[r] = make_float2(st.mq, lsq);
    a.lse_p[r] = make_float2(st.mp, lsp);
}

// This lane's share of one row pair: vectors lane, lane + G, ... in groups of U when
// both rows have the same 16-byte phase, element by element otherwise.
template <typename T, int G, int U>
__device__ __forceinline__ void kl_stream_row(const T* qrow, const T* prow, int64_t V, int lane, KLState& st) {
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
            kl_add<U * kVec>(st, fq, fp);
        }
        for (; j < sp.nvec; j += G) {
            float fq[kVec], fp[kVec];
            Elem<T>::unpack(load_u4_stream(qb + j * 16), fq);
            Elem<T>::unpack(load_u4_stream(pb + j * 16), fp);
            kl_add<kVec>(st, fq, fp);
        }
        const int64_t ns = sp.n_scalar(V);
        for (int64_t k = lane; k < ns; k += G) {
            const int64_t i = sp.scalar_index(k);
            const float fq[1] = {Elem<T>::load1(qrow + i)}, fp[1] = {Elem<T>::load1(prow + i)};
            kl_add<1>(st, fq, fp);
        }
    } else {
        for (int64_t i = lane; i < V; i += G) {
            const float fq[1] = {Elem<T>::load1(qrow + i)}, fp[1] = {Elem<T>::load1(prow + i)};
            kl_add<1>(st, fq, fp);
        }
    }
}

template <typename T, int G, int U>
__global__ __launch_bounds__(kBlock) void kl_fwd_lanes(KLFwdArgs a) {
    constexpr int kRowsPerBlock = kBlock / G;
    const int lane = threadIdx.x % G;
    const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
    for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / G; r < a.n_rows; r += stride) {
        const T* q = static_cast<const T*>(a.q) + row_offset(r, a.ql);
        const T* p = static_cast<const T*>(a.p) + row_offset(r, a.pl);
        KLState st = kl_empty();
        kl_stream_row<T, G, U>(q, p, a.V, lane, st);
        st = kl_group_reduce<G>(st);
        if (lane == 0) kl_store(a, r, st);
    }
}

template <typename T, int NW, int U>
__global__ __launch_bounds__(64 * NW) void kl_fwd_rowwg(KLFwdArgs a) {
    constexpr int G = 64 * NW;
    // One state per wave; the slots alternate between two buffers from row to row, so a
    // wave that runs ahead to the next row writes the other buffer, and that row's
    // barrier keeps it from coming back to this one before wave 0 has read it.
    __shared__ KLState slots[2][NW];
    const int tid = threadIdx.x;
    const int wave = tid / 64;
    const int lane = tid % 64;
    int parity = 0;
    for (int64_t r = blockIdx.x; r < a.n_rows; r += gridDim.x, parity ^= 1) {
        const T* q = static_cast<const T*>(a.q) + row_offset(r, a.ql);
        const T* p = static_cast<const T*>(a.p) + row_offset(r, a.pl);
        KLState st = kl_empty();
        kl_stream_row<T, G, U>(q, p, a.V, tid, st);
        st = kl_group_reduce<64>(st);
        if (lane == 0) slots[parity][wave] = st;
        __syncthreads();
        if (wave == 0) {
            KLState t = lane < NW ? slots[parity][lane] : kl_empty();
            t = kl_group_reduce<NW>(t);
            if (lane == 0) kl_store(a, r, t);
        }
    }
}

// ---- VJP --------------------------------------------------------------------------

struct KLVjpArgs {
    const void* q;
    RowLayout ql;
    const void* p;
    RowLayout pl;
    const float2* lse_q;
    const float2* lse_p;
    const float* g;
    int64_t n_rows;
    int64_t V;
    void* dq;
    RowLayout dl;
};

// Per-row constants on the output type's exponent shift S (out_shift): both softmax
// values come out times 2^S and g is taken times 2^-S.
struct KLRow {
    float mq, cq;  // student max, S - log s_q * log2(e)
    float mp, cp;  // teacher max, S - log s_p * log2(e)
    float g;       // g 2^-S
};

template <typename T>
__device__ __forceinline__ KLRow kl_row(float2 lq, float2 lp, float g) {
    const int S = out_shift<T>(g);
    return KLRow{lq.x, (float)S - lq.y * kLog2e, lp.x, (float)S - lp.y * kLog2e, __builtin_ldexpf(g, -S)};
}

// softmax value times 2^S from (z - m) and the row's constant: (z - m) is formed first.
__device__ __forceinline__ float soft(float z, float m, float c) {
    return __builtin_amdgcn_exp2f(__builtin_fmaf(z - m, kLog2e, c));
}

__device__ __forceinline__ float kl_grad(float q, float p, const KLRow& r) {
    return r.g * (soft(q, r.mq, r.cq) - soft(p, r.mp, r.cp));
}

template <typename T, int G, int U>
__global__ __launch_bounds__(G > kBlock ? G : kBlock) void kl_vjp_lanes(KLVjpArgs a) {
    constexpr int kVec = Elem<T>::kVec;
    constexpr int kThreads = G > kBlock ? G : kBlock;
    constexpr int kRowsPerBlock = kThreads / G;
    const int lane = threadIdx.x % G;
    const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
    for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / G; r < a.n_rows; r += stride) {
        const T* q = static_cast<const T*>(a.q) + row_offset(r, a.ql);
        const T* p = static_cast<const T*>(a.p) + row_offset(r, a.pl);
        T* d = static_cast<T*>(a.dq) + row_offset(r, a.dl);
        const float2 lq = a.lse_q[r], lp = a.lse_p[r];
        const KLRow rw = kl_row<T>(lq, lp, a.g[r]);
        const uintptr_t aq = (uintptr_t)q, ap = (uintptr_t)p, ad = (uintptr_t)d;
        if (((aq ^ ap) & 15u) == 0 && ((aq ^ ad) & 15u) == 0) {
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
                for (int u = 0; u < U; ++u) {
                    float fq[kVec], fp[kVec], o[kVec];
                    Elem<T>::unpack(bq[u], fq);
                    Elem<T>::unpack(bp[u], fp);
#pragma unroll
                    for (int k = 0; k < kVec; ++k) o[k] = kl_grad(fq[k], fp[k], rw);
                    store_u4(db + (j + (int64_t)u * G) * 16, Elem<T>::pack(o));
                }
            }
            for (; j < sp.nvec; j += G) {
                float fq[kVec], fp[kVec], o[kVec];
                Elem<T>::unpack(load_u4_stream(qb + j * 16), fq);
                Elem<T>::unpack(load_u4_stream(pb + j * 16), fp);
#pragma unroll
                for (int k = 0; k < kVec; ++k) o[k] = kl_grad(fq[k], fp[k], rw);
                store_u4(db + j * 16, Elem<T>::pack(o));
            }
            const int64_t ns = sp.n_scalar(a.V);
            for (int64_t k = lane; k < ns; k += G) {
                const int64_t i = sp.scalar_index(k);
                Elem<T>::store1(d + i, kl_grad(Elem<T>::load1(q + i), Elem<T>::load1(p + i), rw));
            }
        } else {
            for (int64_t i = lane; i < a.V; i += G)
                Elem<T>::store1(d + i, kl_grad(Elem<T>::load1(q + i), Elem<T>::load1(p + i), rw));
        }
    }
}

// Long rows: the VJP is elementwise, so each row is cut into chunks of kChunkVec vectors
// and every (row, chunk) pair is one work item of a 256-thread workgroup.  With few rows,
// one workgroup per row leaves too few workgroups for the memory system; many short
// work items keep it full.  Chunk 0 of a row also takes the row's unaligned head and
// tail elements.
template <typename T, int U>
__global__ __launch_bounds__(kBlock) void kl_vjp_chunks(KLVjpArgs a, int64_t chunks_per_row) {
    constexpr int kVec = Elem<T>::kVec;
    constexpr int64_t kChunkVec = (int64_t)kBlock * U;
    const int t = threadIdx.x;
    const int64_t items = a.n_rows * chunks_per_row;
    for (int64_t w = blockIdx.x; w < items; w += gridDim.x) {
        const int64_t r = w / chunks_per_row;
        const int64_t c = w - r * chunks_per_row;
        const T* q = static_cast<const T*>(a.q) + row_offset(r, a.ql);
        const T* p = static_cast<const T*>(a.p) + row_offset(r, a.pl);
        T* d = static_cast<T*>(a.dq) + row_offset(r, a.dl);
        const float2 lq = a.lse_q[r], lp = a.lse_p[r];
        const KLRow rw = kl_row<T>(lq, lp, a.g[r]);
        const uintptr_t aq = (uintptr_t)q, ap = (uintptr_t)p, ad = (uintptr_t)d;
        if (((aq ^ ap) & 15u) == 0 && ((aq ^ ad) & 15u) == 0) {
            RowSplit<T> sp(q, a.V);
            const char* qb = reinterpret_cast<const char*>(q + sp.head);
            const char* pb = reinterpret_cast<const char*>(p + sp.head);
            char* db = reinterpret_cast<char*>(d + sp.head);
            const int64_t v0 = c * kChunkVec + t;
            if (c * kChunkVec + kChunkVec <= sp.nvec) {
                U4 bq[U], bp[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    bq[u] = load_u4_stream(qb + (v0 + (int64_t)u * kBlock) * 16);
                    bp[u] = load_u4_stream(pb + (v0 + (int64_t)u * kBlock) * 16);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float fq[kVec], fp[kVec], o[kVec];
                    Elem<T>::unpack(bq[u], fq);
                    Elem<T>::unpack(bp[u], fp);
#pragma unroll
                    for (int k = 0; k < kVec; ++k) o[k] = kl_grad(fq[k], fp[k], rw);
                    store_u4(db + (v0 + (int64_t)u * kBlock) * 16, Elem<T>::pack(o));
                }
            } else {
                for (int64_t j = v0; j < sp.nvec; j += kBlock) {
                    float fq[kVec], fp[kVec], o[kVec];
                    Elem<T>::unpack(load_u4_stream(qb + j * 16), fq);
                    Elem<T>::unpack(load_u4_stream(pb + j * 16), fp);
#pragma unroll
                    for (int k = 0; k < kVec; ++k) o[k] = kl_grad(fq[k], fp[k], rw);
                    store_u4(db + j * 16, Elem<T>::pack(o));
                }
            }
            if (c == 0) {
                const int64_t ns = sp.n_scalar(a.V);
                for (int64_t k = t; k < ns; k += kBlock) {
                    const int64_t i = sp.scalar_index(k);
                    Elem<T>::store1(d + i, kl_grad(Elem<T>::load1(q + i), Elem<T>::load1(p + i), rw));
                }
            }
        } else {
            const int64_t e0 = c * kChunkVec * kVec;
            const int64_t e1 = e0 + kChunkVec * kVec < a.V ? e0 + kChunkVec * kVec : a.V;
            for (int64_t i = e0 + t; i < e1; i += kBlock)
                Elem<T>::store1(d + i, kl_grad(Elem<T>::load1(q + i), Elem<T>::load1(p + i), rw));
        }
    }
}

RowLayout kl_layout(const HostLayout& h) {
    return RowLayout{h.rows_per_batch, h.row_stride, h.batch_stride, h.uniform};
}

template <typename T>
hipError_t kl_fwd_typed(const KLFwdCall& c) {
    KLFwdArgs a{c.q, kl_layout(c.ql), c.p, kl_layout(c.pl), c.n_rows, c.V, c.kl,
                reinterpret_cast<float2*>(c.lse_q), reinterpret_cast<float2*>(c.lse_p)};
    const dim3 grid((unsigned)c.plan.blocks);
    constexpr int kU = Elem<T>::kVec == 8 ? 1 : 2;  // 8 elements of each row per fold
    switch (c.plan.lanes) {
        case 1: hipLaunchKernelGGL((kl_fwd_lanes<T, 1, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 2: hipLaunchKernelGGL((kl_fwd_lanes<T, 2, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 4: hipLaunchKernelGGL((kl_fwd_lanes<T, 4, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 8: hipLaunchKernelGGL((kl_fwd_lanes<T, 8, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 16: hipLaunchKernelGGL((kl_fwd_lanes<T, 16, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 32: hipLaunchKernelGGL((kl_fwd_lanes<T, 32, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 64: hipLaunchKernelGGL((kl_fwd_lanes<T, 64, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 128: hipLaunchKernelGGL((kl_fwd_rowwg<T, 2, kU>), grid, dim3(128), 0, c.stream, a); break;
        case 256: hipLaunchKernelGGL((kl_fwd_rowwg<T, 4, kU>), grid, dim3(256), 0, c.stream, a); break;
        case 512: hipLaunchKernelGGL((kl_fwd_rowwg<T, 8, kU>), grid, dim3(512), 0, c.stream, a); break;
        case 1024: hipLaunchKernelGGL((kl_fwd_rowwg<T, 16, kU>), grid, dim3(1024), 0, c.stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t kl_vjp_typed(const KLVjpCall& c) {
    KLVjpArgs a{c.q, kl_layout(c.ql), c.p, kl_layout(c.pl), reinterpret_cast<const float2*>(c.lse_q),
                reinterpret_cast<const float2*>(c.lse_p), c.g, c.n_rows, c.V, c.dq, kl_layout(c.dl)};
    const dim3 grid((unsigned)c.plan.blocks);
    if (c.plan.chunks > 0) {
        hipLaunchKernelGGL((kl_vjp_chunks<T, kChunkU>), grid, dim3(kBlock), 0, c.stream, a, c.plan.chunks);
        return hipGetLastError();
    }
    constexpr int kU = Elem<T>::kVec == 8 ? 1 : 2;
    switch (c.plan.lanes) {
        case 1: hipLaunchKernelGGL((kl_vjp_lanes<T, 1, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 2: hipLaunchKernelGGL((kl_vjp_lanes<T, 2, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 4: hipLaunchKernelGGL((kl_vjp_lanes<T, 4, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 8: hipLaunchKernelGGL((kl_vjp_lanes<T, 8, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 16: hipLaunchKernelGGL((kl_vjp_lanes<T, 16, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 32: hipLaunchKernelGGL((kl_vjp_lanes<T, 32, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 64: hipLaunchKernelGGL((kl_vjp_lanes<T, 64, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 128: hipLaunchKernelGGL((kl_vjp_lanes<T, 128, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 256: hipLaunchKernelGGL((kl_vjp_lanes<T, 256, kU>), grid, dim3(256), 0, c.stream, a); break;
        case 512: hipLaunchKernelGGL((kl_vjp_lanes<T, 512, kU>), grid, dim3(512), 0, c.stream, a); break;
        case 1024: hipLaunchKernelGGL((kl_vjp_lanes<T, 1024, kU>), grid, dim3(1024), 0, c.stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kl_forward(const KLFwdCall& c) {
    switch (c.dt) {
        case Dt::F32: return kl_fwd_typed<float>(c);
        case Dt::F16: return kl_fwd_typed<_Float16>(c);
        case Dt::BF16: return kl_fwd_typed<__bf16>(c);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_kl_vjp(const KLVjpCall& c) {
    switch (c.dt) {
        case Dt::F32: return kl_vjp_typed<float>(c);
        case Dt::F16: return kl_vjp_typed<_Float16>(c);
        case Dt::BF16: return kl_vjp_typed<__bf16>(c);
    }
    return hipErrorInvalidValue;
}

}  // namespace ce
