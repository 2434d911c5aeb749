// Softmax cross-entropy forward and vector-Jacobian product for gfx950.
//
// Forward (per row z, target y):  m = max_j z_j,  s = sum_j exp(z_j - m),
//   loss = (m - z_y) + log s,  lse = (m, log s).
//   Ineshin, "A fused linear cross-entropy forward kernel for Apple GPUs", section 1
//   (loss from the log-sum-exp and the target logit; online (m, s) update); MLX PR
//   #4188 "Shift by the max in cross_entropy", Proposed changes (the max is taken
//   out before the target score, so the gap between logits survives at any
//   magnitude).
// VJP:  dlogits_j = g * (exp((z_j - m) - log s) - [j == y]), from the saved pair.
//
// Three row layouts, all HBM streaming with 16-byte loads coalesced across lanes:
//   * narrow: rows of 1, 2, 4 or 8 aligned vectors; one lane per row and several
//     rows per lane in flight.  The default takes it for forward rows of up to 2
//     vectors (the 1,048,576 x 8 fp32 shape has 2) and VJP rows of 1; for longer rows
//     one lane's vectors are 32 B or more apart and the instructions touch part lines;
//   * lanes:  G lanes per row (G <= 64), 64 / G rows per wavefront, online state
//     per lane, then a butterfly merge of (m, s) pairs across the G lanes;
//   * rowwg:  one workgroup of 64 * NW threads per row for long rows, per-wave
//     butterfly merge, then one exchange of (m, s) pairs through LDS.
// Every row loop is a grid-stride loop over 64-bit row indices, so the launch grid
// never has to cover all rows (MLX PR #4776 "fast.cross_entropy silently skips
// rows when the Metal grid gets too large", Issue).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace ce {
namespace {

constexpr int kBlock = 256;

struct FwdArgs {
    const void* logits;
    RowLayout in;
    const int32_t* targets;
    int64_t n_rows;
    int64_t V;
    float* loss;
    float2* lse;
};

struct VjpArgs {
    const void* logits;
    RowLayout in;
    const int32_t* targets;
    const float2* lse;
    const float* g;
    int64_t n_rows;
    int64_t V;
    void* dlogits;
    RowLayout out;
};

__device__ __forceinline__ bool target_ok(int32_t y, int64_t V) { return y >= 0 && (int64_t)y < V; }

__device__ __forceinline__ void store_forward(const FwdArgs& a, int64_t r, MS st, float zy, bool ok) {
    float ls = log_e(st.s);
    a.loss[r] = ok ? (st.m - zy) + ls : __builtin_nanf("");
    a.lse[r] = make_float2(st.m, ls);
}

// Streams this lane's share of one row into `st`: vectors lane, lane + G, ... in
// groups of U loads issued together, then the scalar head and tail elements.  There
// is no software pipelining across groups on purpose: a second group buffer would
// push the kernel past 64 VGPRs and halve the workgroups resident per CU, and the
// other resident waves hide load latency better than one wave's own prefetch does.
template <typename T, int U>
__device__ __forceinline__ void fold_group(MS& st, const U4 (&buf)[U]) {
    constexpr int kVec = Elem<T>::kVec;
    float f[U * kVec];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float t[kVec];
        Elem<T>::unpack(buf[u], t);
#pragma unroll
        for (int k = 0; k < kVec; ++k) f[u * kVec + k] = t[k];
    }
    ms_add<U * kVec>(st, f);
}

// Keep = true loads without the non-temporal hint, for a row that is read again.
template <bool Keep>
__device__ __forceinline__ U4 load_row_vec(const char* p) {
    return Keep ? load_u4(p) : load_u4_stream(p);
}

template <typename T, int G, int U, bool Keep = false>
__device__ __forceinline__ void stream_row(const T* row, int64_t V, int lane, MS& st) {
    constexpr int kVec = Elem<T>::kVec;
    RowSplit<T> sp(row, V);
    const char* vb = reinterpret_cast<const char*>(row + sp.head);
    int64_t j = lane;
    for (; j + (int64_t)(U - 1) * G < sp.nvec; j += (int64_t)U * G) {
        U4 buf[U];
#pragma unroll
        for (int u = 0; u < U; ++u) buf[u] = load_row_vec<Keep>(vb + (j + (int64_t)u * G) * 16);
        fold_group<T, U>(st, buf);
    }
    for (; j < sp.nvec; j += G) {
        float f[kVec];
        Elem<T>::unpack(load_row_vec<Keep>(vb + j * 16), f);
        ms_add<kVec>(st, f);
    }
    const int64_t ns = sp.n_scalar(V);
    for (int64_t k = lane; k < ns; k += G) ms_add1(st, Elem<T>::load1(row + sp.scalar_index(k)));
}

// ---- forward: one lane per short aligned row ------------------------------------

template <typename T, int NV, int UR>
__global__ __launch_bounds__(kBlock) void ce_fwd_narrow(FwdArgs a) {
    constexpr int kVec = Elem<T>::kVec;
    constexpr int kN = NV * kVec;
    const int64_t nthreads = (int64_t)gridDim.x * kBlock;
    const T* base = static_cast<const T*>(a.logits);
    for (int64_t r0 = (int64_t)blockIdx.x * kBlock + threadIdx.x; r0 < a.n_rows; r0 += nthreads * UR) {
        U4 buf[UR][NV];
        int32_t ys[UR];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int64_t r = r0 + u * nthreads;
            if (r < a.n_rows) {
                const char* row = reinterpret_cast<const char*>(base + row_offset(r, a.in));
#pragma unroll
                for (int v = 0; v < NV; ++v) buf[u][v] = load_u4_stream(row + v * 16);
                ys[u] = a.targets[r];
            }
        }
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int64_t r = r0 + u * nthreads;
            if (r < a.n_rows) {
                float f[kN];
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    float t[kVec];
                    Elem<T>::unpack(buf[u][v], t);
#pragma unroll
                    for (int k = 0; k < kVec; ++k) f[v * kVec + k] = t[k];
                }
                MS st = ms_empty();
                ms_add<kN>(st, f);
                // the target logit is already in registers
                const int32_t y = ys[u];
                float zy = 0.0f;
#pragma unroll
                for (int k = 0; k < kN; ++k) zy = (y == k) ? f[k] : zy;
                store_forward(a, r, st, zy, target_ok(y, kN));
            }
        }
    }
}

// ---- forward: G lanes per row, 64 / G rows per wavefront -------------------------

template <typename T, int G, int U>
__global__ __launch_bounds__(kBlock) void ce_fwd_lanes(FwdArgs a) {
    constexpr int kRowsPerBlock = kBlock / G;
    const int lane = threadIdx.x % G;
    const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
    for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / G; r < a.n_rows; r += stride) {
        const T* row = static_cast<const T*>(a.logits) + row_offset(r, a.in);
        const int32_t y = a.targets[r];
        const bool ok = target_ok(y, a.V);
        float zy = 0.0f;
        if (lane == 0 && ok) zy = Elem<T>::load1(row + y);
        MS st = ms_empty();
        stream_row<T, G, U>(row, a.V, lane, st);
        st = ms_group_reduce<G>(st);
        if (lane == 0) store_forward(a, r, st, zy, ok);
    }
}

// ---- forward: one workgroup of 64 * NW threads per row ---------------------------

template <typename T, int NW, int U>
__global__ __launch_bounds__(64 * NW) void ce_fwd_rowwg(FwdArgs a) {
    constexpr int G = 64 * NW;
    // One (m, s) slot per wave.  Each row is one exchange of pairs: lane 0 of every
    // wave writes its slot, one barrier, then wave 0 reads all slots.  The slots
    // alternate between two buffers from row to row, so a wave that races ahead to
    // the next row writes the other buffer, and the barrier of that next row keeps
    // it from reaching this buffer again before wave 0 has read it.  ("One barrier
    // short", sections "Sixty-four floats" and "The fix": reusing one scratch slot
    // for two exchanges without a barrier between them corrupted the row maximum.)
    __shared__ MS slots[2][NW];
    const int tid = threadIdx.x;
    const int wave = tid / 64;
    const int lane = tid % 64;
    int parity = 0;
    for (int64_t r = blockIdx.x; r < a.n_rows; r += gridDim.x, parity ^= 1) {
        const T* row = static_cast<const T*>(a.logits) + row_offset(r, a.in);
        const int32_t y = a.targets[r];
        const bool ok = target_ok(y, a.V);
        float zy = 0.0f;
        if (tid == 0 && ok) zy = Elem<T>::load1(row + y);
        MS st = ms_empty();
        stream_row<T, G, U>(row, a.V, tid, st);
        st = ms_group_reduce<64>(st);
        if (lane == 0) slots[parity][wave] = st;
        __syncthreads();
        if (wave == 0) {
            MS t = lane < NW ? slots[parity][lane] : ms_empty();
            t = ms_group_reduce<NW>(t);
            if (lane == 0) store_forward(a, r, t, zy, ok);
        }
    }
}

// ---- VJP ------------------------------------------------------------------------

// Per-row constants of the gradient, on the output type's exponent shift S (out_shift):
// the kernels form g p as (g 2^-S) (2^S p) and g (p - 1) as (g 2^-S) (2^S p - 2^S).
struct RowGrad {
    float m;    // row maximum, or NaN for a row whose target is out of range
    float c;    // S - log(s) log2(e)
    float g;    // g 2^-S
    float one;  // 2^S
    int32_t y;
};

template <typename T>
__device__ __forceinline__ void set_row_scale(RowGrad& rg, float ls, float g) {
    const int S = out_shift<T>(g);
    rg.c = (float)S - ls * kLog2e;
    rg.g = __builtin_ldexpf(g, -S);
    rg.one = __builtin_ldexpf(1.0f, S);
}

template <typename T>
__device__ __forceinline__ RowGrad load_row_grad(const VjpArgs& a, int64_t r) {
    RowGrad rg;
    rg.y = a.targets[r];
    const float2 l = a.lse[r];
    rg.m = target_ok(rg.y, a.V) ? l.x : __builtin_nanf("");
    set_row_scale<T>(rg, l.y, a.g[r]);
    return rg;
}

// softmax probability of logit z, times 2^S: exp((z - m) - log s) 2^S = 2^((z - m) log2 e +
// S - log s log2 e).  z - m is formed first (exact for nearby logits), and one fused
// multiply-add applies log2 e and the row's constant: no large magnitude ever meets the
// small gap.
__device__ __forceinline__ float prob(float z, const RowGrad& rg) {
    return __builtin_amdgcn_exp2f(__builtin_fmaf(z - rg.m, kLog2e, rg.c));
}

__device__ __forceinline__ float grad_elem(float z, const RowGrad& rg, bool is_target) {
    const float p = prob(z, rg);
    return rg.g * (is_target ? p - rg.one : p);
}

// Gradient of one 16-byte vector of logits, written to `dst` inside output row `orow`.  Every element is
// stored as g * p first; the one lane whose vector holds the target column (elements
// first .. first + kVec - 1) then stores that element again as g * (p - 1).  Both
// stores come from the same lane to the same address, so they land in program order,
// and the common path carries no per-element target test.
template <typename T>
__device__ __forceinline__ void grad_store_vec(const U4& in, const RowGrad& rg, int64_t first, char* dst,
                                               T* orow) {
    constexpr int kVec = Elem<T>::kVec;
    float f[kVec], out[kVec];
    Elem<T>::unpack(in, f);
#pragma unroll
    for (int k = 0; k < kVec; ++k) out[k] = rg.g * prob(f[k], rg);
    store_u4(dst, Elem<T>::pack(out));
    const int64_t rel = (int64_t)rg.y - first;
    if ((uint64_t)rel < (uint64_t)kVec) {
        float zy = f[0];
#pragma unroll
        for (int k = 1; k < kVec; ++k) zy = rel == k ? f[k] : zy;
        Elem<T>::store1(orow + rg.y, grad_elem(zy, rg, true));
    }
}

template <typename T, int NV, int UR>
__global__ __launch_bounds__(kBlock) void ce_vjp_narrow(VjpArgs a) {
    constexpr int kVec = Elem<T>::kVec;
    const int64_t nthreads = (int64_t)gridDim.x * kBlock;
    const T* base = static_cast<const T*>(a.logits);
    T* obase = static_cast<T*>(a.dlogits);
    for (int64_t r0 = (int64_t)blockIdx.x * kBlock + threadIdx.x; r0 < a.n_rows; r0 += nthreads * UR) {
        U4 buf[UR][NV];
        RowGrad rg[UR];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int64_t r = r0 + u * nthreads;
            if (r < a.n_rows) {
                const char* row = reinterpret_cast<const char*>(base + row_offset(r, a.in));
#pragma unroll
                for (int v = 0; v < NV; ++v) buf[u][v] = load_u4_stream(row + v * 16);
                rg[u] = load_row_grad<T>(a, r);
            }
        }
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int64_t r = r0 + u * nthreads;
            if (r < a.n_rows) {
                char* orow = reinterpret_cast<char*>(obase + row_offset(r, a.out));
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    grad_store_vec<T>(buf[u][v], rg[u], (int64_t)v * kVec, orow + v * 16,
                                      reinterpret_cast<T*>(orow));
            }
        }
    }
}

// Gradient of one row, on the G lanes (lane = 0 .. G - 1) that share it.
template <typename T, int G, int U>
__device__ __forceinline__ void grad_row(const T* row, T* orow, int64_t V, int lane, const RowGrad& rg) {
    constexpr int kVec = Elem<T>::kVec;
    const bool same_phase = (((uintptr_t)row ^ (uintptr_t)orow) & 15u) == 0;
    if (same_phase) {
        RowSplit<T> sp(row, V);
        const char* vb = reinterpret_cast<const char*>(row + sp.head);
        char* ob = reinterpret_cast<char*>(orow + sp.head);
        int64_t j = lane;
        for (; j + (int64_t)(U - 1) * G < sp.nvec; j += (int64_t)U * G) {
            U4 buf[U];
#pragma unroll
            for (int u = 0; u < U; ++u) buf[u] = load_u4_stream(vb + (j + (int64_t)u * G) * 16);
#pragma unroll
            for (int u = 0; u < U; ++u)
                grad_store_vec<T>(buf[u], rg, sp.head + (j + (int64_t)u * G) * kVec,
                                  ob + (j + (int64_t)u * G) * 16, orow);
        }
        for (; j < sp.nvec; j += G)
            grad_store_vec<T>(load_u4_stream(vb + j * 16), rg, sp.head + j * kVec, ob + j * 16, orow);
        const int64_t ns = sp.n_scalar(V);
        for (int64_t k = lane; k < ns; k += G) {
            const int64_t idx = sp.scalar_index(k);
            Elem<T>::store1(orow + idx, grad_elem(Elem<T>::load1(row + idx), rg, idx == rg.y));
        }
    } else {
        // input and output rows differ in 16-byte phase: element by element
        for (int64_t idx = lane; idx < V; idx += G)
            Elem<T>::store1(orow + idx, grad_elem(Elem<T>::load1(row + idx), rg, idx == rg.y));
    }
}

template <typename T, int G, int U>
__global__ __launch_bounds__(G > kBlock ? G : kBlock) void ce_vjp_lanes(VjpArgs a) {
    constexpr int kThreads = G > kBlock ? G : kBlock;
    constexpr int kRowsPerBlock = kThreads / G;
    const int lane = threadIdx.x % G;
    const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
    for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / G; r < a.n_rows; r += stride) {
        const T* row = static_cast<const T*>(a.logits) + row_offset(r, a.in);
        T* orow = static_cast<T*>(a.dlogits) + row_offset(r, a.out);
        grad_row<T, G, U>(row, orow, a.V, lane, load_row_grad<T>(a, r));
    }
}

// Long rows: the VJP is elementwise, so each row is cut into chunks of 256 * U vectors
// and every (row, chunk) pair is one work item of a 256-thread workgroup.  With few
// rows, one workgroup per row leaves too few workgroups for the memory system; many
// short work items keep it full.  The target column lies in exactly one chunk (or among
// the row's unaligned head and tail elements, which chunk 0 takes), so it is stored
// again exactly once, as in the row-wide layouts.
template <typename T, int U>
__global__ __launch_bounds__(kBlock) void ce_vjp_chunks(VjpArgs a, int64_t chunks_per_row) {
    constexpr int kVec = Elem<T>::kVec;
    constexpr int64_t kChunkVec = (int64_t)kBlock * U;
    const int t = threadIdx.x;
    const int64_t items = a.n_rows * chunks_per_row;
    for (int64_t w = blockIdx.x; w < items; w += gridDim.x) {
        const int64_t r = w / chunks_per_row;
        const int64_t c = w - r * chunks_per_row;
        const T* row = static_cast<const T*>(a.logits) + row_offset(r, a.in);
        T* orow = static_cast<T*>(a.dlogits) + row_offset(r, a.out);
        const RowGrad rg = load_row_grad<T>(a, r);
        if (((((uintptr_t)row) ^ ((uintptr_t)orow)) & 15u) == 0) {
            RowSplit<T> sp(row, a.V);
            const char* vb = reinterpret_cast<const char*>(row + sp.head);
            char* ob = reinterpret_cast<char*>(orow + sp.head);
            const int64_t v0 = c * kChunkVec + t;
            if (c * kChunkVec + kChunkVec <= sp.nvec) {
                U4 buf[U];
#pragma unroll
                for (int u = 0; u < U; ++u) buf[u] = load_u4_stream(vb + (v0 + (int64_t)u * kBlock) * 16);
#pragma unroll
                for (int u = 0; u < U; ++u)
                    grad_store_vec<T>(buf[u], rg, sp.head + (v0 + (int64_t)u * kBlock) * kVec,
                                      ob + (v0 + (int64_t)u * kBlock) * 16, orow);
            } else {
                for (int64_t j = v0; j < sp.nvec; j += kBlock)
                    grad_store_vec<T>(load_u4_stream(vb + j * 16), rg, sp.head + j * kVec, ob + j * 16, orow);
            }
            if (c == 0) {
                const int64_t ns = sp.n_scalar(a.V);
                for (int64_t k = t; k < ns; k += kBlock) {
                    const int64_t idx = sp.scalar_index(k);
                    Elem<T>::store1(orow + idx, grad_elem(Elem<T>::load1(row + idx), rg, idx == rg.y));
                }
            }
        } else {
            const int64_t e0 = c * kChunkVec * kVec;
            const int64_t e1 = e0 + kChunkVec * kVec < a.V ? e0 + kChunkVec * kVec : a.V;
            for (int64_t idx = e0 + t; idx < e1; idx += kBlock)
                Elem<T>::store1(orow + idx, grad_elem(Elem<T>::load1(row + idx), rg, idx == rg.y));
        }
    }
}

// ---- forward and VJP in one kernel ----------------------------------------------
//
// For a caller that knows the upstream gradient g when it runs the forward (a summed or
// averaged loss): each row's (m, log s) is reduced exactly as the forward reduces it,
// then the same lanes sweep the row again and write g * (softmax - onehot).  The first
// sweep loads without the non-temporal hint, so the second finds the row in L2 or the
// Infinity Cache and HBM carries one read and one write of each row instead of the
// forward's read plus the VJP's read and write.  The loss, the pair and the gradient
// equal those of the forward followed by the VJP bit for bit wherever both take the
// same layout, because every float32 operation is the same and in the same order.

struct FusedArgs {
    const void* logits;
    RowLayout in;
    const int32_t* targets;
    const float* g;
    int64_t n_rows;
    int64_t V;
    float* loss;
    float2* lse;
    void* dlogits;
    RowLayout out;
};

// Writes the row's loss and pair and returns what the gradient needs, as the forward's
// store and the VJP's reading of the pair would give them.
template <typename T>
__device__ __forceinline__ RowGrad fused_finish(const FusedArgs& a, int64_t r, MS st, float zy, int32_t y,
                                                bool ok, bool writer) {
    const float ls = log_e(st.s);
    if (writer) {
        a.loss[r] = ok ? (st.m - zy) + ls : __builtin_nanf("");
        a.lse[r] = make_float2(st.m, ls);
    }
    RowGrad rg;
    rg.y = y;
    rg.m = ok ? st.m : __builtin_nanf("");
    set_row_scale<T>(rg, ls, a.g[r]);
    return rg;
}

template <typename T, int NV, int UR>
__global__ __launch_bounds__(kBlock) void ce_fused_narrow(FusedArgs a) {
    constexpr int kVec = Elem<T>::kVec;
    constexpr int kN = NV * kVec;
    const int64_t nthreads = (int64_t)gridDim.x * kBlock;
    const T* base = static_cast<const T*>(a.logits);
    T* obase = static_cast<T*>(a.dlogits);
    for (int64_t r0 = (int64_t)blockIdx.x * kBlock + threadIdx.x; r0 < a.n_rows; r0 += nthreads * UR) {
        U4 buf[UR][NV];
        int32_t ys[UR];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int64_t r = r0 + u * nthreads;
            if (r < a.n_rows) {
                const char* row = reinterpret_cast<const char*>(base + row_offset(r, a.in));
#pragma unroll
                for (int v = 0; v < NV; ++v) buf[u][v] = load_u4_stream(row + v * 16);
                ys[u] = a.targets[r];
            }
        }
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int64_t r = r0 + u * nthreads;
            if (r < a.n_rows) {
                float f[kN];
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    float t[kVec];
                    Elem<T>::unpack(buf[u][v], t);
#pragma unroll
                    for (int k = 0; k < kVec; ++k) f[v * kVec + k] = t[k];
                }
                MS st = ms_empty();
                ms_add<kN>(st, f);
                const int32_t y = ys[u];
                float zy = 0.0f;
#pragma unroll
                for (int k = 0; k < kN; ++k) zy = (y == k) ? f[k] : zy;
                const RowGrad rg = fused_finish<T>(a, r, st, zy, y, target_ok(y, kN), true);
                // the row is still in registers: no second read
                char* orow = reinterpret_cast<char*>(obase + row_offset(r, a.out));
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    grad_store_vec<T>(buf[u][v], rg, (int64_t)v * kVec, orow + v * 16, reinterpret_cast<T*>(orow));
            }
        }
    }
}

// G lanes per row: up to 64 they are part of one wavefront (256-thread workgroups of
// 256 / G rows); above 64 one workgroup of G threads holds the row and the waves
// exchange their (m, s) pairs through LDS as the forward's row-per-workgroup layout
// does, except that every wave folds the slots itself (in the same order, so all get
// the bits wave 0 of the forward gets) instead of waiting on a second barrier.
template <typename T, int G, int U>
__global__ __launch_bounds__(G > kBlock ? G : kBlock) void ce_fused_rows(FusedArgs a) {
    constexpr int kThreads = G > 64 ? G : kBlock;
    constexpr int kRowsPerBlock = kThreads / G;
    constexpr int NW = G > 64 ? G / 64 : 1;
    // Double-buffered as in the forward's row-per-workgroup layout: a wave that is a
    // row ahead writes the other buffer, and cannot come back to this one before every
    // wave has passed the next row's barrier, after reading this row's slots.
    __shared__ MS slots[2][NW];
    const int lane = threadIdx.x % G;
    const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
    int parity = 0;
    for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / G; r < a.n_rows;
         r += stride, parity ^= 1) {
        const T* row = static_cast<const T*>(a.logits) + row_offset(r, a.in);
        T* orow = static_cast<T*>(a.dlogits) + row_offset(r, a.out);
        const int32_t y = a.targets[r];
        const bool ok = target_ok(y, a.V);
        float zy = 0.0f;
        if (lane == 0 && ok) zy = Elem<T>::load1(row + y);
        MS st = ms_empty();
        stream_row<T, G, U, true>(row, a.V, lane, st);
        if constexpr (G <= 64) {
            st = ms_group_reduce<G>(st);
        } else {
            const int wave = threadIdx.x / 64;
            const int wl = threadIdx.x % 64;
            st = ms_group_reduce<64>(st);
            if (wl == 0) slots[parity][wave] = st;
            __syncthreads();
            MS t = wl < NW ? slots[parity][wl] : ms_empty();
            t = ms_group_reduce<NW>(t);
            st = MS{__shfl(t.m, 0), __shfl(t.s, 0)};
        }
        grad_row<T, G, U>(row, orow, a.V, lane, fused_finish<T>(a, r, st, zy, y, ok, lane == 0));
    }
}

// Rows of up to G * NV vectors whose input and output share a 16-byte phase: one
// workgroup of G threads (the forward's lanes for the row: 512 or 1024) per row, and the
// whole row is loaded into registers at once: vector j = tid + k * G sits in buf[k], the row's unaligned head and tail
// elements in one register each of threads 0 .. ns - 1.  With the row in registers
// the max and the sum are two passes over them (m = max z, then s = sum exp(z - m)),
// each with its own exchange through LDS, rather than the online fold: the fold's
// rescaled groups would need 8 * U more live registers than the row leaves.  The
// gradient is then computed from the same registers, so HBM sees one read and one
// write of each row.  All loads of a row complete before its first store, so the output
// may be the input itself, and each register takes the next row's vector once its
// gradient has been stored.  The loads are buffer accesses with one per-thread offset
// register and the k * 16 KiB step as a scalar offset, so the held row costs no address
// registers.
typedef uint32_t V4U32 __attribute__((ext_vector_type(4)));

// One element through a buffer descriptor, rounded to T as Elem<T>::store1 rounds it.
template <typename T>
__device__ __forceinline__ void store_elem(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, int soff, float v) {
    if constexpr (sizeof(T) == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rsrc, voff, soff, 0);
    } else {
        const T h = (T)v;
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, h), rsrc, voff, soff, 0);
    }
}

// An empty asm step on each held word: the compiler then cannot carry a pass's unpacked
// floats (8 registers per 16-bit vector) over to the next pass in place of the 4
// packed words.
template <int NV>
__device__ __forceinline__ void opaque(U4 (&buf)[NV]) {
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) __asm__ volatile("" : "+v"(buf[k].w[e]));
}

template <typename T, int G, int NV>
__global__ __launch_bounds__(G) void ce_fused_regs(FusedArgs a) {
    constexpr int kVec = Elem<T>::kVec;
    constexpr int NW = G / 64;
    // Two exchanges per row, each with its own slots.  A wave writes the max slots of the
    // next row only after the sum barrier of this row, which every wave reaches after
    // reading this row's max slots; it writes the sum slots of the next row only after
    // the next row's max barrier, which every wave reaches after reading this row's sum
    // slots.  So no slot is overwritten before it has been read ("One barrier short",
    // sections "Sixty-four floats" and "The fix").
    __shared__ float max_slots[NW];
    __shared__ float sum_slots[NW];
    const int tid = threadIdx.x;
    const int wave = tid / 64;
    const int wl = tid % 64;
    const uint32_t voff = (uint32_t)tid * 16u;
    int64_t r = blockIdx.x;
    if (r >= a.n_rows) return;
    // Software pipeline: the loads of the block's next row are issued into each register
    // as soon as that register's gradient has been stored, so one row's writes and the
    // next row's reads are in flight together.  Rows share one 16-byte phase (the host
    // checks the strides), so every row has the same head and vector count.
    const T* row = static_cast<const T*>(a.logits) + row_offset(r, a.in);
    const RowSplit<T> sp(row, a.V);
    const int nvec = (int)sp.nvec;  // at most G * NV
    const int64_t ns = sp.n_scalar(a.V);
    const int64_t sidx = tid < ns ? sp.scalar_index(tid) : 0;
    U4 buf[NV];
    {
        const __amdgpu_buffer_rsrc_t src =
            __builtin_amdgcn_make_buffer_rsrc((void*)(row + sp.head), (short)0, nvec * 16, 0x00020000);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            if (tid + k * G < nvec) {
                const V4U32 v = __builtin_amdgcn_raw_buffer_load_b128(src, voff, k * G * 16, 0);
                buf[k] = U4{{v.x, v.y, v.z, v.w}};
            }
        }
    }
    float sval = tid < ns ? Elem<T>::load1(row + sidx) : kNegInf;
    for (;;) {
        T* orow = static_cast<T*>(a.dlogits) + row_offset(r, a.out);
        const int32_t y = a.targets[r];
        const bool ok = target_ok(y, a.V);
        float zy = 0.0f;
        if (tid == 0 && ok) zy = Elem<T>::load1(row + y);
        // pass 1: the row maximum
        float m = sval;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            if (tid + k * G < nvec) {
                float f[kVec];
                Elem<T>::unpack(buf[k], f);
#pragma unroll
                for (int e = 0; e < kVec; ++e) m = fmaxf(m, f[e]);
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        if (wl == 0) max_slots[wave] = m;
        __syncthreads();
        m = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) m = fmaxf(m, max_slots[w]);
        // pass 2: s = sum exp(z - m), pairwise inside each vector
        opaque(buf);
        const float ref = ref_point(m);
        float s = tid < ns ? exp_e(sval - ref) : 0.0f;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            if (tid + k * G < nvec) {
                float f[kVec];
                Elem<T>::unpack(buf[k], f);
#pragma unroll
                for (int e = 0; e < kVec; ++e) f[e] = exp_e(f[e] - ref);
#pragma unroll
                for (int w = 1; w < kVec; w *= 2)
#pragma unroll
                    for (int e = 0; e + w < kVec; e += 2 * w) f[e] += f[e + w];
                s += f[0];
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
        if (wl == 0) sum_slots[wave] = s;
        __syncthreads();
        s = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) s += sum_slots[w];
        const RowGrad rg = fused_finish<T>(a, r, MS{m, s}, zy, y, ok, tid == 0);
        // pass 3: the gradient from the held registers; each register then takes the
        // next row's vector
        opaque(buf);
        const int64_t rn = r + gridDim.x;
        const bool more = rn < a.n_rows;
        const T* nrow = more ? static_cast<const T*>(a.logits) + row_offset(rn, a.in) : row;
        const __amdgpu_buffer_rsrc_t nsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)(nrow + sp.head), (short)0, nvec * 16, 0x00020000);
        const __amdgpu_buffer_rsrc_t dst =
            __builtin_amdgcn_make_buffer_rsrc((void*)(orow + sp.head), (short)0, nvec * 16, 0x00020000);
        // in 32 bits: the row holds at most G * NV * kVec elements
        const int rel0 = rg.y - (int)sp.head - tid * kVec;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            if (tid + k * G < nvec) {
                float f[kVec], o[kVec];
                Elem<T>::unpack(buf[k], f);
#pragma unroll
                for (int e = 0; e < kVec; ++e) o[e] = rg.g * prob(f[e], rg);
                const U4 u = Elem<T>::pack(o);
                // The store's whole offset is in the VGPR, with a zero scalar offset: with
                // the step in an SGPR the compiler treats a 16-byte buffer store as free of
                // the store-data hazard and lets the next instruction overwrite the data
                // registers while the store may still be reading them, which corrupted
                // the stored words on gfx950.
                const uint32_t vo = voff + (uint32_t)(k * G * 16);
                __builtin_amdgcn_raw_buffer_store_b128(V4U32{u.w[0], u.w[1], u.w[2], u.w[3]}, dst, vo, 0, 0);
                // the target element again, as the VJP does it: a second store from the
                // same lane through the same descriptor, which lands after the first
                const int rel = rel0 - k * G * kVec;
                if ((uint32_t)rel < (uint32_t)kVec) {
                    float zt = f[0];
#pragma unroll
                    for (int e = 1; e < kVec; ++e) zt = rel == e ? f[e] : zt;
                    store_elem<T>(dst, vo + (uint32_t)rel * (uint32_t)sizeof(T), 0, grad_elem(zt, rg, true));
                }
                if (more) {
                    const V4U32 v = __builtin_amdgcn_raw_buffer_load_b128(nsrc, voff, k * G * 16, 0);
                    buf[k] = U4{{v.x, v.y, v.z, v.w}};
                }
            }
        }
        if (tid < ns) Elem<T>::store1(orow + sidx, grad_elem(sval, rg, sidx == rg.y));
        if (!more) break;
        r = rn;
        row = nrow;
        sval = tid < ns ? Elem<T>::load1(row + sidx) : kNegInf;
    }
}

// ---- dispatch -------------------------------------------------------------------

RowLayout dev_layout(const HostLayout& h) {
    return RowLayout{h.rows_per_batch, h.row_stride, h.batch_stride, h.uniform};
}

template <typename T>
hipError_t fwd_typed(const FwdCall& c) {
    FwdArgs a{c.logits, dev_layout(c.in), c.targets, c.n_rows, c.V, c.loss, reinterpret_cast<float2*>(c.lse)};
    const dim3 grid((unsigned)c.plan.blocks);
    constexpr int kU = Elem<T>::kVec == 8 ? 4 : 8;  // 32 elements in flight per lane per step
    if (c.plan.narrow_nv > 0) {
        switch (c.plan.narrow_nv) {
            case 1: hipLaunchKernelGGL((ce_fwd_narrow<T, 1, 4>), grid, dim3(kBlock), 0, c.stream, a); break;
            case 2: hipLaunchKernelGGL((ce_fwd_narrow<T, 2, 2>), grid, dim3(kBlock), 0, c.stream, a); break;
            case 4: hipLaunchKernelGGL((ce_fwd_narrow<T, 4, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
            case 8: hipLaunchKernelGGL((ce_fwd_narrow<T, 8, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (c.plan.lanes) {
        case 1: hipLaunchKernelGGL((ce_fwd_lanes<T, 1, 2>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 2: hipLaunchKernelGGL((ce_fwd_lanes<T, 2, 2>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 4: hipLaunchKernelGGL((ce_fwd_lanes<T, 4, 2>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 8: hipLaunchKernelGGL((ce_fwd_lanes<T, 8, 4>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 16: hipLaunchKernelGGL((ce_fwd_lanes<T, 16, 4>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 32: hipLaunchKernelGGL((ce_fwd_lanes<T, 32, 4>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 64: hipLaunchKernelGGL((ce_fwd_lanes<T, 64, 4>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 128: hipLaunchKernelGGL((ce_fwd_rowwg<T, 2, kU>), grid, dim3(128), 0, c.stream, a); break;
        case 256: hipLaunchKernelGGL((ce_fwd_rowwg<T, 4, kU>), grid, dim3(256), 0, c.stream, a); break;
        case 512: hipLaunchKernelGGL((ce_fwd_rowwg<T, 8, kU>), grid, dim3(512), 0, c.stream, a); break;
        case 1024: hipLaunchKernelGGL((ce_fwd_rowwg<T, 16, kU>), grid, dim3(1024), 0, c.stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t vjp_typed(const VjpCall& c) {
    VjpArgs a{c.logits, dev_layout(c.in), c.targets, reinterpret_cast<const float2*>(c.lse), c.g,
              c.n_rows, c.V, c.dlogits, dev_layout(c.out)};
    const dim3 grid((unsigned)c.plan.blocks);
    constexpr int kU = Elem<T>::kVec == 8 ? 4 : 8;
    if (c.plan.chunks > 0) {
        hipLaunchKernelGGL((ce_vjp_chunks<T, kChunkU>), grid, dim3(kBlock), 0, c.stream, a, c.plan.chunks);
        return hipGetLastError();
    }
    if (c.plan.narrow_nv > 0) {
        switch (c.plan.narrow_nv) {
            case 1: hipLaunchKernelGGL((ce_vjp_narrow<T, 1, 4>), grid, dim3(kBlock), 0, c.stream, a); break;
            case 2: hipLaunchKernelGGL((ce_vjp_narrow<T, 2, 2>), grid, dim3(kBlock), 0, c.stream, a); break;
            case 4: hipLaunchKernelGGL((ce_vjp_narrow<T, 4, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
            case 8: hipLaunchKernelGGL((ce_vjp_narrow<T, 8, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (c.plan.lanes) {
        case 1: hipLaunchKernelGGL((ce_vjp_lanes<T, 1, 2>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 2: hipLaunchKernelGGL((ce_vjp_lanes<T, 2, 2>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 4: hipLaunchKernelGGL((ce_vjp_lanes<T, 4, 2>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 8: hipLaunchKernelGGL((ce_vjp_lanes<T, 8, 4>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 16: hipLaunchKernelGGL((ce_vjp_lanes<T, 16, 4>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 32: hipLaunchKernelGGL((ce_vjp_lanes<T, 32, 4>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 64: hipLaunchKernelGGL((ce_vjp_lanes<T, 64, 4>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 128: hipLaunchKernelGGL((ce_vjp_lanes<T, 128, kU>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 256: hipLaunchKernelGGL((ce_vjp_lanes<T, 256, kU>), grid, dim3(256), 0, c.stream, a); break;
        case 512: hipLaunchKernelGGL((ce_vjp_lanes<T, 512, kU>), grid, dim3(512), 0, c.stream, a); break;
        case 1024: hipLaunchKernelGGL((ce_vjp_lanes<T, 1024, kU>), grid, dim3(1024), 0, c.stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t fused_typed(const FusedCall& c) {
    FusedArgs a{c.logits, dev_layout(c.in), c.targets, c.g, c.n_rows, c.V, c.loss,
                reinterpret_cast<float2*>(c.lse), c.dlogits, dev_layout(c.out)};
    const dim3 grid((unsigned)c.plan.blocks);
    constexpr int kU = Elem<T>::kVec == 8 ? 4 : 8;  // as the forward: the same fold order
    if (c.plan.narrow_nv > 0) {
        switch (c.plan.narrow_nv) {
            case 1: hipLaunchKernelGGL((ce_fused_narrow<T, 1, 4>), grid, dim3(kBlock), 0, c.stream, a); break;
            case 2: hipLaunchKernelGGL((ce_fused_narrow<T, 2, 2>), grid, dim3(kBlock), 0, c.stream, a); break;
            case 4: hipLaunchKernelGGL((ce_fused_narrow<T, 4, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
            case 8: hipLaunchKernelGGL((ce_fused_narrow<T, 8, 1>), grid, dim3(kBlock), 0, c.stream, a); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (c.plan.regs_nv > 0 && c.plan.lanes == 512) {
        if (c.plan.regs_nv != 8) return hipErrorInvalidValue;
        hipLaunchKernelGGL((ce_fused_regs<T, 512, 8>), grid, dim3(512), 0, c.stream, a);
        return hipGetLastError();
    }
    if (c.plan.regs_nv > 0) {
        if constexpr (Elem<T>::kVec == 8) {
            switch (c.plan.regs_nv) {
                case 8: hipLaunchKernelGGL((ce_fused_regs<T, 1024, 8>), grid, dim3(1024), 0, c.stream, a); break;
                case 12: hipLaunchKernelGGL((ce_fused_regs<T, 1024, 12>), grid, dim3(1024), 0, c.stream, a); break;
                case 16: hipLaunchKernelGGL((ce_fused_regs<T, 1024, 16>), grid, dim3(1024), 0, c.stream, a); break;
                case 20: hipLaunchKernelGGL((ce_fused_regs<T, 1024, 20>), grid, dim3(1024), 0, c.stream, a); break;
                default: return hipErrorInvalidValue;
            }
        } else {
            switch (c.plan.regs_nv) {
                case 8: hipLaunchKernelGGL((ce_fused_regs<T, 1024, 8>), grid, dim3(1024), 0, c.stream, a); break;
                case 16: hipLaunchKernelGGL((ce_fused_regs<T, 1024, 16>), grid, dim3(1024), 0, c.stream, a); break;
                default: return hipErrorInvalidValue;
            }
        }
        return hipGetLastError();
    }
    switch (c.plan.lanes) {
        case 1: hipLaunchKernelGGL((ce_fused_rows<T, 1, 2>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 2: hipLaunchKernelGGL((ce_fused_rows<T, 2, 2>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 4: hipLaunchKernelGGL((ce_fused_rows<T, 4, 2>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 8: hipLaunchKernelGGL((ce_fused_rows<T, 8, 4>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 16: hipLaunchKernelGGL((ce_fused_rows<T, 16, 4>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 32: hipLaunchKernelGGL((ce_fused_rows<T, 32, 4>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 64: hipLaunchKernelGGL((ce_fused_rows<T, 64, 4>), grid, dim3(kBlock), 0, c.stream, a); break;
        case 128: hipLaunchKernelGGL((ce_fused_rows<T, 128, kU>), grid, dim3(128), 0, c.stream, a); break;
        case 256: hipLaunchKernelGGL((ce_fused_rows<T, 256, kU>), grid, dim3(256), 0, c.stream, a); break;
        case 512: hipLaunchKernelGGL((ce_fused_rows<T, 512, kU>), grid, dim3(512), 0, c.stream, a); break;
        case 1024: hipLaunchKernelGGL((ce_fused_rows<T, 1024, kU>), grid, dim3(1024), 0, c.stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ce_forward(const FwdCall& c) {
    switch (c.dt) {
        case Dt::F32: return fwd_typed<float>(c);
        case Dt::F16: return fwd_typed<_Float16>(c);
        case Dt::BF16: return fwd_typed<__bf16>(c);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_ce_vjp(const VjpCall& c) {
    switch (c.dt) {
        case Dt::F32: return vjp_typed<float>(c);
        case Dt::F16: return vjp_typed<_Float16>(c);
        case Dt::BF16: return vjp_typed<__bf16>(c);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_ce_fused(const FusedCall& c) {
    switch (c.dt) {
        case Dt::F32: return fused_typed<float>(c);
        case Dt::F16: return fused_typed<_Float16>(c);
        case Dt::BF16: return fused_typed<__bf16>(c);
    }
    return hipErrorInvalidValue;
}

}  // namespace ce
