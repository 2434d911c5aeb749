// Linear cross-entropy backward: dH = dZ W and dW = dZ^T H for the objective
// sum_i g_i loss_i, with dZ = diag(g) (softmax(Z) - onehot(y)) and Z = H W^T.
//
// Ineshin, "A fused linear cross-entropy forward kernel for Apple GPUs", section 1:
// training saves the forward's log-sum-exp and a chunked backward regenerates the
// logits it needs tile by tile.  Here each chunk of 8192 vocabulary columns (the
// page's dispatch tile) is one launch of the MFMA tile kernel whose epilogue turns the
// regenerated logits straight into dZ (bf16, from the saved (m, log s) pair), written
// both row-major and transposed, followed by two plain GEMMs on rocBLAS, accumulated
// in fp32:
//   dH        += dZ_c  W_c       (N x D, every chunk adds its share)
//   dW[c0:c1]  = dZ_c^T H        (the chunk's own rows of dW)
// With both layouts neither GEMM reads a transposed operand (rocBLAS's kernel for
// dZ_c^T H from the row-major chunk ran about 25% slower than the one without).
// Everything runs on the caller's stream; the two dZ chunks and rocBLAS's scratch live
// in the caller's workspace.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include "launch.h"

namespace ce {
namespace {

constexpr int64_t kChunk = 8192;            // vocabulary columns per chunk
constexpr size_t kBlasBytes = 64ull << 20;  // rocBLAS scratch inside the workspace
constexpr int kMaxDevices = 64;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// One rocBLAS handle per thread and device, created on first use and kept for the life
// of the thread (rocBLAS handles must not be used by two threads at once).  The handle
// is told to use the caller's workspace, so rocBLAS allocates no scratch of its own.
struct Handles {
    rocblas_handle h[kMaxDevices] = {};
    void* ws[kMaxDevices] = {};
};

rocblas_status handle_for(int dev, void* ws, rocblas_handle* out) {
    thread_local Handles hs;
    if (!hs.h[dev]) {
        rocblas_status s = rocblas_create_handle(&hs.h[dev]);
        if (s != rocblas_status_success) {
            hs.h[dev] = nullptr;
            return s;
        }
        hs.ws[dev] = nullptr;
    }
    if (hs.ws[dev] != ws) {
        rocblas_status s = rocblas_set_workspace(hs.h[dev], ws, kBlasBytes);
        if (s != rocblas_status_success) return s;
        hs.ws[dev] = ws;
    }
    *out = hs.h[dev];
    return rocblas_status_success;
}

}  // namespace

size_t lce_backward_workspace_bytes(int64_t N, int64_t D, int64_t V) {
    (void)D;
    (void)V;
    return 2 * align256((size_t)N * kChunk * 2) + kBlasBytes;
}

LceBackwardStatus run_lce_backward(const LceBackwardCall& c) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LceBackwardStatus::kHip;
    char* ws = static_cast<char*>(c.workspace);
    const size_t chunk_bytes = align256((size_t)c.N * kChunk * 2);
    void* G = ws;
    void* GT = ws + chunk_bytes;
    void* blas_ws = ws + 2 * chunk_bytes;
    rocblas_handle h = nullptr;
    if (handle_for(dev, blas_ws, &h) != rocblas_status_success) return LceBackwardStatus::kBlas;
    if (rocblas_set_stream(h, c.stream) != rocblas_status_success) return LceBackwardStatus::kBlas;

    const char* Hb = static_cast<const char*>(c.H);
    const char* Wb = static_cast<const char*>(c.W);
    const float one = 1.0f, zero = 0.0f;
    const rocblas_int n = (rocblas_int)c.N, d = (rocblas_int)c.D, ldg = (rocblas_int)kChunk;
    for (int64_t c0 = 0; c0 < c.V; c0 += kChunk) {
        const int64_t w = c.V - c0 < kChunk ? c.V - c0 : kChunk;
        LceGradChunk gc{c.H, c.W, c.targets, c.lse, c.g, c.N, c.D, c.V, c0, w, G, kChunk, GT, c.N, c.stream};
        if (launch_lce_grad_chunk(gc) != hipSuccess) return LceBackwardStatus::kHip;
        // rocBLAS is column-major: a row-major [r][cols] array with leading dimension L
        // is a column-major cols x r matrix with the same L.
        // dH^T (D x N) += W_c^T (D x w) * dZ_c^T (w x N)
        if (rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, d, n, (rocblas_int)w, &one,
                            Wb + c0 * c.D * 2, rocblas_datatype_bf16_r, d, G, rocblas_datatype_bf16_r, ldg,
                            c0 == 0 ? &zero : &one, c.dH, rocblas_datatype_f32_r, d, c.dH,
                            rocblas_datatype_f32_r, d, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0,
                            0) != rocblas_status_success)
            return LceBackwardStatus::kBlas;
        // dW_c^T (D x w) = H^T (D x N) * dZ_c (N x w), dZ_c being the transposed chunk read
        // as a column-major N x w matrix
        if (rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, d, (rocblas_int)w, n, &one,
                            Hb, rocblas_datatype_bf16_r, d, GT, rocblas_datatype_bf16_r, n, &zero,
                            c.dW + c0 * c.D, rocblas_datatype_f32_r, d, c.dW + c0 * c.D, rocblas_datatype_f32_r,
                            d, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0) != rocblas_status_success)
            return LceBackwardStatus::kBlas;
    }
    return LceBackwardStatus::kOk;
}

}  // namespace ce
