// Internal interface between the C ABI (abi.cpp) and the kernel launchers.
// Everything here has already been validated by abi.cpp.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "plan.h"

namespace ce {

enum class Dt : int { F32 = 0, F16 = 1, BF16 = 2 };

struct HostLayout {
    int64_t rows_per_batch;
    int64_t row_stride;
    int64_t batch_stride;
    int32_t uniform;
};

struct FwdCall {
    const void* logits;
    HostLayout in;
    Dt dt;
    const int32_t* targets;
    int64_t n_rows;
    int64_t V;
    float* loss;
    float* lse;
    Plan plan;
    hipStream_t stream;
};

struct VjpCall {
    const void* logits;
    HostLayout in;
    Dt dt;
    const int32_t* targets;
    const float* lse;
    const float* g;
    int64_t n_rows;
    int64_t V;
    void* dlogits;
    HostLayout out;
    Plan plan;
    hipStream_t stream;
};

// ce_forward and ce_vjp in one kernel, with g known up front.
struct FusedCall {
    const void* logits;
    HostLayout in;
    Dt dt;
    const int32_t* targets;
    const float* g;
    int64_t n_rows;
    int64_t V;
    float* loss;
    float* lse;
    void* dlogits;
    HostLayout out;
    Plan plan;
    hipStream_t stream;
};

hipError_t launch_ce_forward(const FwdCall& c);
hipError_t launch_ce_vjp(const VjpCall& c);
hipError_t launch_ce_fused(const FusedCall& c);

// KL divergence of the teacher rows p from the student rows q (same dtype, own views).
struct KLFwdCall {
    const void* q;
    HostLayout ql;
    const void* p;
    HostLayout pl;
    Dt dt;
    int64_t n_rows;
    int64_t V;
    float* kl;
    float* lse_q;
    float* lse_p;
    Plan plan;
    hipStream_t stream;
};

struct KLVjpCall {
    const void* q;
    HostLayout ql;
    const void* p;
    HostLayout pl;
    Dt dt;
    const float* lse_q;
    const float* lse_p;
    const float* g;
    int64_t n_rows;
    int64_t V;
    void* dq;
    HostLayout dl;
    Plan plan;
    hipStream_t stream;
};

// Jensen-Shannon (js_kernels.hip): hq is the student's half H per row.
struct JSFwdCall {
    const void* q;
    HostLayout ql;
    const void* p;
    HostLayout pl;
    Dt dt;
    int64_t n_rows;
    int64_t V;
    float* js;
    float* lse_q;
    float* lse_p;
    float* hq;
    Plan plan;
    hipStream_t stream;
};

struct JSVjpCall {
    const void* q;
    HostLayout ql;
    const void* p;
    HostLayout pl;
    Dt dt;
    const float* lse_q;
    const float* lse_p;
    const float* hq;
    const float* g;
    int64_t n_rows;
    int64_t V;
    void* dq;
    HostLayout dl;
    Plan plan;
    hipStream_t stream;
};

hipError_t launch_js_forward(const JSFwdCall& c);
hipError_t launch_js_vjp(const JSVjpCall& c);

// Cross-entropy options (ce_options.hip).  t != NULL selects probability targets;
// otherwise y holds class-index targets.
struct OptFwdCall {
    const void* z;
    HostLayout zl;
    const void* t;
    HostLayout tl;
    Dt dt;
    const int32_t* y;
    int64_t n_rows;
    int64_t V;
    float eps;
    float* loss;
    float* lse;
    float* wsum;
    Plan plan;
    hipStream_t stream;
};

struct OptVjpCall {
    const void* z;
    HostLayout zl;
    const void* t;
    HostLayout tl;
    Dt dt;
    const int32_t* y;
    const float* lse;
    const float* wsum;
    const float* g;
    const int64_t* count;
    int64_t n_rows;
    int64_t V;
    int32_t reduction;
    int32_t ignore_index;
    int32_t has_ignore;
    float eps;
    void* d;
    HostLayout dl;
    Plan plan;
    hipStream_t stream;
};


struct ReduceCall {
    float* loss;
    const int32_t* y;  // NULL: every row counts
    int64_t n_rows;
    int32_t ignore_index;
    bool has_ignore;
    int32_t reduction;  // 0 none (ignore_index fix-up only), 1 sum, 2 mean
    float* total;
    int64_t* count;
    void* workspace;
    hipStream_t stream;
};

int64_t reduce_parts(int64_t n_rows);
hipError_t launch_opt_forward(const OptFwdCall& c);
hipError_t launch_opt_vjp(const OptVjpCall& c);
hipError_t launch_loss_reduce(const ReduceCall& c);
// This device's fixed reduction scratch (kReduceWorkspaceBytes, 256-byte aligned): its
// device address, taken once per device with that device current.
hipError_t reduce_scratch(void** ptr, size_t* bytes);

hipError_t launch_kl_forward(const KLFwdCall& c);
hipError_t launch_kl_vjp(const KLVjpCall& c);

// lce_forward.  Workspace layout is described in lce_kernels.hip.
struct LceCall {
    const void* H;
    const void* W;
    const int32_t* targets;
    int64_t N;
    int64_t D;
    int64_t V;
    float* loss;
    float* lse;
    void* workspace;
    int cu_count;
    hipStream_t stream;
};

size_t lce_workspace_bytes(int64_t N, int64_t D, int64_t V);
hipError_t launch_lce_forward(const LceCall& c);
// Work-items of an MFMA tile launch over rows x cols (one workgroup per 256 x 256 tile,
// in whole super-blocks).  A dispatch holds at most kMaxGridItems; the tile kernels do
// not loop over tiles, so a larger product is rejected before any launch.
constexpr int64_t kMaxGridItems = ((int64_t)1 << 32) - 1;
int64_t lce_tile_grid_items(int64_t rows, int64_t cols);

// dZ for vocabulary columns [c0, c0 + width) of all N rows, bf16, row r at G + r * ldG.
struct LceGradChunk {
    const void* H;
    const void* W;
    const int32_t* targets;
    const float* lse;
    const float* g;
    int64_t N;
    int64_t D;
    int64_t V;
    int64_t c0;
    int64_t width;
    void* G;      // dZ chunk, row-major [N][ldG]
    int64_t ldG;
    void* GT;     // the same chunk transposed, [width][ldGT]
    int64_t ldGT;
    void* WT;     // W's rows c0 .. c0 + width - 1 transposed, [D][ldWT], zero up to the
    int64_t ldWT; // next multiple of 8 columns
    hipStream_t stream;
};

hipError_t launch_lce_grad_chunk(const LceGradChunk& c);

// C[r][c] (+)= sum_k A[r][k] B[c][k] for r < M, c < Ncols: bf16 A [M][lda] and B [Ncols][ldb],
// both K-contiguous, K a multiple of 8 (lda, ldb too), fp32 C [M][ldc] with ldc a
// multiple of 4 and C 16-byte aligned.
struct LceGemm {
    const void* A;
    int64_t lda;
    const void* B;
    int64_t ldb;
    int64_t M;
    int64_t Ncols;
    int64_t K;
    float* C;
    int64_t ldc;
    bool accumulate;
    hipStream_t stream;
};

hipError_t launch_lce_gemm(const LceGemm& c);
// Two independent products in one launch (both on p.stream).
hipError_t launch_lce_gemm2(const LceGemm& p, const LceGemm& q);

// bf16 dst[c][r] = src[r][c] for r < R, c < C, and 0 for R <= r < Rpad; C, lds, ldd and
// Rpad are multiples of 8, both pointers 16-byte aligned.
hipError_t launch_transpose_bf16(const void* src, int64_t R, int64_t C, int64_t lds, void* dst, int64_t ldd,
                                 int64_t Rpad, hipStream_t stream);
// bf16 p[r][c] = 0 for r < rows, c_from <= c < c_to.
hipError_t launch_zero_cols_bf16(void* p, int64_t rows, int64_t ld, int64_t c_from, int64_t c_to,
                                 hipStream_t stream);

// Writes n zeros (a kernel, not a memset, so a captured graph replays it safely).
hipError_t launch_fill_zero_f32(float* p, int64_t n, hipStream_t stream);

struct LceBackwardCall {
    const void* H;
    const void* W;
    const int32_t* targets;
    const float* lse;
    const float* g;
    int64_t N;
    int64_t D;
    int64_t V;
    float* dH;
    float* dW;
    void* workspace;
    size_t workspace_bytes;  // at least lce_backward_workspace_bytes; with
                             // lce_backward_workspace_bytes_one_pass or more, one chunk
    hipStream_t stream;
};

enum class LceBackwardStatus { kOk, kHip };

// Workspace of chunks of 8192 vocabulary columns (the least a call needs), of one chunk
// over the whole vocabulary, and the part of `workspace_bytes` a call uses.
size_t lce_backward_workspace_bytes(int64_t N, int64_t D, int64_t V);
size_t lce_backward_workspace_bytes_one_pass(int64_t N, int64_t D, int64_t V);
// Whether the chunked layout's launches fit a dispatch (see kMaxGridItems).
bool lce_backward_grids_fit(int64_t N, int64_t D, int64_t V);
size_t lce_backward_workspace_used(int64_t N, int64_t D, int64_t V, size_t workspace_bytes);
LceBackwardStatus run_lce_backward(const LceBackwardCall& c);

}  // namespace ce
