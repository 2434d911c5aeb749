// Linear cross-entropy backward: dH = dZ W and dW = dZ^T H for the objective
// sum_i g_i loss_i, with dZ = diag(g) (softmax(Z) - onehot(y)) and Z = H W^T.
//
// Ineshin, "A fused linear cross-entropy forward kernel for Apple GPUs", section 1:
// training saves the forward's log-sum-exp and a chunked backward regenerates the
// logits it needs tile by tile.  Here each chunk of vocabulary columns is one launch of
// the MFMA tile kernel whose epilogue turns the regenerated logits straight into dZ
// (bf16, from the saved (m, log s) pair), written both row-major and transposed,
// followed by two products on the same MFMA K loop, accumulated in fp32:
//   dH        += dZ_c  W_c       (N x D, every chunk adds its share)
//   dW[c0:c1]  = dZ_c^T H        (the chunk's own rows of dW)
// The K loop reads both operands K-contiguous, so W_c and H enter these products
// transposed: H^T once per call (lce_transpose), W_c^T by the dZ tiles themselves from
// the W rows they stage through LDS.  K is padded to a multiple of 8 with zeros in both
// operands.
//
// Two chunk widths, chosen by the workspace the caller passes: 8192 columns (the page's
// tile; the workspace holds one chunk's dZ, about 2 x 128 MiB at N = 8192), or the
// whole vocabulary as one chunk when the workspace holds all of dZ (about 5.9 GiB at
// N = 8192, V = 151,936).  One chunk writes dH once instead of reading and rewriting it
// per chunk, and launches each product once; its results are the same bit for bit,
// since a chunk's tiles start from the float32 dH the previous chunk stored and the
// float32 additions run in the same order.  Everything runs on the caller's stream in
// the caller's workspace; nothing is allocated and no state is kept between calls.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace ce {
namespace {

constexpr int64_t kChunkCols = 8192;  // the page's tile: vocabulary columns per chunk
// One chunk over the whole vocabulary reads dZ and W^T rows of 2 * round256(V) bytes
// through a buffer descriptor of 256 such rows and 32-bit offsets: V at most 2^22.
constexpr int64_t kMaxOnePassV = (int64_t)1 << 22;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
int64_t round8(int64_t x) { return (x + 7) & ~(int64_t)7; }
int64_t round256(int64_t x) { return (x + 255) & ~(int64_t)255; }

struct Layout {
    int64_t chunk;
    size_t g, gt, ht, wt, total;  // byte offsets of the four bf16 buffers
};

// dZ chunk [N][chunk]; its transpose [chunk][N8]; H^T [D][N8]; W_c^T [D][chunk].
Layout layout(int64_t N, int64_t D, int64_t chunk) {
    const int64_t n8 = round8(N);
    Layout l;
    l.chunk = chunk;
    l.g = 0;
    l.gt = l.g + align256((size_t)N * chunk * 2);
    l.ht = l.gt + align256((size_t)chunk * n8 * 2);
    l.wt = l.ht + align256((size_t)D * n8 * 2);
    l.total = l.wt + align256((size_t)D * chunk * 2);
    return l;
}

Layout chunked(int64_t N, int64_t D, int64_t V) {
    const int64_t v256 = round256(V);
    return layout(N, D, v256 < kChunkCols ? v256 : kChunkCols);
}

// Whether a call with chunks of `chunk` columns fits the dispatches: the gradient tiles
// over N x chunk, and the two products over N x D and chunk x D in one launch.
bool grids_fit(int64_t N, int64_t D, int64_t chunk) {
    return lce_tile_grid_items(N, chunk) <= kMaxGridItems &&
           lce_tile_grid_items(N, D) + lce_tile_grid_items(chunk, D) <= kMaxGridItems;
}

// The layout a call with `bytes` of workspace runs: the whole vocabulary as one chunk
// when the workspace holds it (and its grids fit a dispatch), else chunks of 8192 columns.
Layout pick(int64_t N, int64_t D, int64_t V, size_t bytes) {
    if (V <= kMaxOnePassV && grids_fit(N, D, round256(V))) {
        const Layout one = layout(N, D, round256(V));
        if (bytes >= one.total) return one;
    }
    return chunked(N, D, V);
}

}  // namespace

size_t lce_backward_workspace_bytes(int64_t N, int64_t D, int64_t V) { return chunked(N, D, V).total; }

bool lce_backward_grids_fit(int64_t N, int64_t D, int64_t V) { return grids_fit(N, D, chunked(N, D, V).chunk); }

size_t lce_backward_workspace_bytes_one_pass(int64_t N, int64_t D, int64_t V) {
    return pick(N, D, V, SIZE_MAX).total;
}

size_t lce_backward_workspace_used(int64_t N, int64_t D, int64_t V, size_t workspace_bytes) {
    return pick(N, D, V, workspace_bytes).total;
}

LceBackwardStatus run_lce_backward(const LceBackwardCall& c) {
    const Layout l = pick(c.N, c.D, c.V, c.workspace_bytes);
    const int64_t kChunk = l.chunk;
    char* ws = static_cast<char*>(c.workspace);
    void* G = ws + l.g;
    void* GT = ws + l.gt;
    void* HT = ws + l.ht;
    void* WT = ws + l.wt;
    const int64_t n8 = round8(c.N);
    auto ok = [](hipError_t e) { return e == hipSuccess; };
    // H^T with zero columns N .. N8 - 1, and the same zero columns in the transposed dZ
    // chunk (the tile kernel writes only columns below N): the K padding of dW's product
    if (!ok(launch_transpose_bf16(c.H, c.N, c.D, c.D, HT, n8, n8, c.stream))) return LceBackwardStatus::kHip;
    if (!ok(launch_zero_cols_bf16(GT, kChunk, n8, c.N, n8, c.stream))) return LceBackwardStatus::kHip;
    for (int64_t c0 = 0; c0 < c.V; c0 += kChunk) {
        const int64_t w = c.V - c0 < kChunk ? c.V - c0 : kChunk;
        const int64_t w8 = round8(w);
        // dZ_c in both layouts, and W_c^T [D][w8] (zero past w) written by the same tiles
        LceGradChunk gc{c.H, c.W, c.targets, c.lse, c.g, c.N, c.D, c.V, c0, w, G, kChunk, GT, n8, WT, kChunk, c.stream};
        if (!ok(launch_lce_grad_chunk(gc))) return LceBackwardStatus::kHip;
        // dZ_c's columns w .. w8 - 1 (stale from an earlier chunk, or never written) zeroed,
        // so the padded K adds nothing
        if (w8 > w && !ok(launch_zero_cols_bf16(G, c.N, kChunk, w, w8, c.stream))) return LceBackwardStatus::kHip;
        // dH [N][D] (+)= dZ_c [N][w8] . (W_c^T [D][w8])^T, and
        // dW[c0 : c0 + w] [w][D] = dZ_c^T [w][N8] . (H^T [D][N8])^T, in one launch
        LceGemm p1{G, kChunk, WT, kChunk, c.N, c.D, w8, c.dH, c.D, c0 > 0, c.stream};
        LceGemm p2{GT, n8, HT, n8, w, c.D, n8, c.dW + c0 * c.D, c.D, false, c.stream};
        if (!ok(launch_lce_gemm2(p1, p2))) return LceBackwardStatus::kHip;
    }
    return LceBackwardStatus::kOk;
}

}  // namespace ce
