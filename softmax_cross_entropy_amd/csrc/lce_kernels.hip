// Fused linear cross-entropy forward for gfx950: loss and log-sum-exp of Z = H W^T
// without materialising Z.
//
// Ineshin, "A fused linear cross-entropy forward kernel for Apple GPUs", section 1:
// each vocabulary tile of Z is folded into a running per-row state (m, s),
// m' = max(m, m_t), s' = s exp(m - m') + sum_j exp(z_j - m'), and the target logit
// is captured by the tile that holds the target column.
//
// Two kernels:
//   lce_tile   one 256 x 256 tile of Z per workgroup (bf16 MFMA, fp32 accumulate,
//              K = D streamed through LDS in 64-wide double-buffered stages).  Its
//              epilogue turns the fp32 accumulators straight into one (m, s) pair per
//              row for each 128-column slab, and stores the target logit from the
//              same accumulator when the target column is in the slab.
//   lce_merge  folds the slabs of each row in slab order into (m, s), then
//              loss = (m - z_y) + log s and lse = (m, log s).
// Workspace: partial (m, s) float2 [n_slabs][N], then z_y float [N].
//
// The page's kernel merges fixed 8192-column tiles in a chain of dependent
// dispatches.  Here every tile of the grid is independent (the merge is associative,
// and the fixed slab order of lce_merge keeps the result deterministic), which lets
// 256 compute units work on the whole vocabulary at once.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace ce {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int BM = 256;              // rows of H per tile
constexpr int BN = 256;              // rows of W (vocabulary columns) per tile
constexpr int BK = 64;               // reduction depth per LDS stage
constexpr int kThreads = 256;        // 4 waves as 2 x 2, each owning 128 x 128 of the tile
constexpr int WT = 128;              // wave tile edge
constexpr int FB = WT / 16;          // 8 x 8 MFMA 16x16 blocks per wave
constexpr int kStageBytes = BM * BK * 2;  // 32 KiB per operand per stage
constexpr int kTilesPerGroup = 32;   // tiles per super-block (one per CU of an XCD)
constexpr int kXcds = 8;

struct TileArgs {
    const __bf16* H;
    const __bf16* W;
    const int32_t* targets;
    int64_t N;
    int64_t D;
    int64_t V;
    int n_row_tiles, n_col_tiles;
    int gr, gc;      // super-block shape in tiles (gr * gc == 32)
    int n_rg, n_sb;  // row groups, super-blocks
    float2* partial;  // [n_slabs][N]
    float* zy;        // [N]
};

// LDS layout of one operand stage: 256 rows x 8 chunks of 16 bytes (8 bf16 along K).
// The chunk index is XORed with (row / 2) % 8 so that the 16 rows an MFMA operand
// read touches at one K chunk land in 16 different 16-byte bank groups:
//   byte offset of (row, chunk) = row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4).

__global__ __launch_bounds__(kThreads, 1) void lce_tile(TileArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[2][2][kStageBytes];  // [stage][A|B]

    // ---- which tile: XCD-aware super-blocks ----------------------------------
    // Consecutive workgroups go to the 8 XCDs in turn.  The k-th workgroup an XCD
    // receives is given position k % 32 of super-block k / 32 of that XCD, so the 32
    // workgroups an XCD runs together share gr row tiles of H and gc column tiles of W
    // through its L2, and the 8 XCDs work on neighbouring super-blocks of the same W
    // columns at the same time.
    const int b = blockIdx.x;
    const int xcd = b % kXcds;
    const int local = b / kXcds;
    const int sb = (local / kTilesPerGroup) * kXcds + xcd;
    if (sb >= a.n_sb) return;
    const int pos = local % kTilesPerGroup;
    const int cg = sb / a.n_rg, rg = sb % a.n_rg;
    const int row_tile = rg * a.gr + pos / a.gc;
    const int col_tile = cg * a.gc + pos % a.gc;
    if (row_tile >= a.n_row_tiles || col_tile >= a.n_col_tiles) return;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int64_t row0 = (int64_t)row_tile * BM;
    const int64_t col0 = (int64_t)col_tile * BN;

    // ---- global -> LDS loads: each wave fills 64 rows of A and of B per stage ----
    // One global_load_lds_dwordx4 writes 64 lanes x 16 bytes = 8 LDS rows; lane i lands
    // at (row = first + i / 8, physical chunk i % 8), so it fetches the logical chunk
    // that the swizzle maps there.  Rows past N (or V) re-read the last valid row; their
    // results are never stored (columns past V are masked in the epilogue).
    const __bf16* a_src[8];
    const __bf16* b_src[8];
    int koff[2];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int r = wave * 64 + q * 8 + (lane >> 3);
        int64_t ra = row0 + r;
        ra = ra < a.N ? ra : a.N - 1;
        int64_t rb = col0 + r;
        rb = rb < a.V ? rb : a.V - 1;
        a_src[q] = a.H + ra * a.D;
        b_src[q] = a.W + rb * a.D;
    }
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int r = par * 8 + (lane >> 3);  // (r >> 1) & 7 for the two row parities
        koff[par] = ((lane & 7) ^ ((r >> 1) & 7)) * 8;
    }
    const int nk = (int)((a.D + BK - 1) / BK);

    auto issue = [&](int kt, int buf) {
        const int64_t k0 = (int64_t)kt * BK;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            int64_t k = k0 + koff[q & 1];
            k = k < a.D ? k : a.D - 8;  // K tail: a valid chunk, zeroed after the LDS read
            char* dst_a = &lds[buf][0][(wave * 64 + q * 8) * 128];
            char* dst_b = &lds[buf][1][(wave * 64 + q * 8) * 128];
            __builtin_amdgcn_global_load_lds((const void*)(a_src[q] + k), (lds_void_t*)dst_a, 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)(b_src[q] + k), (lds_void_t*)dst_b, 16, 0, 0);
        }
    };

    f32x4 acc[FB][FB];
#pragma unroll
    for (int i = 0; i < FB; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int wm = wave >> 1, wn = wave & 1;
    const int q16 = lane & 15, g4 = lane >> 4;
    const int rd_row = q16 * 128;
    const int sw = q16 >> 1;

    issue(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        // Stage kt was issued one iteration earlier.  Issue stage kt + 1, then wait until
        // at most its 16 loads are outstanding (loads retire in order), and meet the
        // other waves at a plain barrier: no fence, so the next stage stays in flight.
        if (kt + 1 < nk) {
            issue(kt + 1, cur ^ 1);
            asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const char* As = &lds[cur][0][wm * WT * 128];
        const char* Bs = &lds[cur][1][wn * WT * 128];
        const int64_t kvalid = a.D - (int64_t)kt * BK;  // >= BK except in a K tail
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            const int c = kk * 4 + g4;
            const int off = rd_row + ((c ^ sw) << 4);
            const bool kok = (int64_t)c * 8 < kvalid;
            bf16x8 af[FB], bfr[FB];
#pragma unroll
            for (int i = 0; i < FB; ++i) {
                af[i] = *reinterpret_cast<const bf16x8*>(As + i * 16 * 128 + off);
                bfr[i] = *reinterpret_cast<const bf16x8*>(Bs + i * 16 * 128 + off);
            }
            if (!kok) {
#pragma unroll
                for (int i = 0; i < FB; ++i) {
                    af[i] = bf16x8{};
                    bfr[i] = bf16x8{};
                }
            }
#pragma unroll
            for (int i = 0; i < FB; ++i)
#pragma unroll
                for (int j = 0; j < FB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        // every wave has consumed its LDS reads of this buffer (the MFMAs used them)
        // before any wave issues the loads that overwrite it
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }

    // ---- epilogue: (m, s) per row over this wave's 128 columns ----------------
    // acc[i][j][e] holds Z[row = wm*128 + i*16 + g4*4 + e][col = wn*128 + j*16 + q16].
    const int64_t wcol0 = col0 + wn * WT;
    bool col_ok[FB];
#pragma unroll
    for (int j = 0; j < FB; ++j) col_ok[j] = wcol0 + j * 16 + q16 < a.V;

    // target logits: captured from the accumulator that holds the target column
    const int64_t wrow0 = row0 + wm * WT;
#pragma unroll
    for (int i = 0; i < FB; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t r = wrow0 + i * 16 + g4 * 4 + e;
            if (r < a.N) {
                const int64_t yrel = (int64_t)a.targets[r] - wcol0;
                if (yrel >= 0 && yrel < WT && (int)(yrel & 15) == q16) {
                    const int jj = (int)(yrel >> 4);
                    float v = 0.f;
#pragma unroll
                    for (int j = 0; j < FB; ++j) v = (j == jj) ? acc[i][j][e] : v;
                    a.zy[r] = v;
                }
            }
        }
    }

    MS st[32];  // state index i * 4 + e
#pragma unroll
    for (int i = 0; i < FB; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v[FB];
#pragma unroll
            for (int j = 0; j < FB; ++j) v[j] = col_ok[j] ? acc[i][j][e] : kNegInf;
            MS s0 = ms_empty();
            ms_add<FB>(s0, v);
            st[i * 4 + e] = s0;
        }
    }
    // Reduce-scatter across the 16 lanes that share a row set (lane bits 3..0): at each
    // step a lane keeps one half of its states, sends the other half to its partner and
    // merges what it receives.  After four steps lane q16 holds rows 2*q16 and 2*q16+1.
#pragma unroll
    for (int step = 0; step < 4; ++step) {
        const int mask = 8 >> step;
        const int half = 16 >> step;  // states held before this step: 2 * half
        const bool upper = (lane & mask) != 0;
#pragma unroll
        for (int k = 0; k < half; ++k) {
            const MS lo = st[k], hi = st[k + half];
            const MS keep = upper ? hi : lo;
            const MS send = upper ? lo : hi;
            MS recv{__shfl_xor(send.m, mask, 16), __shfl_xor(send.s, mask, 16)};
            st[k] = ms_merge(keep, recv);
        }
    }
    // state index 2*q16 + t  ->  i = q16 / 2, e = 2 * (q16 % 2) + t
    const int64_t slab = (int64_t)col_tile * 2 + wn;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int64_t r = wrow0 + (q16 >> 1) * 16 + g4 * 4 + 2 * (q16 & 1) + t;
        if (r < a.N) a.partial[slab * a.N + r] = make_float2(st[t].m, st[t].s);
    }
}

constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void lce_merge(const float2* __restrict__ partial,
                                                            const float* __restrict__ zy,
                                                            const int32_t* __restrict__ targets, int64_t N,
                                                            int n_slabs, int64_t V, float* loss, float2* lse) {
    const int64_t r = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
    if (r >= N) return;
    MS st = ms_empty();
    int s = 0;
    for (; s + 8 <= n_slabs; s += 8) {
        float2 p[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) p[u] = partial[(int64_t)(s + u) * N + r];
#pragma unroll
        for (int u = 0; u < 8; ++u) st = ms_merge(st, MS{p[u].x, p[u].y});
    }
    for (; s < n_slabs; ++s) {
        const float2 p = partial[(int64_t)s * N + r];
        st = ms_merge(st, MS{p.x, p.y});
    }
    const int32_t y = targets[r];
    const bool ok = y >= 0 && (int64_t)y < V;
    const float ls = log_e(st.s);
    loss[r] = ok ? (st.m - zy[r]) + ls : __builtin_nanf("");
    lse[r] = make_float2(st.m, ls);
}

struct Geometry {
    int n_row_tiles, n_col_tiles, gr, gc, n_rg, n_cg, n_sb, n_slabs;
    int64_t blocks;
};

Geometry geometry(int64_t N, int64_t V) {
    Geometry g;
    g.n_row_tiles = (int)((N + BM - 1) / BM);
    g.n_col_tiles = (int)((V + BN - 1) / BN);
    g.gr = g.n_row_tiles >= 4 ? 4 : (g.n_row_tiles >= 2 ? 2 : 1);
    g.gc = kTilesPerGroup / g.gr;
    g.n_rg = (g.n_row_tiles + g.gr - 1) / g.gr;
    g.n_cg = (g.n_col_tiles + g.gc - 1) / g.gc;
    g.n_sb = g.n_rg * g.n_cg;
    g.n_slabs = g.n_col_tiles * 2;
    g.blocks = (int64_t)((g.n_sb + kXcds - 1) / kXcds) * kXcds * kTilesPerGroup;
    return g;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t lce_workspace_bytes(int64_t N, int64_t D, int64_t V) {
    (void)D;
    const Geometry g = geometry(N, V);
    return align256((size_t)g.n_slabs * (size_t)N * sizeof(float2)) + align256((size_t)N * sizeof(float));
}

hipError_t launch_lce_forward(const LceCall& c) {
    const Geometry g = geometry(c.N, c.V);
    char* ws = static_cast<char*>(c.workspace);
    float2* partial = reinterpret_cast<float2*>(ws);
    float* zy = reinterpret_cast<float*>(ws + align256((size_t)g.n_slabs * (size_t)c.N * sizeof(float2)));
    TileArgs a{static_cast<const __bf16*>(c.H), static_cast<const __bf16*>(c.W), c.targets, c.N, c.D, c.V,
               g.n_row_tiles, g.n_col_tiles, g.gr, g.gc, g.n_rg, g.n_sb, partial, zy};
    hipLaunchKernelGGL(lce_tile, dim3((unsigned)g.blocks), dim3(kThreads), 0, c.stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t mblocks = (c.N + kMergeThreads - 1) / kMergeThreads;
    hipLaunchKernelGGL(lce_merge, dim3((unsigned)mblocks), dim3(kMergeThreads), 0, c.stream, partial, zy,
                       c.targets, c.N, g.n_slabs, c.V, c.loss, reinterpret_cast<float2*>(c.lse));
    return hipGetLastError();
}

}  // namespace ce
