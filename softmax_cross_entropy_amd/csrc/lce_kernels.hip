// Fused linear cross-entropy forward for gfx950: loss and log-sum-exp of Z = H W^T
// without materialising Z, and the kernels of its backward.
//
// Ineshin, "A fused linear cross-entropy forward kernel for Apple GPUs", section 1:
// each vocabulary tile of Z is folded into a running per-row state (m, s),
// m' = max(m, m_t), s' = s exp(m - m') + sum_j exp(z_j - m'), and the target logit
// is captured by the tile that holds the target column.
//
// Kernels:
//   lce_tile<kTileFwd>   one 256 x 256 tile of Z per workgroup (bf16 MFMA 32x32x16, fp32
//                    accumulate, K streamed through LDS in 64-wide stages, two buffers
//                    for H's rows and three for W's).  Its epilogue turns the fp32
//                    accumulators straight into one (m, s) pair per row for each
//                    128-column slab (exact slab maximum, then one exponential per
//                    logit), and stores the target logit from the same accumulator when
//                    the target column is in the slab.
//   lce_merge        folds the slabs of each row in slab order into (m, s), then
//                    loss = (m - z_y) + log s and lse = (m, log s).
//   lce_tile<kTileGrad>  the same tile of Z turned into the bf16 gradient of the logits (the
//                    backward's regenerated logits), row-major and transposed.
//   lce_tile<kTileGemm>  the same K loop as a plain product C (+)= A B^T of two K-contiguous
//                    bf16 operands into fp32: the backward's dH = dZ W and dW = dZ^T H,
//                    with W and H transposed beforehand by lce_transpose.
// Forward workspace: partial (m, s) float2 [N][n_slabs], then z_y float [N].
//
// The page's kernel merges fixed 8192-column tiles in a chain of dependent
// dispatches.  Here every tile of the grid is independent (the merge is associative,
// and the fixed slab order of lce_merge keeps the result deterministic), which lets
// 256 compute units work on the whole vocabulary at once.
#include <hip/hip_runtime.h>

#include <utility>

#include "device_common.h"
#include "launch.h"

namespace ce {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr int BM = 256;              // rows of H per tile
constexpr int BN = 256;              // rows of W (vocabulary columns) per tile
constexpr int BK = 64;               // reduction depth per LDS stage
constexpr int kThreads = 256;        // 4 waves as 2 x 2, each owning 128 x 128 of the tile
constexpr int WT = 128;              // wave tile edge
constexpr int FB = WT / 32;          // 4 x 4 MFMA 32x32 blocks per wave
constexpr int kStageBytes = BM * BK * 2;  // 32 KiB per operand per stage
// LDS rings: two stages of A and three of B (160 KiB, all of a compute unit's LDS).  The
// third B buffer lets a stage's B rows be loaded a whole stage earlier than its A rows,
// so the loads spread over all four K16 steps of a stage (see the K loop).
constexpr int kBufA = 2;
constexpr int kBufB = 3;
constexpr int kStageArea = (kBufA + kBufB) * kStageBytes;
// The gradient epilogue stages each wave's 128 x 128 bf16 block of dZ through LDS,
// column-major with a column pitch of 136 elements (272 bytes: 16-byte aligned columns,
// and the two half-waves' columns four apart land in different banks).
constexpr int kTPitch = WT + 8;
constexpr int kWaveStaging = WT * kTPitch * 2;
constexpr int kStagingBytes = 4 * kWaveStaging;
constexpr int kTilesPerGroup = 32;   // tiles per super-block (one per CU of an XCD)
constexpr int kXcds = 8;

enum TileMode { kTileFwd = 0, kTileGrad = 1, kTileGemm = 2 };

// The tile computes Z[r][c] = sum_k A[r][k] B[c][k] over K for A rows r < N and B rows
// c in [c0, c_end), both operands bf16 and K-contiguous (an NT product).  In the lce
// calls A = H and B = W (K = D); a plain product passes its own operands.
struct TileArgs {
    const __bf16* H;    // A: row r at H + r * lda
    const __bf16* W;    // B: row c at W + c * ldb
    const int32_t* targets;
    int64_t N;          // rows of A
    int64_t K;          // reduction length (a multiple of 8)
    int64_t lda, ldb;   // row strides of A and B, elements (multiples of 8)
    int64_t V;
    int64_t c0, c_end;  // B rows (vocabulary columns) [c0, c_end) this launch covers
    int n_row_tiles, n_col_tiles;
    int gr, gc;      // super-block shape in tiles (gr * gc == 32)
    int n_rg, n_sb;  // row groups, super-blocks
    // forward
    int n_slabs;
    float2* partial;  // [N][n_slabs]
    float* zy;        // [N]
    // gradient of the logits
    const float2* lse;  // [N] saved (m, log s)
    const float* g;     // [N]
    __bf16* G;          // [N][ldG], column c at c - c0
    int64_t ldG;
    __bf16* GT;         // the same chunk transposed: [width][ldGT], column c as row c - c0
    int64_t ldGT;
    __bf16* WT;         // the W chunk transposed: [K][ldWT], W row c as column c - c0, zero
    int64_t ldWT;       // up to the next multiple of 8 columns
    // plain product: C[r][c - c0] (+)= Z[r][c], fp32, row r at C + r * ldc
    float* C;
    int64_t ldc;
    int32_t accumulate;
};

// LDS layout of one operand stage: 256 rows x 8 chunks of 16 bytes (8 bf16 along K).
// The chunk index is XORed with (row / 2) % 8 so that the 16 rows an MFMA operand
// read touches at one K chunk land in 16 different 16-byte bank groups:
//   byte offset of (row, chunk) = row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4).

// kTileFwd: the forward epilogue ((m, s) per row per 128-column slab, target logit).
// kTileGrad: the same tile of Z turned into dZ = g (exp((z - m) - log s) - [col = y])
// with the saved (m, log s), stored in bf16 (the logits regenerated for the backward),
// both row-major and transposed: each of the two products of the backward then reads
// it K-contiguous.  The transposed copy is staged through LDS and leaves in 16-byte
// stores of 8 rows of a column.
// kTileGemm: the tile stored (or added) into an fp32 matrix.
template <int kMode>
__global__ __launch_bounds__(kThreads, 1) void lce_tile(TileArgs a0, TileArgs a1, int split) {
    constexpr bool kGrad = kMode == kTileGrad;
    constexpr bool kGemm = kMode == kTileGemm;
    // A plain-product launch may carry two independent products: workgroups below
    // `split` compute the first, the rest the second (split is a multiple of 8, so both
    // keep the XCD-aware tile order).  One grid of both products' tiles leaves fewer
    // idle compute units at the end than two launches of two tiles per unit each.
    const bool second = kGemm && (int)blockIdx.x >= split;
    const TileArgs a = second ? a1 : a0;
    // One LDS object (the compiler then sees the DMA writes and the fragment reads as
    // one array and inserts no waits of its own): the A and B stage rings (or, in the
    // gradient epilogue, the dZ staging blocks).
    constexpr int kData = kGrad && kStagingBytes > kStageArea ? kStagingBytes : kStageArea;
    __shared__ __attribute__((aligned(16))) char smem[kData];
    auto lds_a = [&](int buf) { return smem + buf * kStageBytes; };
    auto lds_b = [&](int buf) { return smem + (kBufA + buf) * kStageBytes; };

    // ---- which tile: XCD-aware super-blocks ----------------------------------
    // Consecutive workgroups go to the 8 XCDs in turn.  The k-th workgroup an XCD
    // receives is given position k % 32 of super-block k / 32 of that XCD, so the 32
    // workgroups an XCD runs together share gr row tiles of H and gc column tiles of W
    // through its L2, and the 8 XCDs work on neighbouring super-blocks of the same W
    // columns at the same time.
    const int b = (int)blockIdx.x - (second ? split : 0);
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
    // Wave index read into a scalar register, so that the per-load LDS destinations (M0)
    // are computed with scalar adds instead of a vector add and a v_readfirstlane each.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int64_t row0 = (int64_t)row_tile * BM;
    const int64_t col0 = a.c0 + (int64_t)col_tile * BN;

    // ---- global -> LDS loads: each wave fills 64 rows of A and of B per stage ----
    // One buffer_load_dwordx4 ... lds writes 64 lanes x 16 bytes = 8 LDS rows; lane i lands
    // at (row = first + i / 8, physical chunk i % 8), so it fetches the logical chunk
    // that the swizzle maps there.  Rows past N (or V) re-read the last valid row; their
    // results are never stored (columns past V are masked in the epilogue).
    const int lrow = wave * 64 + (lane >> 3);  // LDS row of load q = 0; q adds 8 rows
    int koff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int r = par * 8 + (lane >> 3);  // (row >> 1) & 7 depends only on q's parity
        koff[par] = ((lane & 7) ^ ((r >> 1) & 7)) * 8;
    }
    // Addresses: a buffer descriptor per operand tile (its first row, its valid rows)
    // plus a 32-bit per-lane byte offset; rows past N (or V) are clamped to the last
    // valid row, so every load stays inside its descriptor's range.
    const int64_t a_rows = a.N - row0 < BM ? a.N - row0 : BM;  // valid rows in this tile
    const int64_t b_rows = a.c_end - col0 < BN ? a.c_end - col0 : BN;
    const uint32_t a_row_bytes = (uint32_t)(a.lda * 2);
    const uint32_t b_row_bytes = (uint32_t)(a.ldb * 2);
    const char* a_tile = reinterpret_cast<const char*>(a.H + row0 * a.lda);
    const char* b_tile = reinterpret_cast<const char*>(a.W + col0 * a.ldb);
    // The DMA goes through buffer_load_dwordx4 ... lds rather than global_load_lds: the
    // compiler counts LDS reads precisely only while no FLAT-encoded instruction is in
    // flight, and with the global form pending it waited for all LDS reads
    // (s_waitcnt lgkmcnt(0)) before every group of MFMAs, including the reads issued
    // for later K16 steps.  Word 3 of the descriptor: raw 32-bit data, no swizzle.
    const __amdgpu_buffer_rsrc_t rsrc_a =
        __builtin_amdgcn_make_buffer_rsrc((void*)a_tile, (short)0, (int)((uint32_t)a_rows * a_row_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsrc_b =
        __builtin_amdgcn_make_buffer_rsrc((void*)b_tile, (short)0, (int)((uint32_t)b_rows * b_row_bytes), 0x00020000);

    // The LDS destination of group q is the group-0 slot plus q * 1 KiB; the instruction's
    // immediate offset moves the LDS and the global address together, so every group
    // shares one LDS base (M0) and the global address is pre-biased by -q KiB.
    // DMA of one stage, group by group: groups 0..7 load A rows into buffer `buf` of the A
    // ring, 8..15 load W rows into buffer `buf` of the B ring.  Group q fills LDS rows
    // wave * 64 + (q % 8) * 8 .. + 7.  The byte offset into the tile is row * 2D + K
    // bytes, below (valid rows) * 2D.
    auto dma_group = [&](auto qc, int kt, int buf) {
        constexpr int q = decltype(qc)::value % 8;
        constexpr bool is_b = decltype(qc)::value >= 8;
        const int64_t k0 = (int64_t)kt * BK;
        const int r = lrow + q * 8;
        const int64_t nrows = is_b ? b_rows : a_rows;
        const int rr = r < nrows ? r : (int)nrows - 1;
        // K tail: past K, re-read this row's last chunk; zeroed in LDS once it lands
        const uint32_t kb = (uint32_t)(k0 + koff[q & 1] < a.K ? koff[q & 1] : a.K - 8 - k0) * 2;
        const uint32_t voff = (uint32_t)(k0 * 2) + ((uint32_t)rr * (is_b ? b_row_bytes : a_row_bytes) + kb);
        char* dst = (is_b ? lds_b(buf) : lds_a(buf)) + (wave * 64 + q * 8) * 128;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(is_b ? rsrc_b : rsrc_a, (lds_void_t*)dst, 16, voff, 0, 0, 0);
    };
    // all of stage kt's A rows (groups 0..7) or B rows (8..15)
    auto issue = [&](auto bc, int kt, int buf) {
        constexpr int q0 = decltype(bc)::value ? 8 : 0;
        [&]<int... Q>(std::integer_sequence<int, Q...>) {
            (dma_group(std::integral_constant<int, q0 + Q>{}, kt, buf), ...);
        }(std::make_integer_sequence<int, 8>{});
    };
    // Waits are written with the builtin, which the compiler's own wait insertion sees
    // (an inline-asm wait is opaque to it, so it added lgkmcnt(0) waits of its own after
    // the barrier); the empty asm statements keep LDS accesses from moving across them.
    // s_waitcnt immediates on gfx9: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
    constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0)
    constexpr int kWaitVm8 = 0x0F78;    // vmcnt(8): one operand's loads of a stage pending
    constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)
    // Waits until every DMA issued has landed (loads retire in order).
    auto wait_all = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        asm volatile("" ::: "memory");
    };
    // Waits until all but the last 8 loads issued have landed: in the loop, those 8 are
    // the B rows of the stage after next, issued during this stage's first two steps.
    auto wait_but_next_b = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitVm8);
        asm volatile("" ::: "memory");
    };
    auto lds_barrier = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // In a K-tail stage the chunks past D hold copies of a valid chunk: overwrite this
    // lane's slots with zeros after its loads have landed, before the barrier that
    // publishes the stage (A buffer abuf, B buffer bbuf).
    auto zero_tail = [&](int kt, int abuf, int bbuf) {
        const int64_t k0 = (int64_t)kt * BK;
        if (k0 + BK <= a.K) return;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (k0 + koff[q & 1] >= a.K) {
                const int o = (wave * 64 + q * 8) * 128 + lane * 16;
                *reinterpret_cast<U4*>(lds_a(abuf) + o) = U4{{0u, 0u, 0u, 0u}};
                *reinterpret_cast<U4*>(lds_b(bbuf) + o) = U4{{0u, 0u, 0u, 0u}};
            }
        }
    };

    // v_mfma_f32_32x32x16_bf16: lane l supplies row l % 32 of the A block and column
    // l % 32 of the B block, K elements 8 * (l / 32) .. + 7 of the 16; it receives
    // D[row = 8 * (e / 4) + 4 * (l / 32) + e % 4][col = l % 32] in element e.  The two
    // operands have the same register layout, so the W fragment is passed as A and the
    // H fragment as B: D is then a block of Z^T, and each lane collects 16 vocabulary
    // columns of one token row per block, which keeps the epilogue's row reductions
    // inside the lane.
    f32x16 acc[FB][FB];
#pragma unroll
    for (int i = 0; i < FB; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h2 = lane >> 5;
    const int sw = (l32 >> 1) & 7;
    int off[4];  // byte offset of this lane's operand row and chunk for K16 step kk
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) off[kk] = l32 * 128 + (((kk * 2 + h2) ^ sw) << 4);

    auto read_frags = [&](int abuf, int bbuf, int kk, bf16x8 (&fa)[FB], bf16x8 (&fb)[FB]) {
        const char* As = lds_a(abuf) + wm * WT * 128;
        const char* Bs = lds_b(bbuf) + wn * WT * 128;
#pragma unroll
        for (int i = 0; i < FB; ++i) {
            fa[i] = *reinterpret_cast<const bf16x8*>(As + i * 32 * 128 + off[kk]);
            fb[i] = *reinterpret_cast<const bf16x8*>(Bs + i * 32 * 128 + off[kk]);
        }
    };
    auto mfma_all = [&](const bf16x8 (&fa)[FB], const bf16x8 (&fb)[FB]) {
#pragma unroll
        for (int i = 0; i < FB; ++i)
#pragma unroll
            for (int j = 0; j < FB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    };
    // One K16 step is 16 MFMAs and 8 LDS reads: one read after every 2 MFMAs.
    auto interleave = [&]() {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        }
    };
    // One K16 step: its 16 MFMAs (on fa, fb) in 8 chunks of 2, each chunk followed by one
    // LDS read of a later step's fragments (into na, nb from A buffer rabuf and B buffer
    // rbbuf, K16 step rkk), and every other chunk by one DMA load, group q0 + chunk / 2,
    // of stage kt_load into buffer lbuf of that group's ring.  The scheduler keeps the
    // chunk order, so the DMA issue never idles the matrix pipe.  A stage's 16 loads are
    // spread over all four K16 steps, 4 per step: B rows in the two steps before the
    // barrier, A rows in the two after.  Issued 16 to a step they filled the
    // vector-memory address queues (the counters showed them full a tenth of the
    // kernel's time) and stalled the MFMAs queued behind them.
    auto step = [&](auto q0c, const bf16x8 (&fa)[FB], const bf16x8 (&fb)[FB], int rabuf, int rbbuf, int rkk,
                    bf16x8 (&na)[FB], bf16x8 (&nb)[FB], int kt_load, int lbuf) {
        constexpr int q0 = decltype(q0c)::value;
        const char* As = lds_a(rabuf) + wm * WT * 128;
        const char* Bs = lds_b(rbbuf) + wn * WT * 128;
        auto chunk = [&](auto cc) {
            constexpr int c = decltype(cc)::value;
            constexpr int i = c / 2, j0 = 2 * (c % 2);
            acc[i][j0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j0], fa[i], acc[i][j0], 0, 0, 0);
            acc[i][j0 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j0 + 1], fa[i], acc[i][j0 + 1], 0, 0, 0);
            if constexpr (c < 4)
                na[c] = *reinterpret_cast<const bf16x8*>(As + c * 32 * 128 + off[rkk]);
            else
                nb[c - 4] = *reinterpret_cast<const bf16x8*>(Bs + (c - 4) * 32 * 128 + off[rkk]);
            if constexpr (c % 2 == 1) dma_group(std::integral_constant<int, q0 + c / 2>{}, kt_load, lbuf);
            __builtin_amdgcn_sched_barrier(0);
        };
        [&]<int... C>(std::integer_sequence<int, C...>) {
            (chunk(std::integral_constant<int, C>{}), ...);
        }(std::make_integer_sequence<int, 8>{});
    };
    // kTileGrad also writes the W chunk transposed (the B operand of the dH product),
    // from the stage buffers, so no separate transpose pass reads W again: stage s of
    // the K loop is written by the tile whose row tile is s % n_row_tiles, so the row
    // tiles of a column tile share the work.  ds_read_b64_tr_b16 transposes within each
    // 16-lane group: output lane j, element e takes element j % 4 of the 8 bytes that
    // lane j / 4 + 4 e addresses.  Lane j of group g addresses tile row cb + j / 4 and
    // K values kb + 4 (j % 4) .. + 3, so it receives K value kb + j of tile rows
    // cb .. cb + 3; a second read gives rows cb + 4 .. cb + 7, and the lane stores the 8
    // of them as 16 bytes of WT row kb + j.  Columns past the chunk are stored as zeros
    // up to the next multiple of 8 (the K padding of the dH product).  A stage is read
    // for this when its loads have landed and before the barrier that frees its buffer.
    // The two reads of a step are inline assembly that waits for them in the same
    // statement: through the builtin, the compiler waited for every stage load in flight
    // first (vmcnt(0)), since it cannot tell which LDS bytes the builtin reads, and the B
    // rows of the stage after next are always in flight here (into another buffer).
    auto put_wt = [&](int s, int buf) {
        const char* Bs = lds_b(buf);
        const int g4 = lane >> 4, j = lane & 15;
        const int64_t wt_w8 = (a.c_end - a.c0 + 7) & ~(int64_t)7;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int kb = 16 * (it >> 1);
            const int cb = wave * 64 + 32 * (it & 1) + 8 * g4;
            const int kk = kb + 4 * (j & 3);
            auto off = [&](int row) { return row * 128 + (((kk >> 3) ^ ((row >> 1) & 7)) << 4) + (kk & 7) * 2; };
            v4i16 lo, hi;
            {
                const uint32_t alo = (uint32_t)(uintptr_t)(Bs + off(cb + (j >> 2)));
                const uint32_t ahi = (uint32_t)(uintptr_t)(Bs + off(cb + 4 + (j >> 2)));
                asm volatile("ds_read_b64_tr_b16 %0, %2\n\tds_read_b64_tr_b16 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                             : "=&v"(lo), "=&v"(hi) : "v"(alo), "v"(ahi) : "memory");
            }
            const int64_t kg = (int64_t)s * BK + kb + j;
            const int64_t cg = col0 + cb;  // vocabulary column of the first of the 8
            if (kg < a.K && cg - a.c0 < wt_w8) {
                // the 8 columns cg .. cg + 7: lo holds the first 4, hi the next 4; columns
                // at or past the chunk's end are stored as 0
                const short e[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                U4 v;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint32_t e0 = cg + 2 * t < a.c_end ? (uint16_t)e[2 * t] : 0u;
                    const uint32_t e1 = cg + 2 * t + 1 < a.c_end ? (uint16_t)e[2 * t + 1] : 0u;
                    v.w[t] = e0 | (e1 << 16);
                }
                store_u4(reinterpret_cast<uint16_t*>(a.WT) + kg * a.ldWT + (cg - a.c0), v);
            }
        }
    };
    auto owns_stage = [&](int s) { return s % a.n_row_tiles == row_tile; };

    // The barrier of stage kt (A buffer ca, B buffer cb): stage kt + 1 (A buffer na, B
    // buffer nb) has landed, with only the B rows of stage kt + 2 still in flight; after
    // it every wave has finished reading stage kt's buffers, which then take the A rows
    // of stage kt + 2 and the B rows of stage kt + 3.
    auto sync_stage = [&](int kt, int cb, int na, int nb, int nk) {
        wait_but_next_b();
        if (kt + 1 < nk) zero_tail(kt + 1, na, nb);
        if constexpr (kGrad)
            if (owns_stage(kt)) put_wt(kt, cb);
        lds_barrier();
    };

    // Pipeline: the fragments of a K16 step are read from LDS two steps ahead, into four
    // rotating sets, so each wave keeps twice as many reads in flight (one wave per SIMD
    // is bound by LDS read latency).  A stage's single barrier sits between its steps 1
    // and 2: by then every wave has read all four steps of the stage (steps 2 and 3 during
    // steps 0 and 1), so its buffers are free, and stage kt + 1 has landed, so steps 2
    // and 3 can read the next stage's first two steps.  The A rows of stage kt + 2 are
    // loaded during steps 2 and 3 into stage kt's A buffer, and have two to three K16
    // steps to land.  The B rows of stage kt + 2 are loaded during steps 0 and 1, into
    // the third B buffer (stage kt - 1's, free since the previous barrier), and have five
    // to six steps.  So each K16 step issues 4 of a stage's 16 loads.
    const int nk = (int)((a.K + BK - 1) / BK);
    bf16x8 fa0[FB], fb0[FB], fa1[FB], fb1[FB], fa2[FB], fb2[FB], fa3[FB], fb3[FB];
    issue(std::false_type{}, 0, 0);
    issue(std::true_type{}, 0, 0);
    if constexpr (kGemm) {
        // An accumulating product starts from C's old values, loaded while the first
        // stage's DMA is in flight, so its epilogue only stores.  (Read and added in the
        // epilogue, every load waited for the store before it: the compiler does not move
        // a load across a store to the same array.)  A row block's 16 vectors are loaded
        // together, the next block's while this one moves into the accumulators.
        if (a.accumulate) {
            const int64_t r0w = row0 + wm * WT, c0w = col0 + wn * WT;
            if (c0w + WT <= a.c_end) {
                float4 buf[2][FB * 4];
                auto load_block = [&](int i, float4 (&b)[FB * 4]) {
                    const int64_t row = r0w + i * 32 + l32;
                    const float* crow = a.C + (row < a.N ? row : a.N - 1) * a.ldc - a.c0 + c0w + 4 * h2;
#pragma unroll
                    for (int jq = 0; jq < FB * 4; ++jq)
                        b[jq] = *reinterpret_cast<const float4*>(crow + (jq / 4) * 32 + 8 * (jq % 4));
                };
                load_block(0, buf[0]);
#pragma unroll
                for (int i = 0; i < FB; ++i) {
                    if (i + 1 < FB) load_block(i + 1, buf[(i + 1) & 1]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int jq = 0; jq < FB * 4; ++jq) {
                        const float4 o = buf[i & 1][jq];
                        const int j = jq / 4, q = jq % 4;
                        acc[i][j][4 * q] = o.x;
                        acc[i][j][4 * q + 1] = o.y;
                        acc[i][j][4 * q + 2] = o.z;
                        acc[i][j][4 * q + 3] = o.w;
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < FB; ++i) {
                    const int64_t row = r0w + i * 32 + l32;
                    const float* crow = a.C + (row < a.N ? row : a.N - 1) * a.ldc - a.c0;
#pragma unroll
                    for (int j = 0; j < FB; ++j)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int64_t c = c0w + j * 32 + 8 * (e / 4) + 4 * h2 + e % 4;
                            acc[i][j][e] = c < a.c_end ? crow[c] : 0.f;
                        }
                }
            }
        }
    }
    wait_all();
    zero_tail(0, 0, 0);
    lds_barrier();
    // stage 1: B rows, then A rows (the loop's first wait leaves only later loads pending)
    if (nk > 1) {
        issue(std::true_type{}, 1, 1);
        issue(std::false_type{}, 1, 1);
    }
    read_frags(0, 0, 0, fa0, fb0);
    read_frags(0, 0, 1, fa1, fb1);
    int cb = 0;  // B buffer of stage kt: kt % 3
    for (int kt = 0; kt + 1 < nk; ++kt) {
        const int ca = kt & 1;
        const int b_next = cb == 2 ? 0 : cb + 1, b_load = b_next == 2 ? 0 : b_next + 1;
        // the last iteration re-issues stage nk - 1 into free buffers, which are never
        // read: no branch around the DMA, so it can interleave with the MFMAs
        const int kt_load = kt + 2 < nk ? kt + 2 : nk - 1;
        step(std::integral_constant<int, 8>{}, fa0, fb0, ca, cb, 2, fa2, fb2, kt_load, b_load);
        step(std::integral_constant<int, 12>{}, fa1, fb1, ca, cb, 3, fa3, fb3, kt_load, b_load);
        sync_stage(kt, cb, ca ^ 1, b_next, nk);
        step(std::integral_constant<int, 0>{}, fa2, fb2, ca ^ 1, b_next, 0, fa0, fb0, kt_load, ca);
        step(std::integral_constant<int, 4>{}, fa3, fb3, ca ^ 1, b_next, 1, fa1, fb1, kt_load, ca);
        cb = b_next;
    }
    // The forward's epilogue takes its rows' targets from LDS once the K loop is done
    // (held in registers through the epilogue, they pushed it into spills): thread t loads
    // row t's before the last stage, and stores it once every wave is past the loop.
    int32_t my_target = -1;
    if constexpr (kMode == kTileFwd) my_target = row0 + tid < a.N ? a.targets[row0 + tid] : -1;
    {
        const int ca = (nk - 1) & 1;
        read_frags(ca, cb, 2, fa2, fb2);
        mfma_all(fa0, fb0);
        interleave();
        read_frags(ca, cb, 3, fa3, fb3);
        mfma_all(fa1, fb1);
        interleave();
        mfma_all(fa2, fb2);
        mfma_all(fa3, fb3);
    }
    // the last loop iteration's (redundant) DMA must land before the workgroup can end
    wait_all();
    if constexpr (kGrad)
        if (owns_stage(nk - 1)) put_wt(nk - 1, cb);
    int32_t* const tile_targets = reinterpret_cast<int32_t*>(smem);
    if constexpr (kMode == kTileFwd) {
        lds_barrier();  // every wave is done with the stage buffers
        tile_targets[tid] = my_target;
        lds_barrier();
    }
    // the gradient epilogue's targets: this lane's four rows, in registers
    int32_t ytile[FB] = {-1, -1, -1, -1};
    if constexpr (kGrad) {
#pragma unroll
        for (int i = 0; i < FB; ++i) {
            const int64_t row = row0 + wm * WT + i * 32 + l32;
            ytile[i] = row < a.N ? a.targets[row] : -1;
        }
    }

    // ---- epilogue: (m, s) per row over this wave's 128 columns ----------------
    // acc[i][j][e] holds Z[row = wrow0 + i*32 + l32][col = wcol0 + j*32 + 8*(e/4) + 4*h2 + e%4]:
    // this lane holds 64 of the wave's 128 columns of 4 rows, lane ^ 32 the other 64.
    const int64_t wcol0 = col0 + wn * WT;
    const int64_t wrow0 = row0 + wm * WT;
    auto col_of = [&](int j, int e) { return j * 32 + 8 * (e / 4) + 4 * h2 + (e % 4); };

    if constexpr (kGemm) {
        // acc[i][j][4q .. 4q + 3] are 4 consecutive columns of one row: 16-byte stores,
        // one row per lane, in a fixed order (an accumulating product started from C's
        // old values).
#pragma unroll
        for (int i = 0; i < FB; ++i) {
            const int64_t row = wrow0 + i * 32 + l32;
            if (row >= a.N) continue;
            float* crow = a.C + row * a.ldc - a.c0;
#pragma unroll
            for (int j = 0; j < FB; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t c = wcol0 + j * 32 + 8 * q + 4 * h2;
                    float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                    if (c + 3 < a.c_end) {
                        *reinterpret_cast<float4*>(crow + c) = make_float4(v[0], v[1], v[2], v[3]);
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            if (c + t < a.c_end) crow[c + t] = v[t];
                    }
                }
        }
    } else if constexpr (kGrad) {
        // dZ for this lane's 4 rows x 64 columns.  A row with an out-of-range target
        // gets m = NaN, so its whole row of dZ is NaN (its loss is NaN too).  The
        // row-major copy is stored directly, 4 columns per store; the transposed copy goes
        // through this wave's LDS block first, so that it leaves in 16-byte stores of 8
        // rows of a column.  After the barrier no wave reads the stage buffers any more
        // (the last DMA has landed: wait_all above).
        // this lane's rows' saved (m, log s) and upstream gradients, loaded together
        float2 lse_r[FB];
        float g_r[FB];
#pragma unroll
        for (int i = 0; i < FB; ++i) {
            const int64_t row = wrow0 + i * 32 + l32;
            const int64_t rr = row < a.N ? row : a.N - 1;
            lse_r[i] = a.lse[rr];
            g_r[i] = a.g[rr];
        }
        lds_barrier();
        char* const tblk = smem + wave * kWaveStaging;
        auto tput = [&](int cl, int rl, uint16_t v) {
            *reinterpret_cast<uint16_t*>(tblk + (cl * kTPitch + rl) * 2) = v;
        };
#pragma unroll
        for (int i = 0; i < FB; ++i) {
            const int lr = wm * WT + i * 32 + l32;
            const int64_t row = row0 + lr;
            if (row >= a.N) continue;
            const int32_t y = ytile[i];
            const float2 l = lse_r[i];
            const float m = (y >= 0 && (int64_t)y < a.V) ? l.x : __builtin_nanf("");
            const float nlsl = -l.y * kLog2e;
            const float gr = g_r[i];
            __bf16* grow = a.G + row * a.ldG - a.c0;
            const int rl = i * 32 + l32;  // row within the wave's block
            auto dz = [&](float z) { return gr * __builtin_amdgcn_exp2f(__builtin_fmaf(z - m, kLog2e, nlsl)); };
#pragma unroll
            for (int j = 0; j < FB; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int cl = j * 32 + 8 * q + 4 * h2;  // 4 consecutive columns of the block
                    const int64_t c = wcol0 + cl;
                    const float v0 = dz(acc[i][j][4 * q]), v1 = dz(acc[i][j][4 * q + 1]);
                    const float v2 = dz(acc[i][j][4 * q + 2]), v3 = dz(acc[i][j][4 * q + 3]);
                    uint2 w;
                    w.x = Elem<__bf16>::bits2(v0, v1);
                    w.y = Elem<__bf16>::bits2(v2, v3);
                    // the block always takes all four; columns past the chunk are never read back
                    tput(cl, rl, (uint16_t)w.x);
                    tput(cl + 1, rl, (uint16_t)(w.x >> 16));
                    tput(cl + 2, rl, (uint16_t)w.y);
                    tput(cl + 3, rl, (uint16_t)(w.y >> 16));
                    if (c + 3 < a.c_end) {
                        *reinterpret_cast<uint2*>(grow + c) = w;
                    } else {
                        const float v[4] = {v0, v1, v2, v3};
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            if (c + t < a.c_end) grow[c + t] = (__bf16)v[t];
                    }
                }
            // the target column: stored again as g (p - 1) by the lane that stored it
            // (same lane, same address, so the second store lands last)
            const int64_t yrel = (int64_t)y - wcol0;
            if (yrel >= 0 && yrel < WT && (((int)yrel >> 2) & 1) == h2) {
                const int cc = (int)yrel;
                const int jj = cc >> 5, ee = (((cc >> 3) & 3) << 2) | (cc & 3);
                float z = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float lo = (jj & 1) ? acc[i][1][e] : acc[i][0][e];
                    const float hi = (jj & 1) ? acc[i][3][e] : acc[i][2][e];
                    z = ee == e ? ((jj & 2) ? hi : lo) : z;
                }
                const __bf16 b = (__bf16)(dz(z) - gr);
                grow[y] = b;
                tput(cc, rl, __builtin_bit_cast(uint16_t, b));  // after this lane's first write of it
            }
        }
        // The transposed copy: lane k of 2048 16-byte pieces takes column k / 16 of the
        // block, rows 8 (k % 16) .. + 7; 16 lanes write one column's 256 bytes.  LDS
        // accesses of one wave complete in order, so the reads see this wave's writes.
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
        uint16_t* const gt = reinterpret_cast<uint16_t*>(a.GT);
        const bool t16 = (a.ldGT % 8) == 0;  // columns of GT start on 16-byte boundaries
#pragma unroll 4
        for (int it = 0; it < WT * WT / 8 / 64; ++it) {
            const int k = it * 64 + lane;
            const int cl = k >> 4, rc = (k & 15) * 8;
            const int64_t c = wcol0 + cl;
            const int64_t r = wrow0 + rc;
            if (c >= a.c_end || r >= a.N) continue;
            const U4 v = *reinterpret_cast<const U4*>(tblk + (cl * kTPitch + rc) * 2);
            uint16_t* dst = gt + (c - a.c0) * a.ldGT + r;
            if (t16 && r + 8 <= a.N) {
                store_u4(dst, v);
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    if (r + t < a.N) dst[t] = (uint16_t)(v.w[t >> 1] >> (16 * (t & 1)));
            }
        }
    } else {
        // target logits: the lane holding the target column of a row stores it.  A row's
        // target lies in this wave's columns for about one wave in ten, so the select runs
        // rarely and only in those lanes: column c = j*32 + 8*(e/4) + 4*h2 + e%4 gives
        // j = c / 32 and e = 4 * ((c / 8) % 4) + c % 4; pick j first, then e.
    #pragma unroll
        for (int i = 0; i < FB; ++i) {
            const int lr = wm * WT + i * 32 + l32;
            const int64_t yrel = (int64_t)tile_targets[lr] - wcol0;
            if (yrel >= 0 && yrel < WT && (((int)yrel >> 2) & 1) == h2) {
                const int c = (int)yrel;
                const int jj = c >> 5, ee = (((c >> 3) & 3) << 2) | (c & 3);
                float v = 0.f;
    #pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float lo = (jj & 1) ? acc[i][1][e] : acc[i][0][e];
                    const float hi = (jj & 1) ? acc[i][3][e] : acc[i][2][e];
                    v = ee == e ? ((jj & 2) ? hi : lo) : v;
                }
                a.zy[row0 + lr] = v;  // a valid target implies a valid row
            }
        }

        // Per row: the exact maximum over the 128 columns (this lane's 64, then lane ^ 32's),
        // then sum exp(z - m) with one exponential per logit, and the partner's sum.  Both
        // lanes of a pair end with the same (m, s); the lower one stores it.  Columns past V
        // hold copies of the last W row and count as -inf: only the last column tile has
        // any, so the masked form is a separate instance (the accumulators stay read-only).
        const int64_t slab = (int64_t)col_tile * 2 + wn;
        auto row_states = [&](auto mask_c) {
            constexpr bool kMask = decltype(mask_c)::value;
            auto z = [&](int i, int j, int e) {
                if constexpr (kMask)
                    return wcol0 + col_of(j, e) < a.c_end ? acc[i][j][e] : kNegInf;
                else
                    return acc[i][j][e];
            };
    #pragma unroll
            for (int i = 0; i < FB; ++i) {
                float mj[FB];
    #pragma unroll
                for (int j = 0; j < FB; ++j) {
                    float t = z(i, j, 0);
    #pragma unroll
                    for (int e = 1; e < 16; ++e) t = fmaxf(t, z(i, j, e));
                    mj[j] = t;
                }
                float m = fmaxf(fmaxf(mj[0], mj[1]), fmaxf(mj[2], mj[3]));
                m = fmaxf(m, __shfl_xor(m, 32));
                const float r = ref_point(m);
                float sj[FB];
    #pragma unroll
                for (int j = 0; j < FB; ++j) {
                    float t = 0.f;
    #pragma unroll
                    for (int e = 0; e < 16; ++e) t += exp_e(z(i, j, e) - r);
                    sj[j] = t;
                }
                float s = (sj[0] + sj[1]) + (sj[2] + sj[3]);
                s += __shfl_xor(s, 32);
                const int64_t row = wrow0 + i * 32 + l32;
                if (h2 == 0 && row < a.N) a.partial[row * a.n_slabs + slab] = make_float2(m, s);
            }
        };
        if (wcol0 + WT > a.c_end)
            row_states(std::true_type{});
        else
            row_states(std::false_type{});
    }
}

constexpr int kMergeThreads = 256;
constexpr int kMergeLanes = 16;  // lanes per row; 16 rows per workgroup

// Folds one row's slabs: lane l takes slabs l, l + 16, ... (16 consecutive float2 per
// step across the lanes, one 128-byte line), four at a time with one rescale, then the
// 16 lane states merge by butterfly.  The order is fixed, so the result is too.
__global__ __launch_bounds__(kMergeThreads) void lce_merge(const float2* __restrict__ partial,
                                                            const float* __restrict__ zy,
                                                            const int32_t* __restrict__ targets, int64_t N,
                                                            int n_slabs, int64_t V, float* loss, float2* lse) {
    const int64_t r = (int64_t)blockIdx.x * (kMergeThreads / kMergeLanes) + threadIdx.x / kMergeLanes;
    const int lane = threadIdx.x % kMergeLanes;
    if (r >= N) return;  // the whole 16-lane group leaves together
    const float2* p = partial + r * n_slabs;
    MS st = ms_empty();
    int s = lane;
    for (; s + 3 * kMergeLanes < n_slabs; s += 4 * kMergeLanes) {
        float2 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = p[s + u * kMergeLanes];
        float m = st.m;
#pragma unroll
        for (int u = 0; u < 4; ++u) m = fmaxf(m, v[u].x);
        const float rr = ref_point(m);
        float acc = __fmul_rn(st.s, exp_e(st.m - rr));
#pragma unroll
        for (int u = 0; u < 4; ++u) acc += __fmul_rn(v[u].y, exp_e(v[u].x - rr));
        st = MS{m, acc};
    }
    for (; s < n_slabs; s += kMergeLanes) st = ms_merge(st, MS{p[s].x, p[s].y});
    st = ms_group_reduce<kMergeLanes>(st);
    if (lane == 0) {
        const int32_t y = targets[r];
        const bool ok = y >= 0 && (int64_t)y < V;
        const float ls = log_e(st.s);
        loss[r] = ok ? (st.m - zy[r]) + ls : __builtin_nanf("");
        lse[r] = make_float2(st.m, ls);
    }
}

struct Geometry {
    int n_row_tiles, n_col_tiles, gr, gc, n_rg, n_cg, n_sb, n_slabs;
    int64_t blocks;
};

// Tiles over N rows and `cols` vocabulary columns.
Geometry geometry(int64_t N, int64_t cols) {
    Geometry g;
    g.n_row_tiles = (int)((N + BM - 1) / BM);
    g.n_col_tiles = (int)((cols + BN - 1) / BN);
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

int64_t lce_tile_grid_items(int64_t rows, int64_t cols) {
    // geometry() in 64-bit arithmetic, for sizes whose grid may not fit a dispatch
    const int64_t rt = (rows + BM - 1) / BM, ct = (cols + BN - 1) / BN;
    const int64_t gr = rt >= 4 ? 4 : (rt >= 2 ? 2 : 1), gc = kTilesPerGroup / gr;
    const int64_t sb = ((rt + gr - 1) / gr) * ((ct + gc - 1) / gc);
    return (sb + kXcds - 1) / kXcds * kXcds * kTilesPerGroup * kThreads;
}

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
    TileArgs a{};
    a.H = static_cast<const __bf16*>(c.H);
    a.W = static_cast<const __bf16*>(c.W);
    a.targets = c.targets;
    a.N = c.N;
    a.K = a.lda = a.ldb = c.D;
    a.V = c.V;
    a.c0 = 0;
    a.c_end = c.V;
    a.n_row_tiles = g.n_row_tiles;
    a.n_col_tiles = g.n_col_tiles;
    a.gr = g.gr;
    a.gc = g.gc;
    a.n_rg = g.n_rg;
    a.n_sb = g.n_sb;
    a.n_slabs = g.n_slabs;
    a.partial = partial;
    a.zy = zy;
    hipLaunchKernelGGL(lce_tile<kTileFwd>, dim3((unsigned)g.blocks), dim3(kThreads), 0, c.stream, a, a, (int)g.blocks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int kRowsPerBlock = kMergeThreads / kMergeLanes;
    const int64_t mblocks = (c.N + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(lce_merge, dim3((unsigned)mblocks), dim3(kMergeThreads), 0, c.stream, partial, zy,
                       c.targets, c.N, g.n_slabs, c.V, c.loss, reinterpret_cast<float2*>(c.lse));
    return hipGetLastError();
}

hipError_t launch_lce_grad_chunk(const LceGradChunk& c) {
    const Geometry g = geometry(c.N, c.width);
    TileArgs a{};
    a.H = static_cast<const __bf16*>(c.H);
    a.W = static_cast<const __bf16*>(c.W);
    a.targets = c.targets;
    a.N = c.N;
    a.K = a.lda = a.ldb = c.D;
    a.V = c.V;
    a.c0 = c.c0;
    a.c_end = c.c0 + c.width;
    a.n_row_tiles = g.n_row_tiles;
    a.n_col_tiles = g.n_col_tiles;
    a.gr = g.gr;
    a.gc = g.gc;
    a.n_rg = g.n_rg;
    a.n_sb = g.n_sb;
    a.lse = reinterpret_cast<const float2*>(c.lse);
    a.g = c.g;
    a.G = static_cast<__bf16*>(c.G);
    a.ldG = c.ldG;
    a.GT = static_cast<__bf16*>(c.GT);
    a.ldGT = c.ldGT;
    a.WT = static_cast<__bf16*>(c.WT);
    a.ldWT = c.ldWT;
    hipLaunchKernelGGL(lce_tile<kTileGrad>, dim3((unsigned)g.blocks), dim3(kThreads), 0, c.stream, a, a, (int)g.blocks);
    return hipGetLastError();
}

namespace {
TileArgs gemm_args(const LceGemm& c, const Geometry& g) {
    TileArgs a{};
    a.H = static_cast<const __bf16*>(c.A);
    a.W = static_cast<const __bf16*>(c.B);
    a.N = c.M;
    a.K = c.K;
    a.lda = c.lda;
    a.ldb = c.ldb;
    a.c0 = 0;
    a.c_end = c.Ncols;
    a.n_row_tiles = g.n_row_tiles;
    a.n_col_tiles = g.n_col_tiles;
    a.gr = g.gr;
    a.gc = g.gc;
    a.n_rg = g.n_rg;
    a.n_sb = g.n_sb;
    a.C = c.C;
    a.ldc = c.ldc;
    a.accumulate = c.accumulate ? 1 : 0;
    return a;
}
}  // namespace

hipError_t launch_lce_gemm(const LceGemm& c) {
    const Geometry g = geometry(c.M, c.Ncols);
    const TileArgs a = gemm_args(c, g);
    hipLaunchKernelGGL(lce_tile<kTileGemm>, dim3((unsigned)g.blocks), dim3(kThreads), 0, c.stream, a, a,
                       (int)g.blocks);
    return hipGetLastError();
}

hipError_t launch_lce_gemm2(const LceGemm& p, const LceGemm& q) {
    const Geometry gp = geometry(p.M, p.Ncols), gq = geometry(q.M, q.Ncols);
    hipLaunchKernelGGL(lce_tile<kTileGemm>, dim3((unsigned)(gp.blocks + gq.blocks)), dim3(kThreads), 0, p.stream,
                       gemm_args(p, gp), gemm_args(q, gq), (int)gp.blocks);
    return hipGetLastError();
}

namespace {
__global__ __launch_bounds__(256) void fill_zero_f32(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

// dst[c][r] = src[r][c] for r < R, c < C, and 0 for R <= r < Rpad: one 64 x 64 block of
// src per step of a 256-thread workgroup, staged through LDS (row pitch 72 elements, so
// the 16-byte row pieces stay aligned).  C, lds and ldd are multiples of 8 and Rpad is
// one too, so every 8-element piece is either wholly inside or wholly outside.
constexpr int kTp = 64;
constexpr int kTpPitch = kTp + 8;
__global__ __launch_bounds__(256) void lce_transpose(const uint16_t* __restrict__ src, int64_t R, int64_t C,
                                                     int64_t lds, uint16_t* __restrict__ dst, int64_t ldd,
                                                     int64_t Rpad) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[kTp * kTpPitch];
    const int64_t tr = (Rpad + kTp - 1) / kTp, tc = (C + kTp - 1) / kTp;
    const int t = threadIdx.x;
    for (int64_t b = blockIdx.x; b < tr * tc; b += gridDim.x) {
        const int64_t r0 = (b / tc) * kTp, c0 = (b % tc) * kTp;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int id = t + 256 * k;
            const int rr = id >> 3, cc = (id & 7) * 8;
            const int64_t r = r0 + rr, c = c0 + cc;
            U4 v = U4{{0u, 0u, 0u, 0u}};
            if (r < R && c < C) v = *reinterpret_cast<const U4*>(src + r * lds + c);
            *reinterpret_cast<U4*>(&tile[rr * kTpPitch + cc]) = v;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int id = t + 256 * k;
            const int cc = id >> 3, rr = (id & 7) * 8;
            const int64_t c = c0 + cc, r = r0 + rr;
            if (c < C && r < Rpad) {
                U4 v;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    v.w[u] = (uint32_t)tile[(rr + 2 * u) * kTpPitch + cc] |
                             ((uint32_t)tile[(rr + 2 * u + 1) * kTpPitch + cc] << 16);
                *reinterpret_cast<U4*>(dst + c * ldd + r) = v;
            }
        }
        __syncthreads();
    }
}

// p[r][c] = 0 for r < rows, c_from <= c < c_to (row r at p + r * ld).
__global__ __launch_bounds__(256) void zero_cols_bf16(uint16_t* p, int64_t rows, int64_t ld, int64_t c_from,
                                                      int64_t c_to) {
    const int64_t w = c_to - c_from;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows * w; i += (int64_t)gridDim.x * 256)
        p[(i / w) * ld + c_from + i % w] = 0;
}

unsigned grid_for(int64_t items, int64_t per_block, int64_t cap) {
    const int64_t want = (items + per_block - 1) / per_block;
    return (unsigned)(want < 1 ? 1 : (want < cap ? want : cap));
}
}  // namespace

hipError_t launch_fill_zero_f32(float* p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_f32, dim3(grid_for(n, 256, 16384)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_transpose_bf16(const void* src, int64_t R, int64_t C, int64_t lds, void* dst, int64_t ldd,
                                 int64_t Rpad, hipStream_t stream) {
    if (C <= 0 || Rpad <= 0) return hipSuccess;
    const int64_t tiles = ((Rpad + kTp - 1) / kTp) * ((C + kTp - 1) / kTp);
    hipLaunchKernelGGL(lce_transpose, dim3(grid_for(tiles, 1, 65536)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(src), R, C, lds, static_cast<uint16_t*>(dst), ldd, Rpad);
    return hipGetLastError();
}

hipError_t launch_zero_cols_bf16(void* p, int64_t rows, int64_t ld, int64_t c_from, int64_t c_to,
                                 hipStream_t stream) {
    if (rows <= 0 || c_to <= c_from) return hipSuccess;
    hipLaunchKernelGGL(zero_cols_bf16, dim3(grid_for(rows * (c_to - c_from), 256, 4096)), dim3(256), 0, stream,
                       static_cast<uint16_t*>(p), rows, ld, c_from, c_to);
    return hipGetLastError();
}

}  // namespace ce
