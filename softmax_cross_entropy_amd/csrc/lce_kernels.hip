// Fused linear cross-entropy forward for gfx950: loss and log-sum-exp of Z = H W^T
// without materialising Z.
//
// Ineshin, "A fused linear cross-entropy forward kernel for Apple GPUs", section 1:
// each vocabulary tile of Z is folded into a running per-row state (m, s),
// m' = max(m, m_t), s' = s exp(m - m') + sum_j exp(z_j - m'), and the target logit
// is captured by the tile that holds the target column.
//
// Two kernels:
//   lce_tile   one 256 x 256 tile of Z per workgroup (bf16 MFMA 32x32x16, fp32 accumulate,
//              K = D streamed through LDS in 64-wide double-buffered stages).  Its
//              epilogue turns the fp32 accumulators straight into one (m, s) pair per
//              row for each 128-column slab (exact slab maximum, then one exponential
//              per logit), and stores the target logit from the same accumulator when
//              the target column is in the slab.
//   lce_merge  folds the slabs of each row in slab order into (m, s), then
//              loss = (m - z_y) + log s and lse = (m, log s).
// Workspace: partial (m, s) float2 [N][n_slabs], then z_y float [N].
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

constexpr int BM = 256;              // rows of H per tile
constexpr int BN = 256;              // rows of W (vocabulary columns) per tile
constexpr int BK = 64;               // reduction depth per LDS stage
constexpr int kThreads = 256;        // 4 waves as 2 x 2, each owning 128 x 128 of the tile
constexpr int WT = 128;              // wave tile edge
constexpr int FB = WT / 32;          // 4 x 4 MFMA 32x32 blocks per wave
constexpr int kStageBytes = BM * BK * 2;  // 32 KiB per operand per stage
constexpr int kStageArea = 2 * 2 * kStageBytes;  // two stages of A and B
// The gradient epilogue stages each wave's 128 x 128 bf16 block of dZ through LDS,
// column-major with a column pitch of 136 elements (272 bytes: 16-byte aligned columns,
// and the two half-waves' columns four apart land in different banks).
constexpr int kTPitch = WT + 8;
constexpr int kWaveStaging = WT * kTPitch * 2;
constexpr int kStagingBytes = 4 * kWaveStaging;
constexpr int kTilesPerGroup = 32;   // tiles per super-block (one per CU of an XCD)
constexpr int kXcds = 8;

struct TileArgs {
    const __bf16* H;
    const __bf16* W;
    const int32_t* targets;
    int64_t N;
    int64_t D;
    int64_t V;
    int64_t c0, c_end;  // vocabulary columns [c0, c_end) this launch covers
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
};

// LDS layout of one operand stage: 256 rows x 8 chunks of 16 bytes (8 bf16 along K).
// The chunk index is XORed with (row / 2) % 8 so that the 16 rows an MFMA operand
// read touches at one K chunk land in 16 different 16-byte bank groups:
//   byte offset of (row, chunk) = row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4).

// kGrad = false: the forward epilogue ((m, s) per row per 128-column slab, target logit).
// kGrad = true: the same tile of Z turned into dZ = g (exp((z - m) - log s) - [col = y])
// with the saved (m, log s), stored in bf16 (the logits regenerated for the backward),
// both row-major and transposed: each of the two products of the backward then reads
// its operand without a transpose.  The transposed copy is staged through LDS and
// leaves in 16-byte stores of 8 rows of a column.
template <bool kGrad>
__global__ __launch_bounds__(kThreads, 1) void lce_tile(TileArgs a) {
    // One LDS object (the compiler then sees the DMA writes and the fragment reads as
    // one array and inserts no waits of its own): two stages of A and B (or, in the
    // gradient epilogue, the dZ staging blocks), then targets.
    constexpr int kData = kGrad && kStagingBytes > kStageArea ? kStagingBytes : kStageArea;
    __shared__ __attribute__((aligned(16))) char smem[kData + BM * 4];
    char (*lds)[2][kStageBytes] = reinterpret_cast<char (*)[2][kStageBytes]>(smem);
    int32_t* tile_targets = reinterpret_cast<int32_t*>(smem + kData);

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
    const uint32_t row_bytes = (uint32_t)(a.D * 2);
    const char* a_tile = reinterpret_cast<const char*>(a.H + row0 * a.D);
    const char* b_tile = reinterpret_cast<const char*>(a.W + col0 * a.D);
    // The DMA goes through buffer_load_dwordx4 ... lds rather than global_load_lds: the
    // compiler counts LDS reads precisely only while no FLAT-encoded instruction is in
    // flight, and with the global form pending it waited for all LDS reads
    // (s_waitcnt lgkmcnt(0)) before every group of MFMAs, including the reads issued
    // for later K16 steps.  Word 3 of the descriptor: raw 32-bit data, no swizzle.
    const __amdgpu_buffer_rsrc_t rsrc_a =
        __builtin_amdgcn_make_buffer_rsrc((void*)a_tile, (short)0, (int)((uint32_t)a_rows * row_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsrc_b =
        __builtin_amdgcn_make_buffer_rsrc((void*)b_tile, (short)0, (int)((uint32_t)b_rows * row_bytes), 0x00020000);

    // The LDS destination of group q is the group-0 slot plus q * 1 KiB; the instruction's
    // immediate offset moves the LDS and the global address together, so every group
    // shares one LDS base (M0) and the global address is pre-biased by -q KiB.
    // DMA of one stage, group by group: groups 0..7 load A rows, 8..15 load W rows.
    // Group q fills LDS rows wave * 64 + (q % 8) * 8 .. + 7.  The byte offset into the
    // tile is row * 2D + K bytes, below (valid rows) * 2D.
    auto dma_group = [&](auto qc, int kt, int buf) {
        constexpr int q = decltype(qc)::value % 8;
        constexpr bool is_b = decltype(qc)::value >= 8;
        const int64_t k0 = (int64_t)kt * BK;
        const int r = lrow + q * 8;
        const int64_t nrows = is_b ? b_rows : a_rows;
        const int rr = r < nrows ? r : (int)nrows - 1;
        // K tail: past D, re-read this row's last chunk; zeroed in LDS once it lands
        const uint32_t kb = (uint32_t)(k0 + koff[q & 1] < a.D ? koff[q & 1] : a.D - 8 - k0) * 2;
        const uint32_t voff = (uint32_t)(k0 * 2) + ((uint32_t)rr * row_bytes + kb);
        char* dst = &lds[buf][is_b ? 1 : 0][(wave * 64 + q * 8) * 128];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(is_b ? rsrc_b : rsrc_a, (lds_void_t*)dst, 16, voff, 0, 0, 0);
    };
    auto issue = [&](int kt, int buf) {
        [&]<int... Q>(std::integer_sequence<int, Q...>) {
            (dma_group(std::integral_constant<int, Q>{}, kt, buf), ...);
        }(std::make_integer_sequence<int, 16>{});
    };
    // Waits are written with the builtin, which the compiler's own wait insertion sees
    // (an inline-asm wait is opaque to it, so it added lgkmcnt(0) waits of its own after
    // the barrier); the empty asm statements keep LDS accesses from moving across them.
    // s_waitcnt immediates on gfx9: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
    constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0)
    constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)
    // Waits until the DMA of stage s has landed (loads retire in order; nothing else is
    // in flight by then).
    auto wait_stage = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
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
    // publishes the stage.
    auto zero_tail = [&](int kt, int buf) {
        const int64_t k0 = (int64_t)kt * BK;
        if (k0 + BK <= a.D) return;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (k0 + koff[q & 1] >= a.D) {
                const int o = (wave * 64 + q * 8) * 128 + lane * 16;
                *reinterpret_cast<U4*>(&lds[buf][0][o]) = U4{{0u, 0u, 0u, 0u}};
                *reinterpret_cast<U4*>(&lds[buf][1][o]) = U4{{0u, 0u, 0u, 0u}};
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

    auto read_frags = [&](int buf, int kk, bf16x8 (&fa)[FB], bf16x8 (&fb)[FB]) {
        const char* As = &lds[buf][0][wm * WT * 128];
        const char* Bs = &lds[buf][1][wn * WT * 128];
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
    // One K16 step is 16 MFMAs and 8 LDS reads: one read after every 2 MFMAs.  The step
    // that also issues the next stage's 16 DMA loads spreads them the same way, so the
    // matrix pipe is never left idle while they are issued.
    auto interleave = [&]() {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        }
    };
    // The K16 step after a stage's barrier: its 16 MFMAs (on fa, fb), the 8 LDS reads of
    // the next stage's first fragments (into na, nb from buffer cur ^ 1) and the 16 DMA
    // loads of stage kt_load (into buffer cur), in 8 chunks of 2 MFMAs + 1 read + 2 loads.
    // The scheduler keeps the chunk order, so the DMA issue never idles the matrix pipe.
    auto step_with_dma = [&](int kt_load, int cur, const bf16x8 (&fa)[FB], const bf16x8 (&fb)[FB],
                             bf16x8 (&na)[FB], bf16x8 (&nb)[FB]) {
        const char* As = &lds[cur ^ 1][0][wm * WT * 128];
        const char* Bs = &lds[cur ^ 1][1][wn * WT * 128];
        auto chunk = [&](auto cc) {
            constexpr int c = decltype(cc)::value;
            constexpr int i = c / 2, j0 = 2 * (c % 2);
            acc[i][j0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j0], fa[i], acc[i][j0], 0, 0, 0);
            acc[i][j0 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j0 + 1], fa[i], acc[i][j0 + 1], 0, 0, 0);
            if constexpr (c < 4)
                na[c] = *reinterpret_cast<const bf16x8*>(As + c * 32 * 128 + off[0]);
            else
                nb[c - 4] = *reinterpret_cast<const bf16x8*>(Bs + (c - 4) * 32 * 128 + off[0]);
            dma_group(std::integral_constant<int, 2 * c>{}, kt_load, cur);
            dma_group(std::integral_constant<int, 2 * c + 1>{}, kt_load, cur);
            __builtin_amdgcn_sched_barrier(0);
        };
        [&]<int... C>(std::integer_sequence<int, C...>) {
            (chunk(std::integral_constant<int, C>{}), ...);
        }(std::make_integer_sequence<int, 8>{});
    };
    auto sync_stage = [&](int kt, int cur, int nk) {
        // stage kt + 1 has landed (issued one stage earlier); after this barrier every
        // wave has finished reading buffer `cur`, which then takes stage kt + 2
        wait_stage();
        if (kt + 1 < nk) zero_tail(kt + 1, cur ^ 1);
        lds_barrier();
    };

    // Pipeline: the fragments of a K16 step are read from LDS two steps ahead, into four
    // rotating sets, so each wave keeps twice as many reads in flight (one wave per SIMD
    // is bound by LDS read latency).  A stage's single barrier sits between its steps 1
    // and 2: by then every wave has read all four steps of the stage (steps 2 and 3 during
    // steps 0 and 1), so the DMA of stage kt + 2 can go into its buffer, and stage kt + 1
    // has landed, so steps 2 and 3 can read the next stage's first two steps.  The DMA
    // still has four K16 steps to land.
    const int nk = (int)((a.D + BK - 1) / BK);
    bf16x8 fa0[FB], fb0[FB], fa1[FB], fb1[FB], fa2[FB], fb2[FB], fa3[FB], fb3[FB];
    // targets of this tile's rows, for the epilogue
    tile_targets[tid] = row0 + tid < a.N ? a.targets[row0 + tid] : -1;
    issue(0, 0);
    wait_stage();
    zero_tail(0, 0);
    lds_barrier();
    if (nk > 1) issue(1, 1);
    read_frags(0, 0, fa0, fb0);
    read_frags(0, 1, fa1, fb1);
    for (int kt = 0; kt + 1 < nk; ++kt) {
        const int cur = kt & 1;
        read_frags(cur, 2, fa2, fb2);
        mfma_all(fa0, fb0);
        interleave();
        read_frags(cur, 3, fa3, fb3);
        mfma_all(fa1, fb1);
        interleave();
        sync_stage(kt, cur, nk);
        // the last stage re-issues stage nk - 1 into the free buffer, which is never read:
        // no branch around the DMA, so it can interleave with the MFMAs
        step_with_dma(kt + 2 < nk ? kt + 2 : nk - 1, cur, fa2, fb2, fa0, fb0);
        read_frags(cur ^ 1, 1, fa1, fb1);
        mfma_all(fa3, fb3);
        interleave();
    }
    {
        const int cur = (nk - 1) & 1;
        read_frags(cur, 2, fa2, fb2);
        mfma_all(fa0, fb0);
        interleave();
        read_frags(cur, 3, fa3, fb3);
        mfma_all(fa1, fb1);
        interleave();
        mfma_all(fa2, fb2);
        mfma_all(fa3, fb3);
    }
    // the last loop iteration's (redundant) DMA must land before the workgroup can end
    wait_stage();

    // ---- epilogue: (m, s) per row over this wave's 128 columns ----------------
    // acc[i][j][e] holds Z[row = wrow0 + i*32 + l32][col = wcol0 + j*32 + 8*(e/4) + 4*h2 + e%4]:
    // this lane holds 64 of the wave's 128 columns of 4 rows, lane ^ 32 the other 64.
    const int64_t wcol0 = col0 + wn * WT;
    const int64_t wrow0 = row0 + wm * WT;
    auto col_of = [&](int j, int e) { return j * 32 + 8 * (e / 4) + 4 * h2 + (e % 4); };

    if constexpr (kGrad) {
        // dZ for this lane's 4 rows x 64 columns.  A row with an out-of-range target
        // gets m = NaN, so its whole row of dZ is NaN (its loss is NaN too).  The
        // row-major copy is stored directly, 4 columns per store; the transposed copy goes
        // through this wave's LDS block first, so that it leaves in 16-byte stores of 8
        // rows of a column.  After the barrier no wave reads the stage buffers any more
        // (the last DMA has landed: wait_stage above).
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
            const int32_t y = tile_targets[lr];
            const float2 l = a.lse[row];
            const float m = (y >= 0 && (int64_t)y < a.V) ? l.x : __builtin_nanf("");
            const float nlsl = -l.y * kLog2e;
            const float gr = a.g[row];
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
               0, c.V, g.n_row_tiles, g.n_col_tiles, g.gr, g.gc, g.n_rg, g.n_sb, g.n_slabs, partial, zy,
               nullptr, nullptr, nullptr, 0};
    hipLaunchKernelGGL(lce_tile<false>, dim3((unsigned)g.blocks), dim3(kThreads), 0, c.stream, a);
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
    TileArgs a{static_cast<const __bf16*>(c.H), static_cast<const __bf16*>(c.W), c.targets, c.N, c.D, c.V,
               c.c0, c.c0 + c.width, g.n_row_tiles, g.n_col_tiles, g.gr, g.gc, g.n_rg, g.n_sb, 0, nullptr,
               nullptr, reinterpret_cast<const float2*>(c.lse), c.g, static_cast<__bf16*>(c.G), c.ldG,
               static_cast<__bf16*>(c.GT), c.ldGT};
    hipLaunchKernelGGL(lce_tile<true>, dim3((unsigned)g.blocks), dim3(kThreads), 0, c.stream, a);
    return hipGetLastError();
}

namespace {
__global__ __launch_bounds__(256) void fill_zero_f32(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}
}  // namespace

hipError_t launch_fill_zero_f32(float* p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t want = (n + 255) / 256;
    const unsigned blocks = (unsigned)(want < 16384 ? want : 16384);
    hipLaunchKernelGGL(fill_zero_f32, dim3(blocks), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

}  // namespace ce
