// C ABI of libce_mi355x: argument validation, row-to-lane planning and dispatch.
// Every check runs on the host before anything is enqueued; a failed check returns
// a negative ce_status and touches no device state.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "ce_mi355x.h"
#include "ce_mi355x_testing.h"
#include "launch.h"

namespace {

using ce::Dt;
using ce::HostLayout;
using ce::Plan;

constexpr int kMaxDevices = 64;
constexpr int64_t kMaxV = 0x7fffffff;  // targets are int32
// lce_backward's product over the tokens reads rows of 2 N bytes through 32-bit offsets
constexpr int64_t kMaxBackwardN = (int64_t)1 << 22;

// Per-device CU count, 0 = not looked up yet, -1 = not a gfx950 device.  Racing
// first calls store the same value, so plain relaxed atomics suffice.
std::atomic<int> g_cus[kMaxDevices];

ce_status device_cus(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CE_ERR_DEVICE;
    int v = g_cus[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return CE_ERR_DEVICE;
        v = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? prop.multiProcessorCount : -1;
        if (v == 0) v = -1;
        g_cus[dev].store(v, std::memory_order_relaxed);
    }
    if (v < 0) return CE_ERR_DEVICE;
    *cus = v;
    return CE_OK;
}

int esize(ce_dtype dt) { return dt == CE_F32 ? 4 : 2; }

bool valid_dtype(int dt) { return dt == CE_F32 || dt == CE_F16 || dt == CE_BF16; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Byte range [lo, hi) covered by n_rows rows of V elements under layout L.
struct Extent {
    uintptr_t lo, hi;
};

int64_t row_off(const ce_layout& L, int64_t r) {
    const int64_t b = r / L.rows_per_batch;
    return b * L.batch_stride + (r - b * L.rows_per_batch) * L.row_stride;
}

Extent view_extent(const void* base, const ce_layout& L, int64_t n_rows, int64_t V, int es) {
    // offsets grow with the row index inside a batch and with the batch index, so the
    // furthest row is the last row, or the last row of the last full batch
    int64_t far = row_off(L, n_rows - 1);
    const int64_t last_b = (n_rows - 1) / L.rows_per_batch;
    if (last_b >= 1) {
        const int64_t r = last_b * L.rows_per_batch - 1;
        const int64_t o = row_off(L, r);
        if (o > far) far = o;
    }
    const uintptr_t lo = (uintptr_t)base;
    return Extent{lo, lo + (uintptr_t)((far + V) * es)};
}

Extent flat_extent(const void* p, int64_t bytes) {
    return Extent{(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes};
}

bool overlaps(Extent a, Extent b) { return a.lo < b.hi && b.lo < a.hi; }

// Strides are in elements.  Inputs may use any non-negative strides (rows may even
// repeat); outputs must give every row its own V elements.
bool layout_ok(const ce_layout& L, int64_t n_rows, int64_t V, bool output) {
    if (L.rows_per_batch < 1 || L.row_stride < 0 || L.batch_stride < 0) return false;
    // byte offsets must fit comfortably in 63 bits
    const double far = (double)L.batch_stride * (double)((n_rows - 1) / L.rows_per_batch + 1) +
                       (double)L.row_stride * (double)L.rows_per_batch + (double)V;
    if (far > 1.0e18) return false;
    if (!output) return true;
    if (L.row_stride < V && n_rows > 1) return false;
    if (n_rows > L.rows_per_batch &&
        L.batch_stride < (L.rows_per_batch - 1) * L.row_stride + V)
        return false;
    return true;
}

HostLayout host_layout(const ce_layout& L, int64_t n_rows) {
    const bool uniform = n_rows <= L.rows_per_batch || L.batch_stride == L.rows_per_batch * L.row_stride;
    return HostLayout{L.rows_per_batch, L.row_stride, L.batch_stride, uniform ? 1 : 0};
}

bool rows_aligned16(const void* base, const ce_layout& L, int64_t n_rows, int es) {
    if (!aligned(base, 16)) return false;
    if ((L.row_stride * es) % 16 != 0) return false;
    if (n_rows > L.rows_per_batch && (L.batch_stride * es) % 16 != 0) return false;
    return true;
}

int pow2_ceil(int64_t x) {
    int p = 1;
    while (p < x && p < 1024) p <<= 1;
    return p;
}

int narrow_rows_per_thread(int nv) { return nv == 1 ? 4 : nv == 2 ? 2 : 1; }

// Picks the row-to-lane mapping and the (capped) grid.  The grid never needs to
// cover every row: all kernels loop over 64-bit row indices.
ce_status make_plan(bool narrow_ok, int64_t V, int es, int64_t n_rows, int32_t lanes_req, bool vjp,
                    int cus, Plan* plan) {
    const int vec = 16 / es;
    const int64_t nvec = (V + vec - 1) / vec;
    Plan p{0, 0, 0, 0, 0};
    if (lanes_req == -1) {
        if (!narrow_ok) return CE_ERR_LAYOUT;
        p.narrow_nv = (int)(V / vec);
    } else if (lanes_req == 0) {
        // One lane per row only where that measured fastest: forward rows of up to two
        // vectors, VJP rows of one.  Otherwise about 8 vectors per lane in a forward and 4
        // in a VJP (while that takes at most 256 lanes), and at least min(nvec, 8) lanes per
        // row, so that the lanes of a row cover whole 128-byte lines in each load and store
        // instruction (a VJP with one lane per 4-vector row ran 1.6x slower, per 8-vector
        // row 2.2x).  On 512 MiB batches of rows of 64 to 256 vectors, 4 vectors per lane
        // instead of 8 ran ce_vjp 7-13% faster VJP after VJP (the same after a clean cache
        // or a forward), kl_vjp, js_vjp and ce_vjp_probs (two rows read per row written)
        // 5-9% faster VJP after VJP and 3-8% after a clean cache, ce_vjp_ex 6-14% faster VJP
        // after VJP; ce_forward gained nothing.  On rows of 512 and 1024 vectors ce_vjp ran
        // 4-7% faster VJP after VJP and 1-4% after a clean cache; at 2000 the same.
        if (narrow_ok && nvec <= (vjp ? 1 : 2)) {
            p.narrow_nv = (int)(V / vec);
        } else {
            const int spread = pow2_ceil(nvec < 8 ? nvec : 8);
            const int per8 = pow2_ceil((nvec + 7) / 8);
            const int per4 = pow2_ceil((nvec + 3) / 4);
            const int per = vjp && per4 <= 256 ? per4 : per8;
            p.lanes = per > spread ? per : spread;
        }
    } else {
        if (lanes_req < 1 || lanes_req > 1024 || (lanes_req & (lanes_req - 1)) != 0) return CE_ERR_SHAPE;
        p.lanes = lanes_req;
    }
    int64_t per_block, threads;
    if (p.narrow_nv > 0) {
        threads = 256;
        per_block = 256 * narrow_rows_per_thread(p.narrow_nv);
    } else if (!vjp && p.lanes > 64) {
        threads = p.lanes;
        per_block = 1;
    } else {
        threads = p.lanes > 256 ? p.lanes : 256;
        per_block = threads / p.lanes;
    }
    const int64_t needed = (n_rows + per_block - 1) / per_block;
    // 256-thread plans whose workgroups move at least 8 KB per pass (one lane per row, one
    // or two lanes per row, or two or more vectors per lane) launch one workgroup per block
    // of rows, up to 2^31 work-items (the dispatch packet holds the grid size in work-items
    // in 32 bits; the kernels loop over whatever rows remain), instead of four rounds of
    // resident workgroups looping over the rows.  Measured on 512 MiB batches: fp32
    // [135,266,304 x 8] forward 11% and VJP 19% faster, the 4- and 8-class rows 6-13%, rows
    // of 2+ vectors per lane about 4%; rows of one vector per lane over 4 or 8 lanes ran
    // 6-10% slower that way (each workgroup then moves only 4 KB), so they, and wider
    // workgroups, keep four rounds.
    const int64_t resident = (int64_t)cus * (2048 / threads);
    const bool open_grid = threads == 256 && (p.narrow_nv > 0 || p.lanes <= 2 || nvec >= 2 * p.lanes);
    const int64_t cap = open_grid ? ((int64_t)1 << 31) / threads : resident * 4;
    p.blocks = needed < cap ? needed : cap;
    if (p.blocks < 1) p.blocks = 1;
    *plan = p;
    return CE_OK;
}

// Chunked layout for the VJP of long rows: work items of one (row, chunk of
// 256 * kChunkU vectors) pair each, on a grid of at most 256 workgroups per CU that
// loops over the rest.  Taken when a row spans at least kChunkMinVec 16-byte vectors
// (counting a partial one); shorter rows keep whole-row layouts.
constexpr int64_t kChunkMinVec = 2048;

bool chunk_plan(int64_t V, int es, int64_t n_rows, int cus, Plan* plan) {
    const int vec = 16 / es;
    const int64_t nvec = (V + vec - 1) / vec;
    if (nvec < kChunkMinVec) return false;
    const int64_t per_chunk = 256 * (int64_t)ce::kChunkU;
    const int64_t chunks = (nvec + per_chunk - 1) / per_chunk;
    const int64_t items = n_rows * chunks;
    const int64_t cap = (int64_t)cus * 256;
    *plan = Plan{0, 0, items < cap ? items : cap, chunks, 0};
    return true;
}

ce_status from_hip(hipError_t e) { return e == hipSuccess ? CE_OK : CE_ERR_LAUNCH; }

ce_status forward_impl(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets,
                       int64_t n_rows, int64_t V, float* loss, float* lse, int32_t lanes,
                       hipStream_t stream) {
    if (!valid_dtype((int)dt)) return CE_ERR_DTYPE;
    if (n_rows < 0 || V < 1 || V > kMaxV) return CE_ERR_SHAPE;
    if (lanes != 0 && lanes != -1 && (lanes < 1 || lanes > 1024 || (lanes & (lanes - 1)) != 0))
        return CE_ERR_SHAPE;
    if (n_rows == 0) return CE_OK;
    if (!logits || !targets || !loss || !lse) return CE_ERR_NULL;
    const int es = esize(dt);
    if (!layout_ok(in, n_rows, V, false) || !aligned(logits, es) || !aligned(targets, 4) ||
        !aligned(loss, 4) || !aligned(lse, 8))
        return CE_ERR_LAYOUT;
    const Extent ex_in = view_extent(logits, in, n_rows, V, es);
    const Extent ex_t = flat_extent(targets, n_rows * 4);
    const Extent ex_loss = flat_extent(loss, n_rows * 4);
    const Extent ex_lse = flat_extent(lse, n_rows * 8);
    if (overlaps(ex_loss, ex_in) || overlaps(ex_loss, ex_t) || overlaps(ex_lse, ex_in) ||
        overlaps(ex_lse, ex_t) || overlaps(ex_loss, ex_lse))
        return CE_ERR_ALIAS;
    int cus = 0;
    if (ce_status s = device_cus(&cus)) return s;
    const bool narrow_ok = rows_aligned16(logits, in, n_rows, es) && V % (16 / es) == 0 &&
                           (V / (16 / es) == 1 || V / (16 / es) == 2 || V / (16 / es) == 4 ||
                            V / (16 / es) == 8);
    Plan plan;
    if (ce_status s = make_plan(narrow_ok, V, es, n_rows, lanes, false, cus, &plan)) return s;
    ce::FwdCall c{logits, host_layout(in, n_rows), (Dt)dt, targets, n_rows, V, loss, lse, plan, stream};
    return from_hip(ce::launch_ce_forward(c));
}

bool same_layout(const ce_layout& a, const ce_layout& b, int64_t n_rows) {
    if (a.row_stride != b.row_stride) return false;
    if (n_rows <= a.rows_per_batch && n_rows <= b.rows_per_batch) return true;
    return a.rows_per_batch == b.rows_per_batch && a.batch_stride == b.batch_stride;
}

ce_status vjp_impl(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets,
                   const float* lse, const float* g, int64_t n_rows, int64_t V, void* dlogits,
                   ce_layout out, int32_t lanes, hipStream_t stream) {
    if (!valid_dtype((int)dt)) return CE_ERR_DTYPE;
    if (n_rows < 0 || V < 1 || V > kMaxV) return CE_ERR_SHAPE;
    if (lanes != 0 && lanes != -1 && (lanes < 1 || lanes > 1024 || (lanes & (lanes - 1)) != 0))
        return CE_ERR_SHAPE;
    if (n_rows == 0) return CE_OK;
    if (!logits || !targets || !lse || !g || !dlogits) return CE_ERR_NULL;
    const int es = esize(dt);
    if (!layout_ok(in, n_rows, V, false) || !layout_ok(out, n_rows, V, true) || !aligned(logits, es) ||
        !aligned(dlogits, es) || !aligned(targets, 4) || !aligned(lse, 8) || !aligned(g, 4))
        return CE_ERR_LAYOUT;
    const Extent ex_in = view_extent(logits, in, n_rows, V, es);
    const Extent ex_out = view_extent(dlogits, out, n_rows, V, es);
    const bool in_place = logits == dlogits && same_layout(in, out, n_rows);
    if (!in_place && overlaps(ex_in, ex_out)) return CE_ERR_ALIAS;
    if (overlaps(ex_out, flat_extent(targets, n_rows * 4)) || overlaps(ex_out, flat_extent(lse, n_rows * 8)) ||
        overlaps(ex_out, flat_extent(g, n_rows * 4)))
        return CE_ERR_ALIAS;
    int cus = 0;
    if (ce_status s = device_cus(&cus)) return s;
    const int vec = 16 / es;
    const bool narrow_ok = rows_aligned16(logits, in, n_rows, es) && rows_aligned16(dlogits, out, n_rows, es) &&
                           V % vec == 0 && (V / vec == 1 || V / vec == 2 || V / vec == 4 || V / vec == 8);
    Plan plan;
    if (lanes != 0 || !chunk_plan(V, es, n_rows, cus, &plan))
        if (ce_status s = make_plan(narrow_ok, V, es, n_rows, lanes, true, cus, &plan)) return s;
    ce::VjpCall c{logits, host_layout(in, n_rows), (Dt)dt, targets, lse, g, n_rows, V, dlogits,
                  host_layout(out, n_rows), plan, stream};
    return from_hip(ce::launch_ce_vjp(c));
}

// Every input row and its output row start at the same offset within 16 bytes.
bool same_phase_rows(const void* x, const ce_layout& in, const void* d, const ce_layout& out, int64_t n_rows,
                     int es) {
    if ((((uintptr_t)x ^ (uintptr_t)d) & 15u) != 0) return false;
    if ((in.row_stride * es) % 16 != 0 || (out.row_stride * es) % 16 != 0) return false;
    if (n_rows > in.rows_per_batch && (in.batch_stride * es) % 16 != 0) return false;
    if (n_rows > out.rows_per_batch && (out.batch_stride * es) % 16 != 0) return false;
    return true;
}

ce_status fused_impl(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets, const float* g,
                     int64_t n_rows, int64_t V, float* loss, float* lse, void* dlogits, ce_layout out,
                     int32_t lanes, hipStream_t stream) {
    if (!valid_dtype((int)dt)) return CE_ERR_DTYPE;
    if (n_rows < 0 || V < 1 || V > kMaxV) return CE_ERR_SHAPE;
    if (lanes != 0 && lanes != -1 && (lanes < 1 || lanes > 1024 || (lanes & (lanes - 1)) != 0))
        return CE_ERR_SHAPE;
    if (n_rows == 0) return CE_OK;
    if (!logits || !targets || !g || !loss || !lse || !dlogits) return CE_ERR_NULL;
    const int es = esize(dt);
    if (!layout_ok(in, n_rows, V, false) || !layout_ok(out, n_rows, V, true) || !aligned(logits, es) ||
        !aligned(dlogits, es) || !aligned(targets, 4) || !aligned(g, 4) || !aligned(loss, 4) || !aligned(lse, 8))
        return CE_ERR_LAYOUT;
    const Extent ex_in = view_extent(logits, in, n_rows, V, es);
    const Extent ex_out = view_extent(dlogits, out, n_rows, V, es);
    const Extent ex_t = flat_extent(targets, n_rows * 4);
    const Extent ex_g = flat_extent(g, n_rows * 4);
    const Extent ex_loss = flat_extent(loss, n_rows * 4);
    const Extent ex_lse = flat_extent(lse, n_rows * 8);
    const bool in_place = logits == dlogits && same_layout(in, out, n_rows);
    if (!in_place && overlaps(ex_in, ex_out)) return CE_ERR_ALIAS;
    const Extent outs[3] = {ex_out, ex_loss, ex_lse};
    for (int i = 0; i < 3; ++i) {
        if (overlaps(outs[i], ex_t) || overlaps(outs[i], ex_g)) return CE_ERR_ALIAS;
        if (i > 0 && overlaps(outs[i], ex_in)) return CE_ERR_ALIAS;
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], outs[j])) return CE_ERR_ALIAS;
    }
    int cus = 0;
    if (ce_status s = device_cus(&cus)) return s;
    const int vec = 16 / es;
    const bool narrow_ok = rows_aligned16(logits, in, n_rows, es) && rows_aligned16(dlogits, out, n_rows, es) &&
                           V % vec == 0 && (V / vec == 1 || V / vec == 2 || V / vec == 4 || V / vec == 8);
    Plan plan;
    if (ce_status s = make_plan(narrow_ok, V, es, n_rows, lanes, false, cus, &plan)) return s;
    // Rows the forward gives a 512- or 1024-thread workgroup, whose input and output rows share
    // their 16-byte phase, and that fit in those threads' registers: the register-resident
    // kernel.  It takes the max and the sum in two passes, so its loss and lse round
    // differently from ce_forward's online fold; its dlogits match ce_vjp's bit for bit
    // for the lse it writes.
    if (lanes == 0 && (plan.lanes == 512 || plan.lanes == 1024) && plan.narrow_nv == 0 &&
        same_phase_rows(logits, in, dlogits, out, n_rows, es)) {
        const int64_t need = ((V + vec - 1) / vec + plan.lanes - 1) / plan.lanes;
        const int* nvs = plan.lanes == 512 ? ce::kRegsNV512 : es == 4 ? ce::kRegsNV32 : ce::kRegsNV16;
        const int cnt = plan.lanes == 512 ? 1
                        : es == 4 ? (int)(sizeof(ce::kRegsNV32) / sizeof(int))
                                  : (int)(sizeof(ce::kRegsNV16) / sizeof(int));
        for (int i = 0; i < cnt; ++i) {
            if (need <= nvs[i]) {
                plan.regs_nv = nvs[i];
                const int64_t cap = (int64_t)cus * 16;
                plan.blocks = n_rows < cap ? n_rows : cap;
                break;
            }
        }
    }
    ce::FusedCall c{logits, host_layout(in, n_rows), (Dt)dt, targets, g, n_rows, V, loss, lse, dlogits,
                    host_layout(out, n_rows), plan, stream};
    return from_hip(ce::launch_ce_fused(c));
}

// ---- cross-entropy options ------------------------------------------------------

bool options_ok(const ce_options& o, bool probs) {
    // NaN fails both comparisons
    if (!(o.label_smoothing >= 0.0f && o.label_smoothing <= 1.0f)) return false;
    if (o.reduction != CE_REDUCE_NONE && o.reduction != CE_REDUCE_SUM && o.reduction != CE_REDUCE_MEAN)
        return false;
    return !probs || o.ignore_index == CE_NO_IGNORE;
}

// True when some output range overlaps an input range or another output range.
bool alias_any(const Extent* outs, int n_out, const Extent* ins, int n_in) {
    for (int i = 0; i < n_out; ++i) {
        for (int j = 0; j < n_in; ++j)
            if (overlaps(outs[i], ins[j])) return true;
        for (int j = i + 1; j < n_out; ++j)
            if (overlaps(outs[i], outs[j])) return true;
    }
    return false;
}

// The two option forwards: class-index targets (use_probs false, `targets`) or
// probability targets (use_probs true, the `probs` view).
ce_status options_forward(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets, bool use_probs,
                          const void* probs, ce_layout pl, int64_t n_rows, int64_t V, ce_options opt, float* loss, float* lse,
                          float* wsum, float* total, int64_t* count, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    if (!valid_dtype((int)dt)) return CE_ERR_DTYPE;
    if (n_rows < 0 || V < 1 || V > kMaxV) return CE_ERR_SHAPE;
    if (!options_ok(opt, use_probs)) return CE_ERR_OPTION;
    const bool reduce = opt.reduction != CE_REDUCE_NONE;
    const bool has_ignore = !use_probs && opt.ignore_index != CE_NO_IGNORE;
    if (reduce) {
        if (!total || !count || !workspace) return CE_ERR_NULL;
        if (workspace_bytes < ce::kReduceWorkspaceBytes) return CE_ERR_WORKSPACE;
        if (!aligned(total, 4) || !aligned(count, 8) || !aligned(workspace, 8)) return CE_ERR_LAYOUT;
    }
    const Extent ex_tot = flat_extent(total, reduce ? 4 : 0);
    const Extent ex_cnt = flat_extent(count, reduce ? 8 : 0);
    const Extent ex_ws = flat_extent(workspace, reduce ? (int64_t)ce::kReduceWorkspaceBytes : 0);
    if (n_rows == 0) {
        if (!reduce) return CE_OK;
        const Extent outs[3] = {ex_tot, ex_cnt, ex_ws};
        if (alias_any(outs, 3, nullptr, 0)) return CE_ERR_ALIAS;
        int cus = 0;
        if (ce_status s = device_cus(&cus)) return s;
        ce::ReduceCall rc{nullptr, nullptr, 0, opt.ignore_index, false, opt.reduction, total, count, workspace, stream};
        return from_hip(ce::launch_loss_reduce(rc));
    }
    if (!logits || !loss || !lse) return CE_ERR_NULL;
    if (use_probs ? (!probs || !wsum) : !targets) return CE_ERR_NULL;
    const int es = esize(dt);
    if (!layout_ok(in, n_rows, V, false) || !aligned(logits, es) || !aligned(loss, 4) || !aligned(lse, 8))
        return CE_ERR_LAYOUT;
    if (use_probs ? (!layout_ok(pl, n_rows, V, false) || !aligned(probs, es) || !aligned(wsum, 4))
                  : !aligned(targets, 4))
        return CE_ERR_LAYOUT;
    const Extent ins[2] = {view_extent(logits, in, n_rows, V, es),
                           use_probs ? view_extent(probs, pl, n_rows, V, es) : flat_extent(targets, n_rows * 4)};
    const Extent outs[6] = {flat_extent(loss, n_rows * 4), flat_extent(lse, n_rows * 8),
                            flat_extent(wsum, use_probs ? n_rows * 4 : 0), ex_tot, ex_cnt, ex_ws};
    if (alias_any(outs, 6, ins, 2)) return CE_ERR_ALIAS;
    int cus = 0;
    if (ce_status s = device_cus(&cus)) return s;
    if (!use_probs && opt.label_smoothing == 0.0f) {
        if (ce_status s = forward_impl(logits, in, dt, targets, n_rows, V, loss, lse, 0, stream)) return s;
    } else {
        Plan plan;
        if (ce_status s = make_plan(false, V, es, n_rows, 0, false, cus, &plan)) return s;
        ce::OptFwdCall c{logits, host_layout(in, n_rows), use_probs ? probs : nullptr,
                         host_layout(use_probs ? pl : in, n_rows), (Dt)dt, targets, n_rows, V, opt.label_smoothing,
                         loss, lse, wsum, plan, stream};
        if (hipError_t e = ce::launch_opt_forward(c)) return from_hip(e);
    }
    if (!reduce && !has_ignore) return CE_OK;
    ce::ReduceCall rc{loss, use_probs ? nullptr : targets, n_rows, opt.ignore_index, has_ignore, opt.reduction,
                      total, count, workspace, stream};
    return from_hip(ce::launch_loss_reduce(rc));
}

ce_status options_vjp(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets, bool use_probs,
                      const void* probs, ce_layout pl, const float* lse, const float* wsum, const float* g, int64_t n_rows, int64_t V,
                      ce_options opt, const int64_t* count, void* dlogits, ce_layout out, hipStream_t stream) {
    if (!valid_dtype((int)dt)) return CE_ERR_DTYPE;
    if (n_rows < 0 || V < 1 || V > kMaxV) return CE_ERR_SHAPE;
    if (!options_ok(opt, use_probs)) return CE_ERR_OPTION;
    if (n_rows == 0) return CE_OK;
    const bool has_ignore = !use_probs && opt.ignore_index != CE_NO_IGNORE;
    if (!use_probs && opt.label_smoothing == 0.0f && !has_ignore && opt.reduction == CE_REDUCE_NONE)
        return vjp_impl(logits, in, dt, targets, lse, g, n_rows, V, dlogits, out, 0, stream);
    if (!logits || !lse || !g || !dlogits) return CE_ERR_NULL;
    if (use_probs ? (!probs || !wsum) : !targets) return CE_ERR_NULL;
    if (opt.reduction == CE_REDUCE_MEAN && !count) return CE_ERR_NULL;
    const int es = esize(dt);
    if (!layout_ok(in, n_rows, V, false) || !layout_ok(out, n_rows, V, true) || !aligned(logits, es) ||
        !aligned(dlogits, es) || !aligned(lse, 8) || !aligned(g, 4) || !aligned(count, 8))
        return CE_ERR_LAYOUT;
    if (use_probs ? (!layout_ok(pl, n_rows, V, false) || !aligned(probs, es) || !aligned(wsum, 4))
                  : !aligned(targets, 4))
        return CE_ERR_LAYOUT;
    const Extent ex_in = view_extent(logits, in, n_rows, V, es);
    const Extent ex_out = view_extent(dlogits, out, n_rows, V, es);
    const bool in_place = logits == dlogits && same_layout(in, out, n_rows);
    if (!in_place && overlaps(ex_in, ex_out)) return CE_ERR_ALIAS;
    const int64_t g_bytes = opt.reduction == CE_REDUCE_NONE ? n_rows * 4 : 4;
    const Extent ins[5] = {use_probs ? view_extent(probs, pl, n_rows, V, es) : flat_extent(targets, n_rows * 4),
                           flat_extent(lse, n_rows * 8), flat_extent(g, g_bytes),
                           flat_extent(wsum, use_probs ? n_rows * 4 : 0),
                           flat_extent(count, opt.reduction == CE_REDUCE_MEAN ? 8 : 0)};
    if (alias_any(&ex_out, 1, ins, 5)) return CE_ERR_ALIAS;
    int cus = 0;
    if (ce_status s = device_cus(&cus)) return s;
    Plan plan;
    if (!chunk_plan(V, es, n_rows, cus, &plan))
        if (ce_status s = make_plan(false, V, es, n_rows, 0, true, cus, &plan)) return s;
    ce::OptVjpCall c{logits, host_layout(in, n_rows), use_probs ? probs : nullptr,
                     host_layout(use_probs ? pl : in, n_rows), (Dt)dt, targets,
                     lse, wsum, g, count, n_rows, V, opt.reduction, opt.ignore_index, has_ignore ? 1 : 0,
                     opt.label_smoothing, dlogits, host_layout(out, n_rows), plan, stream};
    return from_hip(ce::launch_opt_vjp(c));
}

bool lanes_ok_kl(int32_t lanes) {
    return lanes == 0 || (lanes >= 1 && lanes <= 1024 && (lanes & (lanes - 1)) == 0);
}

// The two row-pair divergences share their checks and layouts: the KL forward writes
// (kl, lse_q, lse_p), the Jensen-Shannon forward also the student's half H (`hq`), which
// its VJP reads back.
enum class Div { KL, JS };

ce_status div_forward_impl(Div div, const void* q, ce_layout ql, const void* p, ce_layout pl, ce_dtype dt,
                           int64_t n_rows, int64_t V, float* out, float* lse_q, float* lse_p, float* hq,
                           int32_t lanes, hipStream_t stream) {
    if (!valid_dtype((int)dt)) return CE_ERR_DTYPE;
    if (n_rows < 0 || V < 1 || V > kMaxV || !lanes_ok_kl(lanes)) return CE_ERR_SHAPE;
    if (n_rows == 0) return CE_OK;
    const bool js = div == Div::JS;
    if (!q || !p || !out || !lse_q || !lse_p || (js && !hq)) return CE_ERR_NULL;
    const int es = esize(dt);
    if (!layout_ok(ql, n_rows, V, false) || !layout_ok(pl, n_rows, V, false) || !aligned(q, es) ||
        !aligned(p, es) || !aligned(out, 4) || !aligned(lse_q, 8) || !aligned(lse_p, 8) || !aligned(hq, 4))
        return CE_ERR_LAYOUT;
    const Extent ins[2] = {view_extent(q, ql, n_rows, V, es), view_extent(p, pl, n_rows, V, es)};
    const Extent outs[4] = {flat_extent(out, n_rows * 4), flat_extent(lse_q, n_rows * 8),
                            flat_extent(lse_p, n_rows * 8), flat_extent(hq, js ? n_rows * 4 : 0)};
    if (alias_any(outs, 4, ins, 2)) return CE_ERR_ALIAS;
    int cus = 0;
    if (ce_status s = device_cus(&cus)) return s;
    Plan plan;
    if (ce_status s = make_plan(false, V, es, n_rows, lanes, false, cus, &plan)) return s;
    if (js) {
        ce::JSFwdCall c{q,   host_layout(ql, n_rows), p,     host_layout(pl, n_rows), (Dt)dt, n_rows, V,
                        out, lse_q,                   lse_p, hq,                      plan,   stream};
        return from_hip(ce::launch_js_forward(c));
    }
    ce::KLFwdCall c{q, host_layout(ql, n_rows), p, host_layout(pl, n_rows), (Dt)dt, n_rows, V, out, lse_q, lse_p,
                    plan, stream};
    return from_hip(ce::launch_kl_forward(c));
}

ce_status div_vjp_impl(Div div, const void* q, ce_layout ql, const void* p, ce_layout pl, ce_dtype dt,
                       const float* lse_q, const float* lse_p, const float* hq, const float* g, int64_t n_rows,
                       int64_t V, void* dq, ce_layout dl, int32_t lanes, hipStream_t stream) {
    if (!valid_dtype((int)dt)) return CE_ERR_DTYPE;
    if (n_rows < 0 || V < 1 || V > kMaxV || !lanes_ok_kl(lanes)) return CE_ERR_SHAPE;
    if (n_rows == 0) return CE_OK;
    const bool js = div == Div::JS;
    if (!q || !p || !lse_q || !lse_p || !g || !dq || (js && !hq)) return CE_ERR_NULL;
    const int es = esize(dt);
    if (!layout_ok(ql, n_rows, V, false) || !layout_ok(pl, n_rows, V, false) || !layout_ok(dl, n_rows, V, true) ||
        !aligned(q, es) || !aligned(p, es) || !aligned(dq, es) || !aligned(lse_q, 8) || !aligned(lse_p, 8) ||
        !aligned(g, 4) || !aligned(hq, 4))
        return CE_ERR_LAYOUT;
    const Extent ex_q = view_extent(q, ql, n_rows, V, es);
    const Extent ex_d = view_extent(dq, dl, n_rows, V, es);
    const bool in_place = q == dq && same_layout(ql, dl, n_rows);
    if (!in_place && overlaps(ex_q, ex_d)) return CE_ERR_ALIAS;
    const Extent ins[5] = {view_extent(p, pl, n_rows, V, es), flat_extent(lse_q, n_rows * 8),
                           flat_extent(lse_p, n_rows * 8), flat_extent(g, n_rows * 4),
                           flat_extent(hq, js ? n_rows * 4 : 0)};
    if (alias_any(&ex_d, 1, ins, 5)) return CE_ERR_ALIAS;
    int cus = 0;
    if (ce_status s = device_cus(&cus)) return s;
    Plan plan;
    if (lanes != 0 || !chunk_plan(V, es, n_rows, cus, &plan))
        if (ce_status s = make_plan(false, V, es, n_rows, lanes, true, cus, &plan)) return s;
    if (js) {
        ce::JSVjpCall c{q, host_layout(ql, n_rows), p, host_layout(pl, n_rows), (Dt)dt, lse_q, lse_p, hq, g,
                        n_rows, V, dq, host_layout(dl, n_rows), plan, stream};
        return from_hip(ce::launch_js_vjp(c));
    }
    ce::KLVjpCall c{q,     host_layout(ql, n_rows), p, host_layout(pl, n_rows), (Dt)dt, lse_q, lse_p, g, n_rows,
                    V,     dq, host_layout(dl, n_rows), plan, stream};
    return from_hip(ce::launch_kl_vjp(c));
}

}  // namespace

extern "C" {

ce_status ce_forward(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets, int64_t n_rows,
                     int64_t V, float* loss, float* lse, hipStream_t stream) {
    return forward_impl(logits, in, dt, targets, n_rows, V, loss, lse, 0, stream);
}

ce_status ce_forward_lanes(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets,
                           int64_t n_rows, int64_t V, float* loss, float* lse, int32_t lanes_per_row,
                           hipStream_t stream) {
    return forward_impl(logits, in, dt, targets, n_rows, V, loss, lse, lanes_per_row, stream);
}

ce_status ce_vjp(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets, const float* lse,
                 const float* g, int64_t n_rows, int64_t V, void* dlogits, ce_layout out, hipStream_t stream) {
    return vjp_impl(logits, in, dt, targets, lse, g, n_rows, V, dlogits, out, 0, stream);
}

ce_status ce_vjp_lanes(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets, const float* lse,
                       const float* g, int64_t n_rows, int64_t V, void* dlogits, ce_layout out,
                       int32_t lanes_per_row, hipStream_t stream) {
    return vjp_impl(logits, in, dt, targets, lse, g, n_rows, V, dlogits, out, lanes_per_row, stream);
}

ce_status ce_forward_vjp(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets, const float* g,
                         int64_t n_rows, int64_t V, float* loss, float* lse, void* dlogits, ce_layout out,
                         hipStream_t stream) {
    return fused_impl(logits, in, dt, targets, g, n_rows, V, loss, lse, dlogits, out, 0, stream);
}

ce_status ce_forward_vjp_lanes(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets,
                               const float* g, int64_t n_rows, int64_t V, float* loss, float* lse, void* dlogits,
                               ce_layout out, int32_t lanes_per_row, hipStream_t stream) {
    return fused_impl(logits, in, dt, targets, g, n_rows, V, loss, lse, dlogits, out, lanes_per_row, stream);
}

// The tile kernels take one workgroup per 256 x 256 tile and a dispatch holds at most
// 2^32 - 1 work-items: N x V (or N x D, V x D in the backward's products) is bounded.
bool lce_grid_fits(int64_t N, int64_t V) { return ce::lce_tile_grid_items(N, V) <= ce::kMaxGridItems; }

size_t lce_workspace_size(int64_t N, int64_t D, int64_t V) {
    if (N < 0 || D < 1 || D % 8 != 0 || V < 1 || V > kMaxV || !lce_grid_fits(N, V)) return 0;
    return ce::lce_workspace_bytes(N, D, V);
}

ce_status lce_forward(const void* H, const void* W, const int32_t* targets, int64_t N, int64_t D, int64_t V,
                      float* loss, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (N < 0 || D < 1 || D % 8 != 0 || V < 1 || V > kMaxV || D > (int64_t)1 << 22) return CE_ERR_SHAPE;
    if (!lce_grid_fits(N, V)) return CE_ERR_SHAPE;
    if (N == 0) return CE_OK;
    if (!H || !W || !targets || !loss || !lse) return CE_ERR_NULL;
    if (!workspace || workspace_bytes < ce::lce_workspace_bytes(N, D, V)) return CE_ERR_WORKSPACE;
    if (!aligned(H, 16) || !aligned(W, 16) || !aligned(targets, 4) || !aligned(loss, 4) || !aligned(lse, 8) ||
        !aligned(workspace, 256))
        return CE_ERR_LAYOUT;
    const Extent ex_loss = flat_extent(loss, N * 4);
    const Extent ex_lse = flat_extent(lse, N * 8);
    const Extent ex_ws = flat_extent(workspace, (int64_t)ce::lce_workspace_bytes(N, D, V));
    const Extent ins[3] = {flat_extent(H, N * D * 2), flat_extent(W, V * D * 2), flat_extent(targets, N * 4)};
    for (const Extent& e : ins)
        if (overlaps(ex_loss, e) || overlaps(ex_lse, e) || overlaps(ex_ws, e)) return CE_ERR_ALIAS;
    if (overlaps(ex_loss, ex_lse) || overlaps(ex_loss, ex_ws) || overlaps(ex_lse, ex_ws)) return CE_ERR_ALIAS;
    int cus = 0;
    if (ce_status s = device_cus(&cus)) return s;
    ce::LceCall c{H, W, targets, N, D, V, loss, lse, workspace, cus, stream};
    return from_hip(ce::launch_lce_forward(c));
}

bool lce_backward_shape_ok(int64_t N, int64_t D, int64_t V) {
    return N >= 0 && N <= kMaxBackwardN && D >= 1 && D % 8 == 0 && V >= 1 && V <= kMaxV && D <= (int64_t)1 << 22 &&
           ce::lce_backward_grids_fit(N, D, V);
}

size_t lce_backward_workspace_size(int64_t N, int64_t D, int64_t V) {
    if (!lce_backward_shape_ok(N, D, V)) return 0;
    return ce::lce_backward_workspace_bytes(N, D, V);
}

size_t lce_backward_workspace_size_one_pass(int64_t N, int64_t D, int64_t V) {
    if (!lce_backward_shape_ok(N, D, V)) return 0;
    return ce::lce_backward_workspace_bytes_one_pass(N, D, V);
}

ce_status lce_backward(const void* H, const void* W, const int32_t* targets, const float* lse, const float* g,
                       int64_t N, int64_t D, int64_t V, float* dH, float* dW, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
    if (!lce_backward_shape_ok(N, D, V)) return CE_ERR_SHAPE;
    if (!W || !dW) return CE_ERR_NULL;
    if (N > 0 && (!H || !targets || !lse || !g || !dH)) return CE_ERR_NULL;
    const size_t need = ce::lce_backward_workspace_bytes(N, D, V);
    if (N > 0 && (!workspace || workspace_bytes < need)) return CE_ERR_WORKSPACE;
    if (!aligned(W, 16) || !aligned(dW, 16)) return CE_ERR_LAYOUT;
    if (N > 0 && (!aligned(H, 16) || !aligned(targets, 4) || !aligned(lse, 8) || !aligned(g, 4) ||
                  !aligned(dH, 16) || !aligned(workspace, 256)))
        return CE_ERR_LAYOUT;
    const Extent ex_dW = flat_extent(dW, V * D * 4);
    const Extent ex_W = flat_extent(W, V * D * 2);
    if (overlaps(ex_dW, ex_W)) return CE_ERR_ALIAS;
    if (N > 0) {
        const Extent ex_dH = flat_extent(dH, N * D * 4);
        const Extent ex_ws = flat_extent(workspace, (int64_t)ce::lce_backward_workspace_used(N, D, V, workspace_bytes));
        const Extent ins[5] = {flat_extent(H, N * D * 2), ex_W, flat_extent(targets, N * 4),
                               flat_extent(lse, N * 8), flat_extent(g, N * 4)};
        for (const Extent& e : ins)
            if (overlaps(ex_dH, e) || overlaps(ex_dW, e) || overlaps(ex_ws, e)) return CE_ERR_ALIAS;
        if (overlaps(ex_dH, ex_dW) || overlaps(ex_dH, ex_ws) || overlaps(ex_dW, ex_ws)) return CE_ERR_ALIAS;
    }
    int cus = 0;
    if (ce_status s = device_cus(&cus)) return s;
    if (N == 0) return from_hip(ce::launch_fill_zero_f32(dW, V * D, stream));
    ce::LceBackwardCall c{H, W, targets, lse, g, N, D, V, dH, dW, workspace, workspace_bytes, stream};
    return ce::run_lce_backward(c) == ce::LceBackwardStatus::kOk ? CE_OK : CE_ERR_LAUNCH;
}

ce_status kl_forward(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                     int64_t n_rows, int64_t V, float* kl, float* lse_q, float* lse_p, hipStream_t stream) {
    return div_forward_impl(Div::KL, q, q_layout, p, p_layout, dt, n_rows, V, kl, lse_q, lse_p, nullptr, 0,
                            stream);
}

ce_status kl_forward_lanes(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                           int64_t n_rows, int64_t V, float* kl, float* lse_q, float* lse_p, int32_t lanes_per_row,
                           hipStream_t stream) {
    return div_forward_impl(Div::KL, q, q_layout, p, p_layout, dt, n_rows, V, kl, lse_q, lse_p, nullptr,
                            lanes_per_row, stream);
}

ce_status kl_vjp(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                 const float* lse_q, const float* lse_p, const float* g, int64_t n_rows, int64_t V, void* dq,
                 ce_layout dq_layout, hipStream_t stream) {
    return div_vjp_impl(Div::KL, q, q_layout, p, p_layout, dt, lse_q, lse_p, nullptr, g, n_rows, V, dq, dq_layout,
                        0, stream);
}

ce_status kl_vjp_lanes(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                       const float* lse_q, const float* lse_p, const float* g, int64_t n_rows, int64_t V, void* dq,
                       ce_layout dq_layout, int32_t lanes_per_row, hipStream_t stream) {
    return div_vjp_impl(Div::KL, q, q_layout, p, p_layout, dt, lse_q, lse_p, nullptr, g, n_rows, V, dq, dq_layout,
                        lanes_per_row, stream);
}

ce_status js_forward(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                     int64_t n_rows, int64_t V, float* js, float* lse_q, float* lse_p, float* hq,
                     hipStream_t stream) {
    return div_forward_impl(Div::JS, q, q_layout, p, p_layout, dt, n_rows, V, js, lse_q, lse_p, hq, 0, stream);
}

ce_status js_forward_lanes(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                           int64_t n_rows, int64_t V, float* js, float* lse_q, float* lse_p, float* hq,
                           int32_t lanes_per_row, hipStream_t stream) {
    return div_forward_impl(Div::JS, q, q_layout, p, p_layout, dt, n_rows, V, js, lse_q, lse_p, hq, lanes_per_row,
                            stream);
}

ce_status js_vjp(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                 const float* lse_q, const float* lse_p, const float* hq, const float* g, int64_t n_rows, int64_t V,
                 void* dq, ce_layout dq_layout, hipStream_t stream) {
    return div_vjp_impl(Div::JS, q, q_layout, p, p_layout, dt, lse_q, lse_p, hq, g, n_rows, V, dq, dq_layout, 0,
                        stream);
}

ce_status js_vjp_lanes(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                       const float* lse_q, const float* lse_p, const float* hq, const float* g, int64_t n_rows,
                       int64_t V, void* dq, ce_layout dq_layout, int32_t lanes_per_row, hipStream_t stream) {
    return div_vjp_impl(Div::JS, q, q_layout, p, p_layout, dt, lse_q, lse_p, hq, g, n_rows, V, dq, dq_layout,
                        lanes_per_row, stream);
}

size_t ce_reduce_workspace_size(void) { return ce::kReduceWorkspaceBytes; }

ce_status ce_forward_ex(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets, int64_t n_rows,
                        int64_t V, ce_options opt, float* loss, float* lse, float* total, int64_t* count,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return options_forward(logits, in, dt, targets, false, nullptr, in, n_rows, V, opt, loss, lse, nullptr, total,
                           count, workspace, workspace_bytes, stream);
}

ce_status ce_forward_ex_noalloc(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets,
                                int64_t n_rows, int64_t V, ce_options opt, float* loss, float* lse, float* total,
                                int64_t* count, hipStream_t stream) {
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (opt.reduction != CE_REDUCE_NONE) {
        if (hipError_t e = ce::reduce_scratch(&ws, &ws_bytes)) {
            (void)e;
            return CE_ERR_DEVICE;
        }
        // the scratch holds the reduction's need at every size; this cannot fail
        if (ws_bytes < ce::kReduceWorkspaceBytes) return CE_ERR_WORKSPACE;
    }
    return options_forward(logits, in, dt, targets, false, nullptr, in, n_rows, V, opt, loss, lse, nullptr, total,
                           count, ws, ws_bytes, stream);
}

ce_status ce_vjp_ex(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets, const float* lse,
                    const float* g, int64_t n_rows, int64_t V, ce_options opt, const int64_t* count, void* dlogits,
                    ce_layout out, hipStream_t stream) {
    return options_vjp(logits, in, dt, targets, false, nullptr, in, lse, nullptr, g, n_rows, V, opt, count, dlogits,
                       out, stream);
}

ce_status ce_forward_probs(const void* logits, ce_layout in, ce_dtype dt, const void* probs, ce_layout probs_layout,
                           int64_t n_rows, int64_t V, ce_options opt, float* loss, float* lse, float* wsum,
                           float* total, int64_t* count, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    return options_forward(logits, in, dt, nullptr, true, probs, probs_layout, n_rows, V, opt, loss, lse, wsum, total,
                           count, workspace, workspace_bytes, stream);
}

ce_status ce_vjp_probs(const void* logits, ce_layout in, ce_dtype dt, const void* probs, ce_layout probs_layout,
                       const float* lse, const float* wsum, const float* g, int64_t n_rows, int64_t V, ce_options opt,
                       const int64_t* count, void* dlogits, ce_layout out, hipStream_t stream) {
    return options_vjp(logits, in, dt, nullptr, true, probs, probs_layout, lse, wsum, g, n_rows, V, opt, count,
                       dlogits, out, stream);
}

const char* ce_status_string(ce_status s) {
    switch (s) {
        case CE_OK: return "CE_OK: success";
        case CE_ERR_NULL: return "CE_ERR_NULL: a required pointer is NULL";
        case CE_ERR_SHAPE: return "CE_ERR_SHAPE: a size or lane count is out of range";
        case CE_ERR_DTYPE: return "CE_ERR_DTYPE: unknown element type";
        case CE_ERR_LAYOUT: return "CE_ERR_LAYOUT: bad strides or misaligned pointer";
        case CE_ERR_WORKSPACE: return "CE_ERR_WORKSPACE: workspace missing or too small";
        case CE_ERR_LAUNCH: return "CE_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
        case CE_ERR_ALIAS: return "CE_ERR_ALIAS: an output overlaps an input";
        case CE_ERR_DEVICE: return "CE_ERR_DEVICE: no gfx950 HIP device is current";
        case CE_ERR_OPTION: return "CE_ERR_OPTION: label_smoothing outside [0, 1], an unknown reduction, or an ignore_index with probability targets";
    }
    return "unknown ce_status";
}

}  // extern "C"
