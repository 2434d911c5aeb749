/*
 * ce_mi355x.h: C ABI of the MI355X (gfx950) fused softmax cross-entropy library.
 *
 * The operations, computed by hand-written HIP kernels in libce_mi355x.so:
 *
 *   ce_forward    per-row loss and log-sum-exp of a [rows, V] logits view
 *   ce_vjp        dlogits = g_i * (softmax(z_i) - onehot(y_i)) from the saved log-sum-exp
 *   ce_forward_vjp  ce_forward and ce_vjp in one kernel, for a g known before the forward
 *   lce_forward   per-row loss and log-sum-exp of H.W^T, streamed over vocabulary
 *                 tiles without materialising the N x V logits
 *   lce_backward  dH and dW of sum_i g_i loss_i for lce_forward's loss; the logits
 *                 are regenerated chunk by chunk (8192 columns, or the whole vocabulary
 *                 when the workspace holds it), and the two products with the
 *                 regenerated gradient chunk run on the same MFMA tile kernel
 *   kl_forward    per-row KL divergence of a teacher logits row from a student row
 *   kl_vjp        dq = g_i * (softmax(q_i) - softmax(p_i)) from the saved pairs
 *   js_forward    per-row Jensen-Shannon divergence of a student row and a teacher row
 *   js_vjp        its gradient with respect to the student logits
 *   ce_forward_ex / ce_vjp_ex        ce_forward / ce_vjp with label smoothing,
 *                                    ignore_index and an in-library sum or mean
 *   ce_forward_probs / ce_vjp_probs  the same with probability targets
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers to tensors are DEVICE pointers owned by the caller.  The library keeps
 *   no pointer after a call returns and allocates no device memory: the only scratch
 *   is the caller's workspace (lce_forward, lce_backward, and a sum or mean of the
 *   _ex and _probs forwards), or, for ce_forward_ex_noalloc, a fixed 16 KiB array the
 *   library holds on each GPU.
 * - Work is enqueued on `stream` (NULL = the default stream) and the call returns
 *   without synchronising.  Outputs are valid once the stream has been synchronised.
 * - Every argument is checked on the host before any launch.  A failed check returns
 *   a negative ce_status and enqueues nothing.  n_rows == 0 (or N == 0) is a no-op
 *   that returns CE_OK, except that lce_backward still writes dW = 0.  A failed
 *   launch returns CE_ERR_LAUNCH.  No C++ exception crosses this boundary.  The
 *   library's only mutable state is set once per GPU and then read (the GPU's compute
 *   unit count, and the address of ce_forward_ex_noalloc's array), so the calls may be
 *   made from several host threads at once.
 * - Rows are indexed with 64-bit integers end to end; no launch wraps a 32-bit
 *   grid, however many rows there are.  (MLX PR #4776 "fast.cross_entropy silently
 *   skips rows when the Metal grid gets too large", Issue: a 32-bit grid of
 *   rows x threads-per-row silently dropped rows past 2^32 threads.)
 * - Targets are contiguous int32 [n_rows].  A target outside [0, V) never causes an
 *   out-of-bounds read: that row's loss, and its dlogits row, are written as NaN
 *   (unless it is the ignore_index of a ce_forward_ex / ce_vjp_ex call).
 * - ce_forward and ce_vjp produce per-row outputs only; the _ex and _probs calls can
 *   also reduce the losses to their sum or mean on the device.
 */
#ifndef CE_MI355X_H
#define CE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of logits and dlogits (fp16 and bf16 are IEEE binary16 and bfloat16). */
typedef enum { CE_F32 = 0, CE_F16 = 1, CE_BF16 = 2 } ce_dtype;

/*
 * Strided [batches x rows_per_batch x V] view of logits, in ELEMENTS.
 * Logical row r (0 <= r < n_rows) starts at
 *     base + (r / rows_per_batch) * batch_stride + (r % rows_per_batch) * row_stride
 * and its V columns are contiguous (column stride 1).  A plain contiguous [n_rows, V]
 * tensor is {rows_per_batch = n_rows, row_stride = V, batch_stride = n_rows * V}.
 * The slice x[:, :-1] of a contiguous [B, L, V] tensor is
 * {rows_per_batch = L - 1, row_stride = V, batch_stride = L * V} with n_rows = B * (L - 1).
 * Views are read in place: the library never copies a view to a temporary.
 * (MLX issue #4686 "fast.cross_entropy VJP returns wrong gradients for large
 * non-contiguous inputs on Metal", Describe the bug: the gradient of the
 * next-token loss over the view logits[:, :-1] came back wrong when the view was
 * copied into a temporary whose buffer the output shared.)
 * Requirements: rows_per_batch >= 1, row_stride >= 0, batch_stride >= 0, and the
 * base pointer aligned to the element size.  An input view may overlap itself (for
 * example row_stride 0 repeats one row).  An output view (dlogits) must not: when it
 * has more than one row, row_stride >= V, and when it spans more than one batch,
 * batch_stride >= (rows_per_batch - 1) * row_stride + V.  A layout that breaks these
 * rules, or whose furthest element lies beyond 1e18 elements, returns CE_ERR_LAYOUT.
 */
typedef struct {
    int64_t rows_per_batch;
    int64_t row_stride;
    int64_t batch_stride;
} ce_layout;

typedef enum {
    CE_OK = 0,
    CE_ERR_NULL = -1,      /* a required pointer is NULL                                   */
    CE_ERR_SHAPE = -2,     /* n_rows < 0, V < 1, D < 1, V or D out of supported range      */
    CE_ERR_DTYPE = -3,     /* dtype is not a ce_dtype                                      */
    CE_ERR_LAYOUT = -4,    /* bad strides, or a pointer not aligned as required            */
    CE_ERR_WORKSPACE = -5, /* lce workspace NULL or smaller than the *_workspace_size()    */
    CE_ERR_LAUNCH = -6,    /* the HIP runtime rejected a kernel launch                     */
    CE_ERR_ALIAS = -7,     /* an output overlaps an input it may not overlap               */
    CE_ERR_DEVICE = -8,    /* no usable HIP device, or the device is not gfx950            */
    CE_ERR_OPTION = -9     /* a ce_options field out of range (see ce_options)             */
} ce_status;

/*
 * ce_forward: loss_i = logsumexp(z_i) - z_{i, y_i} for each row of a logits view.
 *
 * Source: Ineshin, "A fused linear cross-entropy forward kernel for Apple GPUs",
 * section 1 (the loss needs only the row's log-sum-exp and target logit; the
 * online log-sum-exp keeps a running maximum m and a sum s rescaled to it).  MLX PR
 * #4188 "Shift by the max in cross_entropy", Proposed changes: the row maximum is
 * taken out before the target score is subtracted, so the loss is assembled as
 * (m - z_y) + log s and two equal logits give log 2 at any magnitude.
 *
 *   logits  [n_rows rows of V] of dtype `dt`, addressed through `in`.
 *   targets int32 [n_rows], contiguous.
 *   loss    float32 [n_rows], contiguous (written).
 *   lse     float32 [n_rows][2], contiguous, 8-byte aligned (written): lse[i][0] = m_i,
 *           the row maximum (a stored logit, exactly), and lse[i][1] = log s_i with
 *           s_i = sum_j exp(z_ij - m_i).  The log-sum-exp is lse[i][0] + lse[i][1].
 *           Keeping the pair lets ce_vjp form exp((z - m) - log s) without the
 *           cancellation that a single float32 lse suffers at large magnitudes.
 * Accumulation is float32 whatever dt is.  Rows holding only -inf, or any +inf or
 * NaN, give a NaN loss.  -inf entries carry zero probability.
 * Outputs must not overlap the logits, the targets or each other (CE_ERR_ALIAS).
 */
ce_status ce_forward(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets,
                     int64_t n_rows, int64_t V, float* loss, float* lse, hipStream_t stream);

/*
 * ce_vjp: dlogits_ij = g_i * (exp((z_ij - m_i) - log s_i) - [j == y_i]).
 *
 * The vector-Jacobian product of ce_forward's per-row loss with upstream gradient g.
 * Source: Ineshin (above), section 1: the backward reuses the log-sum-exp saved by
 * the forward; MLX issue #4686 (above) for the strided-view case.
 *
 *   logits  as in ce_forward (same view, same dt).
 *   targets int32 [n_rows]; lse float32 [n_rows][2] as written by ce_forward;
 *   g       float32 [n_rows], contiguous.
 *   dlogits [n_rows rows of V] of dtype `dt`, addressed through `out` (written).
 *           Values are computed in float32 and rounded to dt to nearest, ties to even.
 *           bf16 results in the subnormal range (below 2^-126) are delivered too,
 *           for |g| < 2^103; this holds for every VJP in this header that writes bf16.
 * dlogits may be the logits themselves (an in-place VJP) only with an identical
 * layout; otherwise it must not overlap the logits, targets, lse or g (CE_ERR_ALIAS).
 * The output is always the caller's buffer: no library temporary is ever shared
 * with it.
 */
ce_status ce_vjp(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets,
                 const float* lse, const float* g, int64_t n_rows, int64_t V, void* dlogits,
                 ce_layout out, hipStream_t stream);

/*
 * ce_forward_vjp: ce_forward and ce_vjp in one kernel, for a caller that knows the
 * upstream gradient g before the forward runs (a loss summed or averaged over the
 * rows, as the next-token loss ".sum()" of MLX issue #4686 (above), Describe the bug).
 *
 * Source: Ineshin (above), section 1: the loss needs only the row's log-sum-exp and
 * target logit, and the backward only that log-sum-exp; "One barrier short", first
 * section: mlx-lm computes its divergences and their gradients in one fused pass so
 * that the log-softmax rows never exist in memory.
 * Rows of more than 2048 and at most 20480 16-byte vectors (16384 for fp32) whose
 * input and output rows share their 16-byte phase are held in the registers of one
 * workgroup of 512 or 1024 threads: the row max and the sum of exponentials are two passes over
 * those registers and the gradient a third, so HBM carries one read and one write of
 * the logits instead of ce_forward's read plus ce_vjp's read and write.  Other rows
 * are reduced as ce_forward reduces them and then swept a second time by the same
 * lanes, mostly from the GPU's caches.
 *
 *   logits, targets  as in ce_forward.
 *   g        float32 [n_rows], contiguous: the upstream gradient of each row's loss.
 *   loss, lse        written as by ce_forward.
 *   dlogits  written as by ce_vjp with that lse and g, through `out`.
 * dlogits always equal ce_vjp's for the lse this call writes, bit for bit.  Loss and
 * lse equal ce_forward's bit for bit except for rows held in registers (their two-pass
 * sum rounds differently, within float32 accumulation error) and for rows of 1 or 2
 * aligned 16-byte vectors whose dlogits rows are not 16-byte aligned (ce_forward then
 * takes one lane per row, this call a lane group).  dlogits may be the logits themselves (in place) only with an
 * identical layout; otherwise no output may overlap the logits, targets, g or another
 * output (CE_ERR_ALIAS).  Errors as ce_forward and ce_vjp.
 */
ce_status ce_forward_vjp(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets, const float* g,
                         int64_t n_rows, int64_t V, float* loss, float* lse, void* dlogits, ce_layout out,
                         hipStream_t stream);

/*
 * lce_workspace_size: bytes of device workspace lce_forward needs for (N, D, V).
 * Returns 0 for arguments lce_forward would reject.
 */
size_t lce_workspace_size(int64_t N, int64_t D, int64_t V);

/*
 * lce_forward: per-row loss and log-sum-exp of Z = H.W^T without materialising Z.
 *
 * Source: Ineshin (above), section 1: for each vocabulary tile the kernel merges the
 * tile into the running (m, s) of every row, m' = max(m, m_t),
 * s' = s * exp(m - m') + sum_j exp(z_j - m'), and captures z_{i, y_i} when y_i falls
 * in the tile; after the last tile the log-sum-exp is m + log s.
 *
 *   H        bf16 [N][D], row-major, contiguous, 16-byte aligned.
 *   W        bf16 [V][D], row-major, contiguous, 16-byte aligned.
 *   targets  int32 [N].
 *   loss     float32 [N] (written); lse float32 [N][2] as in ce_forward (written).
 *   workspace, workspace_bytes: device scratch of at least lce_workspace_size(N, D, V)
 *            bytes, 256-byte aligned; its contents on entry are ignored.
 * The product accumulates in float32 on the matrix cores (bf16 in, fp32 out).  The
 * target logit is taken from the same float32 accumulator that feeds (m, s).
 * Requires D % 8 == 0 (16-byte rows), D <= 2^22 and V < 2^31, and a tile grid that
 * fits one dispatch: one 256-thread workgroup per 256 x 256 tile of N x V, in whole
 * groups of 256 tiles, under 2^32 work-items (up to 2^24 tiles, about N V <= 2^40).
 * Larger shapes return CE_ERR_SHAPE.
 */
ce_status lce_forward(const void* H, const void* W, const int32_t* targets, int64_t N, int64_t D,
                      int64_t V, float* loss, float* lse, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * lce_backward_workspace_size: bytes of device workspace lce_backward needs for
 * (N, D, V): with C = min(8192, V rounded up to 256) columns per chunk and N8 = N
 * rounded up to 8, four bf16 arrays, each starting on a 256-byte boundary: the logits
 * gradient chunk [N][C], its transpose [C][N8], H^T [D][N8] and the W chunk's transpose
 * [D][C] (384 MiB at N = 8192, D = 4096).  This is the least lce_backward accepts.
 * Returns 0 for arguments lce_backward would reject.
 */
size_t lce_backward_workspace_size(int64_t N, int64_t D, int64_t V);

/*
 * lce_backward_workspace_size_one_pass: bytes with which lce_backward runs the whole
 * vocabulary as one chunk: the same four arrays with C = V rounded up to 256 (5.9 GiB
 * at N = 8192, D = 4096, V = 151,936).  One chunk writes dH once instead of reading and
 * rewriting it per chunk, which measured 3% faster at that shape, with identical
 * results.  For V > 2^22 (the one-chunk layout addresses rows of 2 C bytes with 32-bit
 * offsets), for V <= 8192, and where the one-chunk grids would not fit one dispatch
 * (N x V, or N x D and V x D together, past 2^24 tiles as in lce_forward) it equals
 * lce_backward_workspace_size.  Returns 0 for arguments lce_backward would reject.
 * Source: the chunk width is a choice of the implementation; Ineshin (above), section 1,
 * fixes only that the backward regenerates the logits chunk by chunk.
 */
size_t lce_backward_workspace_size_one_pass(int64_t N, int64_t D, int64_t V);

/*
 * lce_backward: gradients of sum_i g_i loss_i, with loss_i as lce_forward computes it,
 * with respect to H and W:
 *   dZ = diag(g) (softmax(Z) - onehot(y)),   dH = dZ W,   dW = dZ^T H,   Z = H.W^T.
 *
 * Source: Ineshin (above), section 1: training saves the forward's log-sum-exp and a
 * separate chunked backward regenerates the logits it needs tile by tile.  For each
 * chunk of vocabulary columns (8192, the page's tile width, or the whole vocabulary when
 * the workspace holds lce_backward_workspace_size_one_pass bytes), the forward's MFMA
 * tile kernel recomputes the chunk of Z and its epilogue writes
 * dZ = g_i (exp((z - m_i) - log s_i) - [col == y_i]) in bf16 (round to nearest even)
 * into the workspace, row-major and transposed, and the same tiles write the W chunk
 * transposed from the W rows they stage.  The same MFMA K loop then adds dZ_c W_c into
 * dH and writes dZ_c^T H into the chunk's rows of dW, both with float32 accumulation
 * (dH is one sequential sum over the vocabulary: each chunk's tiles start from its
 * previous value); H enters through a transposed copy made once per call.  The call is
 * made of kernels only (no library calls, no memsets), so it can be captured in a HIP
 * graph.
 *
 *   H, W, targets  as in lce_forward.
 *   lse      float32 [N][2], the (m, log s) pairs lce_forward wrote for the same H, W.
 *   g        float32 [N], the upstream gradient of each row's loss.
 *   dH       float32 [N][D], row-major, 16-byte aligned (written).
 *   dW       float32 [V][D], row-major, 16-byte aligned (written).
 *   workspace, workspace_bytes: device scratch of at least
 *            lce_backward_workspace_size(N, D, V) bytes, 256-byte aligned.  With at
 *            least lce_backward_workspace_size_one_pass(N, D, V) bytes the call runs one
 *            chunk; otherwise chunks of 8192 columns.  It uses the first bytes of that
 *            size and leaves the rest untouched; only those must be free of overlap.
 * A row whose target lies outside [0, V) has a NaN loss, so its dZ row is NaN: its
 * dH row and every entry of dW come out NaN.  dH and dW must not overlap the inputs,
 * the workspace or each other (CE_ERR_ALIAS).  Requirements on N, D, V as in
 * lce_forward, N <= 2^22 (the product over the tokens addresses rows of 2 N bytes
 * with 32-bit offsets), and the two products' tiles (N x D and 8192 x D, in groups of
 * 256 as in lce_forward) together under 2^24; larger shapes return CE_ERR_SHAPE.
 */
ce_status lce_backward(const void* H, const void* W, const int32_t* targets, const float* lse,
                       const float* g, int64_t N, int64_t D, int64_t V, float* dH, float* dW,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kl_forward: kl_i = sum_j softmax(p_i)_j (log softmax(p_i)_j - log softmax(q_i)_j), the
 * KL divergence of the teacher row p_i from the student row q_i.
 *
 * Source: "One barrier short", section "Run it yourself" (the reference the fused
 * kernel is checked against: kl = sum exp(lp) (lp - lq) with lq, lp the log-softmaxes
 * of the student and teacher logits), and section "Sixty-four floats" (one pass per
 * row with an online log-sum-exp per distribution, combined across waves through
 * shared memory).  Each lane keeps (m_q, s_q), (m_p, s_p) and
 * t = sum_j exp(p_j - m_p) ((p_j - m_p) - (q_j - m_q)), every term taken against its own
 * row's running maximum (and t moved with them when either maximum rises), so rows
 * with different offsets lose nothing to cancellation; then kl = t / s_p + log s_q - log s_p.
 *
 *   q, p     student and teacher logits, [n_rows rows of V] of dtype `dt`, each
 *            addressed through its own layout (as the logits of ce_forward).
 *   kl       float32 [n_rows] (written).
 *   lse_q, lse_p  float32 [n_rows][2] (written): (m, log s) of q and of p, as
 *            ce_forward's lse, kept for kl_vjp.
 * A teacher entry of -inf has zero probability and adds nothing; a student entry of
 * -inf where the teacher has mass makes kl_i = +inf; a row with +inf or NaN, or an
 * all -inf teacher row, gives NaN.  Outputs must not overlap q, p or each other.
 */
ce_status kl_forward(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                     int64_t n_rows, int64_t V, float* kl, float* lse_q, float* lse_p, hipStream_t stream);

/*
 * kl_vjp: dq_ij = g_i * (exp((q_ij - m_q,i) - log s_q,i) - exp((p_ij - m_p,i) - log s_p,i)),
 * the gradient of sum_i g_i kl_i with respect to the student logits (the page's
 * reference gradient exp(lq) - exp(lp)).
 *
 *   q, p, dt, layouts  as in kl_forward; lse_q, lse_p as kl_forward wrote them.
 *   g        float32 [n_rows].
 *   dq       [n_rows rows of V] of dtype `dt`, through `dq_layout` (written); computed
 *            in float32 and rounded to nearest, ties to even.
 * dq may be q itself (same layout); otherwise it must not overlap q.  It must never
 * overlap p, lse_q, lse_p or g (CE_ERR_ALIAS).
 */
ce_status kl_vjp(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                 const float* lse_q, const float* lse_p, const float* g, int64_t n_rows, int64_t V, void* dq,
                 ce_layout dq_layout, hipStream_t stream);

/*
 * js_forward: js_i = 1/2 KL(P_i || M_i) + 1/2 KL(Q_i || M_i), M = (P + Q) / 2, with
 * P = softmax(p_i) (teacher) and Q = softmax(q_i) (student).
 *
 * Source: "One barrier short", first section: mlx-lm fuses the Jensen-Shannon divergence
 * of a student and a teacher the way it fuses the KL one; section "The fix": at a logit
 * scale of 20 the loss overflowed to non-finite values until a numerically stable
 * softplus was used.  log M is formed as log Q + softplus(log P - log Q) - log 2 with
 * softplus(x) = max(x, 0) + log(1 + e^-|x|), which cannot overflow.
 *
 *   q, q_layout, p, p_layout, dt, n_rows, V  as in kl_forward.
 *   js     float32 [n_rows] (written).
 *   lse_q, lse_p  float32 [n_rows][2] (written): (m, log s) of q and p.
 *   hq     float32 [n_rows] (written): H = 1/2 KL(Q || M), the student's half, which
 *          js_vjp needs.
 * Each row is read twice: the terms need both normalisers first.  A row pair where either
 * row has no softmax (all -inf, or a +inf / NaN entry) gives NaN.  Zero probabilities
 * contribute nothing (0 log 0 = 0); js is always finite otherwise, in [0, ln 2].
 * Outputs must not overlap the inputs or each other (CE_ERR_ALIAS).
 */
ce_status js_forward(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                     int64_t n_rows, int64_t V, float* js, float* lse_q, float* lse_p, float* hq,
                     hipStream_t stream);

/*
 * js_vjp: dq_ik = g_i Q_ik (h_ik - H_i), h_ik = (log Q_ik - log M_ik) / 2, the gradient of
 * sum_i g_i js_i with respect to the student logits, from js_forward's lse_q, lse_p, hq.
 *   g   float32 [n_rows].  dq  [n_rows rows of V] of dtype `dt` through `dq_layout`
 *       (written; may be q itself with an identical layout, must not overlap p, lse_q,
 *       lse_p, hq or g).
 */
ce_status js_vjp(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                 const float* lse_q, const float* lse_p, const float* hq, const float* g, int64_t n_rows, int64_t V,
                 void* dq, ce_layout dq_layout, hipStream_t stream);

/*
 * ---- Cross-entropy options --------------------------------------------------------
 *
 * Source: MLX PR #4188 "Shift by the max in cross_entropy", Proposed changes: the
 * cross-entropy takes class-index or probability targets, a label smoothing whose
 * term subtracts the mean logit, and the reductions 'none', 'sum' and 'mean', all
 * checked against PyTorch; the max shift serves every one of these paths.  With target
 * weights w_j the loss of a row is -sum_j w_j log p_j, where
 *     class index y:   w = (1 - eps) onehot(y) + eps / V
 *     probabilities t: w = (1 - eps) t + eps / V,
 * and the gradient of sum_i g_i loss_i is g_i (W_i p_ij - w_ij), W_i = sum_j w_ij.
 * A zero weight contributes nothing even where p_j = 0 (0 log 0 = 0).
 */
typedef enum { CE_REDUCE_NONE = 0, CE_REDUCE_SUM = 1, CE_REDUCE_MEAN = 2 } ce_reduction;

/* ignore_index value that ignores nothing. */
#define CE_NO_IGNORE ((int32_t)INT32_MIN)

/*
 * label_smoothing  eps in [0, 1].
 * ignore_index     class-index targets only: a row whose target equals it has loss 0
 *                  and gradient 0 and does not count towards a mean (PyTorch's
 *                  convention).  Any value may be given, also one inside [0, V).  Must be
 *                  CE_NO_IGNORE for probability targets.
 * reduction        a ce_reduction.  'sum' adds the losses of the rows that count,
 *                  'mean' divides that sum by their number (NaN when none counts).
 * Anything else returns CE_ERR_OPTION.
 */
typedef struct {
    float label_smoothing;
    int32_t ignore_index;
    int32_t reduction;
} ce_options;

/* Bytes of device workspace a CE_REDUCE_SUM or CE_REDUCE_MEAN forward needs (a constant). */
size_t ce_reduce_workspace_size(void);

/*
 * ce_forward_ex: ce_forward with options.
 *
 *   logits, in, dt, targets, n_rows, V, loss, lse  as in ce_forward.  loss holds the
 *           per-row losses whatever the reduction (0 on ignored rows); lse is the pair
 *           (m, log s) of every row.
 *   total   float32 [1]: the sum or mean (written; may be NULL with CE_REDUCE_NONE).
 *   count   int64 [1]: the number of rows that count (written; may be NULL with
 *           CE_REDUCE_NONE).  ce_vjp_ex reads it for a mean.
 *   workspace, workspace_bytes  device scratch of at least ce_reduce_workspace_size()
 *           bytes, 8-byte aligned, for a sum or mean (may be NULL otherwise).
 * The sum is formed in float64 over a fixed split of the rows that depends on n_rows
 * alone, so results are bitwise reproducible.  With n_rows == 0 and a reduction, total
 * is 0 (sum) or NaN (mean) and count is 0.  Outputs, the workspace included, must not
 * overlap the inputs or each other (CE_ERR_ALIAS).
 */
ce_status ce_forward_ex(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets, int64_t n_rows,
                        int64_t V, ce_options opt, float* loss, float* lse, float* total, int64_t* count,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ce_forward_ex_noalloc: ce_forward_ex for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The same call as ce_forward_ex without the workspace arguments: a sum or mean keeps
 * its partials in a fixed array of ce_reduce_workspace_size() = 16 KiB that the library
 * holds on each GPU it runs on, from its first such call on that GPU until the process
 * ends.  That size covers the reduction at every n_rows and V (the rows are split into
 * at most 1024 parts), so no input is too large for it.  The call allocates nothing and
 * issues no memset; nothing in the array needs to start at zero (every partial is
 * written before it is read).  Results are those of ce_forward_ex bit for bit.
 * Every call on one GPU shares that GPU's array, which keeps the last call's partials:
 * calls that overlap in time on one GPU (on different streams, or from different host
 * threads without ordering) race on it and must not be made.  With CE_REDUCE_NONE the
 * array is not used.  Errors as ce_forward_ex; CE_ERR_DEVICE also if the array's
 * address cannot be had on the current device.
 */
ce_status ce_forward_ex_noalloc(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets,
                                int64_t n_rows, int64_t V, ce_options opt, float* loss, float* lse, float* total,
                                int64_t* count, hipStream_t stream);

/*
 * ce_vjp_ex: dlogits_ij = g_i ((1 - eps) (p_ij - [j == y_i]) + eps (p_ij - 1 / V)), the
 * gradient of ce_forward_ex's loss, from the saved lse.
 *
 *   g       float32: [n_rows] per-row upstream gradients for CE_REDUCE_NONE; [1], the
 *           gradient of the total, for a sum or mean.
 *   count   int64 [1] as ce_forward_ex wrote it; read for CE_REDUCE_MEAN (g / count per
 *           row), otherwise may be NULL.
 *   The rest as in ce_vjp.  Ignored rows get dlogits 0; their logits are not read.
 */
ce_status ce_vjp_ex(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets, const float* lse,
                    const float* g, int64_t n_rows, int64_t V, ce_options opt, const int64_t* count, void* dlogits,
                    ce_layout out, hipStream_t stream);

/*
 * ce_forward_probs: loss_i = -sum_j w_ij log p_ij with probability targets.
 *
 *   probs        [n_rows rows of V] of dtype `dt` (the logits' type), read through
 *                `probs_layout` (a ce_layout like `in`).  Rows need not sum to 1.
 *   wsum         float32 [n_rows] (written): W_i = sum_j w_ij, which ce_vjp_probs needs.
 *   The rest as in ce_forward_ex; opt.ignore_index must be CE_NO_IGNORE, and a mean
 *   divides by n_rows.
 */
ce_status ce_forward_probs(const void* logits, ce_layout in, ce_dtype dt, const void* probs, ce_layout probs_layout,
                           int64_t n_rows, int64_t V, ce_options opt, float* loss, float* lse, float* wsum,
                           float* total, int64_t* count, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * ce_vjp_probs: dlogits_ij = g_i (W_i p_ij - w_ij), from ce_forward_probs's lse and wsum.
 * g and count as in ce_vjp_ex; dlogits as in ce_vjp (it may be the logits, in place,
 * and must not overlap probs).
 */
ce_status ce_vjp_probs(const void* logits, ce_layout in, ce_dtype dt, const void* probs, ce_layout probs_layout,
                       const float* lse, const float* wsum, const float* g, int64_t n_rows, int64_t V, ce_options opt,
                       const int64_t* count, void* dlogits, ce_layout out, hipStream_t stream);

/* Static, human-readable text for a status code (never NULL). */
const char* ce_status_string(ce_status status);

#ifdef __cplusplus
}
#endif

#endif /* CE_MI355X_H */
