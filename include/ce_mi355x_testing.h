/*
 * ce_mi355x_testing.h: test and tuning entry points of libce_mi355x.so.
 *
 * These calls are the product calls of ce_mi355x.h with the row-to-lane mapping
 * forced by the caller, so that tests can reach every kernel layout at small sizes and
 * compare the layouts bit for bit.  They are not part of the product interface: a
 * caller of the library uses ce_mi355x.h, whose calls pick the mapping themselves.
 * Every convention of ce_mi355x.h (device pointers, streams, error codes, aliasing
 * rules) applies unchanged.
 */
#ifndef CE_MI355X_TESTING_H
#define CE_MI355X_TESTING_H

#include "ce_mi355x.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * ce_forward_lanes: ce_forward with the row-to-lane mapping chosen by the caller.
 * lanes_per_row = 0 picks the mapping from V and dt exactly as ce_forward does.
 * A power of two in [1, 1024] assigns that many lanes to each row (up to 64 lanes:
 * 64 / lanes rows per wavefront; above 64: one row per workgroup of that many
 * threads, combined through LDS).  -1 asks for the one-lane-per-row path for
 * short aligned rows and fails with CE_ERR_LAYOUT where that path does not apply.
 * Results agree with ce_forward up to float32 summation order.  Intended for tests
 * and tuning; any other value returns CE_ERR_SHAPE.
 */
ce_status ce_forward_lanes(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets,
                           int64_t n_rows, int64_t V, float* loss, float* lse,
                           int32_t lanes_per_row, hipStream_t stream);

/*
 * ce_vjp_lanes: ce_vjp with lanes_per_row chosen as in ce_forward_lanes.  With
 * lanes_per_row = 0 a row spanning at least 2048 16-byte vectors is cut into chunks
 * of 512 vectors, each handled by its own 256-thread workgroup (ce_vjp does the
 * same); a power of two keeps whole rows on that many lanes.  Every layout computes
 * each element with the same float32 operations, so all give identical bits.
 */
ce_status ce_vjp_lanes(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets,
                       const float* lse, const float* g, int64_t n_rows, int64_t V, void* dlogits,
                       ce_layout out, int32_t lanes_per_row, hipStream_t stream);

/*
 * ce_forward_vjp_lanes: ce_forward_vjp with lanes_per_row chosen as in ce_forward_lanes
 * (0: as ce_forward_vjp; a power of two in [1, 1024]; -1: one lane per row, which needs
 * rows of 1, 2, 4 or 8 aligned 16-byte vectors in both views).  For tests and tuning.
 */
ce_status ce_forward_vjp_lanes(const void* logits, ce_layout in, ce_dtype dt, const int32_t* targets,
                               const float* g, int64_t n_rows, int64_t V, float* loss, float* lse, void* dlogits,
                               ce_layout out, int32_t lanes_per_row, hipStream_t stream);


/* kl_forward with lanes_per_row as in ce_forward_lanes (-1 is not accepted here). */
ce_status kl_forward_lanes(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                           int64_t n_rows, int64_t V, float* kl, float* lse_q, float* lse_p,
                           int32_t lanes_per_row, hipStream_t stream);

/* kl_vjp with lanes_per_row as in ce_vjp_lanes (-1 is not accepted here). */
ce_status kl_vjp_lanes(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                       const float* lse_q, const float* lse_p, const float* g, int64_t n_rows, int64_t V,
                       void* dq, ce_layout dq_layout, int32_t lanes_per_row, hipStream_t stream);

/* js_forward with lanes_per_row as in kl_forward_lanes. */
ce_status js_forward_lanes(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                           int64_t n_rows, int64_t V, float* js, float* lse_q, float* lse_p, float* hq,
                           int32_t lanes_per_row, hipStream_t stream);

/* js_vjp with lanes_per_row as in kl_vjp_lanes. */
ce_status js_vjp_lanes(const void* q, ce_layout q_layout, const void* p, ce_layout p_layout, ce_dtype dt,
                       const float* lse_q, const float* lse_p, const float* hq, const float* g, int64_t n_rows,
                       int64_t V, void* dq, ce_layout dq_layout, int32_t lanes_per_row, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CE_MI355X_TESTING_H */
