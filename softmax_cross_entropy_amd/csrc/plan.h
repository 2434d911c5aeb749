// Launch plans and the constants the kernels are built around (shared by the kernels
// and the host-side planner).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace ce {

// How rows map onto lanes.  narrow_nv > 0: one lane per row, each row exactly
// narrow_nv aligned 16-byte vectors.  Otherwise `lanes` lanes per row (a power of two
// in [1, 1024]); above 64 one workgroup of `lanes` threads holds each row.
struct Plan {
    int narrow_nv;
    int lanes;
    int64_t blocks;
    int64_t chunks;  // VJP only: > 0 cuts each row into this many chunks of kChunkU * 256 vectors
    int regs_nv;     // ce_forward_vjp only: > 0 holds each row in the registers of `lanes`
                     // threads, regs_nv 16-byte vectors per thread (see kRegsNV16)
};

// Vectors per thread the register-resident one-pass kernel is built for: 16-bit types
// (groups of 4 vectors), then fp32 (groups of 8).  A row of nvec vectors takes the
// smallest that holds it, ceil(nvec / 1024) <= regs_nv.
constexpr int kRegsNV16[] = {8, 12, 16, 20};
constexpr int kRegsNV32[] = {8, 16};
// Rows the forward gives 512 lanes (2049 to 4096 vectors) take 512 threads of 8 vectors.
constexpr int kRegsNV512[] = {8};

// Vectors per thread in one chunk of the chunked VJP layout.
constexpr int kChunkU = 2;

// Sum / mean of the per-row losses: float64 partial sums over at most kReduceMaxParts
// blocks of at least kReduceRowsMin rows (a split that depends on n_rows alone), then one
// fixed-order fold.  The workspace holds the partials: kReduceMaxParts doubles, then as
// many int64 counts.
constexpr int64_t kReduceMaxParts = 1024;
constexpr int64_t kReduceRowsMin = 4096;
constexpr size_t kReduceWorkspaceBytes = (size_t)kReduceMaxParts * 16;

}  // namespace ce
