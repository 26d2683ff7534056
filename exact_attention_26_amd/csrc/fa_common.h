// Every internal problem description and launcher, for the host entry points
// (fa_api.hip). The kernels include only their own header, so that a change to
// one kernel's description leaves the others' sources untouched. Not part of
// the public ABI (that is include/fa.h).
#pragma once

#include "fa_bwd_params.h"
#include "fa_fwd_params.h"
#include "fa_kvouter_params.h"
#include "fa_norm_params.h"

#include <stdint.h>

namespace fa {

// prepare_bwd's status for an empty problem (a zero size): nothing to launch.
constexpr int kEmptyProblem = 1;
// Rows (B*H*N) of the static scratch buffer behind fa_bwd_noalloc: one fp32
// D value per row, 16 MiB per GPU.
constexpr int64_t kBwdScratchRows = int64_t{1} << 22;

// Validates a dense backward problem and fills p, making no HIP call. With
// caller_delta the caller's delta buffer is checked and used for D; without
// it delta is ignored (p.delta stays null for the caller to set) and the
// problem must fit kBwdScratchRows. Returns FA_OK, kEmptyProblem or an
// fa_status error.
int prepare_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                const float* L, void* dQ, void* dK, void* dV, const float* delta,
                bool caller_delta, int B, int H, int N, int d, float scale, int dtype,
                BwdParams& p);

}  // namespace fa
