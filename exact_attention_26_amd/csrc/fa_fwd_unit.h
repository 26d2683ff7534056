// Workgroup -> work unit (query block of one (batch or sequence, head)) for the
// forward kernels. Internal to the library.
#pragma once

#include "fa_device.h"
#include "fa_fwd_params.h"

namespace fa {

// One work unit: `rows_per_block` query rows of one (batch or sequence, head).
struct WorkUnit {
  int n;             // keys (= queries) of this sequence/head
  int q0;            // first query row of the unit
  int64_t base;      // element offset of row 0 of this head in Q/K/V/O
  int64_t lse_base;  // element offset of row 0 of this head in L
};

// Logical id order: the Q-blocks of one (batch or sequence, head) are
// consecutive, so xcd_remap keeps them on one XCD (one L2 holds that head's
// K/V). Dense units run batch-major; varlen units run head-major, so that
// every XCD's contiguous share of units holds all sequences (for a few
// heads) and the XCDs get equal work whatever the length mix.
// Returns false when the unit lies past the end of its sequence (varlen).
template <bool VARLEN>
__device__ __forceinline__ bool resolve_unit(const FwdParams& p, int rows_per_block,
                                             WorkUnit& u) {
  const int id = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int qb = id % p.q_blocks;
  const int rest = id / p.q_blocks;
  const int h = VARLEN ? rest / p.B : rest % p.H;
  const int b = VARLEN ? rest % p.B : rest / p.H;
  u.q0 = qb * rows_per_block;
  if (VARLEN) {
    const int start = p.cu_seqlens[b];
    u.n = p.cu_seqlens[b + 1] - start;
    u.base = (int64_t)start * p.row_stride + (int64_t)h * p.head_stride;
    u.lse_base = (int64_t)h * p.total_tokens + start;
  } else {
    u.n = p.N;
    u.base = (int64_t)b * p.batch_stride + (int64_t)h * p.head_stride;
    u.lse_base = ((int64_t)b * p.H + h) * p.N;
  }
  return u.q0 < u.n;
}

}  // namespace fa
