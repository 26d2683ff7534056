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
//
// Varlen with units_per_head > 0: within a head, unit j counts the query
// blocks of the sequences taken in order of decreasing length (ties by index),
// at most q_blocks per sequence. Every unit of a sequence visits all of its
// keys, so this dispatches the largest units first and leaves the smallest
// for the end of the launch (longest-processing-time list scheduling), and the
// grid holds no workgroups for blocks past a sequence's end. Lane i ranks
// sequence i against the others with lane reads (nseq <= 64), so every wave
// finds its unit without shared memory or a barrier.
// Returns false when the workgroup has no unit (varlen).
template <bool VARLEN>
__device__ __forceinline__ bool resolve_unit(const FwdParams& p, int rows_per_block,
                                             WorkUnit& u) {
  const int id = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  int qb, h, b;
  if (VARLEN && p.units_per_head > 0) {
    h = id / p.units_per_head;
    const int j = id - h * p.units_per_head;
    const int lane = (int)(threadIdx.x & 63);
    int ni = -1, ci = 0;
    if (lane < p.B) {
      ni = p.cu_seqlens[lane + 1] - p.cu_seqlens[lane];
      ci = min((ni + rows_per_block - 1) / rows_per_block, p.q_blocks);
    }
    int first = 0;  // units of the sequences ordered ahead of this lane's
    for (int s = 0; s < p.B; ++s) {
      const int ns = __builtin_amdgcn_readlane(ni, s);
      const int cs = __builtin_amdgcn_readlane(ci, s);
      first += (ns > ni || (ns == ni && s < lane)) ? cs : 0;
    }
    const unsigned long long own = __ballot(lane < p.B && first <= j && j < first + ci);
    if (own == 0) return false;  // past the head's last unit
    b = __builtin_ctzll(own);
    qb = j - __builtin_amdgcn_readlane(first, b);
  } else {
    qb = id % p.q_blocks;
    const int rest = id / p.q_blocks;
    h = VARLEN ? rest / p.B : rest % p.H;
    b = VARLEN ? rest % p.B : rest / p.H;
  }
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
