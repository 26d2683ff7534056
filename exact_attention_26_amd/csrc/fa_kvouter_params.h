// K/V-outer forward problem description shared by the host entry point and
// its kernel.
// Internal to the library, not part of the public ABI (that is include/fa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// One K/V-outer forward problem (dense [B,H,N,d], 16-bit storage), already
// validated: the key/value tiles are the outer loop and every query row's
// running output and statistics round-trip HBM once per tile.
struct KvOuterParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* oacc;          // [B,H,N,d] fp32 running output (caller's scratch)
  float* mstat;         // [B,H,N] running max (scratch)
  float* lstat;         // [B,H,N] running sum (scratch)
  int64_t head_stride;  // N*d elements
  int BH;
  int N;
  int groups;           // workgroups (query-row groups) per (batch, head)
  int rows_per_group;   // multiple of 32
  int tiles;            // ceil(N / 64)
  float scale;
  float scale_log2;
};

// Returns 0 on success or a hipError_t from the launch.
hipError_t launch_fwd_kv_outer(const KvOuterParams& p, int d, bool bf16, hipStream_t stream);

}  // namespace fa
