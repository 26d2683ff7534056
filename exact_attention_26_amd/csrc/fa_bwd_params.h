// Backward problem description shared by the host entry point and the
// backward kernels.
// Internal to the library, not part of the public ABI (that is include/fa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// One backward problem (dense [B,H,N,d]), already validated on the host.
// Element (b,h,n,k) of Q/K/V/O/dO/dQ/dK/dV at (b*H + h)*head_stride + n*d + k;
// L and delta at (b*H + h)*N + n.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;
  int64_t head_stride;  // N*d elements
  int64_t rows;         // B*H*N
  int BH;
  int N;
  int kblocks;          // key blocks per head (dK/dV kernel)
  int qblocks;          // query blocks per head (dQ kernel)
  float scale;
  float scale_log2;
};

// The three backward kernels in order: D = rowsum(dO * O), dK/dV, dQ.
// Returns 0 on success or a hipError_t from a launch.
hipError_t launch_bwd(const BwdParams& p, int d, bool bf16, hipStream_t stream);
// Keys per dK/dV workgroup and queries per dQ workgroup (size the grids).
constexpr int kBwdKeysPerBlock = 128;
constexpr int kBwdQueriesPerBlock = 128;

}  // namespace fa
