// Fused dropout + residual + norm problem description shared by the host entry
// point and its kernel.
// Internal to the library, not part of the public ABI (that is include/fa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// One fused dropout + residual + LayerNorm/RMSNorm problem ([rows, hidden],
// 16-bit storage), already validated. Optional tensors are nullptr.
struct NormParams {
  const void* x0;
  const void* x1;        // second (parallel) branch
  const void* res;       // residual
  const void* g0;
  const void* b0;
  const void* g1;        // second weight set: y1
  const void* b1;
  void* y0;
  void* y1;
  void* z;               // dropout(x0) + dropout(x1) + residual, storage dtype
  float* mean;           // [rows], LayerNorm only
  float* rstd;           // [rows]
  unsigned char* mask;   // [rows, hidden] keep bytes of x0, then of x1
  int64_t rows;
  int hidden;            // multiple of 8, <= 8192
  uint32_t thr;          // keep when the Philox word is >= thr (0: no dropout)
  float keep_scale;      // 1 / (1 - p)
  uint32_t key0, key1;   // seed
  uint32_t ctr2, ctr3;   // offset
  float eps;
  int rms;
};

// Returns 0 on success or a hipError_t from the launch.
hipError_t launch_dropout_add_norm(const NormParams& p, bool bf16, hipStream_t stream);

}  // namespace fa
