// Internal declarations shared by the host entry points and the kernels of
// the gfx950 FlashAttention-2 forward library. Not part of the public ABI
// (that is include/fa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// One forward problem, already validated on the host.
//
// Dense:  Q/K/V/O [B,H,N,d];  element (b,h,n,k) at b*batch_stride +
//         h*head_stride + n*row_stride + k;  L [B,H,N].
// Varlen: Q/K/V/O [T,H,d];   sequence s = "b" starts at token cu_seqlens[s];
//         element (s,h,n,k) at (cu[s]+n)*row_stride + h*head_stride + k;
//         L [H,T] at h*total_tokens + cu[s] + n.  N holds max_seqlen.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* cu_seqlens;  // varlen only, else nullptr
  int64_t batch_stride;       // elements (dense only)
  int64_t head_stride;        // elements
  int row_stride;             // elements between consecutive tokens
  int B;                      // batch (dense) or number of sequences (varlen)
  int H;
  int N;                      // sequence length (dense) or max_seqlen (varlen)
  int total_tokens;           // varlen: T
  int q_blocks;               // ceil(N / rows per workgroup)
  float scale;                // softmax scale applied to q.k
  float scale_log2;           // scale * log2(e): exp(x*scale) = exp2(x*scale_log2)
  int window;                 // banded (dense 16-bit only): row r sees keys |r - c| <= window,
                              // 0 <= window <= N; -1 = every key
};

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

// Launchers; return 0 on success or a hipError_t from the launch.
hipError_t launch_fwd_f32(const FwdParams& p, int d, bool varlen, hipStream_t stream);
// waves: 8 (ping-pong, 256-row workgroups) or 4 (banded only, 128-row workgroups);
// p.q_blocks must count blocks of 32 * waves rows.
hipError_t launch_fwd_mfma16(const FwdParams& p, int d, bool bf16, bool varlen, int waves,
                             hipStream_t stream);
hipError_t launch_dropout_add_norm(const NormParams& p, bool bf16, hipStream_t stream);
hipError_t launch_fwd_kv_outer(const KvOuterParams& p, int d, bool bf16, hipStream_t stream);
// The three backward kernels in order: D = rowsum(dO * O), dK/dV, dQ.
hipError_t launch_bwd(const BwdParams& p, int d, bool bf16, hipStream_t stream);
// Keys per dK/dV workgroup and queries per dQ workgroup (size the grids).
constexpr int kBwdKeysPerBlock = 128;
constexpr int kBwdQueriesPerBlock = 128;

// Rows of Q owned by one workgroup of each kernel (sizes the grid). The
// 16-bit kernel runs kWaves16 waves of 32 query rows each, or 4 waves (128
// rows) for short sequences and narrow bands (thresholds below).
#ifndef FA_WAVES16
#define FA_WAVES16 8
#endif
constexpr int kWaves16 = FA_WAVES16;
constexpr int kRowsPerBlockF32 = 128;
constexpr int kRowsPerBlock16 = 32 * kWaves16;
// Banded forward: windows up to this many keys run the 4-wave variant
// (measured faster from w = 0, 1.56x, to w = 2048, 1.02x; slower from 4096).
#ifndef FA_BAND_NARROW_MAX
#define FA_BAND_NARROW_MAX 2048
#endif
constexpr int kBandNarrowMax = FA_BAND_NARROW_MAX;
constexpr int kBandNarrowWaves = 4;
// Dense and packed forward: sequences up to these lengths run the 4-wave
// variant too (measured back to back: dense d = 64, N = 512 +12 %, N = 2048
// +10 %; d = 128, N = 1024 +5 %, N = 4096 -2 %, N = 8192 -3 %; varlen with
// lengths 64..4096 +4 %, 64..1024 +29 %). Outputs are bitwise identical.
#ifndef FA_DENSE_NARROW_MAX_N
#define FA_DENSE_NARROW_MAX_N 2048
#endif
#ifndef FA_VARLEN_NARROW_MAX_N
#define FA_VARLEN_NARROW_MAX_N 4096
#endif
constexpr int kDenseNarrowMaxN = FA_DENSE_NARROW_MAX_N;
constexpr int kVarlenNarrowMaxN = FA_VARLEN_NARROW_MAX_N;

}  // namespace fa
