// Forward problem description shared by the host entry points and the forward
// kernels (dense, packed variable-length and banded).
// Internal to the library, not part of the public ABI (that is include/fa.h).
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
  int units_per_head;         // varlen: > 0 runs each head's units longest sequence
                              // first, this many workgroups per head (at least the
                              // head's units); 0 = one workgroup per (block, seq, head)
  int key_split;              // fp32 dense only: > 0 runs the key-split kernel, this many
                              // waves sharing each 32-row block (q_blocks counts 32-row
                              // blocks); 0 = the 128-row kernel
};

// Packed batches of at most this many sequences take the longest-first order.
constexpr int kLptMaxSeqs = 64;

// Workgroups of one forward launch.
inline int64_t fwd_grid(const FwdParams& p) {
  return p.units_per_head > 0 ? (int64_t)p.units_per_head * p.H
                              : (int64_t)p.q_blocks * p.H * p.B;
}

// Launchers; return 0 on success or a hipError_t from the launch.
hipError_t launch_fwd_f32(const FwdParams& p, int d, bool varlen, hipStream_t stream);
// Phase trace of the 16-bit forward (debug build only): steps recorded per
// wave, and the setter; workgroup -1 turns it off. Without FA_DEBUG_TRACE the
// setter returns hipErrorNotSupported.
constexpr int kTraceSteps = 64;
hipError_t set_fwd_trace(int workgroup, unsigned long long* buffer);
// waves: 8 (ping-pong, 256-row workgroups) or 4 (one wave group, 128-row
// workgroups); p.q_blocks must count blocks of 32 * waves rows.
hipError_t launch_fwd_mfma16(const FwdParams& p, int d, bool bf16, bool varlen, int waves,
                             hipStream_t stream);

// Query rows per workgroup of the fp32 kernel (sizes its grid), and of its
// key-split form, which runs when the 128-row grid would hold fewer
// workgroups than the chip has CUs.
constexpr int kRowsPerBlockF32 = 128;
constexpr int kRowsPerBlockF32Split = 32;
constexpr int kF32SplitBelowBlocks = 256;
// Waves per 32-row block of the key-split form (its LDS holds one K/V tile
// per wave).
constexpr int f32_key_split(int d) { return d == 64 ? 8 : 4; }

}  // namespace fa
