// Fused dropout + residual add + LayerNorm / RMSNorm for bf16 / fp16 rows on
// gfx950 (MI355X).
//
// The op (flash-attention's documentation, the paragraph on its fused
// dropout / residual / LayerNorm extension: one fused op, pre- and post-norm,
// RMSNorm as an option, parallel residuals, hidden sizes up to 8192 in
// multiples of 8), per row of `hidden` values:
//
//   z  = dropout(x0) + dropout(x1) + residual      (x1, residual optional)
//   y0 = norm(z) * gamma0 + beta0,  y1 = norm(z) * gamma1 + beta1 (optional)
//   LayerNorm: norm(z) = (z - mean) * rstd,  rstd = 1 / sqrt(var + eps)
//   RMSNorm:   norm(z) = z * rstd,           rstd = 1 / sqrt(mean(z^2) + eps)
//
// with z also written (the pre-norm residual stream), and mean / rstd per
// row. Dropout keeps element e of branch s when word e % 4 of Philox4x32-10
// (Salmon, Moraes, Dror, Shaw, SC'11) at counter (e / 4, offset + s * 2^32),
// key seed, is >= floor(p * 2^32), and scales kept values by 1 / (1 - p).
//
// It is bound by HBM: every input element is read once and every output
// element written once, with z held in registers between the statistics and
// the normalisation. One row is spread over W waves (W = 1, 2, 4 by hidden
// size) so that a lane holds at most 32 values: lane i of wave part w takes
// the 8-element chunks (64*w + i) + 64*W*k, k < K, loaded and stored as
// 16-byte vectors. Row sums are wave reductions plus, for W > 1, an exchange
// of the W partial sums through LDS. Mean and variance are two passes over
// the registers (no cancellation from E[z^2] - E[z]^2).
#include "fa_device.h"
#include "fa_lanes.h"
#include "fa_norm_params.h"

// Build option FA_NORM_NT (1): row loads and stores are non-temporal (every
// row element is touched once; measured 6-9 % faster than plain accesses).
#ifndef FA_NORM_NT
#define FA_NORM_NT 1
#endif

namespace fa {
namespace {

constexpr int kWavesN = 4;
constexpr int kThreadsN = 64 * kWavesN;

// 16-byte row loads and stores.
__device__ __forceinline__ u32x4 ld16(const unsigned short* p) {
#if FA_NORM_NT
  return __builtin_nontemporal_load((const u32x4*)p);
#else
  return *(const u32x4*)p;
#endif
}
__device__ __forceinline__ void st16(unsigned short* p, u32x4 v) {
#if FA_NORM_NT
  __builtin_nontemporal_store(v, (u32x4*)p);
#else
  *(u32x4*)p = v;
#endif
}

// Philox4x32-10: ten rounds of two 32x32->64-bit products by 0xD2511F53 and
// 0xCD9E8D57; the key is bumped by 0x9E3779B9 / 0xBB67AE85 between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = (uint32_t)p1;
    c[2] = n2;
    c[3] = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

template <bool BF16>
__device__ __forceinline__ float to_f32(unsigned short h) {
  if constexpr (BF16)
    return __uint_as_float((uint32_t)h << 16);
  else
    return (float)__builtin_bit_cast(_Float16, h);
}

// Eight 16-bit values of a 16-byte vector, in memory order.
template <bool BF16>
__device__ __forceinline__ void unpack8(const u32x4 v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = to_f32<BF16>((unsigned short)(v[i] & 0xFFFFu));
    f[2 * i + 1] = to_f32<BF16>((unsigned short)(v[i] >> 16));
  }
}

template <bool BF16>
__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack2<BF16>(f[2 * i], f[2 * i + 1]);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return lanes_sum<64>(v); }

// Keep bits of the 8 elements starting at flat index e0 (a multiple of 8)
// of branch `stream`, as one bit per element in bits 0..7.
__device__ __forceinline__ unsigned keep8(const NormParams& p, uint64_t e0, uint32_t stream) {
  unsigned bits = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint64_t q = (e0 >> 2) + h;
    uint32_t c[4] = {(uint32_t)q, (uint32_t)(q >> 32), p.ctr2, p.ctr3 + stream};
    philox4x32_10(c, p.key0, p.key1);
#pragma unroll
    for (int j = 0; j < 4; ++j) bits |= (c[j] >= p.thr ? 1u : 0u) << (4 * h + j);
  }
  return bits;
}

// Row sum over the W waves that share a row: wave reduction, then (W > 1)
// the partial sums through LDS. Every wave of the workgroup calls it.
template <int W>
__device__ __forceinline__ float row_sum(float v, float* red, int wave) {
  v = wave_sum(v);
  if constexpr (W == 1) {
    return v;
  } else {
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    const int base = wave - wave % W;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < W; ++i) s += red[base + i];
    __syncthreads();  // red is reused by the next reduction
    return s;
  }
}

template <bool BF16, int W, int K>
__global__ __launch_bounds__(kThreadsN) void norm_kernel(NormParams p) {
  __shared__ float red[kWavesN];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * (kWavesN / W) + wave / W;
  const int part = wave % W;
  const bool row_ok = row < p.rows;  // no early return: the LDS exchange has barriers
  const int H = p.hidden;
  const int chunks = H >> 3;
  const int64_t rbase = row * H;
  const bool drop = p.thr != 0u;
  const unsigned short* X0 = (const unsigned short*)p.x0 + rbase;
  const unsigned short* X1 = (const unsigned short*)p.x1 + rbase;
  const unsigned short* R = (const unsigned short*)p.res + rbase;

  float z[K][8];
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int c = part * 64 + lane + 64 * W * k;
#pragma unroll
    for (int j = 0; j < 8; ++j) z[k][j] = 0.f;
    if (!row_ok || c >= chunks) continue;
    const uint64_t e0 = (uint64_t)(rbase + 8 * c);
    float f[8];
    unpack8<BF16>(ld16(X0 + 8 * c), f);
    unsigned keep = drop ? keep8(p, e0, 0u) : 0xFFu;
#pragma unroll
    for (int j = 0; j < 8; ++j) z[k][j] = (keep >> j & 1u) ? f[j] * p.keep_scale : 0.f;
    if (p.mask) {
      u32x2 m;
      m[0] = (keep & 1u) | (keep >> 1 & 1u) << 8 | (keep >> 2 & 1u) << 16 | (keep >> 3 & 1u) << 24;
      m[1] = (keep >> 4 & 1u) | (keep >> 5 & 1u) << 8 | (keep >> 6 & 1u) << 16 | (keep >> 7 & 1u) << 24;
      *(u32x2*)(p.mask + e0) = m;
    }
    if (p.x1) {
      unpack8<BF16>(ld16(X1 + 8 * c), f);
      keep = drop ? keep8(p, e0, 1u) : 0xFFu;
#pragma unroll
      for (int j = 0; j < 8; ++j) z[k][j] += (keep >> j & 1u) ? f[j] * p.keep_scale : 0.f;
      if (p.mask) {
        u32x2 m;
        m[0] = (keep & 1u) | (keep >> 1 & 1u) << 8 | (keep >> 2 & 1u) << 16 | (keep >> 3 & 1u) << 24;
        m[1] = (keep >> 4 & 1u) | (keep >> 5 & 1u) << 8 | (keep >> 6 & 1u) << 16 | (keep >> 7 & 1u) << 24;
        *(u32x2*)(p.mask + (uint64_t)p.rows * H + e0) = m;
      }
    }
    if (p.res) {
      unpack8<BF16>(ld16(R + 8 * c), f);
#pragma unroll
      for (int j = 0; j < 8; ++j) z[k][j] += f[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += z[k][j];
  }

  const float inv_h = 1.f / (float)H;
  const float mu = p.rms ? 0.f : row_sum<W>(sum, red, wave) * inv_h;
  float sq = 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int c = part * 64 + lane + 64 * W * k;
    if (!row_ok || c >= chunks) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float t = z[k][j] - mu;
      sq = fmaf(t, t, sq);
    }
  }
  const float rstd = 1.f / sqrtf(row_sum<W>(sq, red, wave) * inv_h + p.eps);
  if (!row_ok) return;  // past the last barrier

  const unsigned short* G0 = (const unsigned short*)p.g0;
  const unsigned short* B0 = (const unsigned short*)p.b0;
  const unsigned short* G1 = (const unsigned short*)p.g1;
  const unsigned short* B1 = (const unsigned short*)p.b1;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int c = part * 64 + lane + 64 * W * k;
    if (c >= chunks) continue;
    float n[8], g[8], b[8], y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) n[j] = (z[k][j] - mu) * rstd;
    unpack8<BF16>(*(const u32x4*)(G0 + 8 * c), g);
    if (B0) {
      unpack8<BF16>(*(const u32x4*)(B0 + 8 * c), b);
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = fmaf(n[j], g[j], b[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = n[j] * g[j];
    }
    st16((unsigned short*)p.y0 + rbase + 8 * c, pack8<BF16>(y));
    if (G1) {
      unpack8<BF16>(*(const u32x4*)(G1 + 8 * c), g);
      if (B1) {
        unpack8<BF16>(*(const u32x4*)(B1 + 8 * c), b);
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = fmaf(n[j], g[j], b[j]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = n[j] * g[j];
      }
      st16((unsigned short*)p.y1 + rbase + 8 * c, pack8<BF16>(y));
    }
    if (p.z) st16((unsigned short*)p.z + rbase + 8 * c, pack8<BF16>(z[k]));
  }
  if (lane == 0 && part == 0) {
    if (p.mean && !p.rms) p.mean[row] = mu;
    if (p.rstd) p.rstd[row] = rstd;
  }
}

template <bool BF16>
const void* pick_norm(int chunks, int& rows_per_block) {
  if (chunks <= 64) { rows_per_block = 4; return (const void*)norm_kernel<BF16, 1, 1>; }
  if (chunks <= 128) { rows_per_block = 4; return (const void*)norm_kernel<BF16, 1, 2>; }
  if (chunks <= 256) { rows_per_block = 4; return (const void*)norm_kernel<BF16, 1, 4>; }
  if (chunks <= 512) { rows_per_block = 2; return (const void*)norm_kernel<BF16, 2, 4>; }
  rows_per_block = 1;
  return (const void*)norm_kernel<BF16, 4, 4>;
}

}  // namespace

hipError_t launch_dropout_add_norm(const NormParams& p, bool bf16, hipStream_t stream) {
  int rpb = 1;
  const int chunks = p.hidden >> 3;
  const void* fn = bf16 ? pick_norm<true>(chunks, rpb) : pick_norm<false>(chunks, rpb);
  const dim3 grid((unsigned)((p.rows + rpb - 1) / rpb));
  const dim3 block(kThreadsN);
  NormParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace fa
