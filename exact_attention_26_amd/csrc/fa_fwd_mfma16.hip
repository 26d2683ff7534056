// FlashAttention-2 forward for bf16 / fp16 storage on gfx950 (MI355X).
//
// The method ("Kernel visualization: Flash Attention 2", sections "Steps"
// through "Write the data back to HBM"): one workgroup owns a block of
// query rows from start to finish; it streams K/V tiles, computes the score
// tile S = scale * Qi Kj^T, updates the per-row running max m, running sum
// l and unnormalised output O (rescaling both by exp(m_old - m_new) when the
// max moves), divides by l once at the end and writes O and L = m + ln l.
// Scores never leave the chip.
//
// How it maps onto CDNA4:
//  * 256 threads = 4 waves; each wave owns 32 query rows, so a workgroup
//    owns Br = 128 rows. Keys are streamed in tiles of Bc = 64.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_{bf16,f16}: the accumulator puts one query per
//    lane (column n = lane % 32) and 16 keys per lane, so the row max and
//    row sum are in-lane reductions plus one exchange with lane ^ 32.
//  * Q stays in VGPRs for the whole loop as the B operand of S^T.
//  * P = exp2(S*c - m*c) (c = scale*log2 e) is rounded to the storage dtype
//    and fed from the S^T accumulator registers straight into the P.V
//    MFMA as its B operand (O^T = V^T P^T): no LDS round trip for P.
//  * K tiles sit in LDS row-major (row padded by 16 bytes against bank
//    conflicts); V tiles are written to LDS transposed, V^T[d][key], with
//    the keys of each 16-key group permuted so that the 8 keys one lane
//    needs for a P.V MFMA are contiguous (one 16-byte LDS read).
//  * Two LDS stages: tile j+1 is fetched from HBM into registers while tile
//    j is computed, then written to the other stage; one barrier per tile.
//  * O (fp32) lives in MFMA accumulators for the whole loop, one query per
//    lane, so the rescale by alpha is a per-lane scalar multiply.
#include <type_traits>

#include "fa_device.h"

// Optionally raise the wave priority around MFMA bursts (s_setprio). Off by
// default: with two waves per SIMD it measured no faster on MI355X.
#ifndef FA_SETPRIO
#define FA_SETPRIO 0
#endif
#if FA_SETPRIO
#define FA_PRIO_HI() __builtin_amdgcn_s_setprio(1)
#define FA_PRIO_LO() __builtin_amdgcn_s_setprio(0)
#else
#define FA_PRIO_HI()
#define FA_PRIO_LO()
#endif

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int BR = kRowsPerBlock16;  // query rows per workgroup (32 per wave)
constexpr int BC = 64;               // keys per tile

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
  using vec8 = bf16x8;
};
template <>
struct Elem<false> {
  using vec8 = f16x8;
};

template <bool BF16>
__device__ __forceinline__ f32x16 mfma32x32x16(typename Elem<BF16>::vec8 a,
                                               typename Elem<BF16>::vec8 b, f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Two fp32 values -> two 16-bit values of the storage dtype (round to
// nearest even), packed low-first into one dword.
template <bool BF16>
__device__ __forceinline__ unsigned pack2(float a, float b) {
  if constexpr (BF16) {
    typedef __bf16 v2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
    v2 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return __builtin_bit_cast(unsigned, r);
  } else {
    typedef _Float16 v2 __attribute__((__vector_size__(2 * sizeof(_Float16))));
    v2 r;
    r[0] = (_Float16)a;
    r[1] = (_Float16)b;
    return __builtin_bit_cast(unsigned, r);
  }
}

template <int C>
struct VChunk;
template <>
struct VChunk<8> {
  using type = u32x4;
};
template <>
struct VChunk<4> {
  using type = u32x2;
};

template <typename T>
__device__ __forceinline__ unsigned half16(const T& v, int c) {
  const unsigned w = v[c >> 1];
  return (c & 1) ? (w >> 16) : (w & 0xffffu);
}

template <bool BF16, int D, bool VARLEN>
__global__ __launch_bounds__(kThreads, 2) void fwd16_kernel(FwdParams p) {
  using vec8 = typename Elem<BF16>::vec8;
  constexpr int KSTR = D + 8;   // 16-bit elements per K row in LDS
  constexpr int VSTR = BC + 8;  // 16-bit elements per V^T row in LDS
  constexpr int KT = BC * KSTR;
  constexpr int VT = D * VSTR;
  constexpr int STAGE = KT + VT;
  __shared__ __attribute__((aligned(16))) unsigned short lds[2 * STAGE];

  WorkUnit u;
  if (!resolve_unit<VARLEN>(p, BR, u)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int n = u.n;
  const int rs = p.row_stride;

  const unsigned short* __restrict__ Qg = (const unsigned short*)p.q + u.base;
  const unsigned short* __restrict__ Kg = (const unsigned short*)p.k + u.base;
  const unsigned short* __restrict__ Vg = (const unsigned short*)p.v + u.base;
  unsigned short* __restrict__ Og = (unsigned short*)p.o + u.base;

  // Q fragment of this lane: query row qrow, elements 16s + 8g .. 16s + 8g + 7.
  const int qrow = u.q0 + wave * 32 + l32;
  vec8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qrow < n) w = *(const u32x4*)(Qg + qrow * rs + 16 * s + 8 * g);
    qf[s] = __builtin_bit_cast(vec8, w);
  }

  // Tile fetch assignments. K: 16-byte chunks, row-major. V: each thread
  // owns 4 consecutive keys x VC columns, which it writes transposed.
  constexpr int CPR = D / 8;                 // 16-byte chunks per K row
  constexpr int KCH = BC * CPR / kThreads;   // K chunks per thread
  constexpr int VC = D / 16;                 // V columns per thread
  using vchunk = typename VChunk<VC>::type;
  // The 16 lanes that share an LDS write pass hold the 16 key groups of one
  // column group, so each transposed ds_write_b64 pass fills one 128-byte
  // V^T row segment: no bank conflicts.
  const int vkg = tid & 15;   // V key group: keys 4*vkg .. 4*vkg+3
  const int vcg = tid >> 4;   // V column group
  // Position of key 4*vkg in the permuted V^T row: key 16t+8h+4q+r is stored
  // at 16t+8q+4h+r, so lane group q of a P.V MFMA reads 8 contiguous keys.
  const int vpos = ((4 * vkg) & ~15) | (((4 * vkg) & 4) << 1) | (((4 * vkg) & 8) >> 1);
  int krow[KCH], kcol[KCH];
#pragma unroll
  for (int r = 0; r < KCH; ++r) {
    krow[r] = (tid + kThreads * r) / CPR;
    kcol[r] = ((tid + kThreads * r) % CPR) * 8;
  }

  u32x4 kr[KCH];
  vchunk vr[4];

  // Global -> registers for the tile starting at key kb. In the ragged last
  // tile (tail) rows past the end are clamped to row n-1: the loads stay in
  // bounds and those keys are masked out of the scores.
  auto fetch = [&](int kb, bool tail) {
    const unsigned short* Kt = Kg + (int64_t)kb * rs;
    const unsigned short* Vt = Vg + (int64_t)kb * rs;
    if (!tail) {
#pragma unroll
      for (int r = 0; r < KCH; ++r) kr[r] = *(const u32x4*)(Kt + (krow[r] * rs + kcol[r]));
#pragma unroll
      for (int r = 0; r < 4; ++r) vr[r] = *(const vchunk*)(Vt + ((4 * vkg + r) * rs + vcg * VC));
    } else {
      const int last = n - 1 - kb;
#pragma unroll
      for (int r = 0; r < KCH; ++r)
        kr[r] = *(const u32x4*)(Kt + (min(krow[r], last) * rs + kcol[r]));
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vr[r] = *(const vchunk*)(Vt + (min(4 * vkg + r, last) * rs + vcg * VC));
    }
  };
  auto stash = [&](int stage) {
    unsigned short* Ks = lds + stage * STAGE;
    unsigned short* Vs = Ks + KT;
#pragma unroll
    for (int r = 0; r < KCH; ++r) *(u32x4*)(Ks + krow[r] * KSTR + kcol[r]) = kr[r];
#pragma unroll
    for (int c = 0; c < VC; ++c) {
      u32x2 w;
      w[0] = half16(vr[0], c) | (half16(vr[1], c) << 16);
      w[1] = half16(vr[2], c) | (half16(vr[3], c) << 16);
      *(u32x2*)(Vs + (vcg * VC + c) * VSTR + vpos) = w;
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  float m = -INFINITY;  // running max of raw q.k (scale > 0)
  float l = 0.f;        // running sum of this lane's half of the keys
  const float c2 = p.scale_log2;

  // One key tile: scores, online softmax update, P.V. MASKED marks the
  // ragged last tile (keys >= n get probability 0).
  auto step = [&](auto masked, int stage, int kb) {
    constexpr bool MASKED = decltype(masked)::value;
    const unsigned short* Ks = lds + stage * STAGE;
    const unsigned short* Vs = Ks + KT;

    // S^T tile: two 32-key MFMA tiles; lane holds query l32, keys
    // kt*32 + 8*(i/4) + 4*g + (i%4) in register i.
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
    FA_PRIO_HI();
#pragma unroll
    for (int ss = 0; ss < D / 16; ++ss)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const vec8 a = *(const vec8*)(Ks + (kt * 32 + l32) * KSTR + 16 * ss + 8 * g);
        s[kt] = mfma32x32x16<BF16>(a, qf[ss], s[kt]);
      }
    FA_PRIO_LO();

    if constexpr (MASKED) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb + kt * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key >= n) s[kt][i] = -INFINITY;
        }
    }

    // Row max: four independent max3 chains, then one exchange with lane ^ 32.
    float mq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x16& a = s[q >> 1];
      const int b = 8 * (q & 1);
      mq[q] = fmaxf(fmaxf(fmaxf(a[b + 0], a[b + 1]), fmaxf(a[b + 2], a[b + 3])),
                    fmaxf(fmaxf(a[b + 4], a[b + 5]), fmaxf(a[b + 6], a[b + 7])));
    }
    float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    const bool grew = mnew > m;
    const float alpha = grew ? __builtin_amdgcn_exp2f((m - mnew) * c2) : 1.f;
    const float mc = mnew * c2;
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[kt][i], c2, -mc));
        s[kt][i] = e;
        ls[i & 3] += e;
      }
    l = l * alpha + ((ls[0] + ls[1]) + (ls[2] + ls[3]));
    m = mnew;
    // Rescale the running output only if some lane's max moved (alpha != 1).
    if (__any(grew)) {
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
    }

    // O^T += V^T P^T over the 64 keys, 16 keys per MFMA. Slot jj of lane
    // group g in MFMA t is key 16t + 8*(jj/4) + 4g + jj%4, which is S^T
    // register 8*(t%2) + jj of key tile t/2.
    vec8 pb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 pw;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        pw[q] = pack2<BF16>(s[t >> 1][8 * (t & 1) + 2 * q], s[t >> 1][8 * (t & 1) + 2 * q + 1]);
      pb[t] = __builtin_bit_cast(vec8, pw);
    }
    FA_PRIO_HI();
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const vec8 a = *(const vec8*)(Vs + (dt * 32 + l32) * VSTR + 16 * t + 8 * g);
        o[dt] = mfma32x32x16<BF16>(a, pb[t], o[dt]);
      }
    FA_PRIO_LO();
  };

  const int nfull = n / BC;                  // tiles with all BC keys valid
  const int tiles = (n + BC - 1) / BC;
  fetch(0, nfull == 0);
  stash(0);
  __syncthreads();
  for (int j = 0; j < nfull; ++j) {
    const bool more = (j + 1) < tiles;
    if (more) fetch((j + 1) * BC, j + 1 == nfull);
    step(std::false_type{}, j & 1, j * BC);
    if (more) stash((j + 1) & 1);
    __syncthreads();
  }
  if (nfull < tiles) step(std::true_type{}, nfull & 1, nfull * BC);

  // Write-back: divide once by l, L = m*scale + ln l.
  l += __shfl_xor(l, 32);
  if (qrow < n) {
    const float inv = 1.f / l;
    unsigned short* orow = Og + qrow * rs;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        u32x2 w;
        w[0] = pack2<BF16>(o[dt][4 * blk + 0] * inv, o[dt][4 * blk + 1] * inv);
        w[1] = pack2<BF16>(o[dt][4 * blk + 2] * inv, o[dt][4 * blk + 3] * inv);
        *(u32x2*)(orow + dt * 32 + 8 * blk + 4 * g) = w;
      }
    if (g == 0) p.lse[u.lse_base + qrow] = m * p.scale + logf(l);
  }
}

template <bool BF16, int D>
const void* pick(bool varlen) {
  return varlen ? (const void*)fwd16_kernel<BF16, D, true>
                : (const void*)fwd16_kernel<BF16, D, false>;
}

}  // namespace

hipError_t launch_fwd_mfma16(const FwdParams& p, int d, bool bf16, bool varlen,
                             hipStream_t stream) {
  const void* fn = nullptr;
  if (bf16)
    fn = (d == 64) ? pick<true, 64>(varlen) : pick<true, 128>(varlen);
  else
    fn = (d == 64) ? pick<false, 64>(varlen) : pick<false, 128>(varlen);
  const dim3 grid((unsigned)((int64_t)p.q_blocks * p.H * p.B));
  const dim3 block(kThreads);
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace fa
