// FlashAttention-2 forward for fp32 storage on gfx950 (MI355X).
//
// Same method and work decomposition as the 16-bit kernel ("Kernel
// visualization: Flash Attention 2": one workgroup per block of query
// rows, K/V tiles streamed through on-chip memory, running max / sum /
// unnormalised output, one division at write-back, L = m + ln l), on the
// fp32 matrix cores: v_mfma_f32_32x32x2f32 with fp32 products and fp32
// accumulation. The pages' kernel is fp32 throughout; this path keeps it so.
//
//  * 4 waves x 32 query rows = 128 rows per workgroup; key tiles of 32.
//  * S^T = K Q^T: one query per lane, 16 keys per lane, so the row max and
//    sum are in-lane reductions plus one exchange with lane ^ 32.
//  * Each lane holds one element per MFMA operand, so P (fp32) goes from
//    the S^T accumulator register straight into the P.V MFMA and V is read
//    from LDS in its natural row-major order.
//  * K rows are padded by one float in LDS (conflict-free column reads),
//    V rows by four floats; two LDS stages, one barrier per tile.
#include "fa_fwd_unit.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int BR = kRowsPerBlockF32;
constexpr int BC = 32;

// Combine a lane's value with that of lane l ^ 32. v_permlane32_swap
// exchanges the two half-waves in one VALU instruction (no LDS crossbar);
// of its two results one is the lane's own value and the other its
// partner's, in an order that depends on the half, so both are combined.
__device__ __forceinline__ float halves_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

template <int D, bool VARLEN>
__global__ __launch_bounds__(kThreads, 2) void fwd_f32_kernel(FwdParams p) {
  constexpr int KSTR = D + 1;
  constexpr int VSTR = D + 4;
  constexpr int KT = BC * KSTR;
  constexpr int VT = BC * VSTR;
  constexpr int STAGE = KT + VT;
  __shared__ __attribute__((aligned(16))) float lds[2 * STAGE];

  WorkUnit u;
  if (!resolve_unit<VARLEN>(p, BR, u)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int n = u.n;
  const int rs = p.row_stride;

  const float* __restrict__ Qg = (const float*)p.q + u.base;
  const float* __restrict__ Kg = (const float*)p.k + u.base;
  const float* __restrict__ Vg = (const float*)p.v + u.base;
  float* __restrict__ Og = (float*)p.o + u.base;

  // Q fragment: element 2s + g of query row qrow, for s = 0 .. D/2-1.
  const int qrow = u.q0 + wave * 32 + l32;
  float qf[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; ++s) qf[s] = (qrow < n) ? Qg[(int64_t)qrow * rs + 2 * s + g] : 0.f;

  constexpr int CPR = D / 4;               // 16-byte chunks per row
  constexpr int NCH = BC * CPR / kThreads;  // chunks per thread per tensor
  f32x4 kr[NCH], vr[NCH];

  auto fetch = [&](int kb) {
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      const int c = tid + kThreads * r;
      const int key = kb + c / CPR;
      const int col = (c % CPR) * 4;
      f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
      if (key < n) {
        a = *(const f32x4*)(Kg + (int64_t)key * rs + col);
        b = *(const f32x4*)(Vg + (int64_t)key * rs + col);
      }
      kr[r] = a;
      vr[r] = b;
    }
  };
  auto stash = [&](int stage) {
    float* Ks = lds + stage * STAGE;
    float* Vs = Ks + KT;
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      const int c = tid + kThreads * r;
      const int key = c / CPR;
      const int col = (c % CPR) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) Ks[key * KSTR + col + e] = kr[r][e];
      *(f32x4*)(Vs + key * VSTR + col) = vr[r];
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  float m = -INFINITY;
  float l = 0.f;
  const float c2 = p.scale_log2;

  const int tiles = (n + BC - 1) / BC;
  fetch(0);
  stash(0);
  __syncthreads();

  for (int j = 0; j < tiles; ++j) {
    const int kb = j * BC;
    const bool more = (j + 1) < tiles;
    if (more) fetch(kb + BC);

    const float* Ks = lds + (j & 1) * STAGE;
    const float* Vs = Ks + KT;

    // S^T: register i of lane (l32, g) holds key 8*(i/4) + 4g + i%4, query l32.
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ss = 0; ss < D / 2; ++ss)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[l32 * KSTR + 2 * ss + g], qf[ss], s, 0, 0, 0);

    if (kb + BC > n) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb + 8 * (i >> 2) + 4 * g + (i & 3) >= n) s[i] = -INFINITY;
    }

    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = halves_max(mx);
    const float mnew = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - mnew) * c2);
    const float mc = mnew * c2;
    float rsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -mc));
      s[i] = e;
      rsum += e;
    }
    l = l * alpha + rsum;
    m = mnew;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[t][i] *= alpha;

    // O^T += V^T P^T: MFMA t pairs key 8*(t/4) + 4g + t%4 (register t).
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int key = 8 * (t >> 2) + 4 * g + (t & 3);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * VSTR + dt * 32 + l32], s[t], o[dt],
                                                     0, 0, 0);
    }

    if (more) stash((j + 1) & 1);
    __syncthreads();
  }

  l = halves_sum(l);
  if (qrow < n) {
    const float inv = 1.f / l;
    float* orow = Og + (int64_t)qrow * rs;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = o[dt][4 * blk + e] * inv;
        *(f32x4*)(orow + dt * 32 + 8 * blk + 4 * g) = w;
      }
    if (g == 0) p.lse[u.lse_base + qrow] = m * p.scale + logf(l);
  }
}


// Key-split form for small problems. With 128-row workgroups a single head
// of a few hundred rows gives the chip one or two workgroups, so a handful
// of SIMDs do all the work. Here a workgroup owns 32 query rows and NS
// waves; wave w streams key tiles w, w + NS, w + 2 NS, ... of the head with
// its own running max, sum and unnormalised output (the online update of
// "Kernel visualization: Flash Attention 2", "Iteration j = 1", on its share
// of the keys). The NS partial states are then merged once through LDS: each
// is brought to the rows' overall max by exp(m_w - m) and summed, the exact
// combine of partial softmax states ("FlashAttention -- for programmers, not
// researchers", STAGE 3), and O and L are written as in the 128-row kernel.
//
// Each wave stages its own K/V tile in a private LDS region, so the key loop
// needs no workgroup barrier: LDS instructions of one wave execute in order,
// so its reads see its own writes, and the next tile's writes follow the
// last reads of the previous one.
template <int D>
__global__ __launch_bounds__(64 * f32_key_split(D)) void fwd_f32_split_kernel(FwdParams p) {
  constexpr int NS = f32_key_split(D);
  constexpr int KSTR = D + 1;
  constexpr int VSTR = D + 4;
  constexpr int KT = BC * KSTR;
  constexpr int VT = BC * VSTR;
  constexpr int REG = KT + VT;  // floats per wave region
  // Merge area, aliasing the regions after a barrier: per wave 32 rows of
  // O (row stride D + 4) followed by m[32] and l[32].
  constexpr int MSTR = D + 4;
  constexpr int MREG = 32 * MSTR + 64;
  static_assert(MREG <= REG, "merge area fits a wave's region");
  static_assert(NS * REG * 4 <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) float lds[NS * REG];

  WorkUnit u;
  if (!resolve_unit<false>(p, kRowsPerBlockF32Split, u)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int n = u.n;
  const int rs = p.row_stride;

  const float* __restrict__ Qg = (const float*)p.q + u.base;
  const float* __restrict__ Kg = (const float*)p.k + u.base;
  const float* __restrict__ Vg = (const float*)p.v + u.base;
  float* __restrict__ Og = (float*)p.o + u.base;

  const int qrow = u.q0 + l32;
  float qf[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; ++s) qf[s] = (qrow < n) ? Qg[(int64_t)qrow * rs + 2 * s + g] : 0.f;

  float* Ks = lds + wave * REG;
  float* Vs = Ks + KT;
  constexpr int CPR = D / 4;            // 16-byte chunks per row
  constexpr int NCH = BC * CPR / 64;    // chunks per lane per tensor

  f32x16 o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  float m = -INFINITY;
  float l = 0.f;
  const float c2 = p.scale_log2;
  const int tiles = (n + BC - 1) / BC;

  for (int j = wave; j < tiles; j += NS) {
    const int kb = j * BC;
    f32x4 kr[NCH], vr[NCH];
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      const int c = lane + 64 * r;
      const int key = kb + c / CPR;
      const int col = (c % CPR) * 4;
      f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
      if (key < n) {
        a = *(const f32x4*)(Kg + (int64_t)key * rs + col);
        b = *(const f32x4*)(Vg + (int64_t)key * rs + col);
      }
      kr[r] = a;
      vr[r] = b;
    }
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      const int c = lane + 64 * r;
      const int key = c / CPR;
      const int col = (c % CPR) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) Ks[key * KSTR + col + e] = kr[r][e];
      *(f32x4*)(Vs + key * VSTR + col) = vr[r];
    }

    // S^T: register i of lane (l32, g) holds key 8*(i/4) + 4g + i%4, query l32.
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ss = 0; ss < D / 2; ++ss)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[l32 * KSTR + 2 * ss + g], qf[ss], s, 0, 0, 0);
    if (kb + BC > n) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb + 8 * (i >> 2) + 4 * g + (i & 3) >= n) s[i] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = halves_max(mx);
    const float mnew = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - mnew) * c2);
    const float mc = mnew * c2;
    float rsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -mc));
      s[i] = e;
      rsum += e;
    }
    l = l * alpha + rsum;
    m = mnew;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int key = 8 * (t >> 2) + 4 * g + (t & 3);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * VSTR + dt * 32 + l32], s[t], o[dt],
                                                     0, 0, 0);
    }
  }
  l = halves_sum(l);

  // Merge. A wave with no tile (fewer tiles than waves) holds m = -inf,
  // l = 0 and O = 0, which weigh exp2(-inf) = 0; wave 0 always holds tile 0,
  // so every row's overall max is finite.
  __syncthreads();  // every wave is done with its K/V region
  {
    float* mw = lds + wave * MREG;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = o[dt][4 * blk + e];
        *(f32x4*)(mw + l32 * MSTR + dt * 32 + 8 * blk + 4 * g) = w;
      }
    if (g == 0) {
      mw[32 * MSTR + l32] = m;
      mw[32 * MSTR + 32 + l32] = l;
    }
  }
  __syncthreads();
  constexpr int CH = 32 * D / (64 * NS);  // output floats per thread
  static_assert(CH % 4 == 0 && D % CH == 0, "whole 16-byte chunks of one row per thread");
  constexpr int TPR = D / CH;             // threads per row
  const int r = tid / TPR;
  const int c0 = (tid % TPR) * CH;
  float mall = -INFINITY;
#pragma unroll
  for (int w = 0; w < NS; ++w) mall = fmaxf(mall, lds[w * MREG + 32 * MSTR + r]);
  float wt[NS];
  float lsum = 0.f;
#pragma unroll
  for (int w = 0; w < NS; ++w) {
    wt[w] = __builtin_amdgcn_exp2f((lds[w * MREG + 32 * MSTR + r] - mall) * c2);
    lsum += lds[w * MREG + 32 * MSTR + 32 + r] * wt[w];
  }
  const float inv = 1.f / lsum;
  const int row = u.q0 + r;
  if (row < n) {
#pragma unroll
    for (int c = 0; c < CH; c += 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NS; ++w) {
        const f32x4 x = *(const f32x4*)(lds + w * MREG + r * MSTR + c0 + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(x[e], wt[w], acc[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] *= inv;
      *(f32x4*)(Og + (int64_t)row * rs + c0 + c) = acc;
    }
    if (c0 == 0) p.lse[u.lse_base + row] = mall * p.scale + logf(lsum);
  }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, int d, bool varlen, hipStream_t stream) {
  if (p.key_split > 0) {
    const void* fn = d == 64 ? (const void*)fwd_f32_split_kernel<64>
                             : (const void*)fwd_f32_split_kernel<128>;
    const dim3 grid((unsigned)fwd_grid(p));
    const dim3 block(64 * f32_key_split(d));
    FwdParams arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
  }
  const void* fn;
  if (d == 64)
    fn = varlen ? (const void*)fwd_f32_kernel<64, true> : (const void*)fwd_f32_kernel<64, false>;
  else
    fn = varlen ? (const void*)fwd_f32_kernel<128, true> : (const void*)fwd_f32_kernel<128, false>;
  const dim3 grid((unsigned)fwd_grid(p));
  const dim3 block(kThreads);
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace fa
