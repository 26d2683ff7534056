// Attention forward in the K/V-outer loop order, for bf16 / fp16 storage on
// gfx950: the traffic experiment beside the Q-outer (FlashAttention-2)
// kernel.
//
// Why it exists. "Kernel visualization: Flash Attention 2" ("Counting trips
// across HBM") credits the Q-outer order with keeping each query block's
// running output O and statistics m, l on chip from start to finish, so that
// they are written once and never read back. This kernel runs the other
// order, with the key/value tiles on the outer loop: for every tile, each
// query row reads Q, reads back its running O (fp32), m and l from HBM,
// applies the same online-softmax update ("FlashAttention -- for
// programmers, not researchers", STAGE 3-4), and writes them out again; the
// last tile writes the final O / l and L = m + ln l instead. It computes the
// same function as the Q-outer kernel; only the traffic differs, which
// rocprof's byte counters then show.
//
// Mapping. A workgroup (4 waves) owns one (batch, head) and one group of
// query rows (a multiple of 32); the groups of a head are consecutive
// logical ids, kept on one XCD by xcd_remap so they share the K/V tiles in
// its L2. For each 64-key tile the workgroup stages K and V in LDS (the same
// XOR-swizzled layout and transposing V reads as the Q-outer kernel), then
// every wave walks its 32-row query blocks: S^T = K Q^T and O^T += V^T P^T on
// v_mfma_f32_32x32x16, one query per lane. The softmax is the exact online
// update (row max every tile).
#include "fa_device.h"
#include "fa_kvouter_params.h"

namespace fa {
namespace {

constexpr int kWavesKV = 4;
constexpr int kThreadsKV = 64 * kWavesKV;
constexpr int BCK = 64;  // keys per tile

// LDS layout of one K (or V) tile of BCK rows for head dimension D.
template <int D>
struct KvLayout {
  static constexpr int ROWB = D * 2;
  static constexpr int TILEB = BCK * ROWB;
  static constexpr int ROWS_PER_256 = 256 / ROWB;
  static constexpr int KCHUNKS = ROWB / 16;
  static constexpr int VCHUNKS = ROWB / 64;
  __device__ static int kswz(int r) { return (r / ROWS_PER_256) & (KCHUNKS - 1); }
  __device__ static int vswz(int r) { return (r / ROWS_PER_256) & (VCHUNKS - 1); }
};

template <bool BF16, int D>
__global__ __launch_bounds__(kThreadsKV, 2) void kvouter_kernel(KvOuterParams p) {
  using vec8 = typename Elem<BF16>::vec8;
  using T = KvLayout<D>;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * T::TILEB];

  const int id = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int bh = id / p.groups;
  const int grp = id % p.groups;
  const int n = p.N;
  const int r_begin = grp * p.rows_per_group;
  const int r_end = min(n, r_begin + p.rows_per_group);
  if (r_begin >= n) return;  // uniform over the workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int64_t base = (int64_t)bh * p.head_stride;
  const unsigned short* __restrict__ Qg = (const unsigned short*)p.q + base;
  const unsigned short* __restrict__ Kg = (const unsigned short*)p.k + base;
  const unsigned short* __restrict__ Vg = (const unsigned short*)p.v + base;
  unsigned short* __restrict__ Og = (unsigned short*)p.o + base;
  float* __restrict__ Acc = p.oacc + base;
  float* __restrict__ Ms = p.mstat + (int64_t)bh * n;
  float* __restrict__ Ls = p.lstat + (int64_t)bh * n;
  float* __restrict__ Lse = p.lse + (int64_t)bh * n;
  const float c2 = p.scale_log2;

  const int kx = T::kswz(l32);
  const int vj = lane & 15, vb = lane >> 4;
  const int vrow = 4 * (vb >> 1) + (vj >> 2);
  const int vin = 32 * (vb & 1) + 8 * (vj & 3);

  for (int j = 0; j < p.tiles; ++j) {
    const int kb = j * BCK;
    __syncthreads();  // the previous tile's LDS reads are done
    // Stage K_j and V_j; rows past the end are clamped to row n-1 (masked).
    for (int c = tid; c < BCK * T::KCHUNKS; c += kThreadsKV) {
      const int row = c / T::KCHUNKS, pos = c % T::KCHUNKS;
      const int key = min(kb + row, n - 1);
      const u32x4 kv = *(const u32x4*)(Kg + (int64_t)key * D + pos * 8);
      const u32x4 vv = *(const u32x4*)(Vg + (int64_t)key * D + pos * 8);
      *(lds_u32x4*)((lds_u8*)lds + row * T::ROWB + ((pos ^ T::kswz(row)) << 4)) = kv;
      const int vpos = (((pos >> 2) ^ T::vswz(row)) << 2) | (pos & 3);
      *(lds_u32x4*)((lds_u8*)lds + T::TILEB + row * T::ROWB + (vpos << 4)) = vv;
    }
    __syncthreads();
    const bool last = j == p.tiles - 1;
    const bool ragged = kb + BCK > n;
    const lds_u8* Ks = (const lds_u8*)lds;
    const lds_u8* Vs = (const lds_u8*)lds + T::TILEB;

    for (int r0 = r_begin + wave * 32; r0 < r_end; r0 += 32 * kWavesKV) {
      const int qrow = r0 + l32;
      const bool valid = qrow < r_end;
      vec8 qf[D / 16];
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (valid) w = *(const u32x4*)(Qg + (int64_t)qrow * D + 16 * s + 8 * g);
        qf[s] = __builtin_bit_cast(vec8, w);
      }
      // Carries: O^T (d = 32*dt + 8*(i/4) + 4g + i%4, query l32), m, and this
      // lane's half of l (the whole l is kept in lane g = 0's half).
      f32x16 o[D / 32];
      float m = -INFINITY, l = 0.f;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
      if (j > 0 && valid) {
        const float* arow = Acc + (int64_t)qrow * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) {
            const f32x4 a = *(const f32x4*)(arow + 32 * dt + 8 * blk + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[dt][4 * blk + e] = a[e];
          }
        m = Ms[qrow];
        l = g == 0 ? Ls[qrow] : 0.f;
      }
      // S^T of this tile: keys kt*32 + 8*(i/4) + 4g + i%4 in register i of s[kt].
      f32x16 s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
      for (int ss = 0; ss < D / 16; ++ss)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const vec8 a = *(const __attribute__((address_space(3))) vec8*)(
              Ks + (kt * 32 + l32) * T::ROWB + (((2 * ss + g) ^ kx) << 4));
          s[kt] = mfma32x32x16<BF16>(a, qf[ss], s[kt]);
        }
      if (ragged) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kb + kt * 32 + 8 * (i >> 2) + 4 * g + (i & 3) >= n) s[kt][i] = -INFINITY;
      }
      // Online update: new row max, rescale of the carried O and l, p.
      float mx = s[0][0];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                         __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float mnew = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f((m - mnew) * c2);  // 0 when m = -inf
      const float mc = mnew * c2;
      float lsum = 0.f;
      vec8 pb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        u32x4 pw;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i0 = 8 * (t & 1) + 2 * q;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[t >> 1][i0], c2, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[t >> 1][i0 + 1], c2, -mc));
          lsum += p0 + p1;
          pw[q] = pack2<BF16>(p0, p1);
        }
        pb[t] = __builtin_bit_cast(vec8, pw);
      }
      l = l * alpha + lsum;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
      // O^T += V^T P^T: lane gets d column 32*dt + l32 of keys 16t + 8h + 4g + 0..3.
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          i16x4 va[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int row = 16 * t + 8 * h + vrow;
            va[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(Vs + row * T::ROWB + ((dt ^ T::vswz(row)) << 6) + vin));
          }
          const i16x8 a8 = {va[0][0], va[0][1], va[0][2], va[0][3],
                            va[1][0], va[1][1], va[1][2], va[1][3]};
          o[dt] = mfma32x32x16<BF16>(__builtin_bit_cast(vec8, a8), pb[t], o[dt]);
        }
      {  // whole l of the row: add the partner half-wave's part
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l),
                                                         false, false);
        l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      if (!valid) continue;
      if (!last) {  // carry to HBM: O^T (fp32), m, l
        float* arow = Acc + (int64_t)qrow * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) {
            f32x4 a;
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = o[dt][4 * blk + e];
            *(f32x4*)(arow + 32 * dt + 8 * blk + 4 * g) = a;
          }
        if (g == 0) {
          Ms[qrow] = mnew;
          Ls[qrow] = l;
        }
      } else {  // final: O / l in the storage dtype, L = m*scale + ln l
        const float inv = 1.f / l;
        unsigned short* orow = Og + (int64_t)qrow * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) {
            u32x2 w;
            w[0] = pack2<BF16>(o[dt][4 * blk + 0] * inv, o[dt][4 * blk + 1] * inv);
            w[1] = pack2<BF16>(o[dt][4 * blk + 2] * inv, o[dt][4 * blk + 3] * inv);
            *(u32x2*)(orow + dt * 32 + 8 * blk + 4 * g) = w;
          }
        if (g == 0) Lse[qrow] = mnew * p.scale + logf(l);
      }
    }
  }
}

}  // namespace

hipError_t launch_fwd_kv_outer(const KvOuterParams& p, int d, bool bf16, hipStream_t stream) {
  const void* fn;
  if (bf16)
    fn = d == 64 ? (const void*)kvouter_kernel<true, 64> : (const void*)kvouter_kernel<true, 128>;
  else
    fn = d == 64 ? (const void*)kvouter_kernel<false, 64> : (const void*)kvouter_kernel<false, 128>;
  const dim3 grid((unsigned)((int64_t)p.BH * p.groups));
  const dim3 block(kThreadsKV);
  KvOuterParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace fa
