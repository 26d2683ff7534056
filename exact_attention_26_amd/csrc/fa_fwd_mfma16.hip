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
//  * K and V tiles travel HBM -> LDS with global_load_lds_dwordx4 (no
//    staging registers, no LDS write instructions). Both stay row-major in
//    LDS with an XOR swizzle of their columns:
//      K: 16-byte chunk c of row r sits at chunk c ^ kswz(r); a lane reads
//         one 16-byte chunk of one key row per S^T MFMA (ds_read_b128);
//      V: 64-byte chunk c of row r sits at chunk c ^ vswz(r); the P.V
//         operand (8 keys of one d column per lane) is read with the gfx950
//         transposing load ds_read_b64_tr_b16: within each 16-lane block,
//         lane l receives element l%4 of the 4-element vectors loaded by
//         lanes l/4, l/4+4, l/4+8 and l/4+12.
//    Both read patterns are free of LDS bank conflicts.
//  * Two LDS stages: tile j+1 streams into one stage while tile j is
//    computed from the other; one barrier per tile.
//  * O (fp32) lives in MFMA accumulators for the whole loop, one query per
//    lane, so the rescale by alpha is a per-lane scalar multiply, skipped
//    when no lane's running max moved.
#include <type_traits>

#include "fa_device.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
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

typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef short i16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

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

// LDS tile geometry for head dimension D (16-bit elements).
template <int D>
struct Tile {
  static constexpr int ROWB = D * 2;                 // bytes per key row
  static constexpr int TILEB = BC * ROWB;            // bytes per K (or V) tile
  static constexpr int STAGEB = 2 * TILEB;           // K tile + V tile
  static constexpr int ROWS_PER_256 = 256 / ROWB;    // rows sharing one 256-byte bank sweep
  static constexpr int KCHUNKS = ROWB / 16;          // 16-byte chunks per row
  static constexpr int VCHUNKS = ROWB / 64;          // 64-byte chunks per row
  static constexpr int DMA_PER_WAVE = TILEB / 1024 / kWaves;  // 1 KiB copies per wave
  // Rows read together get distinct chunk positions, hence distinct banks.
  __device__ static int kswz(int r) { return (r / ROWS_PER_256) & (KCHUNKS - 1); }
  __device__ static int vswz(int r) { return (r / ROWS_PER_256) & (VCHUNKS - 1); }
};

template <bool BF16, int D, bool VARLEN>
__global__ __launch_bounds__(kThreads, 2) void fwd16_kernel(FwdParams p) {
  using vec8 = typename Elem<BF16>::vec8;
  using T = Tile<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * T::STAGEB];

  WorkUnit u;
  if (!resolve_unit<VARLEN>(p, BR, u)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // Direct-to-LDS copies. Copy r of this wave fills bytes
  // [1024*(wave*NDMA + r), +1024) of the K (and of the V) tile; lane i
  // writes 16 bytes at +16*i, i.e. 16-byte slot s of the tile. Slot s is
  // (row, stored chunk); the lane fetches the logical chunk the swizzle
  // stores there.
  constexpr int NDMA = T::DMA_PER_WAVE;
  int drow[NDMA], kcol[NDMA], vcol[NDMA];
#pragma unroll
  for (int r = 0; r < NDMA; ++r) {
    const int s = (wave * NDMA + r) * 64 + lane;
    const int row = s / T::KCHUNKS;
    const int pos = s % T::KCHUNKS;
    drow[r] = row;
    kcol[r] = (pos ^ T::kswz(row)) * 8;
    vcol[r] = ((((pos >> 2) ^ T::vswz(row)) << 2) | (pos & 3)) * 8;
  }
  // Tile at key kb into LDS stage `stage`. In the ragged last tile (tail)
  // rows past the end are clamped to row n-1: loads stay in bounds and those
  // keys are masked out of the scores.
  auto fetch = [&](int stage, int kb, bool tail) {
    const unsigned short* Kt = Kg + (int64_t)kb * rs;
    const unsigned short* Vt = Vg + (int64_t)kb * rs;
    lds_u8* base = (lds_u8*)lds + stage * T::STAGEB + wave * NDMA * 1024;
    const int last = n - 1 - kb;
#pragma unroll
    for (int r = 0; r < NDMA; ++r) {
      const int row = tail ? min(drow[r], last) : drow[r];
      __builtin_amdgcn_global_load_lds((const void*)(Kt + (row * rs + kcol[r])),
                                       (lds_void*)(base + r * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(Vt + (row * rs + vcol[r])),
                                       (lds_void*)(base + T::TILEB + r * 1024), 16, 0, 0);
    }
  };

  // K fragment (S^T A operand): key row kt*32 + l32, logical chunk 2*ss + g,
  // stored at chunk (2*ss + g) ^ kswz(row); kswz(kt*32 + l32) == kswz(l32).
  const int kx = T::kswz(l32);
  // V fragment (P.V A operand, transposing read): lane j of 16-lane block b
  // points at row 16t + 8h + 4*(b/2) + j/4 and columns 32*dt + 16*(b%2) +
  // 4*(j%4) .. +3, so the lane receives d column 32*dt + l32 of keys
  // 16t + 8h + 4g + 0..3: slots 4h .. 4h+3 of P.V MFMA t.
  const int vj = lane & 15, vb = lane >> 4;
  const int vrow = 4 * (vb >> 1) + (vj >> 2);
  const int vin = 32 * (vb & 1) + 8 * (vj & 3);  // byte offset inside the 64-byte chunk

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
    const lds_u8* Ks = (const lds_u8*)lds + stage * T::STAGEB;
    const lds_u8* Vs = Ks + T::TILEB;

    // S^T tile: two 32-key MFMA tiles; lane holds query l32, keys
    // kt*32 + 8*(i/4) + 4*g + (i%4) in register i.
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

    if constexpr (MASKED) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb + kt * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key >= n) s[kt][i] = -INFINITY;
        }
    }

    // Row max: four independent chains, then one exchange with lane ^ 32.
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
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 pw;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        pw[q] = pack2<BF16>(s[t >> 1][8 * (t & 1) + 2 * q], s[t >> 1][8 * (t & 1) + 2 * q + 1]);
      const vec8 pb = __builtin_bit_cast(vec8, pw);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        i16x4 hv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = 16 * t + 8 * h + vrow;
          hv[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(Vs + row * T::ROWB + ((dt ^ T::vswz(row)) << 6) + vin));
        }
        const i16x8 a8 = {hv[0][0], hv[0][1], hv[0][2], hv[0][3],
                          hv[1][0], hv[1][1], hv[1][2], hv[1][3]};
        o[dt] = mfma32x32x16<BF16>(__builtin_bit_cast(vec8, a8), pb, o[dt]);
      }
    }
  };

  const int nfull = n / BC;  // tiles with all BC keys valid
  const int tiles = (n + BC - 1) / BC;
  fetch(0, 0, nfull == 0);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int j = 0; j < nfull; ++j) {
    if (j + 1 < tiles) fetch((j + 1) & 1, (j + 1) * BC, j + 1 == nfull);
    step(std::false_type{}, j & 1, j * BC);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
