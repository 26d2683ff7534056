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
//  * 512 threads = 8 waves (2 per SIMD); each wave owns 32 query rows, so a
//    workgroup owns Br = 256 rows and re-reads K/V once per 256 queries.
//    Keys are streamed in tiles of Bc = 64.
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

// Build options (defaults are the shipped configuration):
//   FA_MFMA_ROWSUM_D64 (0): at d = 64 run the row sums on the matrix cores
//     (a ones-operand MFMA per 16 keys) instead of VALU adds; at d = 128 the
//     extra accumulator does not fit the register budget of 2 waves/SIMD.
//   FA_RESCALE_TAU (0): the running max moves (and O, l are rescaled) when
//     some row's max grew by more than TAU in log2 units of probability; 0 is
//     the method as written (every increase). TAU > 0 defers small rescales
//     (same function, fewer multiplies); it is an experiment, off by default.
#ifndef FA_MFMA_ROWSUM_D64
#define FA_MFMA_ROWSUM_D64 0
#endif
#ifndef FA_RESCALE_TAU
#define FA_RESCALE_TAU 0
#endif
#ifndef FA_SCHED
#define FA_SCHED 0
#endif
#ifndef FA_SCHED_AH
#define FA_SCHED_AH 4
#endif
#ifndef FA_SCHED_VA
#define FA_SCHED_VA 6
#endif
#ifndef FA_SCHED_VB
#define FA_SCHED_VB 3
#endif

namespace fa {
namespace {

constexpr int kWaves = kWaves16;
constexpr int kThreads = 64 * kWaves;
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
  // Consume Q here so the compiler waits for these loads before the key
  // loop; otherwise it places that wait inside the loop, where it would
  // also stall on the prefetch of the next K/V tile.
#pragma unroll
  for (int s = 0; s < D / 16; ++s) __asm__ volatile("" : : "v"(qf[s]));

  // LDS holds two K stages followed by two V stages. K runs one tile ahead
  // of V: while tile j's P.V reads V stage j%2, the S^T of tile j+1 reads K
  // stage (j+1)%2, and the copies in flight fill K stage j%2 (tile j+2) and
  // V stage (j+1)%2 (tile j+1).
  //
  // Direct-to-LDS copies: copy r of this wave fills bytes
  // [1024*(wave*NDMA + r), +1024) of a tile; lane i writes 16 bytes at
  // +16*i, i.e. 16-byte slot s of the tile. Slot s is (row, stored chunk);
  // the lane fetches the logical chunk the swizzle stores there.
  constexpr int NDMA = T::DMA_PER_WAVE;
  // Row and (logical) column of the 16 bytes copy r of this lane moves.
  auto dma_row = [&](int r) { return ((wave * NDMA + r) * 64 + lane) / T::KCHUNKS; };
  auto dma_kcol = [&](int r) {
    const int s = (wave * NDMA + r) * 64 + lane;
    return ((s % T::KCHUNKS) ^ T::kswz(s / T::KCHUNKS)) * 8;
  };
  auto dma_vcol = [&](int r) {
    const int s = (wave * NDMA + r) * 64 + lane;
    const int pos = s % T::KCHUNKS;
    return ((((pos >> 2) ^ T::vswz(s / T::KCHUNKS)) << 2) | (pos & 3)) * 8;
  };
#if FA_DMA_PRECOMPUTE
  unsigned koffb[NDMA], voffb[NDMA];  // byte offsets inside a full tile
#pragma unroll
  for (int r = 0; r < NDMA; ++r) {
    koffb[r] = (unsigned)(dma_row(r) * rs + dma_kcol(r)) * 2u;
    voffb[r] = (unsigned)(dma_row(r) * rs + dma_vcol(r)) * 2u;
  }
#define FA_KOFF(r) koffb[r]
#define FA_VOFF(r) voffb[r]
#else
#define FA_KOFF(r) ((unsigned)(dma_row(r) * rs + dma_kcol(r)) * 2u)
#define FA_VOFF(r) ((unsigned)(dma_row(r) * rs + dma_vcol(r)) * 2u)
#endif
  const unsigned lds0 = (unsigned)(uintptr_t)(lds_u8*)lds + (unsigned)(wave * NDMA * 1024);
  // Copy the K (or V) tile at key kb into LDS at byte `dst`. In the ragged
  // last tile (tail) rows past the end are clamped to row n-1: loads stay in
  // bounds and those keys are masked out of the scores.
  //
  // The copies are inline asm (global_load_lds_dwordx4, LDS destination in
  // M0) so the compiler does not treat them as pending writes to every LDS
  // location and wait for them before unrelated LDS reads; completion is
  // awaited explicitly (vmcnt(0)) before the barrier that publishes a tile.
  auto dma = [&](const unsigned short* Gt, unsigned dst, unsigned off) {
    __asm__ volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "s"(dst), "v"(off), "s"(Gt)
        : "memory", "m0");
  };
  auto fetch_k = [&](int stage, int kb, bool tail) {
    const unsigned short* Gt = Kg + (int64_t)kb * rs;
    const unsigned dst = lds0 + stage * T::TILEB;
    if (!tail) {
#pragma unroll
      for (int r = 0; r < NDMA; ++r) dma(Gt, dst + r * 1024, FA_KOFF(r));
    } else {
      const int last = n - 1 - kb;
#pragma unroll
      for (int r = 0; r < NDMA; ++r)
        dma(Gt, dst + r * 1024, (unsigned)(min(dma_row(r), last) * rs + dma_kcol(r)) * 2u);
    }
  };
  auto fetch_v = [&](int stage, int kb, bool tail) {
    const unsigned short* Gt = Vg + (int64_t)kb * rs;
    const unsigned dst = lds0 + (2 + stage) * T::TILEB;
    if (!tail) {
#pragma unroll
      for (int r = 0; r < NDMA; ++r) dma(Gt, dst + r * 1024, FA_VOFF(r));
    } else {
      const int last = n - 1 - kb;
#pragma unroll
      for (int r = 0; r < NDMA; ++r)
        dma(Gt, dst + r * 1024, (unsigned)(min(dma_row(r), last) * rs + dma_vcol(r)) * 2u);
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

  f32x16 o[D / 32];  // O^T accumulators: d = 32*t + 8*(i/4) + 4g + i%4, query l32
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  // Row sums on the matrix cores: one more P.V MFMA per 16 keys with an
  // all-ones A operand leaves sum_k P[q][k] (over both half-waves' keys) in
  // every register of lacc; only lacc[0] is carried (and rescaled).
  constexpr bool kRowSumMfma = FA_MFMA_ROWSUM_D64 && D == 64;
  f32x16 lacc;
#pragma unroll
  for (int i = 0; i < 16; ++i) lacc[i] = 0.f;
  const vec8 ones = __builtin_bit_cast(
      vec8, (u32x4){pack2<BF16>(1.f, 1.f), pack2<BF16>(1.f, 1.f), pack2<BF16>(1.f, 1.f),
                    pack2<BF16>(1.f, 1.f)});
  float l = 0.f;  // VALU row sums: this lane's half of the keys
  const float c2 = p.scale_log2;

  // S^T of the K tile in stage `stage`: lane holds query l32, keys
  // kt*32 + 8*(i/4) + 4*g + (i%4) in register i of s[kt].
  auto qk = [&](int stage, f32x16 (&s)[2]) {
    const lds_u8* Ks = (const lds_u8*)lds + stage * T::TILEB;
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
  };
  // Keys >= n of the tile at kb score -inf (probability 0).
  auto mask = [&](f32x16 (&s)[2], int kb) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb + kt * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key >= n) s[kt][i] = -INFINITY;
      }
  };
  // Max over this lane's 32 scores, then over the partner lane l ^ 32
  // (v_permlane32_swap exchanges the two half-waves).
  auto rowmax = [&](const f32x16 (&s)[2]) {
    float a = fmaxf(s[0][0], s[0][1]), b = fmaxf(s[1][0], s[1][1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) {
      a = fmaxf(fmaxf(a, s[0][i]), s[0][i + 1]);
      b = fmaxf(fmaxf(b, s[1][i]), s[1][i + 1]);
    }
    const float x = fmaxf(a, b);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                     false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };
  // p = exp2(s*c - m*c) in place; returns this lane's sum of p (VALU sums).
  auto expo = [&](f32x16 (&s)[2], float mc) {
    float ls[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[kt][i] = __builtin_amdgcn_exp2f(fmaf(s[kt][i], c2, -mc));
        if (kt == 0 && i < 4)
          ls[i] = s[kt][i];
        else
          ls[i & 3] += s[kt][i];
      }
    return (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };
  // O^T += V^T P^T over the 64 keys of the V tile in stage `stage`, 16 keys
  // per MFMA, and the row sums. Slot jj of lane group g in MFMA t is key
  // 16t + 8*(jj/4) + 4g + jj%4, which is S^T register 8*(t%2) + jj of key
  // tile t/2.
  auto pv = [&](int stage, const f32x16 (&s)[2]) {
    const lds_u8* Vs = (const lds_u8*)lds + (2 + stage) * T::TILEB;
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
      if constexpr (kRowSumMfma) lacc = mfma32x32x16<BF16>(ones, pb, lacc);
    }
  };

  const int nfull = n / BC;  // tiles with all BC keys valid
  const int tiles = (n + BC - 1) / BC;

  // Prologue: K and V of tile 0 and K of tile 1 in flight, then S^T of
  // tile 0 and its row max.
  fetch_k(0, 0, nfull == 0);
  fetch_v(0, 0, nfull == 0);
  if (tiles > 1) fetch_k(1, BC, nfull == 1);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f32x16 sA[2], sB[2];  // scores of the current / next tile, swapping roles
  qk(0, sA);
  float m = rowmax(sA);  // running max of raw q.k (scale > 0)

  // Iteration j (stage parity P = j % 2): the softmax VALU work of tile j
  // is interleaved with the S^T MFMAs of tile j+1, and the row max of tile
  // j+1 with the P.V MFMAs of tile j. HAS_NEXT: a tile j+1 exists.
  //
  // The ragged last tile needs no special handling until its exponentials:
  // its rows past the end are copies of key row n-1, so their scores equal a
  // real score and leave the running max unchanged; they are masked to
  // probability 0 just before the exp2 in the final iteration.
  auto iteration = [&](auto has_next, auto parity, int j, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    constexpr bool HN = decltype(has_next)::value;
    constexpr int P = decltype(parity)::value;
    // Keep each iteration its own scheduling region (bounds register
    // pressure: the scheduler would otherwise hoist the next iteration's
    // loads and spill).
    if constexpr (HN) {
      if (j + 2 < tiles) fetch_k(P, (j + 2) * BC, j + 2 == nfull);
      fetch_v(1 - P, (j + 1) * BC, j + 1 == nfull);
      qk(1 - P, sn);
    }
    if constexpr (!HN) {
      if (nfull < tiles) mask(sc, j * BC);
    }
    const float lsum = expo(sc, m * c2);
    pv(P, sc);
    if constexpr (!kRowSumMfma) l += lsum;
    if constexpr (HN) {
      // The running max moves when some row of the wave saw a larger score
      // (by more than FA_RESCALE_TAU in log2 units; 0 = any increase): then
      // O and l of every row are brought to its new max by
      // alpha = exp2((m_old - m_new) * c), which is 1 for rows whose max
      // did not move. The branch is uniform across the wave.
      const float mx = rowmax(sn);
#if FA_SCHED
      // Interleave: S^T MFMAs of tile j+1 with the softmax VALU of tile j,
      // then P.V MFMAs of tile j with the row max of tile j+1; LDS reads run
      // a few MFMAs ahead of their use.
      __builtin_amdgcn_sched_group_barrier(0x100, FA_SCHED_AH, 0);
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, FA_SCHED_VA, 0);
        if (i + FA_SCHED_AH < D / 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * FA_SCHED_AH, 0);
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, FA_SCHED_VB, 0);
        if (i + FA_SCHED_AH < D / 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#endif
      if (__any((mx - m) * c2 > (float)FA_RESCALE_TAU)) {
        const float mnew = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f((m - mnew) * c2);
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
        if constexpr (kRowSumMfma)
          lacc[0] *= alpha;
        else
          l *= alpha;
        m = mnew;
      }
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  };
  using T0 = std::integral_constant<int, 0>;
  using T1 = std::integral_constant<int, 1>;
  const std::true_type Y;
  const std::false_type N;

  int j = 0;
  for (; j + 2 < tiles; j += 2) {  // pairs of iterations that both have a next tile
    iteration(Y, T0{}, j, sA, sB);
    iteration(Y, T1{}, j + 1, sB, sA);
  }
  // j is even here and the current scores are in sA.
  if (j + 1 < tiles) {
    iteration(Y, T0{}, j, sA, sB);
    iteration(N, T1{}, j + 1, sB, sA);
  } else {
    iteration(N, T0{}, j, sA, sB);
  }
  if constexpr (kRowSumMfma) {
    l = lacc[0];  // already the sum over both half-waves' keys
  } else {        // add the partner half-wave's partial sum
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l),
                                                     false, false);
    l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }

  // Write-back: divide once by l, L = m*scale + ln l.
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
