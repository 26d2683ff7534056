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
//    and fed from registers straight into the P.V MFMA as its B operand
//    (O^T = V^T P^T): no LDS round trip for P.
//  * Ping-pong between the two waves of a SIMD: waves w and w+4 (measured:
//    they share a SIMD) run half a step apart, and each step of a wave is a
//    matrix half (MFMAs and LDS reads only) and a softmax half (VALU only),
//    separated by workgroup barriers. The softmax of a tile depends on the
//    scores the same wave has just computed, so inside one wave it would
//    wait for them; split across the two waves, the VALU of one runs while
//    the matrix core works for the other (measured faster than interleaving
//    both streams in one wave).
//  * K and V tiles travel HBM -> LDS with global_load_lds_dwordx4 (no
//    staging registers, no LDS write instructions), issued by waves 4-7 at
//    the start of their softmax half. Both stay row-major in LDS with an
//    XOR swizzle of their columns:
//      K: 16-byte chunk c of row r sits at chunk c ^ kswz(r); a lane reads
//         one 16-byte chunk of one key row per S^T MFMA (ds_read_b128);
//      V: 64-byte chunk c of row r sits at chunk c ^ vswz(r); the P.V
//         operand (8 keys of one d column per lane) is read with the gfx950
//         transposing load ds_read_b64_tr_b16: within each 16-lane block,
//         lane l receives element l%4 of the 4-element vectors loaded by
//         lanes l/4, l/4+4, l/4+8 and l/4+12.
//    Both read patterns are free of LDS bank conflicts.
//  * K runs one tile ahead of V. The 8-wave kernel keeps three LDS stages
//    each of K and V (two for 4 waves), so that every wave can read the
//    first operands of its next matrix half during its softmax half and
//    start its MFMAs right after the barrier.
//  * O (fp32) lives in MFMA accumulators for the whole loop, one query per
//    lane, so the rescale by alpha is a per-lane scalar multiply. It and the
//    row max are skipped while the sums of p show that no p exceeds 2^8.
#include <type_traits>

#include "fa_fwd_unit.h"

// Build options (defaults are the shipped configuration):
//   FA_RESCALE_TAU (8): the reference max m of the running sums moves (and
//     O, l are rescaled by exp2((m_old - m_new) * c)) only when some lane's
//     sum of p over a tile exceeds 2^TAU; then m becomes the exact running
//     max. O/l and L = m + ln l are the same for any reference, so this
//     changes rounding only; every p stays at most 2^TAU (no overflow in
//     fp32, bf16 or fp16).
//   FA_PP_PRIO (1): s_setprio of a wave during its matrix half.
//   FA_PP_AHEAD (2): MFMA steps between an LDS operand read and its use.
//   FA_SKIP_IDLE (1): in packed batches, waves whose rows all lie past the
//     end of their sequence skip their MFMAs and softmax (0: they compute on
//     zero rows and discard the result).
#ifndef FA_RESCALE_TAU
#define FA_RESCALE_TAU 8
#endif
static_assert(FA_RESCALE_TAU >= 5 && FA_RESCALE_TAU <= 15, "a lane sums 2^5 values of p; p must fit fp16");
#ifndef FA_PP_PRIO
#define FA_PP_PRIO 1
#endif
#ifndef FA_PP_AHEAD
#define FA_PP_AHEAD 2
#endif
#ifndef FA_SKIP_IDLE
#define FA_SKIP_IDLE 1
#endif

// Phase trace (debug build libfa_trace.so only, FA_DEBUG_TRACE): one chosen
// workgroup records the shader-clock timestamp (s_memtime) of four points of
// each of its first kTraceSteps steps, per wave: the start and end of its
// matrix half, and the start and end of its softmax half. The points sit
// where the wave has no LDS read in flight, since the timestamp's wait
// (lgkmcnt) would otherwise also wait for those reads. Timestamps go to LDS
// and are copied to the host-given buffer at the end of the workgroup,
// followed per wave by s_memtime and the 100 MHz clock (s_memrealtime) at
// its start and end, for the clock rate. Layout (u64): [wave][step][point]
// for 8 waves x kTraceSteps x 4, then [wave][4].
#ifdef FA_DEBUG_TRACE
__device__ unsigned long long* fa_trace_buf;
__device__ int fa_trace_wg = -1;
#define FA_TRACE(pt, tt)                                                     \
  do {                                                                       \
    if (tracing && (tt) >= 0 && (tt) < fa::kTraceSteps) {                    \
      const unsigned long long ts_ = __builtin_amdgcn_s_memtime();           \
      if (lane == 0) trbuf[(wave * fa::kTraceSteps + (tt)) * 4 + (pt)] = ts_; \
    }                                                                        \
  } while (0)
#else
#define FA_TRACE(pt, tt) \
  do {                   \
  } while (0)
#endif

namespace fa {
namespace {

constexpr int BC = 64;               // keys per tile
// Waves that issue the K/V copies (group B, waves 4-7).
constexpr int kDmaWaves = 4;

// LDS tile geometry for head dimension D (16-bit elements).
template <int D>
struct Tile {
  static constexpr int ROWB = D * 2;                 // bytes per key row
  static constexpr int TILEB = BC * ROWB;            // bytes per K (or V) tile
  static constexpr int STAGEB = 2 * TILEB;           // K tile + V tile
  static constexpr int ROWS_PER_256 = 256 / ROWB;    // rows sharing one 256-byte bank sweep
  static constexpr int KCHUNKS = ROWB / 16;          // 16-byte chunks per row
  static constexpr int VCHUNKS = ROWB / 64;          // 64-byte chunks per row
  static constexpr int DMA_PER_WAVE = TILEB / 1024 / kDmaWaves;  // 1 KiB copies per wave
  // Rows read together get distinct chunk positions, hence distinct banks.
  __device__ static int kswz(int r) { return (r / ROWS_PER_256) & (KCHUNKS - 1); }
  __device__ static int vswz(int r) { return (r / ROWS_PER_256) & (VCHUNKS - 1); }
};

// BAND: row r only attends to keys c with |r - c| <= p.window (local
// window; "FlashAttention -- for programmers, not researchers", DEMO 6). The
// workgroup visits only the key tiles that hold a key within the window of
// one of its rows, and masks per element only in the tiles where the band
// edge cuts a wave's 32 x 64 block.
//
// NW: waves per workgroup. 8 (the default) runs the ping-pong of two wave
// groups described below, one workgroup per CU. 4 runs a single group (every
// wave issues its share of the copies and takes both barriers of a step) in
// 128-row workgroups, two per CU: their load, compute and store phases then
// overlap each other, which pays off when a workgroup visits only a few key
// tiles (narrow bands, short sequences).
template <bool BF16, int D, bool VARLEN, bool BAND, int NW>
__global__ __launch_bounds__(64 * NW, 2) void fwd16_kernel(FwdParams p) {
  static_assert(NW == 8 || NW == 4, "8 waves (ping-pong) or 4 (one group)");
  constexpr int BR = 32 * NW;  // query rows per workgroup (32 per wave)
  // LDS stages for K (and for V). The ping-pong needs three so that the
  // first group can read its next operands before the barrier (below).
  constexpr int S = NW == 8 ? 3 : 2;
  using vec8 = typename Elem<BF16>::vec8;
  using T = Tile<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[S * T::STAGEB];

  WorkUnit u;
  if (!resolve_unit<VARLEN>(p, BR, u)) return;
#ifdef FA_DEBUG_TRACE
  __shared__ unsigned long long trbuf[8 * kTraceSteps * 4];
  const bool tracing = (int)blockIdx.x == fa_trace_wg;
  unsigned long long trace_t0 = 0, trace_r0 = 0;
  if (tracing) {
    trace_t0 = __builtin_amdgcn_s_memtime();
    trace_r0 = __builtin_amdgcn_s_memrealtime();
  }
#endif

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
    if (qrow < n) w = *(const u32x4*)(Qg + (int64_t)qrow * rs + 16 * s + 8 * g);
    qf[s] = __builtin_bit_cast(vec8, w);
  }

  // LDS holds S K stages followed by S V stages; tile j of either lives in
  // stage (j + ph) % S (ph below). K runs one tile ahead of V: the matrix
  // half of step j reads K of tile j+1 (for S^T) and V of tile j (for P.V).
  //
  // Direct-to-LDS copies: copy r of this wave fills bytes
  // [1024*(wave*NDMA + r), +1024) of a tile; lane i writes 16 bytes at
  // +16*i, i.e. 16-byte slot s of the tile. Slot s is (row, stored chunk);
  // the lane fetches the logical chunk the swizzle stores there.
  constexpr int NDMA = T::DMA_PER_WAVE;
  const int dwave = wave % kDmaWaves;  // index among the copying waves
  // Row and (logical) column of the 16 bytes copy r of this lane moves.
  auto dma_row = [&](int r) { return ((dwave * NDMA + r) * 64 + lane) / T::KCHUNKS; };
  auto dma_kcol = [&](int r) {
    const int s = (dwave * NDMA + r) * 64 + lane;
    return ((s % T::KCHUNKS) ^ T::kswz(s / T::KCHUNKS)) * 8;
  };
  auto dma_vcol = [&](int r) {
    const int s = (dwave * NDMA + r) * 64 + lane;
    const int pos = s % T::KCHUNKS;
    return ((((pos >> 2) ^ T::vswz(s / T::KCHUNKS)) << 2) | (pos & 3)) * 8;
  };
  // Byte offsets of the full-tile copies relative to the tile's first row.
  // They do not change over the loop; computed once and pinned in registers
  // (opaque to the compiler, which would otherwise recompute them before
  // every copy: ~4 VALU instructions each, one a quarter-rate multiply, in
  // the copying waves' softmax half). Where that would push the kernel past
  // 256 VGPRs (4-wave packed d = 128, banded d = 128) they are recomputed.
  constexpr bool PRE_OFF = !(D == 128 && (BAND || (VARLEN && NW == 4)));
  unsigned koff[PRE_OFF ? NDMA : 1], voff[PRE_OFF ? NDMA : 1];
  if constexpr (PRE_OFF) {
#pragma unroll
    for (int r = 0; r < NDMA; ++r) {
      koff[r] = (unsigned)(dma_row(r) * rs + dma_kcol(r)) * 2u;
      voff[r] = (unsigned)(dma_row(r) * rs + dma_vcol(r)) * 2u;
      __asm__ volatile("" : "+v"(koff[r]), "+v"(voff[r]));
    }
  }
#define FA_KOFF(r) (PRE_OFF ? koff[PRE_OFF ? (r) : 0] : (unsigned)(dma_row(r) * rs + dma_kcol(r)) * 2u)
#define FA_VOFF(r) (PRE_OFF ? voff[PRE_OFF ? (r) : 0] : (unsigned)(dma_row(r) * rs + dma_vcol(r)) * 2u)
  const unsigned lds0 = (unsigned)(uintptr_t)(lds_u8*)lds + (unsigned)(dwave * NDMA * 1024);
  // Copy the K (or V) tile at key kb into LDS at byte `dst`. In the ragged
  // last tile (tail) rows past the end are clamped to row n-1: loads stay in
  // bounds and those keys are masked out of the scores.
  //
  // The copies are inline asm (global_load_lds_dwordx4, LDS destination in
  // M0) so the compiler does not treat them as pending writes to every LDS
  // location and wait for them before unrelated LDS reads; completion is
  // awaited explicitly (vmcnt(0)) before the barrier that publishes a tile.
  auto dma = [&](const unsigned short* Gt, unsigned dst, unsigned off) {
    poison_lds_before_copy<16>(dst);
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
    const unsigned dst = lds0 + (S + stage) * T::TILEB;
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
  // This lane's operand addresses in stage 0: K per 32-element chunk pair
  // ss, V per 32-column block dt (the V swizzle of row 16t + 8h + vrow
  // equals that of vrow, since 16t + 8h spans whole swizzle periods). Every
  // other read adds a constant (stage, key block, row block) that fits the
  // 16-bit offset of the LDS instructions; the empty asm keeps the compiler
  // from re-deriving one base per stage.
  static_assert((8 / T::ROWS_PER_256) % T::VCHUNKS == 0, "V swizzle period");
  const lds_u8* kp[D / 16];
  const lds_u8* vp[D / 32];
#pragma unroll
  for (int ss = 0; ss < D / 16; ++ss) {
    kp[ss] = (const lds_u8*)lds + l32 * T::ROWB + (((2 * ss + g) ^ kx) << 4);
    __asm__ volatile("" : "+v"(kp[ss]));
  }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    vp[dt] = (const lds_u8*)lds + S * T::TILEB + vrow * T::ROWB + ((dt ^ T::vswz(vrow)) << 6) + vin;
    __asm__ volatile("" : "+v"(vp[dt]));
  }

  f32x16 o[D / 32];  // O^T accumulators: d = 32*t + 8*(i/4) + 4g + i%4, query l32
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  float l = 0.f;  // VALU row sums: this lane's half of the keys
  const float c2 = p.scale_log2;

  // S^T of the K tile in stage `stage`: lane holds query l32, keys
  // kt*32 + 8*(i/4) + 4*g + (i%4) in register i of s[kt].
  auto qk = [&](int stage, f32x16 (&s)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
    for (int ss = 0; ss < D / 16; ++ss)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const vec8 a = *(const __attribute__((address_space(3))) vec8*)(
            kp[ss] + stage * T::TILEB + kt * 32 * T::ROWB);
        s[kt] = mfma32x32x16<BF16>(a, qf[ss], s[kt]);
      }
  };
  // Keys >= n of the tile at kb (and, with a band, keys farther than the
  // window from this lane's query row) score -inf (probability 0).
  const int win = BAND ? p.window : 0;
  auto mask = [&](f32x16 (&s)[2], int kb) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb + kt * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
        bool out = key >= n;
        if constexpr (BAND) out = out || (unsigned)(key - qrow + win) > (unsigned)(2 * win);
        if (out) s[kt][i] = -INFINITY;
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

  const int nfull = n / BC;  // tiles with all BC keys valid
  // Key tiles visited: t0 .. t0 + tiles - 1. With a band, only those that
  // hold a key within the window of one of the workgroup's rows (whole
  // tiles outside are skipped; the host caps the window at n).
  int t0 = 0, tiles = (n + BC - 1) / BC;
  if constexpr (BAND) {
    const int lo = max(0, u.q0 - win);
    const int hi = min(n - 1, min(u.q0 + BR, n) - 1 + win);
    t0 = lo / BC;
    tiles = hi / BC - t0 + 1;
  }
  const int rag = nfull - t0;  // visiting index of the ragged tile, if any
  // With a band, whether the edge of the band cuts this wave's block of 32
  // query rows x the 64 keys at kb (then the tile is masked per element).
  const int row0 = u.q0 + wave * 32;
  auto band_edge = [&](int kb) {
    return BAND && (kb + BC - 1 - row0 > win || row0 + 31 - kb > win);
  };

  // Ping-pong: waves 0-3 (group A) and 4-7 (group B) share the four SIMDs,
  // one of each per SIMD, and run half a step apart. Between two workgroup
  // barriers one wave of every SIMD is in its matrix half (MFMAs only: S^T
  // of tile t+1 and P.V of tile t) while the other is in its softmax half
  // (VALU only: row max, rescale, exponentials, row sums, P in the storage
  // dtype); at the next barrier they swap. The matrix core and the VALU of
  // a SIMD thus work for different waves at the same time, and neither
  // waits on the other's results.
  const bool grp_a = NW == 8 && wave < 4;  // with NW = 4 every wave is in group B
  // Packed batches: a wave whose 32 query rows all lie past the end of its
  // sequence (in the ragged last block of a sequence) computes nothing; it
  // only issues its share of the copies and takes every barrier, and its
  // SIMD serves the other workgroup's wave there. Wave-uniform. Measured
  // back to back: +0.1-1.2 % on packed batches; the dense instances keep
  // the unconditional code (the branch cost a d = 64 dense shape 4.8 %
  // through register allocation).
  const bool busy = !(VARLEN && FA_SKIP_IDLE) || row0 < n;
  vec8 pb[4];           // P of the current tile, storage dtype: P.V B operands
  // Running max of raw q.k (scale > 0). With a band it starts at a large
  // finite negative value instead of -inf: a row may meet whole tiles with
  // every key masked before its first in-band key, and exp2(-inf*c - m*c)
  // must then be 0, not NaN. The first in-band key moves m and rescales by
  // exp2((-1e30 - m)*c) = 0, so nothing from before survives.
  float m = BAND ? -1e30f : -INFINITY;
  f32x16 sc[2];         // scores of the next tile

  // Softmax half for the score tile in sc (keys kb..kb+63). Every form keeps
  // each p = exp2(s*c - m*c) at most 2^FA_RESCALE_TAU:
  //  * kSpeculative: no row max. p is formed against the current reference
  //    m and summed per lane; p >= 0, so a lane sum <= 2^FA_RESCALE_TAU
  //    bounds every p of that lane, and when that holds in every lane m
  //    stays. Otherwise (a score came near or above the bound; rare once m
  //    has settled) the row max is taken, O and l are rescaled to it exactly
  //    by alpha = exp2((m_old - m_new)*c), and p is recomputed from the
  //    scores, which are still in sc.
  //  * kMaxFirst (the first tile, where m is still the initial value): the
  //    row max is taken first and becomes m; p is computed once. O and l are
  //    still zero, so nothing is rescaled.
  //  * kAdaptive: kSpeculative while the max has settled; after a tile that
  //    needed the exact path, the speculative pass is skipped and the row
  //    max is taken first (m stays if no lane's max exceeds it by more than
  //    (TAU-5)/c, so that a lane's 32 p sum to at most 2^TAU; otherwise O
  //    and l are rescaled to the new max first) until a tile needs no
  //    rescale. Inputs whose max keeps moving (large logits) then pay one
  //    exponential per score instead of two. Used at d = 64, where the
  //    softmax is the larger share of a step (measured back to back: 13-15 %
  //    faster on large-logit inputs at N = 512, 1.5 % on N(0,1) inputs at
  //    N = 1024, no change at N = 2048). At d = 128 it cost 0.75 % on packed
  //    batches and gained nothing on long sequences, where the max settles
  //    within a few of 32 or more tiles; d = 128 keeps kSpeculative.
  // Then row sums, and P rounded and packed for P.V.
  enum { kSpeculative, kMaxFirst, kAdaptive };
  // kAdaptive: wave-uniform, the last tile needed no rescale. It starts
  // false: the first tile's max (kMaxFirst) says little about whether the
  // second tile will move it, and a failed speculative pass costs a whole
  // pass of exponentials, a row max only a sixth of that.
  bool settled = false;
  auto rescale_to = [&](float mnew) __attribute__((always_inline)) {
    const float alpha = __builtin_amdgcn_exp2f((m - mnew) * c2);
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
    l *= alpha;
    m = mnew;
  };
  auto softmax = [&](auto form, bool ragged, int kb) __attribute__((always_inline)) {
    constexpr int FORM = decltype(form)::value;
    if (ragged || band_edge(kb)) mask(sc, kb);
    f32x16 pf[2];
    // Three groups fenced apart: the 32 exponent arguments, the 32
    // exponentials, then the sums. Left to itself the compiler puts each
    // exponential's consumer right behind it, where it waits for the
    // transcendental unit; grouped, no instruction waits on a result still
    // in flight (measured 0.7-1.2 % faster on the whole kernel).
    auto exps = [&]() {
      const float mc = m * c2;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) pf[kt][i] = fmaf(sc[kt][i], c2, -mc);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) pf[kt][i] = __builtin_amdgcn_exp2f(pf[kt][i]);
      __builtin_amdgcn_sched_barrier(0);
      float ls[4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          ls[i & 3] = (kt == 0 && i < 4) ? pf[kt][i] : ls[i & 3] + pf[kt][i];
      return (ls[0] + ls[1]) + (ls[2] + ls[3]);
    };
    float lsum;
    if constexpr (FORM == kMaxFirst) {
      m = fmaxf(m, rowmax(sc));  // a band's fully masked lane keeps its -1e30
      lsum = exps();
    } else if constexpr (FORM == kAdaptive) {
      // The speculative pass runs only while the max has settled; otherwise
      // (or when it fails) the exact path runs: the row max, a rescale if
      // some lane's max exceeds m by more than (TAU-5)/c (after a failed
      // speculative pass one always does: a lane sum above 2^TAU needs a p
      // above 2^(TAU-5)), and the exponentials against the final m. One
      // rescale site: with two, the compiler copied all of O every tile.
      bool exact = true;
      if (settled) {
        lsum = exps();
        exact = __any(!(lsum <= (float)(1u << FA_RESCALE_TAU)));
      }
      if (exact) {
        const float mx = rowmax(sc);
        // (mx - m)*c is -inf for a lane whose keys here are all masked
        // (band), so only moved maxima count.
        settled = !__any((mx - m) * c2 > (float)(FA_RESCALE_TAU - 5));
        if (!settled) rescale_to(fmaxf(m, mx));
        lsum = exps();
      }
    } else {
      lsum = exps();
      if (__any(!(lsum <= (float)(1u << FA_RESCALE_TAU)))) {
        const float mx = rowmax(sc);
        if (__any(mx > m)) {
          rescale_to(fmaxf(m, mx));
          lsum = exps();
        }
      }
    }
    l += lsum;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 pw;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        pw[q] = pack2<BF16>(pf[t >> 1][8 * (t & 1) + 2 * q], pf[t >> 1][8 * (t & 1) + 2 * q + 1]);
      pb[t] = __builtin_bit_cast(vec8, pw);
      __asm__ volatile("" : "+v"(pb[t]));
    }
    __asm__ volatile("" : "+v"(l));
  };
  using LoopForm = std::integral_constant<int, D == 64 ? kAdaptive : kSpeculative>;
  // Operand registers of the matrix half. Reads run FA_PP_AHEAD MFMA steps
  // ahead of their MFMAs in rotating registers; the first FA_PP_AHEAD reads
  // of a matrix half are issued early, in the wave's preceding softmax half,
  // so that its first MFMAs can start as soon as the barrier releases.
  constexpr int NSTEP = D / 8, DT = D / 32, AH = FA_PP_AHEAD, NB = AH + 1;
  static_assert(AH >= 1 && AH < NSTEP, "read-ahead depth");
  vec8 ka[NB];
  i16x4 va[NB][2];
  // Operands of MFMA step i of a matrix half: the K chunk for S^T of the
  // next tile (K stage KS) and the transposed V rows for P.V (V stage VS).
  auto read = [&](int KS, int VS, int i) __attribute__((always_inline)) {
    const int ss = i >> 1, kt = i & 1;
    ka[i % NB] = *(const __attribute__((address_space(3))) vec8*)(
        kp[ss] + KS * T::TILEB + kt * 32 * T::ROWB);
    const int t = i / DT, dt = i % DT;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      va[i % NB][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(vp[dt] + VS * T::TILEB + (16 * t + 8 * h) * T::ROWB));
  };
  auto preread = [&](int kstage, int vstage) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < AH; ++i) read(kstage, vstage, i);
  };
  // Matrix half of step t: S^T of tile t+1 into sc from K stage KS (when
  // HN) and O^T += V^T P^T of tile t from V stage VS, the two MFMA streams
  // interleaved. The reads of steps 0 .. AH-1 were issued by preread.
  auto matrix = [&](auto has_next, auto kstage, auto vstage) {
    constexpr bool HN = decltype(has_next)::value;
    __builtin_amdgcn_s_setprio(FA_PP_PRIO);
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      if (i + AH < NSTEP) read(decltype(kstage)::value, decltype(vstage)::value, i + AH);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (HN) {
        const int ss = i >> 1, kt = i & 1;
        sc[kt] = mfma32x32x16<BF16>(ka[i % NB], qf[ss], ss == 0 ? f32x16{} : sc[kt]);
      }
      const int t = i / DT, dt = i % DT;
      const i16x8 a8 = {va[i % NB][0][0], va[i % NB][0][1], va[i % NB][0][2], va[i % NB][0][3],
                        va[i % NB][1][0], va[i % NB][1][1], va[i % NB][1][2], va[i % NB][1][3]};
      o[dt] = mfma32x32x16<BF16>(__builtin_bit_cast(vec8, a8), pb[t], o[dt]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // Copies issued in the softmax half of step t (phase F): K of tile t+1+S
  // into K stage (F+1) % S and V of tile t+S into V stage F. Both stages were
  // last read in the matrix halves of step t, which every wave has finished
  // at the barrier before. The copies complete (vmcnt(0)) at the end of the
  // issuing waves' next matrix half, before the barrier after which the
  // earliest reader, a preread, may run.
  auto copies = [&](auto kstage, auto vstage, int t) {
    constexpr int KS = decltype(kstage)::value, VS = decltype(vstage)::value;
    if (t + 1 + S < tiles) fetch_k(KS, (t0 + t + 1 + S) * BC, t + 1 + S == rag);
    if (t + S < tiles) fetch_v(VS, (t0 + t + S) * BC, t + S == rag);
  };
  // Step t (phase F = (t + ph) % S): [matrix(t)] | [softmax of tile t+1] |. With 8
  // waves, group B runs every step one half-step (one barrier) after group
  // A, so on each SIMD the matrix half of one wave meets the softmax half of
  // the other. Group B issues the copies. At the start of its softmax half
  // each wave reads the first operands of its next matrix half (K of tile
  // t+2, V of tile t+1): with three stages those tiles completed a full step
  // earlier, so group A may read them while group B's copies of the step
  // before are still in flight into other stages.
  auto step = [&](auto has_next, auto phase, int t) {
    constexpr int F = decltype(phase)::value;
    using KS = std::integral_constant<int, (F + 1) % S>;
    using VS = std::integral_constant<int, F>;
    using KN = std::integral_constant<int, (F + 2) % S>;
    using VN = std::integral_constant<int, (F + 1) % S>;
    FA_TRACE(0, t);
    if (busy) matrix(has_next, KS{}, VS{});
    FA_TRACE(1, t);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    FA_TRACE(2, t);
    if constexpr (decltype(has_next)::value) {
      if (busy) preread(KN::value, VN::value);
      if (!grp_a) copies(KS{}, VS{}, t);
      if (busy) softmax(LoopForm{}, t + 1 == rag, (t0 + t + 1) * BC);
    }
    FA_TRACE(3, t);
    __syncthreads();
  };

  // Tile j (visiting order) lives in stage (j + ph) % S; every step has a
  // compile-time phase, so every stage offset is an immediate. With PEEL,
  // the r = (tiles-1) % S steps that do not fill a group of S run before
  // the loop, in phases S-r .. S-1, so that the loop runs whole groups in
  // phases 0 .. S-1 and the last step (no next tile: no S^T, no softmax)
  // has phase 0. Otherwise ph = 0 and the remainder follows the loop. A
  // remainder after the loop spilled registers with three stages and with
  // a band (measured: the spills cost HBM writes); with neither it is the
  // faster of the two.
  constexpr bool PEEL = S == 3 || BAND;
  const int r = PEEL ? (tiles - 1) % S : 0;
  const int ph = (S - r) % S;
  auto stage_of = [&](int j) { return (j + ph) % S; };

  // Prologue: tiles 0 .. S-1 of K and 0 .. S-2 of V; S^T and softmax of tile
  // 0; the first operands of matrix half 0 (K of tile 1, V of tile 0); then
  // the copies that step -1 would have issued (K of tile S, V of tile S-1).
  if (!grp_a) {
#pragma unroll
    for (int i = 0; i < S; ++i)
      if (i < tiles) fetch_k(stage_of(i), (t0 + i) * BC, rag == i);
#pragma unroll
    for (int i = 0; i + 1 < S; ++i)
      if (i < tiles) fetch_v(stage_of(i), (t0 + i) * BC, rag == i);
  }
  // Consume Q here, after the first copies are issued, so its load latency
  // overlaps theirs and the compiler waits for these loads before the key
  // loop; otherwise it places that wait inside the loop, where it would
  // also stall on the prefetch of the next K/V tile.
#pragma unroll
  for (int s = 0; s < D / 16; ++s) __asm__ volatile("" : : "v"(qf[s]));
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // The K stage of tile 1 is read even when there is no tile 1: the
  // registers then go unused (matrix half 0 computes no S^T). The stage
  // offsets are computed here, not chosen by a branch on ph: hipcc (ROCm
  // 7.2) miscompiled a three-way branch with a constant-stage read in each
  // arm (the ph == 2 arm read K through an address register it never set).
  if (busy) {
    qk(stage_of(0), sc);
    preread(stage_of(1), stage_of(0));
    softmax(std::integral_constant<int, kMaxFirst>{}, rag == 0, t0 * BC);
  }
  __syncthreads();  // the K stage of tile 0 is free for tile S
  if (!grp_a) {
    if (S < tiles) fetch_k(stage_of(S), (t0 + S) * BC, rag == S);
    if (S - 1 < tiles) fetch_v(stage_of(S - 1), (t0 + S - 1) * BC, rag == S - 1);
    if (NW == 8) __syncthreads();  // group B starts half a step late
  }

  using F0 = std::integral_constant<int, 0>;
  using F1 = std::integral_constant<int, 1>;
  using F2 = std::integral_constant<int, 2 % S>;
  const std::true_type Y;
  const std::false_type N;
  int t = 0;
  if constexpr (PEEL) {
    if constexpr (S == 3) {
      if (r == 2) step(Y, F1{}, t++);
    }
    if (r >= 1) step(Y, std::integral_constant<int, S - 1>{}, t++);
    for (; t + 1 < tiles; t += S) {
      step(Y, F0{}, t);
      step(Y, F1{}, t + 1);
      if constexpr (S == 3) step(Y, F2{}, t + 2);
    }
    step(N, F0{}, t);
  } else {
    for (; t + 2 < tiles; t += 2) {
      step(Y, F0{}, t);
      step(Y, F1{}, t + 1);
    }
    if (t + 1 < tiles) {
      step(Y, F0{}, t);
      step(N, F1{}, t + 1);
    } else {
      step(N, F0{}, t);
    }
  }
  if (grp_a) __syncthreads();  // matches group B's extra barrier
  {  // add the partner half-wave's partial sum
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l),
                                                     false, false);
    l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }

  // Write-back: divide once by l, L = m*scale + ln l.
  //
  // O goes out through LDS so that the global stores are whole 16-byte row
  // chunks: a lane holds 4 consecutive d of its row per register block, so
  // direct stores would be 8-byte pieces of 32 rows each. Every wave has
  // passed the barrier after its last matrix half, so no LDS stage is read
  // any more; each wave writes its 32 rows into a region of its own
  // (rows padded by 16 bytes: the half-waves' 8-byte writes then hit
  // distinct banks, and rows stay 16-byte aligned for the reads), and reads
  // them back in the same wave, so no barrier is needed.
  {
    constexpr int OROWB = 2 * D + 16;  // bytes per staged row
    static_assert(NW * 32 * OROWB <= S * T::STAGEB, "O staging fits the K/V stages");
    lds_u8* ow = (lds_u8*)lds + wave * 32 * OROWB;
    const float inv = 1.f / l;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        u32x2 w;
        w[0] = pack2<BF16>(o[dt][4 * blk + 0] * inv, o[dt][4 * blk + 1] * inv);
        w[1] = pack2<BF16>(o[dt][4 * blk + 2] * inv, o[dt][4 * blk + 3] * inv);
        *(__attribute__((address_space(3))) u32x2*)(ow + l32 * OROWB +
                                                     2 * (dt * 32 + 8 * blk + 4 * g)) = w;
      }
    // Read back: per instruction, 64 / (D/8) rows of D/8 lanes x 16 bytes.
    constexpr int LPR = D / 8;  // lanes per row
    constexpr int RPI = 64 / LPR;
    const int rsub = lane / LPR, cb = (lane % LPR) * 16;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + rsub;
      const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(ow + r * OROWB + cb);
      if (row0 + r < n) *(u32x4*)(Og + (int64_t)(row0 + r) * rs + cb / 2) = v;
    }
    if (qrow < n && g == 0) p.lse[u.lse_base + qrow] = m * p.scale + logf(l);
  }
#ifdef FA_DEBUG_TRACE
  if (tracing) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    unsigned long long* out = fa_trace_buf;
    for (int i = lane; i < kTraceSteps * 4; i += 64)
      out[wave * kTraceSteps * 4 + i] = trbuf[wave * kTraceSteps * 4 + i];
    if (lane < 4)
      out[8 * kTraceSteps * 4 + wave * 4 + lane] =
          lane == 0 ? trace_t0 : lane == 1 ? trace_r0 : lane == 2 ? t1 : r1;
  }
#endif
}

template <bool BF16, int D>
const void* pick(bool varlen, bool band, int waves) {
  if (band)
    return waves == 4 ? (const void*)fwd16_kernel<BF16, D, false, true, 4>
                      : (const void*)fwd16_kernel<BF16, D, false, true, 8>;
  if (varlen)
    return waves == 4 ? (const void*)fwd16_kernel<BF16, D, true, false, 4>
                      : (const void*)fwd16_kernel<BF16, D, true, false, 8>;
  return waves == 4 ? (const void*)fwd16_kernel<BF16, D, false, false, 4>
                    : (const void*)fwd16_kernel<BF16, D, false, false, 8>;
}

}  // namespace

hipError_t set_fwd_trace(int workgroup, unsigned long long* buffer) {
#ifdef FA_DEBUG_TRACE
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(fa_trace_buf), &buffer, sizeof(buffer));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(fa_trace_wg), &workgroup, sizeof(workgroup));
  return e;
#else
  (void)workgroup;
  (void)buffer;
  return hipErrorNotSupported;
#endif
}

hipError_t launch_fwd_mfma16(const FwdParams& p, int d, bool bf16, bool varlen, int waves,
                             hipStream_t stream) {
  const bool band = p.window >= 0;
  const void* fn = nullptr;
  if (bf16)
    fn = (d == 64) ? pick<true, 64>(varlen, band, waves) : pick<true, 128>(varlen, band, waves);
  else
    fn = (d == 64) ? pick<false, 64>(varlen, band, waves) : pick<false, 128>(varlen, band, waves);
  const dim3 grid((unsigned)fwd_grid(p));
  const dim3 block(64 * waves);
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace fa
