// FlashAttention-2 backward for bf16 / fp16 storage on gfx950 (MI355X).
//
// The method ("FlashAttention -- for programmers, not researchers", STAGE 5):
// the probabilities are not kept from the forward; every score tile is
// recomputed and turned into P with the forward's row statistic L, so only
// O(N) extra state exists. The products are the five of the backward list
// in the flash-attention documentation (S = Q K^T, dP = dO V^T, dV = P^T dO,
// dK = dS^T Q, dQ = dS K), with dS = P * (dP - D) and D = rowsum(dO * O).
//
// Three kernels, enqueued in order on one stream:
//  1. delta: D[r] = sum_k dO[r,k] O[r,k] (fp32), one pass over O and dO;
//     it stores -D, and -L[r]*log2 e into the dQ buffer (free until step 3
//     writes dQ), the two per-row offsets the dK/dV kernel adds.
//  2. dK/dV: a workgroup owns 128 keys of one head (4 waves x 32 keys) and
//     streams the head's queries in tiles of 64. Per tile and wave:
//       S  = Q K^T  and  dP = dO V^T   (queries x keys; A = Q / dO rows from
//                                       LDS, B = K / V rows held in VGPRs),
//       P  = exp2(S*c - L*log2 e), dS = P * (dP - D),
//       dV^T += dO^T P  and  dK^T += Q^T dS   (d x keys; A = dO^T / Q^T read
//                                       transposed from LDS, B = P / dS taken
//                                       from the S / dP accumulator registers).
//     dK = scale * dK^T^T and dV are written once at the end.
//  3. dQ: a workgroup owns 128 queries (4 waves x 32) and streams the keys in
//     tiles of 64, as the forward does: S^T = K Q^T and dP^T = V dO^T (Q and
//     dO in VGPRs), P^T, dS^T, then dQ^T += K^T dS^T (K^T read transposed).
//     Held to 2 waves per SIMD (<= 256 VGPRs), so each SIMD has a second
//     wave to issue while one waits.
// No atomics: each gradient element is produced by one workgroup in a fixed
// order, so results are bitwise reproducible. The cost is that S and dP are
// computed in both kernels (7 products instead of 5).
//
// LDS tiles (64 rows) are filled by global_load_lds_dwordx4 copies and read
// both row-wise (ds_read_b128: 8 elements of one row per lane) and
// transposed (ds_read_b64_tr_b16: 4 rows of one column per lane). One XOR
// swizzle serves both without bank conflicts: 16-byte chunk c of row r is
// stored at chunk c ^ f(r), with f(r) = 4*(r%4) + (r/4)%4 for d = 128 (16
// chunks per row) and f(r) = 4*((r/2)%2) + (r/4)%4 for d = 64 (8 chunks per
// row, two rows per 256-byte bank sweep). f takes distinct values over the
// 16 rows a 16-lane row read touches, and its top bits differ over the 4
// consecutive rows a transposed read touches.
#include <type_traits>

#include "fa_bwd_params.h"
#include "fa_device.h"
#include "fa_lanes.h"

namespace fa {
namespace {

constexpr int kWavesB = 4;
constexpr int kThreadsB = 64 * kWavesB;
constexpr int TQ = 64;  // queries per tile (dK/dV kernel)
constexpr int TK = 64;  // keys per tile (dQ kernel)
static_assert(kBwdKeysPerBlock == 32 * kWavesB && kBwdQueriesPerBlock == 32 * kWavesB,
              "one 32-row slice per wave");

template <int D>
struct BTile {
  static constexpr int ROWB = D * 2;            // bytes per row
  static constexpr int KCH = ROWB / 16;         // 16-byte chunks per row
  static constexpr int TILEB = 64 * ROWB;       // bytes per 64-row tile
  static constexpr int CPW = TILEB / 1024 / kWavesB;  // 1 KiB copies per wave and tile
  __device__ static int swz(int r) {
    if constexpr (D == 128)
      return ((r & 3) << 2) | ((r >> 2) & 3);
    else
      return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  // Byte offset of logical byte column cb of row r inside a tile.
  __device__ static int off(int r, int cb) {
    return r * ROWB + ((((cb >> 4) ^ swz(r))) << 4) + (cb & 15);
  }
};

// One 1 KiB copy: lane i moves 16 bytes from gbase + voff to LDS M0 + 16*i.
// Inline asm so the compiler does not make later LDS reads wait for it;
// completion is awaited explicitly (vmcnt) before the publishing barrier.
__device__ __forceinline__ void dma16(const void* gbase, unsigned lds_dst, unsigned voff) {
  poison_lds_before_copy<16>(lds_dst);
  __asm__ volatile(
      "s_mov_b32 m0, %0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds_dst), "v"(voff), "s"(gbase)
      : "memory", "m0");
}
// 64 floats: lane i moves 4 bytes from gbase + voff to LDS M0 + 4*i.
__device__ __forceinline__ void dma4(const void* gbase, unsigned lds_dst, unsigned voff) {
  poison_lds_before_copy<4>(lds_dst);
  __asm__ volatile(
      "s_mov_b32 m0, %0\n\t"
      "global_load_lds_dword %1, %2"
      :
      : "s"(lds_dst), "v"(voff), "s"(gbase)
      : "memory", "m0");
}

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O).
// ---------------------------------------------------------------------------
template <bool BF16, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdParams p) {
  constexpr int LPR = D / 8;        // lanes per row, 8 elements (16 bytes) each
  constexpr int RPB = 256 / LPR;    // rows per block
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < p.rows) {
    const int64_t e = row * D + part * 8;
    const u32x4 a = *(const u32x4*)((const unsigned short*)p.o + e);
    const u32x4 b = *(const u32x4*)((const unsigned short*)p.dout + e);
    using vec8 = typename Elem<BF16>::vec8;
    const vec8 va = __builtin_bit_cast(vec8, a), vb = __builtin_bit_cast(vec8, b);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)va[i], (float)vb[i], acc);
  }
  acc = lanes_sum<LPR>(acc);  // the LPR lanes of a row are an aligned group
  // Stored negated: the key-block kernel starts its dP accumulators at -D,
  // so its MFMAs produce dP - D directly. The same kernel needs -L*log2(e)
  // per query as its exponent offset; that goes to the first B*H*N floats
  // of the dQ buffer, which nothing reads and the dQ kernel (last in the
  // stream) overwrites with dQ. dQ holds B*H*N*d 16-bit values (d >= 64),
  // far more than B*H*N floats.
  if (row < p.rows && part == 0) {
    p.delta[row] = -acc;
    ((float*)p.dq)[row] = -p.lse[row] * 1.4426950408889634f;
  }
}

// ---------------------------------------------------------------------------
// 2. dK, dV: one workgroup per (head, 128 keys).
// ---------------------------------------------------------------------------
template <bool BF16, int D>
__global__ __launch_bounds__(kThreadsB) void bwd_dkdv_kernel(BwdParams p) {
  using vec8 = typename Elem<BF16>::vec8;
  using T = BTile<D>;
  constexpr int STG = 2 * T::TILEB + 512;  // Q tile, dO tile, L[64], D[64]
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * STG];

  const int id = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int kb = id % p.kblocks;  // key blocks of one head are consecutive
  const int bh = id / p.kblocks;
  const int n = p.N;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t hb = (int64_t)bh * p.head_stride;
  const unsigned short* Qg = (const unsigned short*)p.q + hb;
  const unsigned short* Og = (const unsigned short*)p.dout + hb;
  const float* Lg = (const float*)p.dq + (int64_t)bh * n;  // -L*log2(e), staged by the delta kernel
  const float* Dg = p.delta + (int64_t)bh * n;

  // K and V rows of this lane's key as B operands (k = d): elements
  // 16s + 8g .. +7 of key row kr (rows past the end read row n-1; their
  // results are never stored).
  const int kr = kb * kBwdKeysPerBlock + wave * 32 + l32;
  const int krc = min(kr, n - 1);
  vec8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    kf[s] = __builtin_bit_cast(
        vec8, *(const u32x4*)((const unsigned short*)p.k + hb + (int64_t)krc * D + 16 * s + 8 * g));
    vf[s] = __builtin_bit_cast(
        vec8, *(const u32x4*)((const unsigned short*)p.v + hb + (int64_t)krc * D + 16 * s + 8 * g));
    // d = 128 runs one wave per SIMD with more than 256 live registers: the
    // fragments are pinned to AGPRs (MFMA operands may come from there).
    // Otherwise the compiler kept them in AGPRs but copied every one to
    // another AGPR before each use (56 moves per tile).
    if constexpr (D == 128) __asm__ volatile("" : "+a"(kf[s]), "+a"(vf[s]));
  }
  f32x16 dk[D / 32], dv[D / 32];  // dK^T, dV^T: d = 32t + 8(i/4) + 4g + i%4, key l32
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[t][i] = dv[t][i] = 0.f;

  const unsigned ldsb = (unsigned)(uintptr_t)(lds_u8*)lds;
  // Copies of query tile jt into stage st: Q and dO rows (4 waves x CPW
  // copies each; slot s = row*KCH + stored chunk, fetching logical chunk
  // (stored ^ f(row)); rows past the end are clamped), L and D by waves 0/1.
  auto fetch = [&](int st, int jt) {
    const int q0 = jt * TQ, last = n - 1 - q0;
    const unsigned short* Qt = Qg + (int64_t)q0 * D;
    const unsigned short* Ot = Og + (int64_t)q0 * D;
    const unsigned base = ldsb + st * STG;
#pragma unroll
    for (int r = 0; r < T::CPW; ++r) {
      const int s = (wave * T::CPW + r) * 64 + lane;
      const int row = s / T::KCH;
      const int chunk = (s % T::KCH) ^ T::swz(row);
      const unsigned goff = (unsigned)(min(row, last) * D + chunk * 8) * 2u;
      const unsigned dst = (wave * T::CPW + r) * 1024;
      dma16(Qt, base + dst, goff);
      dma16(Ot, base + T::TILEB + dst, goff);
    }
    if (wave < 2) {
      const unsigned voff = (unsigned)min(lane, last) * 4u;
      dma4(wave == 0 ? (const void*)(Lg + q0) : (const void*)(Dg + q0),
           base + 2 * T::TILEB + wave * 256, voff);
    }
  };

  // Transposed-read lane geometry (as the forward's V^T read): lane j of
  // 16-lane block b reads row 16t + 8h + vrow of the tile, logical bytes
  // 64*dt + vin .. +7, and receives column 32*dt + l32 of rows
  // 16t + 8h + 4g + 0..3.
  const int vj = lane & 15, vb = lane >> 4;
  const int vrow = 4 * (vb >> 1) + (vj >> 2);
  const int vin = 32 * (vb & 1) + 8 * (vj & 3);
  const float c2 = p.scale_log2;

  // RAG (compile time): the tile holds queries past the end (only the last
  // tile can); full tiles carry no masking code at all. Left as a runtime
  // test, the compiler turned the mask into selects executed on every tile.
  auto compute = [&](auto stage, int q0, auto rag) {
    constexpr bool RAG = decltype(rag)::value;
    const int st = stage;
    const lds_u8* Qs = (const lds_u8*)lds + st * STG;
    const lds_u8* Os = Qs + T::TILEB;
    const float* Ls = (const float*)(lds + st * STG + 2 * T::TILEB);
    const float* Ds = Ls + 64;
    // Operand rings of the two MFMA chains of a 32-query half, read two
    // steps ahead of their MFMAs: Q / dO rows for S and dP (step ss), and
    // dO^T / Q^T (transposed reads) for dV and dK (step k). The first two
    // reads of each chain are issued early, where their latency hides: the
    // transposed ones before the softmax VALU work, the row reads of the
    // second half during the first half's dV/dK chain. One wave per SIMD
    // leaves nothing else to cover an LDS read at the head of a chain.
    constexpr int NS = D / 16;
    constexpr int NST = 2 * (D / 32);
    vec8 qa[3], oa[3];
    i16x4 ho[3][2], hqv[3][2];
    auto rd_row = [&](int hq, int ss) {
      const int r = hq * 32 + l32, cb = (2 * ss + g) * 16;
      qa[ss % 3] = *(const __attribute__((address_space(3))) vec8*)(Qs + T::off(r, cb));
      oa[ss % 3] = *(const __attribute__((address_space(3))) vec8*)(Os + T::off(r, cb));
    };
    auto rd_tr = [&](int hq, int k) {
      const int t = k / (D / 32), dt = k % (D / 32);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = hq * 32 + 16 * t + 8 * h + vrow;
        const int o = T::off(r, 64 * dt + vin);
        ho[k % 3][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Os + o));
        hqv[k % 3][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Qs + o));
      }
    };
    rd_row(0, 0);
    rd_row(0, 1);
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {  // 32-query halves of the tile
      // rows: query hq*32 + 8(i/4) + 4g + i%4; column: key l32. dp starts
      // at -D of its row (the scratch holds -D), so it ends as dP - D.
      f32x16 s = {}, dp;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 nd = *(const f32x4*)(Ds + hq * 32 + 8 * a + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[4 * a + e] = nd[e];
      }
#pragma unroll
      for (int ss = 0; ss < NS; ++ss) {
        if (ss + 2 < NS) rd_row(hq, ss + 2);
        __builtin_amdgcn_sched_barrier(0);
        s = mfma32x32x16<BF16>(qa[ss % 3], kf[ss], s);
        dp = mfma32x32x16<BF16>(oa[ss % 3], vf[ss], dp);
        __builtin_amdgcn_sched_barrier(0);
      }
      rd_tr(hq, 0);
      rd_tr(hq, 1);
      // Exponent arguments, exponentials, then dS, as three fenced groups so
      // that no instruction waits right behind the exponential it consumes.
      float pr[16], ds[16];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int qi = hq * 32 + 8 * a + 4 * g;
        const f32x4 nl = *(const f32x4*)(Ls + qi);  // -L*log2(e)
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[4 * a + e] = fmaf(s[4 * a + e], c2, nl[e]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) pr[i] = __builtin_amdgcn_exp2f(pr[i]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int qi = hq * 32 + 8 * a + 4 * g;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * a + e;
          if (RAG && q0 + qi + e >= n) pr[i] = 0.f;  // query past the end
          ds[i] = pr[i] * dp[i];
        }
      }
      // P and dS as B operands: slot jj of lane group g in product t is
      // query 16t + 8(jj/4) + 4g + jj%4 of this half = register 8t + jj.
      vec8 pp[2], pd[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 w1, w2;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          w1[q] = pack2<BF16>(pr[8 * t + 2 * q], pr[8 * t + 2 * q + 1]);
          w2[q] = pack2<BF16>(ds[8 * t + 2 * q], ds[8 * t + 2 * q + 1]);
        }
        pp[t] = __builtin_bit_cast(vec8, w1);
        pd[t] = __builtin_bit_cast(vec8, w2);
      }
#pragma unroll
      for (int k = 0; k < NST; ++k) {
        const int t = k / (D / 32), dt = k % (D / 32);
        if (k + 2 < NST)
          rd_tr(hq, k + 2);
        else if (hq == 0)
          rd_row(1, k + 2 - NST);  // the second half's first row operands
        __builtin_amdgcn_sched_barrier(0);
        const i16x8 ao = {ho[k % 3][0][0], ho[k % 3][0][1], ho[k % 3][0][2], ho[k % 3][0][3],
                          ho[k % 3][1][0], ho[k % 3][1][1], ho[k % 3][1][2], ho[k % 3][1][3]};
        const i16x8 aq = {hqv[k % 3][0][0], hqv[k % 3][0][1], hqv[k % 3][0][2], hqv[k % 3][0][3],
                          hqv[k % 3][1][0], hqv[k % 3][1][1], hqv[k % 3][1][2], hqv[k % 3][1][3]};
        dv[dt] = mfma32x32x16<BF16>(__builtin_bit_cast(vec8, ao), pp[t], dv[dt]);
        dk[dt] = mfma32x32x16<BF16>(__builtin_bit_cast(vec8, aq), pd[t], dk[dt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  const int tiles = (n + TQ - 1) / TQ;
  fetch(0, 0);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // Tile jt sits in stage jt & 1. The loop runs two tiles per iteration so
  // that each stage is a compile-time constant and every LDS read address is
  // a fixed per-lane base plus an instruction offset (a runtime stage cost
  // one add per read). Each fetch fills the stage last read in the tile
  // before.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  const std::false_type full;
  auto step = [&](auto st, int jt) {
    fetch(1 - decltype(st)::value, jt + 1);
    compute(st, jt * TQ, full);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  int jt = 0;
  for (; jt + 2 < tiles; jt += 2) {
    step(S0{}, jt);
    step(S1{}, jt + 1);
  }
  if (jt + 1 < tiles) step(S0{}, jt++);
  if (n % TQ == 0)
    compute(jt & 1, jt * TQ, full);
  else
    compute(jt & 1, jt * TQ, std::true_type{});

  if (kr < n) {
    unsigned short* dkr = (unsigned short*)p.dk + hb + (int64_t)kr * D;
    unsigned short* dvr = (unsigned short*)p.dv + hb + (int64_t)kr * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        u32x2 a, b;
        a[0] = pack2<BF16>(dk[dt][4 * blk + 0] * p.scale, dk[dt][4 * blk + 1] * p.scale);
        a[1] = pack2<BF16>(dk[dt][4 * blk + 2] * p.scale, dk[dt][4 * blk + 3] * p.scale);
        b[0] = pack2<BF16>(dv[dt][4 * blk + 0], dv[dt][4 * blk + 1]);
        b[1] = pack2<BF16>(dv[dt][4 * blk + 2], dv[dt][4 * blk + 3]);
        *(u32x2*)(dkr + dt * 32 + 8 * blk + 4 * g) = a;
        *(u32x2*)(dvr + dt * 32 + 8 * blk + 4 * g) = b;
      }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ: one workgroup per (head, 128 queries).
// ---------------------------------------------------------------------------
template <bool BF16, int D>
__global__ __launch_bounds__(kThreadsB) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_kernel(BwdParams p) {
  using vec8 = typename Elem<BF16>::vec8;
  using T = BTile<D>;
  constexpr int STG = 2 * T::TILEB;  // K tile, V tile
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * STG];

  const int id = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int qb = id % p.qblocks;
  const int bh = id / p.qblocks;
  const int n = p.N;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t hb = (int64_t)bh * p.head_stride;
  const unsigned short* Kg = (const unsigned short*)p.k + hb;
  const unsigned short* Vg = (const unsigned short*)p.v + hb;

  // This lane's query: Q and dO rows as B operands, its L and D.
  const int qr = qb * kBwdQueriesPerBlock + wave * 32 + l32;
  vec8 qf[D / 16], of[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (qr < n) {
      a = *(const u32x4*)((const unsigned short*)p.q + hb + (int64_t)qr * D + 16 * s + 8 * g);
      b = *(const u32x4*)((const unsigned short*)p.dout + hb + (int64_t)qr * D + 16 * s + 8 * g);
    }
    qf[s] = __builtin_bit_cast(vec8, a);
    of[s] = __builtin_bit_cast(vec8, b);
  }
  const int qrc = min(qr, n - 1);
  const float lq = p.lse[(int64_t)bh * n + qrc] * 1.4426950408889634f;
  const float dq_nd = p.delta[(int64_t)bh * n + qrc];  // -D of this query
  // d = 64: the dP^T chains start from -D (every accumulator value of a lane
  // belongs to its query), held in 16 registers for the whole kernel, so the
  // MFMAs produce dP - D and dS needs no add per element. At d = 128 the
  // kernel has no 16 registers to spare (2 waves per SIMD) and adds -D.
  constexpr bool ND_INIT = D == 64;
  f32x16 nd16;
#pragma unroll
  for (int i = 0; i < 16; ++i) nd16[i] = dq_nd;
  f32x16 acc[D / 32];  // dQ^T: d = 32t + 8(i/4) + 4g + i%4, query l32
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;

  const unsigned ldsb = (unsigned)(uintptr_t)(lds_u8*)lds;
  auto fetch = [&](int st, int kt) {
    const int k0 = kt * TK, last = n - 1 - k0;
    const unsigned short* Kt = Kg + (int64_t)k0 * D;
    const unsigned short* Vt = Vg + (int64_t)k0 * D;
    const unsigned base = ldsb + st * STG;
#pragma unroll
    for (int r = 0; r < T::CPW; ++r) {
      const int s = (wave * T::CPW + r) * 64 + lane;
      const int row = s / T::KCH;
      const int chunk = (s % T::KCH) ^ T::swz(row);
      const unsigned goff = (unsigned)(min(row, last) * D + chunk * 8) * 2u;
      const unsigned dst = (wave * T::CPW + r) * 1024;
      dma16(Kt, base + dst, goff);
      dma16(Vt, base + T::TILEB + dst, goff);
    }
  };

  const int vj = lane & 15, vb = lane >> 4;
  const int vrow = 4 * (vb >> 1) + (vj >> 2);
  const int vin = 32 * (vb & 1) + 8 * (vj & 3);
  const float c2 = p.scale_log2;

  // RAG (compile time): the tile holds keys past the end (only the last
  // tile can), as in the key-block kernel.
  auto compute = [&](auto stage, int k0, auto rag) {
    constexpr bool RAG = decltype(rag)::value;
    const int st = stage;
    const lds_u8* Ks = (const lds_u8*)lds + st * STG;
    const lds_u8* Vs = Ks + T::TILEB;
    f32x16 s[2] = {}, dp[2] = {};  // rows: key kt*32 + 8(i/4) + 4g + i%4; column: query l32
#pragma unroll
    for (int ss = 0; ss < D / 16; ++ss)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int r = kt * 32 + l32, cb = (2 * ss + g) * 16;
        const vec8 ka = *(const __attribute__((address_space(3))) vec8*)(Ks + T::off(r, cb));
        const vec8 va = *(const __attribute__((address_space(3))) vec8*)(Vs + T::off(r, cb));
        s[kt] = mfma32x32x16<BF16>(ka, qf[ss], s[kt]);
        dp[kt] = mfma32x32x16<BF16>(va, of[ss], (ND_INIT && ss == 0) ? nd16 : dp[kt]);
      }
    // P^T then dS^T, one 32-key half at a time: the half's exponent arguments,
    // its exponentials, then its dS, as three fenced groups, so no instruction
    // waits right behind the exponential it consumes.
    vec8 pb[4];  // dS^T as B operands, 16 keys each (as the forward packs P)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 pe;
#pragma unroll
      for (int i = 0; i < 16; ++i) pe[i] = fmaf(s[kt][i], c2, -lq);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) pe[i] = __builtin_amdgcn_exp2f(pe[i]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float x[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int i = 8 * h + 2 * q + e;
            float pv = pe[i];
            if constexpr (RAG) {
              const int key = k0 + kt * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
              if (key >= n) pv = 0.f;
            }
            x[e] = ND_INIT ? pv * dp[kt][i] : pv * (dp[kt][i] + dq_nd);
          }
          w[q] = pack2<BF16>(x[0], x[1]);
        }
        pb[2 * kt + h] = __builtin_bit_cast(vec8, w);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        i16x4 hk[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = 16 * t + 8 * h + vrow;
          hk[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(Ks + T::off(r, 64 * dt + vin)));
        }
        const i16x8 a8 = {hk[0][0], hk[0][1], hk[0][2], hk[0][3],
                          hk[1][0], hk[1][1], hk[1][2], hk[1][3]};
        acc[dt] = mfma32x32x16<BF16>(__builtin_bit_cast(vec8, a8), pb[t], acc[dt]);
      }
  };

  const int tiles = (n + TK - 1) / TK;
  fetch(0, 0);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // Two tiles per iteration, each stage a compile-time constant (as in the
  // key-block kernel).
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  const std::false_type full;
  auto step = [&](auto st, int kt) {
    fetch(1 - decltype(st)::value, kt + 1);
    compute(st, kt * TK, full);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  int kt = 0;
  for (; kt + 2 < tiles; kt += 2) {
    step(S0{}, kt);
    step(S1{}, kt + 1);
  }
  if (kt + 1 < tiles) step(S0{}, kt++);
  if (n % TK == 0)
    compute(kt & 1, kt * TK, full);
  else
    compute(kt & 1, kt * TK, std::true_type{});

  // The query row again, from the lane count rather than the thread index, so
  // that no per-lane address stays live (and spills) across the key loop.
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int qr_e = qb * kBwdQueriesPerBlock + wave * 32 + (lane_e & 31);
  if (qr_e < n) {
    unsigned short* row = (unsigned short*)p.dq + hb + (int64_t)qr_e * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        u32x2 w;
        w[0] = pack2<BF16>(acc[dt][4 * blk + 0] * p.scale, acc[dt][4 * blk + 1] * p.scale);
        w[1] = pack2<BF16>(acc[dt][4 * blk + 2] * p.scale, acc[dt][4 * blk + 3] * p.scale);
        *(u32x2*)(row + dt * 32 + 8 * blk + 4 * g) = w;
      }
  }
}

template <bool BF16, int D>
hipError_t launch3(const BwdParams& p, hipStream_t stream) {
  BwdParams arg = p;
  void* args[] = {&arg};
  constexpr int RPB = 256 / (D / 8);
  hipError_t e = hipLaunchKernel((const void*)bwd_delta_kernel<BF16, D>,
                                 dim3((unsigned)((p.rows + RPB - 1) / RPB)), dim3(256), args, 0,
                                 stream);
  if (e != hipSuccess) return e;
  e = hipLaunchKernel((const void*)bwd_dkdv_kernel<BF16, D>,
                      dim3((unsigned)((int64_t)p.kblocks * p.BH)), dim3(kThreadsB), args, 0,
                      stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel((const void*)bwd_dq_kernel<BF16, D>,
                         dim3((unsigned)((int64_t)p.qblocks * p.BH)), dim3(kThreadsB), args, 0,
                         stream);
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int d, bool bf16, hipStream_t stream) {
  if (bf16) return d == 64 ? launch3<true, 64>(p, stream) : launch3<true, 128>(p, stream);
  return d == 64 ? launch3<false, 64>(p, stream) : launch3<false, 128>(p, stream);
}

}  // namespace fa
