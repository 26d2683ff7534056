// C-ABI entry points of the FlashAttention-2 library (include/fa.h):
// argument validation, work-grid sizing and dispatch to the gfx950 kernels.
//
// Validation touches no HIP API, so every error path returns before
// anything is enqueued (and can be exercised without a GPU).
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_common.h"

namespace {

// Wave count of the 16-bit forward's workgroups: 8 runs the ping-pong of two
// wave groups (256 rows), 4 a single group (128 rows, two workgroups per CU),
// which wins whenever a workgroup visits few key tiles. Measured back to back,
// with bitwise-identical outputs:
// - banded: faster from w = 0 (1.56x) to w = 2048 (1.02x), slower from 4096;
// - dense: d = 64, N = 512 +12 %, N = 2048 +10 %; d = 128, N = 1024 +5 %,
//   N = 4096 -2 %, N = 8192 -3 %;
// - varlen, 32 sequences of lengths drawn from a range (d = 128): 64..1024
//   +6 %, 64..2048 +1.7 %, 64..2560 and 64..3072 within 0.3 %, 64..4096,
//   1024..4096 and 2048..4096 -1.4 %; packed batches switch to 8 waves
//   above max_seqlen 3072.
#ifndef FA_BAND_NARROW_MAX
#define FA_BAND_NARROW_MAX 2048
#endif
#ifndef FA_DENSE_NARROW_MAX_N
#define FA_DENSE_NARROW_MAX_N 2048
#endif
#ifndef FA_VARLEN_NARROW_MAX_N
#define FA_VARLEN_NARROW_MAX_N 3072
#endif
constexpr int kWavesPingPong = 8;
constexpr int kWavesNarrow = 4;
constexpr int kBandNarrowMax = FA_BAND_NARROW_MAX;     // windows (capped at N)
constexpr int kDenseNarrowMaxN = FA_DENSE_NARROW_MAX_N;
constexpr int kVarlenNarrowMaxN = FA_VARLEN_NARROW_MAX_N;  // max_seqlen
// Largest query block of any forward kernel (the 8-wave 16-bit one).
constexpr int kMaxRowsPerBlock = 256;

constexpr int kVersion = 700;  // 0.7.0: adds fa_debug_fwd_trace (debug build)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Half-open byte ranges [a, a+na) and [b, b+nb) intersect.
bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

int elem_bytes(int dtype) { return dtype == FA_F32 ? 4 : 2; }

bool valid_dtype(int dtype) { return dtype == FA_F32 || dtype == FA_F16 || dtype == FA_BF16; }

// Shared checks on the dense and varlen entry points after the sizes are
// known to be non-negative and non-empty.
int check_buffers(const void* Q, const void* K, const void* V, const void* O, const float* L,
                  uint64_t qkvo_bytes, uint64_t l_bytes) {
  if (!Q || !K || !V || !O || !L) return FA_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(L))
    return FA_ERR_ALIGN;
  if (overlap(O, qkvo_bytes, Q, qkvo_bytes) || overlap(O, qkvo_bytes, K, qkvo_bytes) ||
      overlap(O, qkvo_bytes, V, qkvo_bytes) || overlap(L, l_bytes, Q, qkvo_bytes) ||
      overlap(L, l_bytes, K, qkvo_bytes) || overlap(L, l_bytes, V, qkvo_bytes) ||
      overlap(L, l_bytes, O, qkvo_bytes))
    return FA_ERR_ALIAS;
  return FA_OK;
}

int launch(const fa::FwdParams& p, int d, int dtype, bool varlen, void* stream,
           int waves = kWavesPingPong) {
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == FA_F32)
    e = fa::launch_fwd_f32(p, d, varlen, s);
  else
    e = fa::launch_fwd_mfma16(p, d, dtype == FA_BF16, varlen, waves, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// A launch covers at most 2^32 - 1 work-items (workgroups x threads) in its
// one grid dimension. Every kernel here runs 256-thread workgroups except the
// 8-wave 16-bit forward (512); the fp32 forward's are 256.
constexpr int64_t kMaxWorkItems = (int64_t{1} << 32) - 1;
constexpr int kThreadsDefault = 256;
constexpr int64_t kMaxBlocks = kMaxWorkItems / kThreadsDefault;
bool grid_fits(int64_t blocks, int threads) { return blocks <= kMaxWorkItems / threads; }
// Threads per workgroup of a forward launch with `waves` (fp32 runs 256).
int fwd_threads(int dtype, int waves) { return dtype == FA_F32 ? kThreadsDefault : 64 * waves; }

}  // namespace

namespace fa {

int prepare_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                const float* L, void* dQ, void* dK, void* dV, const float* delta,
                bool caller_delta, int B, int H, int N, int d, float scale, int dtype,
                BwdParams& p) {
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (B == 0 || H == 0 || N == 0) return kEmptyProblem;

  if ((int64_t)N * d >= (int64_t{1} << 31)) return FA_ERR_SIZE;
  const int kb = (N + kBwdKeysPerBlock - 1) / kBwdKeysPerBlock;
  const int qb = (N + kBwdQueriesPerBlock - 1) / kBwdQueriesPerBlock;
  if ((int64_t)kb * H * B > kMaxBlocks || (int64_t)qb * H * B > kMaxBlocks) return FA_ERR_SIZE;
  const int64_t rows = (int64_t)B * H * N;
  if ((rows + 15) / 16 > kMaxBlocks) return FA_ERR_SIZE;  // the D kernel: >= 16 rows per block
  if (!caller_delta && rows > kBwdScratchRows) return FA_ERR_SCRATCH;
  if (!Q || !K || !V || !O || !dO || !L || !dQ || !dK || !dV || (caller_delta && !delta))
    return FA_ERR_NULL;
  const void* all[] = {Q, K, V, O, dO, L, dQ, dK, dV, delta};
  for (const void* ptr : all)
    if (ptr && !aligned16(ptr)) return FA_ERR_ALIGN;  // delta is null only when unused
  const uint64_t tb = (uint64_t)rows * d * 2, rb = (uint64_t)rows * 4;
  const void* in[] = {Q, K, V, O, dO, L};
  const uint64_t in_b[] = {tb, tb, tb, tb, tb, rb};
  const void* out[] = {dQ, dK, dV, delta};
  const uint64_t out_b[] = {tb, tb, tb, caller_delta ? rb : 0};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlap(out[i], out_b[i], in[j], in_b[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(out[i], out_b[i], out[j], out_b[j])) return FA_ERR_ALIAS;
  }

  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.dout = dO;
  p.lse = L;
  p.dq = dQ;
  p.dk = dK;
  p.dv = dV;
  p.delta = const_cast<float*>(delta);
  p.head_stride = (int64_t)N * d;
  p.rows = rows;
  p.BH = B * H;
  p.N = N;
  p.kblocks = kb;
  p.qblocks = qb;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  return FA_OK;
}

}  // namespace fa

extern "C" {

int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* L, int B, int H, int N,
           int d, float scale, int dtype, void* stream) {
  if (!valid_dtype(dtype)) return FA_ERR_DTYPE;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (B == 0 || H == 0 || N == 0) return FA_OK;

  if ((int64_t)N * d >= (int64_t{1} << 31)) return FA_ERR_SIZE;
  const int waves = (dtype != FA_F32 && N <= kDenseNarrowMaxN) ? kWavesNarrow : kWavesPingPong;
  // fp32 problems too small to give every CU a 128-row workgroup run the
  // key-split form: 32-row workgroups whose waves share the keys.
  const bool split = dtype == FA_F32 && (int64_t)((N + fa::kRowsPerBlockF32 - 1) /
                                                   fa::kRowsPerBlockF32) * H * B <
                                            fa::kF32SplitBelowBlocks;
  const int br = dtype == FA_F32 ? (split ? fa::kRowsPerBlockF32Split : fa::kRowsPerBlockF32)
                                 : 32 * waves;
  const int threads = split ? 64 * fa::f32_key_split(d) : fwd_threads(dtype, waves);
  if (!grid_fits((int64_t)((N + br - 1) / br) * H * B, threads)) return FA_ERR_SIZE;
  const uint64_t elems = (uint64_t)B * H * N * d;
  const int st = check_buffers(Q, K, V, O, L, elems * elem_bytes(dtype), (uint64_t)B * H * N * 4);
  if (st != FA_OK) return st;

  fa::FwdParams p{};
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.lse = L;
  p.cu_seqlens = nullptr;
  p.batch_stride = (int64_t)H * N * d;
  p.head_stride = (int64_t)N * d;
  p.row_stride = d;
  p.B = B;
  p.H = H;
  p.N = N;
  p.total_tokens = 0;
  p.q_blocks = (N + br - 1) / br;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.window = -1;
  p.key_split = split ? fa::f32_key_split(d) : 0;
  return launch(p, d, dtype, false, stream, waves);
}

int fa_fwd_banded(const void* Q, const void* K, const void* V, void* O, float* L, int B, int H,
                  int N, int d, int window, float scale, int dtype, void* stream) {
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (B < 0 || H < 0 || N < 0 || window < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (B == 0 || H == 0 || N == 0) return FA_OK;

  if ((int64_t)N * d >= (int64_t{1} << 31)) return FA_ERR_SIZE;
  // Narrow bands visit few key tiles per block: 4-wave, 128-row workgroups
  // (two per CU) overlap one another's loads with compute.
  const int wcap = window < N ? window : N;  // a window of N or more keeps every key
  const int waves = wcap <= kBandNarrowMax ? kWavesNarrow : kWavesPingPong;
  const int br = 32 * waves;
  if (!grid_fits((int64_t)((N + br - 1) / br) * H * B, 64 * waves)) return FA_ERR_SIZE;
  const uint64_t elems = (uint64_t)B * H * N * d;
  const int st = check_buffers(Q, K, V, O, L, elems * 2, (uint64_t)B * H * N * 4);
  if (st != FA_OK) return st;

  fa::FwdParams p{};
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.lse = L;
  p.cu_seqlens = nullptr;
  p.batch_stride = (int64_t)H * N * d;
  p.head_stride = (int64_t)N * d;
  p.row_stride = d;
  p.B = B;
  p.H = H;
  p.N = N;
  p.total_tokens = 0;
  p.q_blocks = (N + br - 1) / br;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.window = wcap;
  return launch(p, d, dtype, false, stream, waves);
}

int fa_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* L,
                  const int32_t* cu_seqlens, int nseq, int total_tokens, int max_seqlen, int H,
                  int d, float scale, int dtype, void* stream) {
  if (!valid_dtype(dtype)) return FA_ERR_DTYPE;
  if (nseq < 0 || total_tokens < 0 || max_seqlen < 0 || H < 0) return FA_ERR_SHAPE;
  if (max_seqlen > total_tokens) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (nseq == 0 || total_tokens == 0 || max_seqlen == 0 || H == 0) return FA_OK;

  // Query rows run up to max_seqlen rounded up to a whole query block (at
  // most 256 rows); the in-sequence row offsets of all of them fit 32 bits.
  const int64_t rows_cap = ((int64_t)max_seqlen + kMaxRowsPerBlock - 1) / kMaxRowsPerBlock *
                           kMaxRowsPerBlock;
  if (rows_cap * H * d >= (int64_t{1} << 31)) return FA_ERR_SIZE;
  const int waves = (dtype != FA_F32 && max_seqlen <= kVarlenNarrowMaxN) ? kWavesNarrow : kWavesPingPong;
  const int br = dtype == FA_F32 ? fa::kRowsPerBlockF32 : 32 * waves;
  // Longest-first order (nseq <= 64): one workgroup per unit, at most
  // floor(T / br) + nseq per head (each sequence adds less than one block to
  // T / br), and at most the q_blocks of every sequence.
  const int64_t qblk = (max_seqlen + br - 1) / br;
  int64_t units = 0;
  if (nseq <= fa::kLptMaxSeqs) {
    units = total_tokens / br + nseq;
    if (units > qblk * nseq) units = qblk * nseq;
  }
  if (!grid_fits(units > 0 ? units * H : qblk * H * nseq, fwd_threads(dtype, waves)))
    return FA_ERR_SIZE;
  if (!cu_seqlens) return FA_ERR_NULL;
  const uint64_t elems = (uint64_t)total_tokens * H * d;
  const int st =
      check_buffers(Q, K, V, O, L, elems * elem_bytes(dtype), (uint64_t)H * total_tokens * 4);
  if (st != FA_OK) return st;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return FA_ERR_ALIGN;
  const uint64_t cu_bytes = (uint64_t)(nseq + 1) * 4;
  if (overlap(O, elems * elem_bytes(dtype), cu_seqlens, cu_bytes) ||
      overlap(L, (uint64_t)H * total_tokens * 4, cu_seqlens, cu_bytes))
    return FA_ERR_ALIAS;

  fa::FwdParams p{};
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.lse = L;
  p.cu_seqlens = cu_seqlens;
  p.batch_stride = 0;
  p.head_stride = d;
  p.row_stride = H * d;
  p.B = nseq;
  p.H = H;
  p.N = max_seqlen;
  p.total_tokens = total_tokens;
  p.q_blocks = (int)qblk;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.window = -1;
  p.units_per_head = (int)units;
  return launch(p, d, dtype, true, stream, waves);
}

int fa_fwd_kv_outer(const void* Q, const void* K, const void* V, void* O, float* L, float* acc,
                    int B, int H, int N, int d, int q_groups, float scale, int dtype,
                    void* stream) {
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (B < 0 || H < 0 || N < 0 || q_groups < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (B == 0 || H == 0 || N == 0) return FA_OK;

  if ((int64_t)N * d >= (int64_t{1} << 31)) return FA_ERR_SIZE;
  const int blocks32 = (N + 31) / 32;
  const int groups_req = q_groups < blocks32 ? q_groups : blocks32;
  const int rows = (blocks32 + groups_req - 1) / groups_req * 32;
  const int groups = (N + rows - 1) / rows;  // non-empty groups only
  if ((int64_t)groups * H * B > kMaxBlocks) return FA_ERR_SIZE;
  if (!Q || !K || !V || !O || !L || !acc) return FA_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(L) ||
      !aligned16(acc))
    return FA_ERR_ALIGN;
  const uint64_t rows_all = (uint64_t)B * H * N;
  const uint64_t tb = rows_all * d * 2, lb = rows_all * 4, ab = rows_all * (d + 2) * 4;
  const void* in[3] = {Q, K, V};
  const void* out[3] = {O, L, acc};
  const uint64_t out_b[3] = {tb, lb, ab};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlap(out[i], out_b[i], in[j], tb)) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(out[i], out_b[i], out[j], out_b[j])) return FA_ERR_ALIAS;
  }

  fa::KvOuterParams p{};
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.lse = L;
  p.oacc = acc;
  p.mstat = acc + rows_all * d;
  p.lstat = acc + rows_all * (d + 1);
  p.head_stride = (int64_t)N * d;
  p.BH = B * H;
  p.N = N;
  p.groups = groups;
  p.rows_per_group = rows;
  p.tiles = (N + 63) / 64;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  const hipError_t e =
      fa::launch_fwd_kv_outer(p, d, dtype == FA_BF16, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_dropout_add_norm(const void* x0, const void* x1, const void* residual, const void* gamma0,
                        const void* beta0, const void* gamma1, const void* beta1, void* y0,
                        void* y1, void* z, float* mean, float* rstd, unsigned char* mask,
                        int rows, int hidden, float dropout_p, uint64_t seed, uint64_t offset,
                        float eps, int norm, int dtype, void* stream) {
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (rows < 0 || hidden < 0 || hidden % 8 != 0 || hidden > 8192) return FA_ERR_SHAPE;
  if (norm != FA_NORM_LAYER && norm != FA_NORM_RMS) return FA_ERR_ARG;
  if (!(dropout_p >= 0.f && dropout_p < 1.f)) return FA_ERR_ARG;
  if (!(eps > 0.f) || !isfinite(eps)) return FA_ERR_ARG;
  if (rows == 0 || hidden == 0) return FA_OK;
  if (rows > kMaxBlocks) return FA_ERR_SIZE;
  if (!x0 || !gamma0 || !y0) return FA_ERR_NULL;
  if ((gamma1 == nullptr) != (y1 == nullptr) || (beta1 && !gamma1)) return FA_ERR_NULL;
  const void* t16[] = {x0, x1, residual, gamma0, beta0, gamma1, beta1, y0, y1, z, mask};
  for (const void* t : t16)
    if (t && !aligned16(t)) return FA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(mean) & 3u) || (reinterpret_cast<uintptr_t>(rstd) & 3u))
    return FA_ERR_ALIGN;
  const uint64_t rb = (uint64_t)rows * hidden * 2, wb = (uint64_t)hidden * 2;
  const void* in[] = {x0, x1, residual, gamma0, beta0, gamma1, beta1};
  const uint64_t in_b[] = {rb, rb, rb, wb, wb, wb, wb};
  const void* out[] = {y0, y1, z, mean, rstd, mask};
  const uint64_t out_b[] = {rb, rb, rb, (uint64_t)rows * 4, (uint64_t)rows * 4,
                            (uint64_t)rows * hidden * (x1 ? 2 : 1)};
  for (int i = 0; i < 6; ++i) {
    if (!out[i]) continue;
    for (int j = 0; j < 7; ++j)
      if (in[j] && overlap(out[i], out_b[i], in[j], in_b[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 6; ++j)
      if (out[j] && overlap(out[i], out_b[i], out[j], out_b[j])) return FA_ERR_ALIAS;
  }

  fa::NormParams p{};
  p.x0 = x0;
  p.x1 = x1;
  p.res = residual;
  p.g0 = gamma0;
  p.b0 = beta0;
  p.g1 = gamma1;
  p.b1 = beta1;
  p.y0 = y0;
  p.y1 = y1;
  p.z = z;
  p.mean = mean;
  p.rstd = rstd;
  p.mask = mask;
  p.rows = rows;
  p.hidden = hidden;
  p.thr = (uint32_t)floor((double)dropout_p * 4294967296.0);
  p.keep_scale = 1.f / (1.f - dropout_p);
  p.key0 = (uint32_t)seed;
  p.key1 = (uint32_t)(seed >> 32);
  p.ctr2 = (uint32_t)offset;
  p.ctr3 = (uint32_t)(offset >> 32);
  p.eps = eps;
  p.rms = norm == FA_NORM_RMS;
  const hipError_t e =
      fa::launch_dropout_add_norm(p, dtype == FA_BF16, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
           const float* L, void* dQ, void* dK, void* dV, float* delta, int B, int H, int N, int d,
           float scale, int dtype, void* stream) {
  fa::BwdParams p{};
  const int st = fa::prepare_bwd(Q, K, V, O, dO, L, dQ, dK, dV, delta, true, B, H, N, d, scale,
                                 dtype, p);
  if (st != FA_OK) return st == fa::kEmptyProblem ? FA_OK : st;
  const hipError_t e =
      fa::launch_bwd(p, d, dtype == FA_BF16, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_debug_fwd_trace(int workgroup, unsigned long long* trace_buffer) {
  if (workgroup < -1) return FA_ERR_ARG;
  if (workgroup >= 0 && !trace_buffer) return FA_ERR_NULL;
  if (workgroup >= 0 && (reinterpret_cast<uintptr_t>(trace_buffer) & 7u) != 0) return FA_ERR_ALIGN;
  const hipError_t e = fa::set_fwd_trace(workgroup, trace_buffer);
  if (e == hipErrorNotSupported) return FA_ERR_UNSUPPORTED;
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: negative or inconsistent sizes or window";
    case FA_ERR_HEADDIM: return "FA_ERR_HEADDIM: head dimension must be 64 or 128";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: dtype not supported by this entry point";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a pointer is not suitably aligned";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: an output overlaps an input or the other output";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: the HIP runtime refused the kernel launch";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite and > 0";
    case FA_ERR_SIZE: return "FA_ERR_SIZE: problem too large for 32-bit in-head offsets or one launch grid";
    case FA_ERR_ARG: return "FA_ERR_ARG: an argument outside its documented range";
    case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH: problem larger than the library's static scratch buffer";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: not available in this build of the library";
    default: return "unknown fa_status";
  }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
