/*
 * fa.h -- C ABI of the MI355X (gfx950) FlashAttention-2 library: forward
 * (dense, packed variable-length and dense banded), dense backward, the
 * K/V-outer forward used to measure the other loop order's traffic, and the
 * fused dropout + residual + LayerNorm/RMSNorm op.
 *
 * What is computed. For every (batch, head) -- or every (sequence, head)
 * in the packed variable-length entry -- and every query row r:
 *
 *     S[r, c] = scale * dot(Q[r, :], K[c, :])         over all keys c
 *     O[r, :] = sum_c softmax(S[r, :])[c] * V[c, :]
 *     L[r]    = max_c S[r, c] + ln( sum_c exp(S[r, c] - max_c S[r, c]) )
 *
 * i.e. the forward pass of "Kernel visualization: Flash Attention 2"
 * (tinyvolt.com): its fa2 kernel takes Q, K, V and writes O and the single
 * array L = m + log(l) (sections "Steps" and "Write the data back to HBM"),
 * with the score scale applied to the dot product (section "Iteration
 * j = 0"). It is the same function as plain softmax attention, not an
 * approximation ("FlashAttention -- for programmers, not researchers",
 * STAGE 4 and DEMO 6). No causal mask, no dropout, no bias; query and
 * key/value head counts are equal. fa_fwd_banded restricts every row to a
 * local window of keys.
 *
 * Conventions shared by every entry point:
 *   - Every tensor argument (Q, K, V, O, L, cu_seqlens, dO, dQ, dK, dV,
 *     delta, acc) is a DEVICE pointer, allocated and owned by the caller.
 *     No entry point allocates device memory or keeps per-call state, and
 *     none synchronises: work is enqueued on `stream` (a hipStream_t passed
 *     as void*; NULL = the default stream) and the caller synchronises.
 *     Calls on one stream run in order. The one piece of library-owned
 *     device memory is fa_bwd_noalloc's static scratch array (below).
 *   - Storage dtype of Q, K, V and O is `dtype` (fa_dtype). Arithmetic:
 *     products of dtype values summed in fp32; softmax statistics m, l in
 *     fp32; for fp16/bf16 the probabilities are rounded to dtype (round to
 *     nearest even) as operands of the P.V product; O is rounded to dtype
 *     once, after the single division by l. L is always fp32, natural log.
 *   - Head dimension d is 64 or 128 (FA_ERR_HEADDIM otherwise).
 *   - `scale` must be finite and > 0 (FA_ERR_SCALE otherwise).
 *   - Q, K, V, O and L must be 16-byte aligned, cu_seqlens 4-byte aligned
 *     (FA_ERR_ALIGN).
 *   - O and L must not overlap Q, K, V or each other (FA_ERR_ALIAS).
 *   - Empty problems (a zero size) return FA_OK without launching.
 *   - Errors are returned, never raised or printed; nothing is enqueued
 *     when a check fails. A kernel launch error is FA_ERR_LAUNCH.
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_F32 = 0,
  FA_F16 = 1,
  FA_BF16 = 2
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,     /* a required pointer is NULL                        */
  FA_ERR_SHAPE = -2,    /* a negative size or window, or inconsistent sizes  */
  FA_ERR_HEADDIM = -3,  /* d not in {64, 128}                                */
  FA_ERR_DTYPE = -4,    /* dtype not an fa_dtype value, or not supported     */
  FA_ERR_ALIGN = -5,    /* a pointer not 16-byte aligned                     */
  FA_ERR_ALIAS = -6,    /* an output overlaps an input or the other output   */
  FA_ERR_LAUNCH = -7,   /* the HIP runtime refused the kernel launch         */
  FA_ERR_SCALE = -8,    /* scale not finite or not > 0                       */
  FA_ERR_SIZE = -9,     /* too large for 32-bit in-head offsets or one grid  */
  FA_ERR_ARG = -10,     /* an argument outside its documented range          */
  FA_ERR_SCRATCH = -11, /* larger than the library's static scratch buffer    */
  FA_ERR_UNSUPPORTED = -12 /* not available in this build of the library       */
} fa_status;

typedef enum {
  FA_NORM_LAYER = 0,    /* LayerNorm: (z - mean) / sqrt(var + eps)           */
  FA_NORM_RMS = 1       /* RMSNorm:   z / sqrt(mean(z^2) + eps)              */
} fa_norm;

/*
 * Dense forward.
 *   Q, K, V, O : contiguous [B, H, N, d] tensors of `dtype`
 *                (element (b,h,n,k) at ((b*H + h)*N + n)*d + k).
 *   L          : contiguous [B, H, N] float32 (natural-log logsumexp).
 *   B, H, N    : >= 0; N*d must be below 2^31.
 * The [KV] kernel signature fa2(Q, K, V, O, L, N, scale) with its per-head
 * offsets bh*N*D and bh*N ("Steps"), widened by batch, heads, d and dtype.
 * Returns an fa_status.
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* L,
           int B, int H, int N, int d, float scale, int dtype, void* stream);

/*
 * Packed variable-length forward (self-attention within each sequence).
 *
 * Basis: the pages describe no variable-length forward. Their kernel runs
 * one (batch, head) of length N per set of blocks ("Kernel visualization:
 * Flash Attention 2", "Steps" and "Same operations in another block"), and
 * the flash-attention documentation mentions packed variable-length batches
 * only for the backward's dq_accum padding. This entry point is that same
 * per-head computation applied to every sequence of a packed batch, laid
 * out the way packed batches commonly are: token-major [T, H, d] tensors,
 * one array of cumulative sequence offsets shared by queries and keys, and
 * L as [H, T].
 *
 * total_tokens is an argument of its own because T = cu_seqlens[nseq] lives
 * in device memory: the host needs T, without a synchronising read of the
 * device, to bound the extents of Q, K, V, O and L for the alias and size
 * checks and to size the launch grid.
 *
 *   Q, K, V, O   : contiguous [T, H, d] tensors of `dtype`; token t of
 *                  head h at (t*H + h)*d. Sequence s owns tokens
 *                  cu_seqlens[s] .. cu_seqlens[s+1]-1 and attends to those
 *                  tokens only (no causal mask).
 *   L            : contiguous [H, T] float32; L[h*T + t].
 *   cu_seqlens   : device int32[nseq + 1], cu_seqlens[0] = 0, non-decreasing,
 *                  cu_seqlens[nseq] = total_tokens = T. Its contents are the
 *                  caller's responsibility: they are read on the device and
 *                  not checked.
 *   max_seqlen   : host-side upper bound of every sequence length; it sizes
 *                  the grid. Of a longer sequence, the first max_seqlen rows
 *                  are computed (against all of its keys), and the rows past
 *                  max_seqlen rounded up to the kernel's query block (128 or
 *                  256 rows) are not written. max_seqlen rounded up to a
 *                  multiple of 256, times H*d, must be below 2^31
 *                  (FA_ERR_SIZE otherwise).
 * Returns an fa_status.
 */
int fa_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* L,
                  const int32_t* cu_seqlens, int nseq, int total_tokens, int max_seqlen,
                  int H, int d, float scale, int dtype, void* stream);

/*
 * Dense banded (local-window) forward: as fa_fwd, except that query row r
 * only attends to the keys c with |r - c| <= window; the scores of all other
 * keys count as -inf before the row softmax:
 *
 *     S[r, c] = scale * dot(Q[r, :], K[c, :])   if |r - c| <= window, else -inf
 *     O, L    as for fa_fwd, over the kept keys only
 *
 * "FlashAttention -- for programmers, not researchers", DEMO 6, where the
 * local window (64 there) is the contrast to exact attention: a different
 * function. The key of a row's own index is always kept, so every O and L
 * is finite. Work grows with the window, not with N: a workgroup reads only
 * the key tiles that reach its rows' windows.
 *   Q, K, V, O, L : as for fa_fwd ([B, H, N, d] and [B, H, N]).
 *   window        : >= 0 (FA_ERR_SHAPE otherwise); window >= N - 1 keeps
 *                   every key and computes the same function as fa_fwd.
 *   dtype         : FA_F16 or FA_BF16 (FA_ERR_DTYPE otherwise).
 * Other checks and conventions as for fa_fwd. Returns an fa_status.
 */
int fa_fwd_banded(const void* Q, const void* K, const void* V, void* O, float* L,
                  int B, int H, int N, int d, int window, float scale, int dtype,
                  void* stream);

/*
 * Dense forward in the K/V-outer loop order (the traffic experiment): the
 * same O and L as fa_fwd, computed with the key/value tiles (64 keys) on the
 * outer loop. For every tile, each query row reads Q and reads back its
 * running output O (fp32) and statistics m, l from `acc`, applies the
 * online-softmax update, and writes them back; the last tile writes O / l
 * and L = m + ln l instead. "Kernel visualization: Flash Attention 2",
 * "Counting trips across HBM", explains why the Q-outer order of fa_fwd
 * never makes those round trips; this entry point exists to measure them.
 *   Q, K, V, O, L : as for fa_fwd ([B, H, N, d] and [B, H, N]).
 *   acc           : float32 scratch owned by the caller, B*H*N*(d + 2)
 *                   floats: the running O [B, H, N, d], then m [B, H, N],
 *                   then l [B, H, N]. Contents on entry are ignored; on
 *                   return they hold the state before the last tile.
 *   q_groups      : >= 1 (FA_ERR_SHAPE otherwise): workgroups that split
 *                   the query rows of one (batch, head); each streams all
 *                   of that head's K/V tiles. Capped at ceil(N / 32).
 *   dtype         : FA_F16 or FA_BF16 (FA_ERR_DTYPE otherwise).
 * All pointers 16-byte aligned; O, L and acc must not overlap each other or
 * Q, K, V (FA_ERR_ALIAS). Other checks as for fa_fwd. Returns an fa_status.
 */
int fa_fwd_kv_outer(const void* Q, const void* K, const void* V, void* O, float* L, float* acc,
                    int B, int H, int N, int d, int q_groups, float scale, int dtype,
                    void* stream);

/*
 * Fused dropout + residual add + LayerNorm / RMSNorm over rows of `hidden`
 * values: the fused op of flash-attention's documentation (the paragraph on
 * its dropout / residual / LayerNorm extension: pre- and post-norm, RMSNorm,
 * parallel residuals, hidden up to 8192 in multiples of 8). Per row:
 *
 *     z  = dropout(x0) + dropout(x1) + residual
 *     y0 = norm(z) * gamma0 + beta0,    y1 = norm(z) * gamma1 + beta1
 *     FA_NORM_LAYER: norm(z) = (z - mean) * rstd, rstd = 1/sqrt(var + eps)
 *     FA_NORM_RMS:   norm(z) = z * rstd,          rstd = 1/sqrt(mean(z^2) + eps)
 *
 * Dropout: element e = row*hidden + col of branch s (0 for x0, 1 for x1) is
 * kept when word e % 4 of Philox4x32-10 (Salmon et al., SC'11) at counter
 * (e / 4 mod 2^32, e / 4 div 2^32, offset mod 2^32, offset div 2^32 + s),
 * key (seed mod 2^32, seed div 2^32), is >= floor(dropout_p * 2^32); kept
 * values are multiplied by 1 / (1 - dropout_p) (fp32). dropout_p = 0 keeps
 * every element without drawing.
 *   x0            : [rows, hidden] of `dtype`; required.
 *   x1, residual  : [rows, hidden] or NULL (no parallel branch / no residual).
 *   gamma0, beta0 : [hidden] of `dtype`; gamma0 required, beta0 NULL = 0.
 *   gamma1, beta1 : second weight set or NULL; y1 is written iff gamma1 is
 *                   given (then y1 must be non-NULL, and beta1 needs gamma1).
 *   y0, y1        : [rows, hidden] outputs of `dtype`.
 *   z             : [rows, hidden] output of `dtype` or NULL (pre-norm keeps
 *                   it as the next residual; post-norm passes NULL).
 *   mean, rstd    : [rows] float32 or NULL; mean is written for LayerNorm only.
 *   mask          : uint8 keep flags or NULL: [rows, hidden] for x0, followed
 *                   by [rows, hidden] for x1 when x1 is given.
 *   hidden        : a multiple of 8, at most 8192 (FA_ERR_SHAPE otherwise).
 *   dropout_p     : 0 <= p < 1; eps > 0 and finite; norm an fa_norm value
 *                   (FA_ERR_ARG otherwise).
 *   dtype         : FA_F16 or FA_BF16 (FA_ERR_DTYPE otherwise).
 * Arithmetic in fp32: z is formed and kept in fp32, then rounded to dtype
 * for the z output only; mean and variance are two passes over z. Tensor
 * pointers 16-byte aligned, mean / rstd 4-byte aligned (FA_ERR_ALIGN);
 * outputs must not overlap inputs or each other (FA_ERR_ALIAS). rows = 0
 * or hidden = 0 is a no-op. Returns an fa_status.
 */
int fa_dropout_add_norm(const void* x0, const void* x1, const void* residual,
                        const void* gamma0, const void* beta0, const void* gamma1,
                        const void* beta1, void* y0, void* y1, void* z, float* mean,
                        float* rstd, unsigned char* mask, int rows, int hidden,
                        float dropout_p, uint64_t seed, uint64_t offset, float eps,
                        int norm, int dtype, void* stream);

/*
 * Dense backward: the gradients of sum(O * dO) with respect to Q, K and V.
 * "FlashAttention -- for programmers, not researchers", STAGE 5: the score
 * tiles are recomputed from the forward's row statistic L rather than kept
 * from the forward; the products are those of the backward list in the
 * flash-attention documentation (S = Q K^T, dP = dO V^T, dV = P^T dO,
 * dK = dS^T Q, dQ = dS K):
 *
 *     P[r, c]  = exp(S[r, c] - L[r])            (S as in the forward)
 *     D[r]     = sum_k dO[r, k] * O[r, k]
 *     dS[r, c] = P[r, c] * (sum_k dO[r, k] * V[c, k] - D[r])
 *     dV = P^T dO,   dQ = scale * dS K,   dK = scale * dS^T Q
 *
 *   Q, K, V, O, dO : contiguous [B, H, N, d] tensors of `dtype`; O and L as
 *                    fa_fwd wrote them for the same Q, K, V and scale.
 *   L              : contiguous [B, H, N] float32, natural-log logsumexp.
 *   dQ, dK, dV     : contiguous [B, H, N, d] tensors of `dtype`, written.
 *                    The first B*H*N*4 bytes of dQ also hold a per-row
 *                    intermediate before dQ itself is written (last).
 *   delta          : contiguous [B, H, N] float32 scratch owned by the
 *                    caller; receives -D (negated, the form the kernels
 *                    consume). Its contents on entry are ignored.
 *   dtype          : FA_F16 or FA_BF16 (FA_ERR_DTYPE otherwise: there is no
 *                    fp32 backward).
 * Arithmetic: products of dtype values summed in fp32; P and dS rounded to
 * dtype (round to nearest even) as operands of the products that consume
 * them; each gradient rounded to dtype once. Every output element is
 * produced by one workgroup in a fixed order, so results are bitwise
 * reproducible. All pointers 16-byte aligned (FA_ERR_ALIGN); dQ, dK, dV and
 * delta must not overlap each other or any input (FA_ERR_ALIAS). Other
 * checks and conventions as for fa_fwd. Returns an fa_status.
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
           const float* L, void* dQ, void* dK, void* dV, float* delta,
           int B, int H, int N, int d, float scale, int dtype, void* stream);

/*
 * Dense backward that allocates nothing: fa_bwd without the delta argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). The same
 * kernels compute the same dQ, dK, dV, bit for bit; -D = -rowsum(dO * O)
 * goes to a static device array of the library instead of caller scratch.
 *   - The array holds 2^22 float32 values (16 MiB): B*H*N must be at most
 *     4,194,304 (FA_ERR_SCRATCH otherwise, before anything is enqueued).
 *     Each GPU the library runs on holds its own copy from the first call on
 *     that device until the process ends.
 *   - The call makes no hipMalloc, hipFree or other allocating call. On its
 *     first use on a device it looks up that device's copy of the array
 *     (hipGetSymbolAddress, with that device current) and keeps the address;
 *     a failed lookup returns FA_ERR_LAUNCH.
 *   - `stream` must belong to the current device (FA_ERR_ARG otherwise).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in
 *     time on one GPU (on different streams, or from different threads
 *     without ordering) race on it and may return wrong gradients. Calls on
 *     one stream run in order and are safe. Every D value is written before
 *     it is read within a call, so nothing needs clearing between calls.
 * Arguments, checks and conventions otherwise as for fa_bwd. Returns an
 * fa_status.
 */
int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* L, void* dQ, void* dK, void* dV,
                   int B, int H, int N, int d, float scale, int dtype, void* stream);

/*
 * Phase trace of the 16-bit forward, for performance work. Only the debug
 * build libfa_trace.so (compiled with FA_DEBUG_TRACE) implements it; the
 * product library returns FA_ERR_UNSUPPORTED and records nothing.
 *
 * After this call, every fa_fwd / fa_fwd_varlen / fa_fwd_banded launch of the
 * 16-bit kernel has its workgroup number `workgroup` (launch order, as
 * blockIdx.x) record, per wave and for each of its first 64 key-tile steps,
 * the shader-clock timestamps (s_memtime) of the start and end of the wave's
 * matrix half and of its softmax half, and write them to `trace_buffer` when
 * it ends. Later launches overwrite the buffer. workgroup = -1 turns the
 * trace off.
 *   trace_buffer : device memory of at least 2080 uint64 values, 8-byte
 *                  aligned, owned by the caller: [wave 0..7][step 0..63]
 *                  [point 0..3], then per wave {s_memtime at the start,
 *                  s_memrealtime (100 MHz) at the start, s_memtime at the
 *                  end, s_memrealtime at the end}. Waves and steps that do not
 *                  exist keep their old contents.
 * The call is synchronous (it copies two values to device symbols) and is
 * not ordered with work already enqueued. Returns FA_ERR_NULL for a NULL
 * buffer with workgroup >= 0, FA_ERR_ALIGN for a misaligned one, FA_ERR_ARG
 * for workgroup < -1, FA_ERR_UNSUPPORTED in the product library,
 * FA_ERR_LAUNCH when the copies fail, else FA_OK.
 */
int fa_debug_fwd_trace(int workgroup, unsigned long long* trace_buffer);

/* Static, NUL-terminated description of an fa_status value. */
const char* fa_strerror(int status);

/* Library version, major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
