/*
 * fa.h -- C ABI of the exact-attention library for AMD Instinct MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention
 *
 *     O = softmax(scale * Q K^T + bias, masked) V
 *
 * the tiled, IO-aware way: Q is cut into row blocks and K/V into column blocks,
 * each score tile lives only in registers, a running row max and row sum rescale
 * the output accumulator (online softmax), and the N x N score matrix never
 * reaches device memory. The backward pass recomputes the score tiles from Q, K
 * and the saved log-sum-exp.
 *
 * Sources (pages cited by title and section):
 *  - "Apakah Konteks Sehari Penuh Mengalahkan Konteks Sepuluh Menit? Perhatian
 *    Kilat dan Pertanyaan Panjang Urutan" (marketmaker.cc blog on Flash
 *    Attention): sections "Algoritma Flash Attention" (tiling and the per-block
 *    loop), "Pengulangan softmax online" (running max/sum rescaling),
 *    "Backward pass: menghitung ulang, bukan menyimpan" (keep only O and the
 *    softmax statistics, recompute tiles), "FA2: paralelisme" (deferred
 *    normalisation, parallelism over query blocks, per-wave query rows),
 *    "Causal masking adalah tempat perdagangan mendapat diskon" (skip tiles in
 *    the future), "Integrasinya delapan baris" ((batch, heads, seq, head_dim)
 *    layout; causal is a flag; never fall back silently to a slow path).
 *  - scifaro.com "related papers: FlashMask: Efficient and Rich Mask Extension
 *    of FlashAttention": attention with an additive bias on the query-key scores.
 *  - briefgpt.xyz page for arXiv 2307.08691, FlashAttention abstract: the
 *    tiled method extends to block-sparse attention.
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, contiguous [B, H, N, d] with d innermost (element
 *    (b,h,n,c) at ((b*H + h)*N + n)*d + c). LSE is [B, H, N_q] float32.
 *  - Pointers named "device" must be device memory of the current HIP device,
 *    16-byte aligned. The caller owns every buffer; the library allocates and
 *    frees nothing and keeps no state between calls (one exception: the fixed
 *    scratch array that fa_bwd_noalloc uses in place of a workspace).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the calls return without synchronising. Inputs must stay valid until the
 *    stream has passed the call.
 *  - Arguments are validated before anything is enqueued. On any error the
 *    call returns a non-zero fa_status and enqueues nothing; there is no
 *    fallback to another algorithm. A launch failure returns FA_ERR_HIP.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of the shared library (it is built with hidden default visibility). */
#define FA_API __attribute__((visibility("default")))

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,       /* B, H, N_q or N_k < 1, or a size overflows 32-bit indexing */
  FA_ERR_DTYPE = 3,       /* unknown dtype or gradient dtype */
  FA_ERR_HEADDIM = 4,     /* d not in {64, 128} */
  FA_ERR_MASK = 5,        /* malformed mask/bias descriptor */
  FA_ERR_ALIGN = 6,       /* a device pointer is misaligned (16 bytes; 4 for float32 arrays
                             such as lse, the bias tensor, dbias and dslopes) */
  FA_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than fa_bwd_workspace_bytes() */
  FA_ERR_UNSUPPORTED = 8, /* a valid combination this build does not implement */
  FA_ERR_HIP = 9,         /* the HIP runtime reported an error at launch */
  FA_ERR_ARG = 10,        /* scale not finite or not positive; a slope not finite; bad phase set */
  FA_ERR_SCRATCH = 11     /* fa_bwd_noalloc: the sizes need more than FA_NOALLOC_SCRATCH_BYTES */
} fa_status;

typedef enum fa_dtype { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

typedef enum fa_bias_kind {
  FA_BIAS_NONE = 0,
  /* bias(h, i, j) = slopes[h] * |i - j|, i and j absolute row/column indices,
     generated on the fly (never stored); added after scaling (see fa_fwd). */
  FA_BIAS_DIST_LINEAR = 1,
  /* bias(b, h, i, j) = bias[b * bias_stride_b + h * bias_stride_h + i * bias_stride_i + j],
     a float32 tensor in device memory (see the descriptor); added after scaling. */
  FA_BIAS_TENSOR = 2
} fa_bias_kind;

#define FA_MAX_SLOPES 256

/* Optional bias and key-range mask.
 *  bias_kind : fa_bias_kind.
 *  slopes    : HOST pointer to n_slopes floats (read during the call only);
 *              n_slopes == 1 applies slopes[0] to every head, n_slopes == H gives
 *              one slope per head (H <= FA_MAX_SLOPES). Ignored for FA_BIAS_NONE.
 *  key_start, key_end : DEVICE pointers to N_q int32 each, or both NULL.
 *              Query row i attends exactly to keys j with
 *              key_start[i] <= j < key_end[i] (one interval per row, shared by
 *              every batch and head). Any int32 values are allowed: the interval
 *              is intersected with [0, N_k); an empty interval gives an empty row.
 *  block_mask : DEVICE pointer to a block-sparse bitmap of bytes, or NULL (then the
 *              five fields below are ignored). The score matrix of every (b, h) is cut
 *              into blocks of block_q query rows by block_k keys; block (r, c) is
 *              visible when
 *                block_mask[b * mask_stride_b + h * mask_stride_h + r * n_kb + c] != 0
 *              with n_kb = ceil(N_k / block_k), r < ceil(N_q / block_q). Entries of an
 *              invisible block are masked like keys outside a row's key range (the
 *              method skips such tiles: briefgpt.xyz page for arXiv 2307.08691, its
 *              FlashAttention abstract on the extension to block-sparse attention, and
 *              the related abstract on sparsity patterns such as key/query dropping).
 *  block_q, block_k : block sizes, multiples of 64 (else FA_ERR_MASK).
 *  mask_stride_b, mask_stride_h : bitmap strides in bytes between batches and heads;
 *              0 shares one bitmap over that axis (negative: FA_ERR_MASK).
 *              The bitmap is read during the enqueued work; it must stay valid until the
 *              stream has passed the call. 16-bit inputs skip the tiles of invisible
 *              blocks; float32 inputs apply the bitmap as a mask (same result).
 *              N_q and N_k at most FA_MAX_SPARSE_N (FA_ERR_UNSUPPORTED beyond).
 *  dslopes : DEVICE pointer to n_slopes floats, or NULL. fa_bwd (and fa_bwd_phases with
 *              FA_BWD_DKDV) writes there the gradient of the same loss with respect to the
 *              bias slopes: dL/dslope_h = sum over b, i, j of dS_{b,h,i,j} |i - j| (dS the
 *              gradient with respect to the scores), or its sum over heads for one shared
 *              slope; it needs FA_BIAS_DIST_LINEAR (else FA_ERR_MASK). The reduction runs
 *              in a fixed order, so the result is deterministic. fa_fwd ignores it.
 *  bias :      FA_BIAS_TENSOR only: DEVICE pointer to float32 values, 4-byte aligned
 *              (NULL: FA_ERR_NULL; misaligned: FA_ERR_ALIGN). Element (b, h, i, j) is read
 *              at the offset given for FA_BIAS_TENSOR; the key index j has stride 1.
 *              Any array the caller can index that way works: a dense [B, H, N_q, N_k]
 *              tensor, or one broadcast over batches, heads or query rows by a zero
 *              stride. Attention with an additive bias matrix on the query-key scores
 *              (scifaro.com related-papers page for FlashMask, arXiv 2410.01359: the
 *              abstract on attention with bias); -inf entries act as a mask; +inf or NaN
 *              entries give undefined results. Read during the enqueued work. Works
 *              together with a block bitmap, dbias and its summed forms included.
 *  bias_stride_b, bias_stride_h, bias_stride_i : element strides, >= 0 (else FA_ERR_MASK);
 *              64 * bias_stride_i + N_k must stay below 2^30 (else FA_ERR_UNSUPPORTED).
 *  dbias :     DEVICE pointer to a dense float32 array (4-byte aligned), or NULL. fa_bwd
 *              (and fa_bwd_phases with FA_BWD_DKDV) writes there the gradient of the loss
 *              with respect to the bias: dS_{b,h,i,j}, the gradient with respect to each
 *              biased score (zero where masked), summed over the axes that dbias_reduce
 *              names. Needs FA_BIAS_TENSOR (else FA_ERR_MASK). fa_fwd ignores it.
 *  dbias_reduce : 0, or an OR of FA_DBIAS_SUM_BATCH, FA_DBIAS_SUM_HEADS, FA_DBIAS_SUM_ROWS
 *              (other bits, or nonzero without dbias: FA_ERR_MASK). dbias is dense
 *              [B', H', N_q', N_k] with B' = 1 when batches are summed (else B), H' = 1
 *              when heads are summed (else H), N_q' = 1 when query rows are summed (else
 *              N_q): the gradient of a bias broadcast over those axes, e.g. [1, H, N_q, N_k]
 *              for one bias matrix per head shared over the batch, [B, 1, 1, N_k] for a
 *              per-key bias. Every element is written (zero where nothing is visible).
 *              The sums run in a fixed order (batches, then heads, then rows), so the
 *              result is deterministic. Summing batches or heads makes one workgroup
 *              compute every (b, h) that shares a dbias slice, one after the other: the
 *              dK/dV launch then has B' H' (not B H) times ceil(N_k / 128) workgroups.
 *  A row with no visible key (after causal, range and block masking) gets O = 0 and
 *  LSE = -inf. */
#define FA_MAX_SPARSE_N 65536
typedef struct fa_mask_bias_desc {
  int32_t bias_kind;
  int32_t n_slopes;
  const float* slopes;
  const int32_t* key_start;
  const int32_t* key_end;
  const uint8_t* block_mask;
  int32_t block_q;
  int32_t block_k;
  int64_t mask_stride_b;
  int64_t mask_stride_h;
  float* dslopes;
  const float* bias;
  int64_t bias_stride_b;
  int64_t bias_stride_h;
  int64_t bias_stride_i;
  float* dbias;
  int32_t dbias_reduce;
} fa_mask_bias_desc;
#define FA_DBIAS_SUM_BATCH 1
#define FA_DBIAS_SUM_HEADS 2
#define FA_DBIAS_SUM_ROWS 4

/* Forward pass.
 *  q [B,H,N_q,d], k and v [B,H,N_k,d]: device, element type `dtype`.
 *  o [B,H,N_q,d]: device, output, element type `dtype` (rounded to nearest even).
 *  lse [B,H,N_q]: device float32 output, natural-log log-sum-exp of each row's
 *                 scaled, biased, masked scores (saved for fa_bwd); may be NULL.
 *  d in {64, 128}; N_q, N_k >= 1 (any value: tail tiles are masked).
 *  scale > 0 and finite (1/sqrt(d) is the usual choice); otherwise FA_ERR_ARG.
 *  causal != 0: query i sees key j only if j <= i + (N_k - N_q) (bottom-right
 *               aligned diagonal; identical to the usual rule when N_q == N_k).
 *  mb: NULL for no bias and no range mask.
 *  Math: s_ij = scale * q_i.k_j + bias(h,i,j), -inf where masked;
 *        O_i = sum_j softmax(s_i)_j v_j ; LSE_i = log sum_j exp(s_ij).
 *  Accumulation is float32 (bf16/f16 inputs go through bf16/f16 MFMA with the
 *  probabilities rounded to the input type before the P.V product). */
FA_API fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N_q, int N_k, int d, float scale, int causal,
                 const fa_mask_bias_desc* mb, fa_dtype dtype, void* stream);

/* Forward with tile counters, to verify that tiles no row can see are neither loaded nor
 * computed (blog "Apakah Konteks Sehari Penuh...", section "Causal masking adalah
 * tempat perdagangan mendapat diskon": key tiles in the future of every query of a block
 * are never loaded or computed, about half of the work for causal attention; the same
 * holds for key ranges and block bitmaps).
 * Computes exactly what fa_fwd computes, with the same launches, and in addition adds
 *  counts[0]: the number of key tiles loaded into on-chip memory, summed over workgroups,
 *  counts[1]: the number of (wave, key tile) score blocks computed, summed over waves,
 * (device, two 8-byte-aligned uint64 the caller has zeroed; atomically added, so calls
 * may accumulate) and writes to the HOST array config the launch's geometry:
 *  config[0] = query rows per workgroup, config[1] = query rows per wave,
 *  config[2] = keys per tile.
 * Without a bitmap a workgroup loads the tiles from the one holding the first key any of
 * its rows can see to the one holding the last, and a wave computes the tiles of that
 * span for its own 32 rows; with a bitmap only tiles whose block byte is set for some
 * wave (workgroup) or for the wave (wave count) are counted. So tiles that no row of the
 * workgroup (wave) can see are never loaded (computed) when the visible keys of its rows
 * form one span, as for causal masks and key ranges of overlapping rows.
 * Errors: as fa_fwd; FA_ERR_NULL without counts or config; FA_ERR_ALIGN for misaligned
 * counts; FA_ERR_UNSUPPORTED for float32 inputs (counted in the 16-bit kernels only). */
FA_API fa_status fa_fwd_tile_counts(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int B, int H, int N_q, int N_k, int d,
                                    float scale, int causal, const fa_mask_bias_desc* mb,
                                    fa_dtype dtype, void* stream, unsigned long long* counts,
                                    int* config);

/* Split-key forward, for shapes with few query rows per head (decode-like: N_q small,
 * N_k long), where one workgroup per (b, h, query block) leaves most compute units idle.
 * The keys of every head are cut into n_split consecutive ranges (multiples of 64 keys);
 * each (b, h, query block, range) computes a partial softmax-normalised output and its
 * LSE into `workspace`, and a second launch merges them with the same rescaling algebra
 * as the online softmax: LSE = log sum_r exp(LSE_r), O = sum_r exp(LSE_r - LSE) O_r.
 * Sources: briefgpt.xyz page for arXiv 2307.08691 (its related abstract on speeding up
 * the decode phase by spreading one sequence's keys over parallel workers); blog
 * "Apakah Konteks Sehari Penuh...", sections "FA2: paralelisme" (parallelise along the
 * sequence when batch x heads alone starves the GPU) and "Pengulangan softmax online"
 * (partial results combine exactly through their running max and sum).
 *  All arguments except the three below mean exactly what they mean for fa_fwd, and the
 *  result equals fa_fwd's up to float32 rounding order.
 *  n_split: requested number of key ranges; 0 picks a count from the shape. Ranges are
 *           whole 64-key tiles of equal length (the last one shorter), so the effective
 *           count (fa_fwd_split_count) can be lower than requested and never exceeds
 *           ceil(N_k / 64). With an effective count of 1 the call is fa_fwd (workspace
 *           unused, may be NULL).
 *  workspace: device, 16-byte aligned, at least fa_fwd_split_workspace_bytes(...) bytes
 *           for the same sizes and n_split; contents on entry do not matter; the call
 *           overwrites it. Calls sharing one workspace must not overlap on the device.
 *  Errors: as fa_fwd; FA_ERR_WORKSPACE if the workspace is NULL or too small (effective
 *  count > 1); FA_ERR_ARG if n_split < 0. */
FA_API fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int N_q, int N_k, int d, float scale, int causal,
                              const fa_mask_bias_desc* mb, fa_dtype dtype, int n_split,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Effective key-range count fa_fwd_split uses for this shape and request (n_split = 0:
 * the automatic choice, about two (b, h, query block, range) units per compute unit,
 * at least four 64-key tiles per range). Returns 0 for invalid sizes. */
FA_API int fa_fwd_split_count(int B, int H, int N_q, int N_k, int d, int n_split);

/* Bytes of workspace fa_fwd_split needs: n * B * H * N_q * (d + 1) float32 partials for
 * the effective count n (0 when n == 1). */
FA_API size_t fa_fwd_split_workspace_bytes(int B, int H, int N_q, int N_k, int d, int n_split);

/* Bytes of device workspace fa_bwd needs for these sizes (caller allocates). */
FA_API size_t fa_bwd_workspace_bytes(int B, int H, int N_q, int N_k, int d);

/* Backward pass by recomputation.
 *  q, k, v, o, dout: device, element type `dtype`, same shapes as in fa_fwd;
 *  lse: device float32 [B,H,N_q] exactly as written by fa_fwd for these inputs.
 *  dq [B,H,N_q,d], dk and dv [B,H,N_k,d]: device outputs of type `grad_dtype`
 *  (FA_F32 or `dtype`); they are fully overwritten.
 *  workspace: device, at least fa_bwd_workspace_bytes(...) bytes, 16-byte aligned;
 *  its contents on entry do not matter.
 *  Gradients of L = sum(O * dout): dV = P^T dO; dP = dO V^T; D_i = rowsum(dO_i * O_i);
 *  dS = P * (dP - D); dQ = scale * dS K; dK = scale * dS^T Q, with
 *  P = exp(S - LSE) recomputed tile by tile. No gradient flows to bias or mask (dbias and
 *  dslopes in the descriptor ask for the bias gradients explicitly).
 *  16-bit inputs: products on 16-bit MFMA with P and dS rounded to the input type,
 *  float32 accumulation. float32 inputs: every product on float32 MFMA, nothing rounded
 *  below float32 (gradients float32). The result is deterministic (a fixed order of every
 *  sum, dbias summed over batches or heads included). */
FA_API fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, fa_dtype grad_dtype,
                 void* workspace, size_t workspace_bytes,
                 int B, int H, int N_q, int N_k, int d, float scale, int causal,
                 const fa_mask_bias_desc* mb, fa_dtype dtype, void* stream);

/* The launches of fa_bwd, selectable for callers that schedule or time them apart:
 *  FA_BWD_PREP: D = rowsum(dO * O) and the key-range summary, into the workspace;
 *  FA_BWD_DKDV: dK and dV (needs a completed FA_BWD_PREP on the same workspace);
 *  FA_BWD_DQ:   dQ (needs a completed FA_BWD_PREP on the same workspace).
 *  FA_BWD_DQ_ATOMIC (with FA_BWD_DKDV, in place of FA_BWD_DQ): the dK/dV launch also
 *               forms dQ = scale dS K for its block of keys and adds it into dq with
 *               float32 atomic adds; dq must be float32 (grad_dtype FA_F32) and is cleared
 *               by the call first. The order of the additions varies from run to run, so
 *               dQ is not bitwise reproducible (dK, dV are). 16-bit inputs without a
 *               block bitmap or a bias tensor (else FA_ERR_UNSUPPORTED); without
 *               FA_BWD_DKDV, or together with FA_BWD_DQ: FA_ERR_ARG. This is the
 *               recomputation backward with the dQ accumulation kept in the key-outer
 *               pass (marketmaker.cc attention page, the section on the backward pass
 *               recomputing rather than storing); FA_BWD_DQ recomputes S and dP in a
 *               query-outer pass instead, deterministically.
 *  Phases given together run in that order. fa_bwd(...) is fa_bwd_phases(FA_BWD_ALL, ...).
 *  `phases` must be a non-empty subset of FA_BWD_ALL | FA_BWD_DQ_ATOMIC (else
 *  FA_ERR_ARG); the other arguments are validated exactly as for fa_bwd. */
#define FA_BWD_PREP 1
#define FA_BWD_DKDV 2
#define FA_BWD_DQ 4
#define FA_BWD_ALL 7
#define FA_BWD_DQ_ATOMIC 8
FA_API fa_status fa_bwd_phases(int phases, const void* q, const void* k, const void* v,
                               const void* o, const float* lse, const void* dout, void* dq,
                               void* dk, void* dv, fa_dtype grad_dtype, void* workspace,
                               size_t workspace_bytes, int B, int H, int N_q, int N_k, int d,
                               float scale, int causal, const fa_mask_bias_desc* mb,
                               fa_dtype dtype, void* stream);

/* Allocation-free backward, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving or training loops, harnesses that forbid hipMalloc.
 * Computes exactly what fa_bwd computes (the same kernels, bit for bit), with the same
 * arguments except the workspace: the library keeps a fixed device array of
 * FA_NOALLOC_SCRATCH_BYTES bytes per GPU (allocated when the library is loaded, held until
 * the process ends) and uses it in place of the caller's workspace. The call itself
 * allocates and frees nothing; the caller still provides every input and output.
 *  Limit: fa_bwd_workspace_bytes(B, H, N_q, N_k, d) <= FA_NOALLOC_SCRATCH_BYTES, i.e. about
 *         2 * 4 bytes per (b, h, query row): B * H * N_q up to about 2 million rows;
 *         larger problems return FA_ERR_SCRATCH (checked before anything is enqueued).
 *  Concurrency: every call on one GPU uses that GPU's one array; calls whose work can
 *         overlap on the device (different streams, or other host threads) race and give
 *         undefined gradients. Calls in order on one stream are safe: each call writes
 *         everything it reads from the array before reading it.
 *  Errors: as fa_bwd (FA_ERR_WORKSPACE never), plus FA_ERR_SCRATCH, and FA_ERR_HIP if the
 *         array's device address cannot be obtained. */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)
FA_API fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, void* dq, void* dk,
                                void* dv, fa_dtype grad_dtype, int B, int H, int N_q, int N_k,
                                int d, float scale, int causal, const fa_mask_bias_desc* mb,
                                fa_dtype dtype, void* stream);

/* Key-range summary of consecutive blocks of `block_rows` query rows.
 *  key_start, key_end: device int32 [N_q] (same meaning as in fa_mask_bias_desc).
 *  out: device int32 [ceil(N_q / block_rows) * 4]; block r gets
 *       {min start, max start, min end, max end} after clamping to [0, N_k].
 *  A column tile [c0, c1) is fully masked for block r if c1 <= min start or
 *  c0 >= max end, and fully visible if max start <= c0 and min end >= c1.
 *  block_rows in [1, 1024]. */
FA_API fa_status fa_mask_summary(const int32_t* key_start, const int32_t* key_end, int N_q, int N_k,
                          int block_rows, int32_t* out, void* stream);

/* ---------------------------------------------------------------------------------
 * FP8 forward with block quantisation and incoherent processing.
 * Source: marketmaker.cc blog on Flash Attention, section "FA3: Mekanika hopper",
 * item 3 (FP8 at twice the 16-bit matrix rate; plain FP8 attention is spoiled by
 * outliers; a random rotation of the vectors before block quantisation spreads an
 * outlier over all coordinates, with a reported 2.6x lower error).
 *
 * Format: OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * largest finite 448; no infinities). A tensor [B,H,N,d] is quantised in blocks of 64
 * rows of one (b, h): N is padded with zero rows to Np = fa_fp8_rows(N) (a multiple of
 * 64), block i covers rows 64i .. 64i+63, and amax[b,h,i] = max |x| over the block.
 * FA_FP8_Q, FA_FP8_K: a value x becomes code RNE(clamp(x * (448 / amax), -448, 448)),
 * whose stored value is decode(c) * amax / 448. FA_FP8_V: the block scale is a power of
 * two, 2^e with e the smallest integer >= -127 such that amax <= 448 * 2^e (e = 0 for an
 * all-zero block); x becomes code RNE(x * 2^-e), stored value decode(c) * 2^e (the P V
 * product of fa_fwd_fp8 applies 2^e as its E8M0 operand scale, exactly). For Q and K
 * the rows may first be rotated:
 * x -> x diag(signs) H_d, with H_d the Sylvester Hadamard matrix (entries +-1,
 * H_d H_d^T = d I) and signs a caller-drawn vector of +-1; Q and K must use the same
 * signs, and then (Q M)(K M)^T = d Q K^T, which fa_fwd_fp8 divides out.
 *
 * Byte layouts of x8 (B*H*Np*d bytes, (b, h) major, then 64-row tiles t of 64*d bytes):
 *  FA_FP8_Q: row-major, row r of tile t at byte 64*t*d + r*d + column.
 *  FA_FP8_K: row r (key 64t + r) at r*d inside its tile; the 16-byte chunk c of the
 *            row (columns 16c .. 16c+15) sits in slot c ^ z(r), z(r) = (r >> 1) & 7 for
 *            d = 128 and (r >> 2) & 3 for d = 64.
 *  FA_FP8_V: transposed: column e of the tile is a 64-byte row at e*64; key 64t + k
 *            sits at position p(k) = 16*(k >> 5) + 32*((k >> 2) & 1) + 4*((k & 31) >> 3)
 *            + (k & 3) of that row, and the row's 16-byte chunk c sits in slot
 *            c ^ ((e >> 2) & 3).
 * (K and V are stored as the forward's LDS tile images, so it copies them linearly.)
 * --------------------------------------------------------------------------------- */
typedef enum fa_fp8_layout { FA_FP8_Q = 0, FA_FP8_K = 1, FA_FP8_V = 2 } fa_fp8_layout;

/* Rows of a quantised tensor with N rows: N rounded up to a multiple of 64 (0 if N < 1). */
FA_API int fa_fp8_rows(int N);

/* Quantise x [B,H,N,d] (device, dtype FA_BF16 or FA_F16, d in {64, 128}) into
 *  x8:   device, B*H*fa_fp8_rows(N)*d bytes, in `layout`'s byte order;
 *  amax: device float32 [B, H, fa_fp8_rows(N)/64], the block amaxes (of the rotated
 *        values when rotating).
 *  signs: HOST pointer to d floats, each exactly +1 or -1 (read during the call), to
 *        rotate (FA_FP8_Q and FA_FP8_K only; NULL: no rotation; with FA_FP8_V: FA_ERR_ARG).
 * The rotation is computed exactly (float64 sums of the 16-bit inputs) and rounded once
 * to float32; amax, 448/amax and the products are float32 (for V the product with
 * 2^-e is exact). One launch, one workgroup per block. */
FA_API fa_status fa_fp8_quantize(const void* x, int B, int H, int N, int d, fa_dtype dtype,
                                 fa_fp8_layout layout, const float* signs, void* x8, float* amax,
                                 void* stream);

/* FP8 forward: O and LSE of attention with scores
 *   s_ij = scale * <q_i, k_j> (divided by d when rotated != 0),
 * from operands quantised by fa_fp8_quantize (q8 with FA_FP8_Q, k8 with FA_FP8_K, v8 with
 * FA_FP8_V; q_amax, k_amax, v_amax their amax arrays; all device). causal as fa_fwd.
 * o [B,H,N_q,d] device in out_dtype (FA_BF16 or FA_F16), lse [B,H,N_q] float32 or NULL.
 * Both products run on E4M3 MFMA with float32 accumulation: S^T = K Q^T on the codes,
 * scaled by the block scales; the probabilities (at most 2^8 with the lazy rescale) are
 * rounded to E4M3 for O^T += V^T P^T (each key tile's V block scale applied by the
 * product), while the row sum uses them unrounded; O is the result over the row sum. */
FA_API fa_status fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_amax,
                            const float* k_amax, const float* v_amax, void* o, float* lse, int B,
                            int H, int N_q, int N_k, int d, float scale, int causal, int rotated,
                            fa_dtype out_dtype, void* stream);

/* Static description of a status code (never NULL). */
FA_API const char* fa_status_string(fa_status s);

/* Library version string, e.g. "fa 0.1.0 gfx950". */
FA_API const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
