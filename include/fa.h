/*
 * fa.h -- C ABI of libfa.so: exact fused attention forward and split-KV
 * decode for AMD Instinct MI355X (gfx950).
 *
 * Pages cited (short names):
 *   [Evolution]  "FlashAttention evolution" (sandeep007734.github.io,
 *                posts/flashattention-evolution)
 *   [Kruglikov]  "Flash Attention" (vladislavkruglikov.com,
 *                articles/flash-attention)
 *   [Comparison] "FlashAttention 1-4 generation comparison"
 *                (phantomic12.github.io, inference-research)
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *     allocates no memory and keeps no state between calls (apart from the
 *     thread-local text of the last HIP error, and the fixed scratch array of
 *     fa_decode_splitkv_noalloc with its per-device address).  Calls from
 *     several host threads are safe, except overlapping calls of
 *     fa_decode_splitkv_noalloc on one GPU.
 *   - Layout: [B][H][N][d] contiguous, d fastest, bf16 (IEEE bfloat16 bit
 *     patterns in 16-bit words).  LSE is fp32.  Every tensor pointer must be
 *     16-byte aligned.
 *   - Calls only enqueue work on `stream` (a hipStream_t; NULL means the
 *     default stream) and return; nothing is synchronised.  A fault inside a
 *     kernel surfaces at the caller's next synchronisation.
 *   - Every argument check runs before any HIP call.  On a negative return
 *     nothing was enqueued and no output byte was written.
 *   - Every kernel-side scratch buffer is a caller workspace argument, except
 *     in fa_decode_splitkv_noalloc.
 *   - Results are deterministic: no atomics, fixed reduction order.
 *   - Non-finite inputs are not checked; the result is then undefined.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = -1,       /* a required pointer is NULL                      */
  FA_ERR_SHAPE = -2,      /* B, H or N <= 0, Hq % Hkv != 0, causal && Nq > Nk,
                             serving decode Nq outside 1..16                 */
  FA_ERR_HEAD_DIM = -3,   /* d not in {32, 64, 128, 256}                     */
  FA_ERR_ALIGN = -4,      /* a tensor pointer is not 16-byte aligned         */
  FA_ERR_WORKSPACE = -5,  /* workspace NULL or smaller than required         */
  FA_ERR_SPLITS = -6,     /* num_splits outside 0 .. fa_decode_max_splits()  */
  FA_ERR_HIP = -7,        /* a HIP launch failed; see fa_last_hip_error()    */
  FA_ERR_SCALE = -8,      /* scale not finite or not > 0                     */
  FA_ERR_ALIAS = -9,      /* an output overlaps an input or another output   */
  FA_ERR_TOO_LARGE = -10, /* sizes exceed the 2^31 grid / 2^62 byte limits   */
  FA_ERR_SCRATCH = -11    /* fa_decode_splitkv_noalloc: the partials need more
                             than FA_DECODE_NOALLOC_SCRATCH_BYTES            */
};

/*
 * fa_fwd -- exact attention forward with per-row log-sum-exp.
 *
 * Computes, for every batch b, query head h, query row i:
 *   O[b,h,i,:] = sum_j P[i,j] V[b,g,j,:],   P = softmax_j(scale * Q K^T)
 *   LSE[b,h,i] = ln sum_{j allowed} exp(scale * q_i . k_j)
 * with g = h / (Hq / Hkv) (grouped-query heads share a KV head).  This is the
 * function of [Evolution] §1 (the equation under "The Invariant and the
 * Moving Bottleneck") with the scale of [Kruglikov]'s scaled dot-product
 * attention; as [Kruglikov] "The IO problem" describes, only O and one
 * number per row (here the natural-log LSE) are written, the score and
 * probability tiles never leave the chip.
 *
 * causal = 1 keeps key j for row i iff j <= i + (Nk - Nq) (bottom-right
 * aligned; j <= i when Nq == Nk).  causal with Nq > Nk is rejected so that no
 * row is empty.
 *
 *   q      bf16 [B][Hq][Nq][d]
 *   k, v   bf16 [B][Hkv][Nk][d]
 *   o      bf16 [B][Hq][Nq][d]   output, rounded to nearest even
 *   lse    fp32 [B][Hq][Nq]      output, natural log
 *   scale  finite, > 0 (1/sqrt(d) for standard attention)
 *   causal 0 or 1
 *   stream hipStream_t or NULL
 * Returns FA_OK or a negative fa_status.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
           int causal, void* stream);

/*
 * fa_fwd_fp8 -- the forward of fa_fwd with fp8 inputs and fp8 products.
 *
 * FlashAttention-3 runs both products in 8-bit floating point ([Evolution]
 * §4; [Comparison] "Notes", FA-3 entry).  Here q, k, v are OCP fp8 e4m3
 * bytes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, largest
 * value 448) with one dequantisation factor per tensor: the real inputs are
 * byte value * q_descale (k_descale, v_descale).  The function computed is
 * fa_fwd's on those real values; inside, S = Q K^T is exact up to fp32
 * accumulation and P is rounded to e4m3 before P V, which bounds the error
 * of each output element by about 2^-4 * max|v| (plus bf16 rounding of O).
 * Incoherent processing (the random Hadamard rotation of Q and K) happens
 * before quantisation, in fa_fp8_quantize below; this call takes the codes.
 *
 *   q         fp8 e4m3 [B][Hq][Nq][d]
 *   k, v      fp8 e4m3 [B][Hkv][Nk][d]
 *   o         bf16 [B][Hq][Nq][d]     output
 *   lse       fp32 [B][Hq][Nq]        output, natural log of the scaled scores
 *   d         32, 64, 128 or 256
 *   scale, q_descale, k_descale, v_descale  finite, > 0
 * Errors as fa_fwd (FA_ERR_HEAD_DIM for d other than 32, 64, 128, 256).
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
               float q_descale, float k_descale, float v_descale, int causal,
               void* stream);

/*
 * fa_fwd_fp8_devscale -- fa_fwd_fp8 with the three dequantisation factors
 * read from device memory when the kernel starts (each a single fp32, as
 * fa_fp8_quantize writes it), so that quantisation and attention run on one
 * stream without a host round trip.  q_descale, k_descale, v_descale are
 * device pointers (4-byte aligned, not overlapping o or lse); their values
 * must be finite and > 0.  Other arguments and errors as fa_fwd_fp8.
 */
int fa_fwd_fp8_devscale(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                        const float* q_descale, const float* k_descale,
                        const float* v_descale, int causal, void* stream);

/*
 * fa_fp8_quantize -- the fp8 input step: incoherent processing and
 * per-tensor e4m3 quantisation ([Comparison] "Notes", FA-3 entry: FP8 with
 * a Hadamard transform; [Evolution] §4).
 *
 * Q and K are rotated along the head dimension by the same random
 * orthogonal matrix R = diag(signs) H_d / sqrt(d), H_d the Sylvester
 * Hadamard matrix (H[i][j] = (-1)^popcount(i & j)), which leaves Q K^T
 * unchanged and spreads one channel's outliers over all d channels; V is
 * quantised without rotation (signs NULL).  For a tensor x of `rows` rows
 * of d values:
 *   y        = x R                (x without signs)
 *   descale  = max |y| / 448      (1 when x is all zero)
 *   codes    = e4m3(y / descale)  round to nearest, ties to even, within
 *                                 +-448; the sign of y is kept (-0 = 0x80)
 * so that codes * descale approximates y to 3 mantissa bits.  The rotation
 * runs in fp32 as a fast Walsh-Hadamard transform; its 1/sqrt(d) goes into
 * descale only.
 *
 *   x         bf16 [rows][d] (any [B][H][N][d] tensor: rows = B*H*N)
 *   codes     fp8 e4m3 [rows][d]    output
 *   descale   device fp32, 1 value  output (feed to fa_fwd_fp8_devscale)
 *   signs     device int8 [d], negative = -1, otherwise +1; or NULL
 *   d         32, 64, 128 or 256
 *   workspace device scratch of at least fa_fp8_quantize_workspace_size(rows,
 *             d) bytes, 16-byte aligned; its contents on entry do not matter
 * Two kernels on `stream`: the first writes one partial maximum per
 * workgroup into the workspace, the second reduces them and writes codes and
 * descale.  Errors: FA_ERR_NULL, FA_ERR_SHAPE (rows <= 0), FA_ERR_HEAD_DIM,
 * FA_ERR_ALIGN (x, codes, workspace not 16-byte or descale not 4-byte
 * aligned), FA_ERR_WORKSPACE, FA_ERR_ALIAS (codes, descale or workspace
 * overlapping each other, x or signs).
 */
size_t fa_fp8_quantize_workspace_size(int rows, int d);
int fa_fp8_quantize(const void* x, void* codes, float* descale, const void* signs, int rows,
                    int d, void* workspace, size_t workspace_bytes, void* stream);

/* Kernel symbol of fa_fp8_quantize: stage 0 the maximum pass, 1 the
 * quantising pass; NULL for an unsupported d. */
const char* fa_fp8_quantize_kernel_name(int d, int stage);

/*
 * Split-KV decode ([Evolution] §6, Flash-Decoding): one query row per
 * sequence against a long KV cache.  The keys are cut into num_splits
 * contiguous chunks; one kernel computes, per (b, KV head, chunk), the
 * chunk-normalised partial output and chunk LSE for all query heads of that
 * KV head (each K/V byte is read once per KV head); a second kernel merges
 * the chunks with the log-sum-exp identity:
 *   M = max_s LSE_s,  w_s = exp(LSE_s - M),
 *   O = sum_s w_s O_s / sum_s w_s,  LSE = M + ln sum_s w_s.
 * Chunks are ceil(Nk / num_splits) keys rounded up to a multiple of 64; a
 * chunk that falls past Nk is empty and gets weight 0.
 *
 *   q         bf16 [B][Hq][d]
 *   k_cache   bf16 [B][Hkv][Nk][d]
 *   v_cache   bf16 [B][Hkv][Nk][d]
 *   o         bf16 [B][Hq][d]       output
 *   lse       fp32 [B][Hq]          output, natural log
 *   num_splits 0 = fa_decode_num_splits(B, Hq, Hkv, Nk, d), else
 *             1 .. fa_decode_max_splits(Nk)
 *   workspace device scratch of at least
 *             fa_decode_workspace_size(B, Hq, d, splits) bytes (splits after
 *             the 0 -> heuristic substitution), 16-byte aligned, owned by the
 *             caller; it must not overlap any tensor argument.  Its contents
 *             on return are unspecified.
 */
int fa_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                      void* o, float* lse, int B, int Hq, int Hkv, int Nk,
                      int d, float scale, int num_splits, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * fa_decode_splitkv_noalloc -- fa_decode_splitkv without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * stream capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * The split partials go to a fixed array inside the library of
 * FA_DECODE_NOALLOC_SCRATCH_BYTES (16 MiB), which every GPU the library runs
 * on holds from the library's load until the process ends.  The call
 * allocates nothing and frees nothing.  The first call on a device looks up
 * that device's copy of the array (with the device current); later calls
 * reuse the address.
 *
 * Arguments, results and errors as fa_decode_splitkv, plus FA_ERR_SCRATCH
 * when fa_decode_workspace_size(B, Hq, d, splits) exceeds
 * FA_DECODE_NOALLOC_SCRATCH_BYTES (e.g. B = 8, Hq = 32, d = 128 allows up to
 * 127 splits).  `stream` must belong to the current device (else FA_ERR_HIP).
 * Outputs equal fa_decode_splitkv's bit for bit for the same split count.
 *
 * Every call on one GPU shares that GPU's array, and the array keeps the last
 * call's contents (nothing needs clearing: each call writes every partial it
 * reads).  Calls that can overlap on one GPU -- on different streams, or
 * from different host threads -- race on it; serialise them (one stream, or
 * events between the streams).
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)
int fa_decode_splitkv_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              void* o, float* lse, int B, int Hq, int Hkv, int Nk, int d,
                              float scale, int num_splits, void* stream);

/*
 * fa_decode_serve -- serving-shaped split-KV decode: Nq (1..16) query rows
 * per sequence and a per-sequence KV length, over a padded cache.
 *
 * The same split/merge method as fa_decode_splitkv ([Evolution] §6) for
 * the decode step of a serving engine ([Evolution] §7 compares one), where
 * each sequence of a batch has its own cache length (up to tens of
 * thousands of tokens, [Evolution] §6) and a step may score several new
 * tokens at once.  For sequence b with n_b =
 * seqlens[b] keys (clamped to 0..Nk; seqlens NULL means n_b = Nk for all b),
 * query row i attends to keys j < n_b, and with causal = 1 only to
 * j <= n_b - Nq + i (the rows are the last Nq positions of the sequence).
 * Each sequence's keys are cut into num_splits chunks of
 * ceil(n_b / num_splits) keys rounded up to a multiple of 64; chunks past
 * n_b are empty and get weight 0.  A row with no allowed key (n_b = 0, or
 * causal rows with n_b - Nq + i < 0) gets O = 0 and LSE = -inf.
 *
 *   q         bf16 [B][Hq][Nq][d]
 *   k_cache   bf16 [B][Hkv][Nk][d]   (Nk = capacity; rows >= n_b are not read)
 *   v_cache   bf16 [B][Hkv][Nk][d]
 *   seqlens   int32 [B] device array, 4-byte aligned, or NULL
 *   o         bf16 [B][Hq][Nq][d]    output
 *   lse       fp32 [B][Hq][Nq]       output, natural log
 *   num_splits 0 = fa_decode_serve_num_splits(...), else 1 .. fa_decode_max_splits(Nk)
 *   workspace at least fa_decode_serve_workspace_size(B, Hq, Nq, d, splits)
 *             bytes, 16-byte aligned, caller-owned, overlapping no tensor.
 */
int fa_decode_serve(const void* q, const void* k_cache, const void* v_cache,
                    const int* seqlens, void* o, float* lse, int B, int Hq, int Hkv,
                    int Nq, int Nk, int d, float scale, int causal, int num_splits,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of serving-decode workspace: 4*B*Hq*Nq*S*(d+1).  0 on invalid sizes. */
size_t fa_decode_serve_workspace_size(int B, int Hq, int Nq, int d, int num_splits);

/* Split count used by fa_decode_serve when num_splits == 0 (as
 * fa_decode_num_splits, for the workgroups the Nq rows need); negative
 * fa_status for invalid sizes. */
int fa_decode_serve_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d);

/* Bytes of decode workspace: fp32 partial outputs [B][Hq][S][d] followed by
 * fp32 partial LSEs [B][Hq][S], i.e. 4*B*Hq*S*(d+1).  0 on invalid sizes. */
size_t fa_decode_workspace_size(int B, int Hq, int d, int num_splits);

/* Split count used when num_splits == 0: enough (b, KV head, chunk) work
 * groups to fill the GPU several times over, chunks of at least 256 keys.
 * Returns a value in 1 .. fa_decode_max_splits(Nk), or a negative fa_status
 * for invalid sizes. */
int fa_decode_num_splits(int B, int Hq, int Hkv, int Nk, int d);

/* Largest accepted num_splits for a cache of Nk keys: ceil(Nk / 64). */
int fa_decode_max_splits(int Nk);

/*
 * fa_bwd -- gradients of fa_fwd's output.
 *
 * For a loss whose gradient with respect to O is dO, computes with
 * P = exp(S - LSE), S = scale * Q K^T (masked keys: P = 0, as in fa_fwd):
 *   dV = P^T dO,  dP = dO V^T,  dS = P (dP - Delta),  Delta_i = dO_i . O_i,
 *   dQ = scale * dS K,  dK = scale * dS^T Q,
 * grouped-query heads summing into their shared KV head's dK, dV.  The pages
 * print no gradient formulas: these are the chain rule applied to fa_fwd's
 * function.  As [Comparison] "Notes" (FlashAttention-1 entry) describes for
 * the backward pass, the probabilities are recomputed from Q, K and the
 * forward's LSE instead of being stored.
 *
 *   q, o, dout bf16 [B][Hq][Nq][d]     (o: fa_fwd's output; dout: dL/dO)
 *   k, v       bf16 [B][Hkv][Nk][d]
 *   lse        fp32 [B][Hq][Nq]        fa_fwd's LSE (natural log)
 *   dq         bf16 [B][Hq][Nq][d]     output
 *   dk, dv     bf16 [B][Hkv][Nk][d]    outputs
 *   d          32, 64, 128 or 256
 *   scale, causal  the values the forward used
 *   workspace  device scratch of at least fa_bwd_workspace_size(B, Hq, Nq)
 *              bytes (Delta, fp32), 16-byte aligned, owned by the caller; it
 *              must not overlap any tensor argument.  Contents on return are
 *              unspecified.
 * Two kernels run in stream order (dQ and Delta, then dK and dV); there are
 * no atomics, so repeated calls give identical bits.
 * Returns FA_OK or a negative fa_status (FA_ERR_WORKSPACE for a NULL or
 * short workspace, FA_ERR_ALIAS if an output or the workspace overlaps an
 * input or another output).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv,
           int Nq, int Nk, int d, float scale, int causal, void* workspace,
           size_t workspace_bytes, void* stream);

/* Bytes of backward workspace: 4*B*Hq*Nq (Delta, fp32).  0 on invalid sizes. */
size_t fa_bwd_workspace_size(int B, int Hq, int Nq);

/* Static text for a status code. */
const char* fa_strerror(int status);

/* Text of the last HIP error seen by this host thread ("" if none). */
const char* fa_last_hip_error(void);

/* 1 for the race-check build of this library (every staged copy into LDS
 * completes, behind waits and workgroup barriers, before anything else
 * runs; its outputs must equal the pipelined build's bit for bit), 0 for
 * the product build. */
int fa_build_is_serial(void);

/* Kernel symbol names, as a profiler reports them, so a benchmark can
 * confirm which kernel ran: [Evolution] §1.1 ("Before comparing versions,
 * identify the kernel") asks every measurement to record the kernel that
 * actually executed.  NULL for an unsupported head dimension or
 * invalid sizes.  fa_fwd_kernel_name: the forward kernel fa_fwd launches for
 * these sizes (the tile depends on d and, for d = 128, on the key length).
 * fa_decode_kernel_name: stage 0 = split kernel (depends on the number of
 * query heads per KV head), stage 1 = merge kernel. */
const char* fa_fwd_kernel_name(int d, int causal, int Nq, int Nk);
const char* fa_decode_kernel_name(int d, int hq_per_kv, int stage);
/* fa_bwd_kernel_name: stage 0 = dQ kernel (also writes Delta), stage 1 =
 * dK/dV kernel. */
const char* fa_bwd_kernel_name(int d, int causal, int stage);
/* fa_decode_serve_kernel_name: stage 0 = split kernel (depends on the query
 * heads per KV head and on Nq), stage 1 = merge kernel. */
const char* fa_decode_serve_kernel_name(int d, int hq_per_kv, int Nq, int stage);
/* fa_fwd_fp8_kernel_name: the fp8 forward kernel for d and causal. */
const char* fa_fwd_fp8_kernel_name(int d, int causal);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
