/*
 * fa.h -- C ABI of libfa.so: exact IO-aware attention (FlashAttention) on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation: for every batch b and head h, with S = scale * Q K^T,
 *   O = softmax(S) V   (softmax over each row of S; causal keeps key j <= query i)
 * computed exactly, in tiles that stay on chip, without ever writing the
 * N x N score matrix to device memory (groundtruth.day, "FlashAttention:
 * making attention fast by respecting the memory hierarchy": paragraphs on the
 * cost of attention, on tiling with an online softmax, and on the payoff in
 * linear memory). The forward saves one softmax statistic per query row, the
 * natural-log logsumexp lse_i = ln sum_j exp(S_ij), and the backward
 * recomputes the score and probability tiles on chip from Q, K, V and lse
 * (michaelc-yu summary of Dao et al., "Backward / recomputation").
 *
 * Layout: q, k, v, o, dout, dq, dk, dv are contiguous [B, H, N, d] arrays
 * (d innermost) of the element type named by `dtype`; lse is a contiguous
 * [B, H, N] float array. Every pointer is a device pointer, 16-byte aligned.
 *
 * Ownership: every buffer belongs to the caller. The library keeps no pointer
 * after a call returns, allocates no device memory and is reentrant; its only
 * global state is the fixed per-device scratch buffer of fa_decode_noalloc (and
 * that buffer's looked-up address per device). Outputs must not overlap inputs.
 *
 * Execution: a call only enqueues kernels on `stream` (a hipStream_t; NULL is
 * the default stream) and returns without synchronising. Device faults show
 * up at the caller's next synchronisation.
 *
 * Errors: every argument is checked before any HIP call. The library never
 * prints, aborts or throws across this boundary; it returns a status code.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v, o, dout, dq, dk, dv. Accumulation is always fp32. */
typedef enum {
    FA_BF16 = 0, /* bfloat16; MFMA bf16 path */
    FA_FP16 = 1, /* IEEE half; MFMA f16 path */
    FA_FP32 = 2  /* IEEE single; exact fp32 vector path, d = 64 only */
} fa_dtype;

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,  /* null or misaligned pointer, B/H/N < 1, causal not 0/1,
                                scale not finite and > 0, overlapping buffers, size overflow */
    FA_ERR_UNSUPPORTED = 2,  /* d not in {64, 128}, unknown dtype, fp32 with d = 128,
                                unknown dQ strategy, FA_DQ_ATOMIC with 16-bit d = 128 */
    FA_ERR_WORKSPACE = 3,    /* workspace null, not 256-byte aligned, or smaller than
                                fa_bwd_workspace_size() */
    FA_ERR_HIP = 4,          /* a kernel launch failed (hipGetLastError after launch) */
    FA_ERR_SCRATCH = 5       /* fa_decode_noalloc: the shape needs more scratch than the
                                library's fixed per-device buffer (FA_DECODE_SCRATCH_BYTES) */
} fa_status;

/* How fa_bwd_dq() forms dQ. */
typedef enum {
    FA_DQ_DEFAULT = 0,   /* the strategy measured fastest on MI355X: FA_DQ_SEPARATE */
    FA_DQ_ATOMIC = 1,    /* fp32 atomic adds into a workspace accumulator, then a convert pass */
    FA_DQ_SEPARATE = 2   /* query workgroups recompute the tiles and write dQ directly, in the
                            same launch as the dK/dV workgroups */
} fa_dq_strategy;

/*
 * Forward pass.
 *   q, k, v : inputs, [B,H,N,d] of `dtype`.
 *   o       : output, [B,H,N,d] of `dtype`, O = softmax(scale Q K^T (+ causal mask)) V.
 *   lse     : output, [B,H,N] float, lse_i = ln sum_j exp(scale q_i.k_j) over visible keys.
 *   scale   : score multiplier (usually 1/sqrt(d)); must be finite and > 0.
 *   causal  : 0 = every key visible, 1 = key j visible to query i iff j <= i.
 *   stream  : hipStream_t to enqueue on.
 * Any N >= 1 is accepted (a partial last tile is masked). Returns a fa_status.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, int dtype, void* stream);

/*
 * Bytes of device workspace the backward needs for this shape, whatever the
 * dQ strategy: D_i = dO_i . O_i ([B,H,N] float), lse_i * log2(e) ([B,H,N]
 * float) and, for bf16/fp16, the fp32 dQ accumulator of FA_DQ_ATOMIC
 * ([B,H,N,d] float), each part rounded up to 256 bytes. All O(N). Returns 0
 * for invalid shapes.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d, int dtype);

/*
 * Backward pass of L = sum(dout * O): writes dq, dk, dv ([B,H,N,d] of `dtype`).
 *   q, k, v, o, lse : the forward's inputs and outputs (o and lse exactly as fa_fwd wrote them).
 *   dout            : upstream gradient dL/dO, [B,H,N,d] of `dtype`.
 *   workspace       : caller-owned device memory of at least fa_bwd_workspace_size() bytes,
 *                     256-byte aligned; its contents on entry do not matter.
 * Reads only q, k, v, o, dout and lse; recomputes every score and probability tile
 * on chip from them (michaelc-yu summary of Dao et al., "Backward / recomputation").
 * 16-bit inputs: d in {64, 128}; fp32: d = 64. Uses the default dQ strategy.
 * Equivalent to fa_bwd_prep() followed by fa_bwd_main(). Returns a fa_status.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           void* workspace, size_t workspace_bytes, void* stream);

/* fa_bwd() with an explicit fa_dq_strategy (ignored for FA_FP32, which has one path;
 * FA_DQ_ATOMIC exists for d = 64 only and returns FA_ERR_UNSUPPORTED for 16-bit d = 128). */
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, void* dq, void* dk, void* dv,
              int B, int H, int N, int d, float scale, int causal, int dtype, int dq_strategy,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * First stage of the backward, for callers that schedule the stages themselves:
 * one pass over o and dout that writes D_i = dO_i . O_i and lse_i * log2(e) into
 * the workspace (and, for FA_DQ_ATOMIC, zeroes its fp32 dQ accumulator). For
 * FA_FP32 it validates and returns (the fp32 backward forms D in fa_bwd_main).
 * Arguments as fa_bwd_dq(). Returns a fa_status.
 */
int fa_bwd_prep(const void* o, const void* dout, const float* lse, int B, int H, int N, int d, int dtype,
                int dq_strategy, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Second stage of the backward: dq, dk, dv from q, k, v, dout and a workspace that
 * fa_bwd_prep() filled, on the same stream, for the same o, dout, lse and strategy
 * (a workspace prepared for another strategy gives wrong results). For bf16/fp16
 * with the default strategy this is a single kernel launch. Arguments as
 * fa_bwd_dq(). Returns a fa_status.
 */
int fa_bwd_main(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv,
                int B, int H, int N, int d, float scale, int causal, int dtype, int dq_strategy,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block-sparse attention (the block-sparse extension of the method that the
 * michaelc-yu summary of Dao et al. names in its abstract without defining it;
 * reading: exact attention with whole blocks of the score matrix dropped).
 * The score matrix of a head is cut into FA_SPARSE_BLOCK x FA_SPARSE_BLOCK
 * blocks, nb = ceil(N / FA_SPARSE_BLOCK) per side. block_mask holds, per
 * mask, nb x nb bytes in row-major order (row = query block, column = key
 * block): a nonzero byte keeps the block, zero drops it (its pairs are masked
 * like the causal upper triangle, and its tiles are never loaded or computed).
 * Causal masking applies on top. A query row that keeps no key gets O = 0,
 * lse = -inf, and no gradient.
 *   block_mask        : device memory, read only; head (b, h) uses the mask that
 *                       starts mask_head_stride * (b * H + h) bytes in.
 *   mask_head_stride  : 0 (one mask for every head) or >= nb * nb.
 *   workspace         : caller-owned device memory, 256-byte aligned, at least
 *                       fa_fwd_sparse_workspace_size() / fa_bwd_sparse_workspace_size()
 *                       bytes; its contents on entry do not matter.
 * bf16/fp16 only (FA_FP32 -> FA_ERR_UNSUPPORTED), d in {64, 128}. Other arguments,
 * errors and semantics as fa_fwd / fa_bwd (overlaps with the mask or the
 * workspace -> FA_ERR_INVALID_ARG; mask_head_stride invalid or mask NULL ->
 * FA_ERR_INVALID_ARG). Returns a fa_status.
 */
#define FA_SPARSE_BLOCK 128

size_t fa_fwd_sparse_workspace_size(int B, int H, int N, long long mask_head_stride);
size_t fa_bwd_sparse_workspace_size(int B, int H, int N, long long mask_head_stride);

int fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int N, int d, float scale, int causal, int dtype,
                  const void* block_mask, long long mask_head_stride,
                  void* workspace, size_t workspace_bytes, void* stream);

int fa_bwd_sparse(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv,
                  int B, int H, int N, int d, float scale, int causal, int dtype,
                  const void* block_mask, long long mask_head_stride,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP8 forward (the lower-precision continuation of the method that the
 * groundtruth.day page names in its lineage paragraph without defining it;
 * reading: the same attention on e4m3 inputs, the softmax in fp32, the weights
 * rounded to e4m3 for the P V product).
 *   q, k, v : [B,H,N,d] OCP e4m3 bytes (1 byte per element), device memory.
 *   *_descale: positive finite fp32 factors; the real inputs are byte value x descale.
 *   o       : [B,H,N,d] bf16 output; lse: [B,H,N] fp32 (natural log of the scaled scores,
 *             as fa_fwd writes it).
 * d in {64, 128}; any N >= 1; causal 0/1; scale as fa_fwd. Rounding the weights to
 * 3 mantissa bits costs about 2 % relative RMS on O for Gaussian inputs. Errors as
 * fa_fwd (non-positive or non-finite descale -> FA_ERR_INVALID_ARG). Returns a fa_status.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               float q_descale, float k_descale, float v_descale, void* stream);

/*
 * Attention of a few new queries over a long key/value cache (decoding; the pages
 * name the cache beside the method, groundtruth.day payoff paragraph). The same
 * exact attention, tiled with an online softmax and split over the keys; the
 * splits are merged with their row statistics (lse = log sum exp lse_s,
 * O = sum exp(lse_s - lse) O_s).
 *   q       : [B,H,Nq,d] of `dtype`, the last Nq positions of the sequence, 1 <= Nq <= 8.
 *   k, v    : [B,H,Nk,d] of `dtype`, the cache (Nk >= 1; causal needs Nk >= Nq).
 *   o, lse  : [B,H,Nq,d] of `dtype` and [B,H,Nq] fp32 (natural log).
 *   causal  : 1 = query t sees keys j <= t + Nk - Nq; 0 = every key.
 *   workspace: caller-owned device memory, 256-byte aligned, at least
 *             fa_decode_workspace_size() bytes (the per-split partial results).
 * bf16/fp16, d in {64, 128} (else FA_ERR_UNSUPPORTED, also for Nq > 8). Errors
 * and semantics otherwise as fa_fwd. Returns a fa_status.
 */
size_t fa_decode_workspace_size(int B, int H, int Nq, int Nk, int d);

int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. The per-split partial results go to a fixed buffer of
 * FA_DECODE_SCRATCH_BYTES that the library holds in each device's memory for
 * the life of the process; the call allocates nothing. Same arguments,
 * semantics and results as fa_decode (the same kernels and split plan), except:
 *   - shapes whose fa_decode_workspace_size() exceeds FA_DECODE_SCRATCH_BYTES are
 *     rejected with FA_ERR_SCRATCH (checked before any HIP call);
 *   - `stream` must belong to the current device (else FA_ERR_INVALID_ARG);
 *   - every call on a device shares that device's buffer: calls that may overlap
 *     on one device (several streams, several host threads) race and must be
 *     serialised by the caller. Calls on different devices do not interact.
 * The buffer's contents between calls are unspecified (each call writes every
 * part it reads). On first use on a device the library looks up the buffer's
 * address there (hipGetSymbolAddress; a failure returns FA_ERR_HIP).
 */
#define FA_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                      void* stream);

/*
 * General shapes for the 16-bit forward: strided layouts (for instance [B,N,H,d]
 * storage, "BSHD", seen as [B,H,N,d]), Nq queries against Nk keys, and
 * sequences of different lengths padded into one batch.
 *   fa_strides      : element strides of a [B,H,N,d] view (the head-dim stride is 1);
 *                     every stride >= 0 and a multiple of 8, the row stride below 2^23,
 *                     each view's base 16-byte aligned.
 *   q, o            : Nq rows per (batch, head); k, v: Nk rows.
 *   lse             : [B,H,Nq] fp32, contiguous.
 *   seqlens_q/_k    : NULL, or device arrays of B ints: sequence b has seqlens_q[b]
 *                     queries and seqlens_k[b] keys (clamped to [0, Nq] / [0, Nk]); rows
 *                     past a sequence's queries are neither computed nor written.
 *   causal          : the queries are the last positions of their sequence: query i of
 *                     sequence b sees keys j <= i + seqlens_k[b] - seqlens_q[b]; a row that
 *                     sees no key gets O = 0 and lse = -inf.
 * dtype bf16/fp16, d in {64, 128}. Errors as fa_fwd (overlapping views, bad strides or
 * misaligned bases -> FA_ERR_INVALID_ARG). Returns a fa_status.
 */
typedef struct {
    long long batch, head, row;
} fa_strides;

int fa_fwd_general(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                   const fa_strides* q_strides, const fa_strides* k_strides,
                   const fa_strides* v_strides, const fa_strides* o_strides,
                   const int* seqlens_q, const int* seqlens_k, void* stream);

/*
 * Bytes of device workspace fa_bwd_general needs: D_i = dO_i . O_i and
 * lse_i * log2(e), [B,H,Nq] float each, each part rounded up to 256 bytes.
 * Returns 0 for invalid shapes.
 */
size_t fa_bwd_general_workspace_size(int B, int H, int Nq);

/*
 * Backward over the general shapes of fa_fwd_general (recomputation from lse as
 * in fa_bwd): strided q, k, v, o, dout, dq, dk, dv views, Nq queries against Nk
 * keys, per-sequence lengths, causal alignment at the end.
 *   q, o, dout, dq  : Nq rows per (batch, head); k, v, dk, dv: Nk rows.
 *   lse             : [B,H,Nq] fp32, contiguous, as fa_fwd_general wrote it.
 *   seqlens_q/_k    : as fa_fwd_general. Rows of dq past a sequence's queries and
 *                     rows of dk, dv past its keys are neither computed nor written;
 *                     a key that no query sees gets dK = dV = 0.
 *   workspace       : caller-owned, 256-byte aligned, at least
 *                     fa_bwd_general_workspace_size() bytes.
 * dtype bf16/fp16, d in {64, 128}. Errors as fa_fwd_general (outputs that overlap
 * each other, an input or the workspace -> FA_ERR_INVALID_ARG). Returns a fa_status.
 */
int fa_bwd_general(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                   const fa_strides* q_strides, const fa_strides* k_strides,
                   const fa_strides* v_strides, const fa_strides* o_strides,
                   const fa_strides* dout_strides, const fa_strides* dq_strides,
                   const fa_strides* dk_strides, const fa_strides* dv_strides,
                   const int* seqlens_q, const int* seqlens_k,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable name of a fa_status value. Never NULL. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
