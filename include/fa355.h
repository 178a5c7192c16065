/*
 * libfa355 -- exact tiled scaled-dot-product attention with online softmax
 * (FlashAttention) for AMD Instinct MI355X (gfx950), forward and backward.
 *
 * What is computed (all pages agree that the tiled method returns the plain
 * definition up to rounding: "FlashAttention and the Kernel Era", The
 * Mathematics, SDPA equation; "FlashAttention 1, 2, and 3 Explained",
 * section 1):
 *
 *     S = scale * Q K^T   (key j hidden from query i when causal and j > i)
 *     P = softmax(S) row by row,   O = P V,   lse_i = ln sum_j exp(S_ij)
 *
 * computed block by block without forming the N x N matrices (running row
 * max and row sum with rescaling of the output accumulator: "FlashAttention
 * and the Kernel Era", The Mathematics, online-softmax equation; "FlashAttention
 * 1, 2, and 3 Explained", section 2), and the backward pass rebuilds P from
 * Q, K and the saved lse instead of storing it ("FlashAttention Kernel"
 * glossary, Recomputation bullet).
 *
 * Layouts (row-major, densely packed, no strides):
 *   q, o, dout, dq : [B, H_q,  N, d]
 *   k, v, dk, dv   : [B, H_kv, N, d]
 *   lse            : [B, H_q,  N] float32, natural log
 * Query head h reads K/V head h / (H_q / H_kv) (grouped-query / multi-query
 * attention, "FlashAttention" glossary, KV-cache paragraph).  All of q, k, v,
 * o, dout, dq, dk, dv share one element type `dtype`.
 *
 * Ownership: every pointer is a device pointer owned by the caller; the
 * library allocates no device memory and keeps no pointer after a call
 * returns.  Inputs are only read.  Outputs must not overlap inputs or each
 * other.  Every buffer must be 16-byte aligned.  The library's only state is
 * a per-device cache of the compute-unit count, for fa_bwd_noalloc one fixed
 * scratch array per device (see there), and two rings of 64 small counter
 * slots per device (part of the code object, not allocated) through which the
 * causal forward and dK/dV kernels hand out their last blocks at run time, so
 * that the chip's faster XCDs take more of them.  Each launch takes the next
 * slot (host-side atomic) and leaves it at zero when it ends; at most 64
 * launches of one of these kernels may be in flight on one device at once.
 * Every cache is initialised once in a thread-safe way.
 *
 * Timing and errors: calls enqueue work on `stream` and return without
 * synchronising.  Argument errors are reported synchronously and nothing is
 * enqueued.  A failed launch returns FA_ERR_HIP.  Faults inside a kernel
 * surface at the caller's next synchronisation.  No C++ exception crosses
 * this interface.
 */
#ifndef FA355_H
#define FA355_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, bad flag, small workspace */
    FA_ERR_UNSUPPORTED = 2, /* head dim or dtype the library has no kernel for */
    FA_ERR_HIP = 3,         /* the HIP runtime refused a launch */
    FA_ERR_TOO_LARGE = 4    /* exceeds the fixed scratch of fa_bwd_noalloc */
} fa_status;

typedef enum {
    FA_DTYPE_FP32 = 0,
    FA_DTYPE_FP16 = 1,
    FA_DTYPE_BF16 = 2
} fa_dtype;

/*
 * Forward pass: O = softmax(scale * Q K^T [causal]) V and lse.
 *
 *   q, k, v   in : see layouts above.
 *   o         out: [B, H_q, N, d], dtype.
 *   lse       out: [B, H_q, N] float32, ln sum_j exp(scale * q_i . k_j) over
 *                  the keys visible to row i.
 *   B, H_q, H_kv, N >= 1; H_q % H_kv == 0; d in {64, 128}.
 *   causal in {0, 1}: when 1, key j is visible to query i iff j <= i.
 *   scale: finite and > 0 (the pages' equation uses 1 / sqrt(d)); any other
 *          value is rejected with FA_ERR_INVALID_ARG.
 * Needs no workspace: memory beyond the inputs and outputs is O(1)
 * ("FlashAttention Kernel" glossary: memory drops from O(N^2) to O(N)).
 */
fa_status fa_fwd(const void* q, const void* k, const void* v,
                 void* o, float* lse,
                 int B, int H_q, int H_kv, int N, int d,
                 int causal, float scale, fa_dtype dtype, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes: the float32 row
 * terms D_i = sum_k dO_ik O_ik, [B, H_q, N], rounded up to 256 bytes.
 * Returns 0 for invalid sizes.  Linear in N.
 */
size_t fa_bwd_workspace_size(int B, int H_q, int H_kv, int N, int d, fa_dtype dtype);

/*
 * Backward pass: gradients of sum(dout * O) with respect to q, k, v
 * (the pages give no gradient formulas; these are the chain rule through
 * O = P V and the row-wise softmax: D_i = sum_k dO_ik O_ik, dP = dO V^T,
 * dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO).
 *
 *   q, k, v, o, lse  in : exactly what fa_fwd took and returned.
 *   dout             in : [B, H_q, N, d], dtype.
 *   dq               out: [B, H_q, N, d], dtype.
 *   dk, dv           out: [B, H_kv, N, d], dtype; for grouped heads each is
 *                         the sum over the H_q / H_kv query heads reading it.
 *   workspace        scratch of at least fa_bwd_workspace_size() bytes,
 *                    owned by the caller; contents on entry are ignored and
 *                    on return are unspecified.
 * P is rebuilt per tile from q, k and lse ("FlashAttention Kernel" glossary,
 * Recomputation bullet), once in a pass over key blocks that accumulates dK
 * and dV, and once in a pass over query blocks that accumulates dQ; every
 * accumulator is float32 until the final rounding to dtype.  Results are
 * deterministic (no atomics).
 */
fa_status fa_bwd(const void* q, const void* k, const void* v,
                 const void* o, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 int B, int H_q, int H_kv, int N, int d,
                 int causal, float scale, fa_dtype dtype, hipStream_t stream);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments and results are those of fa_bwd, and it
 * runs the same kernels; the row terms fa_bwd keeps in `workspace` live in a
 * fixed device array of FA_NOALLOC_SCRATCH_BYTES bytes that the library holds
 * on every device it runs on until the process ends.
 *
 * Limit: fa_bwd_workspace_size(B, H_q, H_kv, N, d, dtype) must not exceed
 * FA_NOALLOC_SCRATCH_BYTES (B * H_q * N <= 4,194,304 rows); larger problems
 * return FA_ERR_TOO_LARGE and enqueue nothing.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).  Every call on one
 * device shares that device's array and leaves its contents behind; each
 * call writes every entry it reads before reading it, so nothing needs
 * clearing.  Calls that overlap on one device (different streams, or
 * threads, without ordering between them) race on the array: order them.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v,
                         const void* o, const float* lse, const void* dout,
                         void* dq, void* dk, void* dv,
                         int B, int H_q, int H_kv, int N, int d,
                         int causal, float scale, fa_dtype dtype, hipStream_t stream);

/*
 * The three phases fa_bwd runs, for callers that schedule them themselves
 * (for example dK/dV and dQ on two streams once the row terms are ready).
 * Arguments mean what they mean for fa_bwd; `delta` is a float32
 * [B, H_q, N] buffer (16-byte aligned), owned by the caller.
 *
 * fa_bwd_prepare: delta_i = sum_k dout_ik o_ik for every query row.
 * fa_bwd_dkdv:    dk, dv from q, k, v, lse, dout and delta (rebuilds P and
 *                 dP per key block; sums grouped query heads).
 * fa_bwd_dq:      dq from q, k, v, lse, dout and delta (rebuilds P and dP per
 *                 query block).
 * fa_bwd_dkdv and fa_bwd_dq only read delta and may run concurrently once
 * fa_bwd_prepare has completed.
 */
fa_status fa_bwd_prepare(const void* o, const void* dout, float* delta,
                         int B, int H_q, int N, int d, fa_dtype dtype, hipStream_t stream);

fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v,
                      const float* lse, const void* dout, const float* delta,
                      void* dk, void* dv,
                      int B, int H_q, int H_kv, int N, int d,
                      int causal, float scale, fa_dtype dtype, hipStream_t stream);

fa_status fa_bwd_dq(const void* q, const void* k, const void* v,
                    const float* lse, const void* dout, const float* delta,
                    void* dq,
                    int B, int H_q, int H_kv, int N, int d,
                    int causal, float scale, fa_dtype dtype, hipStream_t stream);

/*
 * Split-KV forward (FlashDecoding: "FlashAttention" glossary, the
 * FlashDecoding paragraph): the same attention for a few query rows against
 * a long key/value sequence, parallelised over the key length.  The keys are
 * cut into num_splits chunks; each chunk yields a float32 partial output
 * normalised over its own keys and the logsumexp of its scores, and a second
 * pass merges them with the online-softmax rescale ("FlashAttention 1, 2,
 * and 3 Explained", section 2): lse = ln sum_s exp(lse_s),
 * O = sum_s exp(lse_s - lse) O_s.
 *
 *   q         in : [B, H_q, N_q, d], dtype.
 *   k, v      in : [B, H_kv, N_kv, d], dtype.
 *   o         out: [B, H_q, N_q, d], dtype.
 *   lse       out: [B, H_q, N_q] float32, natural log, over the visible keys.
 *   workspace scratch of at least fa_fwd_splitkv_workspace_size() bytes,
 *             16-byte aligned, owned by the caller; its contents on entry are
 *             ignored and on return hold the per-chunk partials:
 *             float32 [num_splits, B * H_q * N_q, d] partial outputs, then
 *             (at the next 256-byte boundary) float32 [num_splits,
 *             B * H_q * N_q] partial logsumexps (-inf for a chunk in which a
 *             row sees no key).
 *   causal in {0, 1}: when 1 the queries are the last N_q positions of the
 *          sequence, so query i sees keys j <= i + N_kv - N_q; requires
 *          N_q <= N_kv.  With N_q == N_kv this is fa_fwd's mask.
 *   num_splits in [1, 1024]: number of key chunks (keys are dealt in chunks
 *          of ceil(N_kv / num_splits) rounded up to the kernel's key tile, so
 *          trailing chunks may be empty); fa_fwd_splitkv_default_splits()
 *          suggests one.
 *   d in {64, 128}; dtype bf16 or fp16 (fp32 returns FA_ERR_UNSUPPORTED).
 *   Other sizes and checks as for fa_fwd.
 */
fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v,
                         void* o, float* lse,
                         void* workspace, size_t workspace_bytes,
                         int B, int H_q, int H_kv, int N_q, int N_kv, int d,
                         int causal, float scale, int num_splits,
                         fa_dtype dtype, hipStream_t stream);

/* Workspace bytes fa_fwd_splitkv needs for these sizes (0 if invalid). */
size_t fa_fwd_splitkv_workspace_size(int B, int H_q, int N_q, int d, int num_splits);

/* A chunk count that fills the device for these sizes (0 if invalid). */
int fa_fwd_splitkv_default_splits(int B, int H_q, int H_kv, int N_q, int N_kv, int d);

/*
 * Attention dropout, fused into the kernels ("FlashAttention Kernel" glossary,
 * opening paragraph; "FlashAttention" glossary, kernel-fusion paragraph;
 * "Flash Attention" (21medien), fusion bullet and the dropout_p argument of
 * its code example):
 *
 *     P = softmax(scale * Q K^T [causal]),   O = (P o Z) V * 256 / t8,
 *
 * Z the keep mask: element (b, h, i, j) (query head h, row i, key j) is kept
 * iff its random byte is below t8 = round((1 - dropout_p) * 256), computed in
 * double from the float dropout_p.  The bytes come from the counter-based
 * generator Philox4x64-10 (Salmon et al., SC 2011) with key (seed, offset) and
 * counter (j / 32, i, b * H_q + h, 0); the four 64-bit outputs are 32 bytes,
 * little-endian, byte j % 32 for key j.  The mask is never stored: the
 * backward pass draws the same bytes again.  lse is that of the undropped
 * scores (as fa_fwd's).
 *
 * fa_fwd_dropout: arguments as fa_fwd, plus dropout_p in [0, 1) leaving
 *   t8 >= 1 (else FA_ERR_INVALID_ARG), seed and offset (any values; change
 *   offset between calls that must draw different masks).  bf16 / fp16 only
 *   (fp32 returns FA_ERR_UNSUPPORTED).
 * fa_bwd_dropout: arguments as fa_bwd, plus the same dropout_p, seed and
 *   offset as the forward call that produced o; gradients of sum(dout * o)
 *   with the same mask: dV = (P o Z)^T dO * 256 / t8, dP = (dO V^T) o Z *
 *   256 / t8, dS = P o (dP - rowsum(dO o O)), dQ = scale dS K,
 *   dK = scale dS^T Q.
 */
fa_status fa_fwd_dropout(const void* q, const void* k, const void* v,
                         void* o, float* lse,
                         int B, int H_q, int H_kv, int N, int d,
                         int causal, float scale, float dropout_p,
                         unsigned long long seed, unsigned long long offset,
                         fa_dtype dtype, hipStream_t stream);

fa_status fa_bwd_dropout(const void* q, const void* k, const void* v,
                         const void* o, const float* lse, const void* dout,
                         void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes,
                         int B, int H_q, int H_kv, int N, int d,
                         int causal, float scale, float dropout_p,
                         unsigned long long seed, unsigned long long offset,
                         fa_dtype dtype, hipStream_t stream);

/*
 * Block-sparse attention: the kernels skip the blocks of the attention matrix
 * that a block mask zeroes ("FlashAttention and the Kernel Era", The
 * Breakthrough: the block-sparse extension of the kernel).
 *
 *   block_mask in: uint8 [mask_heads, nb, nb], nb = ceil(N / 128)
 *                  (FA_SPARSE_BLOCK), row-major, device memory, any
 *                  alignment.  Query i may see key j iff
 *                  block_mask[h_m][i / 128][j / 128] != 0 (and j <= i when
 *                  causal), with h_m = 0 when mask_heads == 1 and the query
 *                  head otherwise.  The same mask serves every batch element.
 *   mask_heads     1 or H_q (else FA_ERR_INVALID_ARG).
 * The softmax runs over the visible keys only.  A row that sees no key gets
 * o = 0 and lse = -inf, and contributes no gradient.  Other arguments, sizes
 * and errors as for fa_fwd / fa_bwd; bf16 / fp16 only (fp32 returns
 * FA_ERR_UNSUPPORTED).  The work (and time) falls with the fraction of
 * blocks set.
 */
#define FA_SPARSE_BLOCK 128

fa_status fa_fwd_blocksparse(const void* q, const void* k, const void* v,
                             void* o, float* lse,
                             const unsigned char* block_mask, int mask_heads,
                             int B, int H_q, int H_kv, int N, int d,
                             int causal, float scale, fa_dtype dtype, hipStream_t stream);

fa_status fa_bwd_blocksparse(const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* dout,
                             void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes,
                             const unsigned char* block_mask, int mask_heads,
                             int B, int H_q, int H_kv, int N, int d,
                             int causal, float scale, fa_dtype dtype, hipStream_t stream);

/*
 * Variable-length batches in the padded layout: batch element b holds
 * seqlens[b] valid tokens (the ragged end of one sequence, generalised to a
 * batch; "Flash Attention" (21medien), the [batch, heads, seq_len, head_dim]
 * layout of its code example).  Queries and keys at positions >= seqlens[b]
 * are padding: they take no part in any softmax, their output rows are 0 with
 * lse -inf, and dq / dk / dv are 0 there.
 *   seqlens in: int32 [B] in device memory, 4-byte aligned, each in [0, N]
 *               (values outside are clamped).
 * Other arguments, sizes and errors as for fa_fwd / fa_bwd; bf16 / fp16 only
 * (fp32 returns FA_ERR_UNSUPPORTED).  The work falls with the lengths.
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v,
                        void* o, float* lse, const int* seqlens,
                        int B, int H_q, int H_kv, int N, int d,
                        int causal, float scale, fa_dtype dtype, hipStream_t stream);

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* dout,
                        void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, const int* seqlens,
                        int B, int H_q, int H_kv, int N, int d,
                        int causal, float scale, fa_dtype dtype, hipStream_t stream);

/*
 * FP8 path ("FlashAttention 1, 2, and 3 Explained", section 4 on
 * FlashAttention-3: FP8 with block quantization and incoherent processing;
 * "FlashAttention" glossary, FlashAttention-3 paragraph).  Low precision:
 * the forward below computes attention of the quantized values, not of the
 * 16-bit inputs.
 *
 * e4m3 codes are the OCP FP8 E4M3 format (1 sign, 4 exponent bits with bias
 * 7, 3 mantissa bits; largest finite value 448; 0x7f / 0xff are NaN and are
 * never produced).  A quantized tensor is a pair:
 *   codes  uint8   [B, H, N, d]          (same layout as the 16-bit tensor)
 *   scales float32 [B, H, ceil(N / 64)]  one scale per block of 64 rows
 * and stands for codes * scales[block of the row] (FA_FP8_BLOCK_ROWS).
 */
#define FA_FP8_BLOCK_ROWS 64

/*
 * Block quantizer.  For each head and block of 64 rows of x (the last block
 * may be shorter):
 *   y      = x, or (x * signs) H / sqrt(d) when signs != NULL: the
 *            incoherent-processing rotation, H the d x d Sylvester Hadamard
 *            matrix, evaluated in float32 as the fast Walsh-Hadamard transform
 *            (butterflies (a, b) -> (a + b, a - b) with strides 1, 2, 4, ...,
 *            then one multiplication by float32(1 / sqrt(d)));
 *   amax   = max |y| over the block;  scale = amax / 448;
 *   codes  = e4m3(clamp(y * (448 / amax), -448, 448)), round to nearest even,
 *            sign bit kept for negative values that round to zero;
 *            a block with amax == 0, or with 448 / amax beyond the float32
 *            range (amax below about 1.3e-36), gets scale 1 and zero codes.
 *   x      in : [B, H, N, d] bf16 or fp16 (`dtype`; fp32 returns
 *               FA_ERR_UNSUPPORTED), finite values, 16-byte aligned.
 *   signs  in : NULL, or d float32 values (+1 / -1), 16-byte aligned.  Pass
 *               the same signs for Q and K (the rotation is orthogonal, so
 *               scores are unchanged) and NULL for V.
 *   codes  out: [B, H, N, d] uint8, 16-byte aligned.
 *   scales out: [B, H, ceil(N / 64)] float32, 4-byte aligned.
 *   B, H, N >= 1 (sizes as for fa_fwd); d in {64, 128}.
 */
fa_status fa_fp8_quantize(const void* x, const float* signs,
                          unsigned char* codes, float* scales,
                          int B, int H, int N, int d, fa_dtype dtype,
                          hipStream_t stream);

/*
 * FP8 forward: O = softmax(scale * Qd Kd^T [causal]) Vd and lse, where Qd,
 * Kd, Vd are the dequantized values of three fa_fp8_quantize outputs.  Both
 * products run on the e4m3 matrix cores; the probabilities enter the P V
 * product rounded to e4m3 (relative error up to 2^-4 each), the row sums and
 * lse are kept in float32 from the unrounded probabilities.
 *   q, k, v   in : e4m3 codes [B, H_q, N, d] / [B, H_kv, N, d] / [B, H_kv, N, d],
 *                  16-byte aligned.
 *   q_scale, k_scale, v_scale in: their block scales [B, H, ceil(N / 64)],
 *                  float32, finite and > 0 (as fa_fp8_quantize writes them),
 *                  4-byte aligned.
 *   o         out: [B, H_q, N, d] in out_dtype (bf16 or fp16; fp32 returns
 *                  FA_ERR_UNSUPPORTED).
 *   lse       out: [B, H_q, N] float32, natural log, of the dequantized scores.
 *   Other arguments and checks as for fa_fwd.  Needs no workspace.
 */
fa_status fa_fwd_fp8(const unsigned char* q, const unsigned char* k, const unsigned char* v,
                     const float* q_scale, const float* k_scale, const float* v_scale,
                     void* o, float* lse,
                     int B, int H_q, int H_kv, int N, int d,
                     int causal, float scale, fa_dtype out_dtype, hipStream_t stream);

/* Static, never-NULL description of a status code. */
const char* fa_status_string(fa_status s);

/* Library version as major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */
