/*
 * attn.h — C ABI of the MI355X (gfx950) fused softmax-attention library.
 *
 * The library computes the attention forward pass
 *     O = softmax(Q K^T * scale + mask) V,   lse_i = ln sum_j exp(S_ij)
 * without ever writing the score matrix to memory: Q tiles stay in registers,
 * K/V tiles stream through LDS, and an online softmax (running row max and
 * row sum, rescaled per tile) keeps the result exact.  Sources:
 *   - "flashattention-kernels" page (cyk1337 paper-daily), §0 and §1: the
 *     tiling + online-softmax dataflow and the parallel work partitioning of
 *     the FlashAttention line; §3: Flash-Decoding (split the KV sequence,
 *     compute partial attention per chunk, reduce) for one-token decode, and
 *     an engine-style interface covering GQA/MQA and prefill/decode;
 *   - "cuda-kernel-pretrain" page (cyk1337 paper-daily), §2 and §3: IO-aware
 *     exact attention; GQA/MQA share one K/V head per group of query heads;
 *     the practice list asks that a low-precision path state its scale
 *     granularity and accumulation precision as part of its contract;
 *   - "GPU kernel overview" page (zhaifeiyue.github.io), SageAttention chain
 *     and the INT-for-QK / FP-for-PV insight: Smooth-K, per-block INT8 Q/K,
 *     FP8 (E4M3) P and V.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronises inside a call (scratch memory is
 *     the caller's `workspace`, sized by the *_workspace_size functions).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  Inputs must stay valid until the work on `stream` completes.
 *   - Layouts are dense row-major (C order):
 *       q [B, H, N, d],  k and v [B, Hkv, N, d],  o [B, H, N, d],  lse [B, H, N].
 *     Query head h reads kv head h / (H / Hkv) (consecutive groups; H % Hkv == 0;
 *     Hkv == H is plain multi-head attention, Hkv == 1 is MQA).
 *   - q, k, v are bf16.  o is bf16 or fp32 (o_dtype).  lse is fp32, natural log,
 *     over the scaled and masked scores; lse may be NULL (not written).
 *   - causal != 0 applies the top-left aligned mask: key j is visible to query
 *     i iff j <= i.
 *   - Every argument is validated before any HIP call: an invalid call returns
 *     an error status and launches nothing.  A failed launch returns
 *     ATTN_ERR_HIP.  No C++ exception crosses this interface.
 *     attn_last_error() gives a human-readable reason for the last failure on
 *     the calling thread.
 */
#ifndef MI355X_ATTN_H
#define MI355X_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, H % Hkv != 0, bad scale */
    ATTN_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. d not in {64, 128}) */
    ATTN_ERR_WORKSPACE = -3,   /* workspace missing or smaller than *_workspace_size */
    ATTN_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} attn_status;

typedef enum {
    /* bf16 inputs, bf16 MFMA for QK^T and PV, fp32 accumulation and softmax. */
    ATTN_MODE_EXACT_BF16 = 0,
    /* SageAttention-style quantised mode ("GPU kernel overview" page, Sage
     * chain): Smooth-K (K minus its per-channel mean over all N tokens of the
     * kv head, in fp32); Q and K' quantised to symmetric INT8 per block of 64
     * consecutive tokens of one (batch, head) with scale max|x|/127; S from an
     * INT8 MFMA with exact int32 accumulation; P quantised to OCP E4M3 as
     * E4M3(448 * exp(S - m_running)), the exponent formed in fp32 to within
     * half a unit of the integer score (times its scale) before the E4M3
     * rounding; V quantised to E4M3 per (batch, kv head,
     * channel) with scale max|V|/448; PV by an FP8 MFMA with fp32
     * accumulation.  lse is the true LSE (the Smooth-K shift q_i . kmean is
     * added back).  Needs a workspace. */
    ATTN_MODE_SAGE_QK_I8_BLK64_PV_FP8_E4M3 = 1,
    /* SageAttention3-style FP4 microscaling on the MX block formats of the
     * gfx950 matrix cores ("gpu-kernel-porting-with-ai-agents" page,
     * SageAttention 3 section; "GPU kernel overview" page, insights on FP4
     * attention): Smooth-K as above; Q and K' in MXFP4 blocks of 32
     * consecutive channels of a token, V in blocks of 32 consecutive tokens
     * of a channel, P = exp(S - m_running) (<= 1 per row) in blocks of 32
     * consecutive keys: OCP E2M1 elements (nearest, ties to even) with one
     * E8M0 scale 2^e per block, e the smallest exponent with
     * max|x| <= 6 * 2^e (no element saturates); S = Q^ K^^T and O = P^ V^ on
     * the FP4 MFMA with fp32 accumulation; l sums the unquantised P; lse is
     * the true LSE.  Prefill only; needs a workspace. */
    ATTN_MODE_SAGE3_QK_MXFP4_PV_MXFP4 = 2,
    /* The same recipe with the MX FP6 element format E2M3 ("GPU kernel
     * overview" page, insights: CDNA4's matrix cores take FP4 and FP6): OCP
     * E2M3 elements (1 sign, 2 exponent, 3 mantissa bits; largest magnitude
     * 7.5; nearest, ties to even), one E8M0 scale 2^e per block of 32, e the
     * smallest exponent with max|x| <= 7.5 * 2^e; the FP6 MFMA runs at the
     * FP4 rate.  Prefill only; needs a workspace. */
    ATTN_MODE_SAGE3_QK_MXFP6_PV_MXFP6 = 3
} attn_mode;

typedef enum { ATTN_OUT_BF16 = 0, ATTN_OUT_FP32 = 1 } attn_dtype;

/*
 * Attention forward pass (prefill: N queries against the same N keys).
 *   q, k, v    device inputs (bf16), layouts above.
 *   o          device output, [B, H, N, d], dtype o_dtype.
 *   lse        device output fp32 [B, H, N], or NULL.
 *   B, H, Hkv, N, d   sizes; d must be 64 or 128; N >= 1.
 *   causal     0 = no mask, else the top-left causal mask.
 *   scale      multiplier of Q K^T (finite, > 0); usually 1/sqrt(d).
 *   mode       attn_mode.
 *   o_dtype    attn_dtype.
 *   workspace  device scratch of at least attn_fwd_workspace_size() bytes
 *              (may be NULL when that size is 0).  Its content on entry is
 *              irrelevant; it is overwritten.
 */
attn_status attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                     int B, int H, int Hkv, int N, int d, int causal, float scale,
                     int mode, int o_dtype, void *workspace, size_t workspace_bytes,
                     void *stream);

/* Bytes of workspace attn_fwd needs for these sizes and mode (0 for the exact
 * mode).  Returns 0 as well for sizes attn_fwd rejects (invalid, d other than
 * 64 or 128, B*H beyond 2^31 - 1 or N beyond 2^24); attn_fwd then reports the
 * error. */
size_t attn_fwd_workspace_size(int B, int H, int Hkv, int N, int d, int mode);

/*
 * The quantisation state a quantised-mode attn_fwd call leaves in its
 * workspace, for inspecting the recipe's numeric path (scale ranges, codes at
 * the ends of their ranges): the "cuda-kernel-pretrain" page's practice list
 * asks that a low-precision path expose numeric counters such as scale
 * distributions and overflow rates.  With nblk = ceil(N / 64) and
 * Npad = 64 * nblk, the pieces are (row-major):
 *   ATTN_SAGE_WS_KMEAN   fp32 [B*Hkv][d]        per-channel mean of K (Smooth-K)
 *   ATTN_SAGE_WS_VSCALE  fp32 [B*Hkv][d]        V scale max|V| / 448 per channel
 *   ATTN_SAGE_WS_QDELTA  fp32 [B*H][nblk]       Q scale max|Q| / 127 per 64-token block
 *   ATTN_SAGE_WS_KDELTA  fp32 [B*Hkv][nblk]     the same for K - kmean
 *   ATTN_SAGE_WS_QHAT    int8 [B*H][Npad][d]    quantised Q (rows >= N are 0)
 *   ATTN_SAGE_WS_KHAT    int8 [B*Hkv][Npad][d]  quantised K - kmean
 *   ATTN_SAGE_WS_VHATT   E4M3 [B*Hkv][d][Npad]  quantised V, feature-major
 * and scratch of the kernels (the other enumerators).  Offsets are in bytes
 * from the start of the workspace.
 */
typedef enum {
    ATTN_SAGE_WS_KSUM_PART = 0,
    ATTN_SAGE_WS_VMAX_PART,
    ATTN_SAGE_WS_KMEAN,
    ATTN_SAGE_WS_VSCALE,
    ATTN_SAGE_WS_VINV,
    ATTN_SAGE_WS_QDELTA,
    ATTN_SAGE_WS_KDELTA,
    ATTN_SAGE_WS_QKDOT,
    ATTN_SAGE_WS_QHAT,
    ATTN_SAGE_WS_KHAT,
    ATTN_SAGE_WS_VHATT,
    ATTN_SAGE_WS_COUNT
} attn_sage_ws_piece;

/* Fills offsets[0 .. ATTN_SAGE_WS_COUNT-1] with the byte offset of each piece
 * for these sizes.  ATTN_ERR_INVALID_ARG for a null offsets or for sizes
 * attn_fwd rejects (as attn_fwd_workspace_size). */
attn_status attn_sage_workspace_layout(int B, int H, int Hkv, int N, int d, size_t *offsets);

/*
 * The quantisation state an MX-mode attn_fwd call (MXFP4 or MXFP6) leaves in
 * its workspace, for the same inspection (the "cuda-kernel-pretrain" page's
 * practice list: scale distributions of a low-precision path).  With Npad =
 * 64 * ceil(N / 64) and F = 4 or 6 bits per element, the pieces are:
 *   ATTN_MX_WS_KSUM_PART  fp64 [B*Hkv][16][d]     partial per-channel K sums
 *   ATTN_MX_WS_KMEAN      fp32 [B*Hkv][d]         per-channel mean of K (Smooth-K)
 *   ATTN_MX_WS_QKDOT      fp32 [B*H][N]           q . kmean per query
 *   ATTN_MX_WS_QHAT       [B*H][Npad * d * F / 8] Q codes (see below)
 *   ATTN_MX_WS_QSC        u8 [B*H][Npad][d/32]    Q block scales, E8M0 (2^(byte - 127))
 *   ATTN_MX_WS_KHAT       [B*Hkv][Npad * d * F / 8] K - kmean codes
 *   ATTN_MX_WS_KSC        u8 [B*Hkv][Npad][d/32]  their block scales
 *   ATTN_MX_WS_VHATT      [B*Hkv][d * Npad * F / 8] V codes, in 64-key tiles
 *   ATTN_MX_WS_VSCT       u8 [B*Hkv][Npad/32][d]  V block scales (32 keys of a channel)
 * Codes are in tiles of 64 tokens.  A block of 32 codes is 16 bytes (E2M1,
 * element i in nibble i % 2 of byte i / 2, low nibble first) or 24 bytes
 * (E2M3, element i in bits 6i .. 6i+5 of the block read as a little-endian
 * 192-bit number).  A Q or K tile holds every block's first 16 bytes as
 * [token][block], then (E2M3) their last 8 bytes as [block][token with
 * bits 4 and 5 swapped].  A V tile holds them as [key block][channel], in
 * the same two parts.  Rows past N hold zero codes.
 */
typedef enum {
    ATTN_MX_WS_KSUM_PART = 0,
    ATTN_MX_WS_KMEAN,
    ATTN_MX_WS_QKDOT,
    ATTN_MX_WS_QHAT,
    ATTN_MX_WS_QSC,
    ATTN_MX_WS_KHAT,
    ATTN_MX_WS_KSC,
    ATTN_MX_WS_VHATT,
    ATTN_MX_WS_VSCT,
    ATTN_MX_WS_COUNT
} attn_mx_ws_piece;

/* Fills offsets[0 .. ATTN_MX_WS_COUNT-1] with the byte offset of each piece
 * for these sizes and MX mode.  ATTN_ERR_INVALID_ARG for a null offsets, for
 * a mode that is not an MX mode, or for sizes attn_fwd rejects. */
attn_status attn_mx_workspace_layout(int B, int H, int Hkv, int N, int d, int mode,
                                     size_t *offsets);

/*
 * Attention forward over a packed batch of variable-length sequences (the
 * exact mode only): each sequence attends to its own tokens, with the same
 * computation as attn_fwd applied sequence by sequence.  Packing without
 * padding is the shape/packing lever the "flashattention-kernels" page
 * (recommendation table) puts before any specialised kernel, and the
 * library interface of its §3 switches between prefill and decode over such
 * batches.
 *   q, o       device [total, H, d] (token-major: the H heads of a token are
 *              adjacent); o has dtype o_dtype.
 *   k, v       device bf16 [total, Hkv, d].
 *   lse        device fp32 [H, total] or NULL.
 *   cu_seqlens device int32 [B + 1]: sequence b holds tokens
 *              [cu_seqlens[b], cu_seqlens[b+1]); cu_seqlens[0] = 0,
 *              non-decreasing, cu_seqlens[B] = total.  Offsets outside
 *              [0, total] are clamped into it, and a sequence longer than
 *              max_seqlen is cut to its first max_seqlen queries and keys
 *              (the result is then unspecified, but no access leaves the
 *              tensors).  Empty sequences are allowed.
 *   total      number of packed tokens (>= 1).
 *   max_seqlen an upper bound of the sequence lengths (>= 1); it sizes the grid.
 *   causal     0 = no mask, else the top-left causal mask inside each sequence.
 *   mode       only ATTN_MODE_EXACT_BF16 (the quantised mode returns
 *              ATTN_ERR_UNSUPPORTED).
 * No workspace.  Errors as for attn_fwd, plus ATTN_ERR_INVALID_ARG for a null
 * cu_seqlens or non-positive total or max_seqlen.
 */
attn_status attn_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                            const int32_t *cu_seqlens, int B, int H, int Hkv, int total,
                            int max_seqlen, int d, int causal, float scale, int mode,
                            int o_dtype, void *stream);

/*
 * One-token decode against per-sequence KV caches with split-KV
 * (Flash-Decoding, "flashattention-kernels" page §3): the valid keys
 * [0, seqlens[b]) of each sequence are split into pieces whose partial
 * attention (O_s, lse_s) is computed in parallel, and the partials are merged
 * by log-sum-exp weights:
 *     M = max_s lse_s,  w_s = exp(lse_s - M),
 *     O = sum_s w_s O_s / sum_s w_s,  lse = M + ln sum_s w_s.
 * The valid keys of all (sequence, kv head) pairs, in that order, are divided
 * into equal contiguous ranges among a fixed set of resident waves, so the
 * work is balanced whatever the length mix.  Inside a range, the keys of each
 * (sequence, kv head) form chunks of split_tokens keys (chunk c holds keys
 * [c*split_tokens, (c+1)*split_tokens)); each chunk's partial is folded into
 * the wave's running partial by the same merge, and a second kernel merges
 * the partials of the waves that share a (sequence, kv head).
 * The single query of sequence b sits at position seqlens[b] - 1 and sees every
 * valid key, so there is no causal argument.
 *   q          device bf16 [B, H, d].
 *   k_cache, v_cache   device bf16 [B, Hkv, N_max, d]; rows >= seqlens[b] are
 *              never read.
 *   seqlens    device int32 [B]; each value must lie in [1, N_max] (values
 *              outside are clamped to that range by the kernels).
 *   o          device output [B, H, d], dtype o_dtype.
 *   lse        device fp32 [B, H] or NULL.
 *   mode       only ATTN_MODE_EXACT_BF16 (others return ATTN_ERR_UNSUPPORTED).
 *   split_tokens   chunk length; a positive multiple of 64.
 *   workspace  at least attn_decode_workspace_size() bytes: fp32 partial
 *              outputs and LSEs of every (wave, sequence, kv head) piece.
 *              Its content on entry is irrelevant.
 * The result does not depend on the order in which waves run: every partial
 * has one writer and the merge order is fixed, so calls are deterministic.
 */
attn_status attn_decode(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *seqlens, void *o, float *lse, int B, int H, int Hkv,
                        int N_max, int d, float scale, int mode, int o_dtype,
                        int split_tokens, void *workspace, size_t workspace_bytes,
                        void *stream);

/* Bytes of workspace attn_decode and attn_decode_paged need (0 for invalid
 * sizes): independent of the cache length and the chunk length. */
size_t attn_decode_workspace_size(int B, int H, int Hkv, int d);

/*
 * attn_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The same kernels and the same result as attn_decode
 * (bit for bit); the partials live in a fixed array of the library,
 * ATTN_DECODE_SCRATCH_BYTES on every GPU it runs on, held until the process
 * ends.  Nothing is allocated or freed.  The caller still passes the inputs
 * and outputs; every partial the merge reads is written by the same call, so
 * the array needs no clearing.
 * Calls on one GPU share its array: calls that overlap in time on one GPU
 * (other streams, other threads) race and must be serialised by the caller.
 * Errors: those of attn_decode (no workspace error), and ATTN_ERR_UNSUPPORTED
 * when attn_decode_workspace_size(B, H, Hkv, d) exceeds the array.
 */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
attn_status attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *seqlens, void *o, float *lse, int B, int H,
                                int Hkv, int N_max, int d, float scale, int mode, int o_dtype,
                                int split_tokens, void *stream);

/*
 * attn_decode over paged KV caches: the cache is a pool of fixed-size pages
 * and a per-sequence page table names the page holding each run of
 * page_size key positions (the non-contiguous KV layout of paged serving
 * caches: "flashattention-kernels" page §3, a library interface covering
 * paged KV; "GPU kernel overview" page, the open gaps on decode with paged,
 * non-contiguous KV memory).  The computation, the work split, the chunking
 * into split_tokens keys and the merge are those of attn_decode: for the same
 * keys and values it returns bit-identical results.
 *   k_pages, v_pages   device bf16 [num_pages, Hkv, page_size, d].
 *   block_table  device int32 [B, max_pages]: key position n of sequence b
 *              (0 <= n < seqlens[b]) is row n % page_size of page
 *              block_table[b * max_pages + n / page_size].  Entries beyond a
 *              sequence's last page are never used.  Entries must lie in
 *              [0, num_pages); the kernels clamp others into that range
 *              (the result is then unspecified, but no access leaves the pool).
 *   seqlens    device int32 [B]; values are clamped to [1, max_pages * page_size].
 *   page_size  a power of two, >= 16.
 *   other arguments as for attn_decode (N_max = max_pages * page_size).
 *   workspace  at least attn_decode_workspace_size(B, H, Hkv, d) bytes.
 * Errors: those of attn_decode; ATTN_ERR_INVALID_ARG for a null block_table,
 * non-positive num_pages or max_pages, or a page_size that is not a power of
 * two; ATTN_ERR_UNSUPPORTED for a page_size below 16 or max_pages * page_size
 * beyond 2^31 - 1.
 */
attn_status attn_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                              const int32_t *block_table, const int32_t *seqlens, void *o,
                              float *lse, int B, int H, int Hkv, int num_pages, int page_size,
                              int max_pages, int d, float scale, int mode, int o_dtype,
                              int split_tokens, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * Backward pass of the exact mode: the gradients dQ, dK, dV of
 * O = softmax(Q K^T * scale + mask) V for an upstream gradient dO, given the
 * forward's O and LSE (the training side of the pages' kernels: "GPU kernel
 * overview" page, SageBwd and the training gaps; "flashattention-kernels"
 * page §0, FA2/FA3 as training kernels).  With P recomputed from the LSE:
 *     dP = dO V^T,  D_i = dO_i . O_i,  dS = P * (dP - D),
 *     dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,
 * and a kv head's dK/dV sum over the query heads of its group.  Deterministic
 * (no atomics).
 *   q, o, dout  device bf16 [B, H, N, d];  k, v  device bf16 [B, Hkv, N, d].
 *   lse        device fp32 [B, H, N] as written by attn_fwd (natural log).
 *   dq         device [B, H, N, d];  dk, dv  device [B, Hkv, N, d]; all of
 *              dtype grad_dtype (attn_dtype).
 *   workspace  at least attn_bwd_workspace_size() bytes (fp32 -D and
 *              -lse/scale per row, each head's rows padded to a multiple
 *              of 64); overwritten.
 *   scale      as attn_fwd, and at least 2^-64 (so that lse/scale stays
 *              finite).
 * Errors: as attn_fwd (d in {64, 128}); null lse, any null tensor or a scale
 * below 2^-64 is ATTN_ERR_INVALID_ARG; a missing or short workspace
 * ATTN_ERR_WORKSPACE.
 */
attn_status attn_bwd(const void *q, const void *k, const void *v, const void *o,
                     const float *lse, const void *dout, void *dq, void *dk, void *dv, int B,
                     int H, int Hkv, int N, int d, int causal, float scale, int grad_dtype,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace attn_bwd needs (0 for invalid sizes and for sizes
 * attn_bwd rejects: N beyond 2^24 or B*H*N beyond 2^31 - 1). */
size_t attn_bwd_workspace_size(int B, int H, int N);

/* Static description of a status code. */
const char *attn_status_string(int status);

/* Detailed message of the last failed call on the calling thread ("" if none). */
const char *attn_last_error(void);

/*
 * Kernel timing hooks for benchmarks.  While enabled, every kernel the library
 * launches on the calling thread is bracketed by a pair of HIP events recorded
 * on the launch stream.  attn_profiler_read() waits for those events, adds each
 * launch's elapsed time to a per-kernel-name total, and clears the record.
 * For i < returned count: names + i*name_stride holds the kernel name
 * (NUL-terminated, truncated to name_stride - 1 chars), total_ms[i] the summed
 * time and launches[i] the number of launches.  Returns the number of distinct
 * kernels (at most cap) or a negative attn_status.
 */
attn_status attn_profiler_enable(int enable);
int attn_profiler_read(char *names, int name_stride, double *total_ms, int *launches, int cap);

/* The recorded launches one by one, in launch order: for i < returned count,
 * names + i*name_stride holds the kernel name and ms[i] its elapsed time.
 * Waits for the events like attn_profiler_read and clears the record (launches
 * beyond cap are dropped).  The events come from a pool created by
 * attn_profiler_enable, so recording creates none while the pool lasts. */
int attn_profiler_launches(char *names, int name_stride, float *ms, int cap);

#ifdef __cplusplus
}
#endif
#endif /* MI355X_ATTN_H */
