/*
 * fa.h -- C ABI of the io_aware_amd FlashAttention forward for gfx950 (MI355X).
 *
 * The operation ("6. FlashAttention 分块逻辑" sections 1-6 and 11;
 * "9.4 FlashAttention 与 FlashMLA" sections 9.4.2-9.4.5; "08. Triton Flash
 * Attention" Steps 1-4): exact softmax attention
 *
 *     O = softmax(scale * Q K^T [+ causal mask]) V,   LSE = m + ln(l)
 *
 * computed per (batch, head) and Q row block, streaming K/V column blocks
 * with the online softmax (running max m, running sum l, accumulator
 * rescaled by exp(m_old - m_new)), so that the Nq x Nk score and probability
 * matrices never reach device memory.  LSE is the per-row natural-log
 * logsumexp of the scaled, masked scores (the statistic the backward pass
 * rebuilds P from; "9.4 FlashAttention 与 FlashMLA", section 9.4.5).
 *
 * Layouts.  q: [B, H, Nq, d]; k, v: [B, H, Nk, d]; out: [B, H, Nq, d], all
 * contiguous row-major (d fastest) in the element type ``dtype``.
 * lse: [B, H, Nq] float32.  Accumulation and the m/l statistics are float32
 * on every path; probabilities are rounded to the input type (nearest-even)
 * before the P.V product, O is divided by the sum of those rounded
 * probabilities (a convex combination of value rows) while LSE comes from
 * the float32 sum, and O is rounded to the input type (nearest-even).
 * (The single-token split-KV path keeps its probabilities in float32.)
 * Range: probabilities are formed against a row max that may lag the
 * exact one; the lag is bounded so that with bf16 inputs O stays finite for
 * |V| up to 2^96 (about 7.9e28) whatever the key count, and with fp16
 * inputs for every finite V.
 *
 * Causal mask (``causal`` = 1): key j is visible to query i iff j <= i
 * (top-left alignment, for any Nq and Nk; "6. FlashAttention 分块逻辑",
 * section 4.1).  Out-of-range keys of a ragged last block are excluded
 * (score -inf), never treated as score 0.
 *
 * Ownership.  Every pointer is device memory owned by the caller; the
 * library never frees or retains it.  out and lse must not overlap q, k or
 * v.  The library owns only the split-KV workspace cache of ``fa_fwd``
 * (decode, and prefill grids too small for the GPU; released by
 * ``fa_release_workspace``).
 *
 * Asynchrony.  Every entry point enqueues its kernels on ``stream`` and
 * returns; results are valid once the stream has completed that work.  A
 * NULL stream is the device's default (null) stream.
 *
 * Threads.  Every entry point may be called from several host threads at
 * once.  The only state shared between calls is the workspace cache of
 * ``fa_fwd``, guarded by a mutex; the error message is per thread.
 *
 * Graph capture.  No kernel clears memory with a memset, so every entry
 * point may be captured into a HIP graph on ``stream`` and replayed.  The
 * split workspace of ``fa_fwd`` is allocated (hipMalloc) by the first call
 * on a stream that needs it: make one such call on the capturing stream
 * before capture.  A captured ``fa_fwd`` holds that workspace's address.  A
 * later call that needs a larger workspace on that stream allocates a new
 * one and keeps the old one alive, so the graph stays valid; only
 * ``fa_release_workspace`` frees them, so do not call it while the graph is
 * in use.  The entry points that take a caller workspace have no such
 * constraint.
 *
 * Errors.  Entry points return an ``fa_status``.  All arguments are checked
 * on the host before any HIP call, so a rejected call has no device side
 * effects.  ``fa_last_error`` returns a message for the calling thread's
 * most recent failure.
 *
 * Index range.  B*H, Nq*d and Nk*d must each fit in 31 bits (one head's
 * rows are addressed with 32-bit byte offsets), and B*H*max(Nq, Nk)*d may
 * not exceed 2^48 elements (far past any device's memory; it keeps every
 * byte count in 64 bits); larger calls return FA_ERR_UNSUPPORTED.  Whole
 * tensors may exceed 2^31 elements: they are indexed with 64-bit offsets.
 */
#ifndef IO_AWARE_AMD_FA_H
#define IO_AWARE_AMD_FA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of q, k, v and out (one type for all four). */
typedef enum fa_dtype {
    FA_F32 = 0,
    FA_F16 = 1,
    FA_BF16 = 2
} fa_dtype;

/* Status codes. */
typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,  /* null pointer, a size < 1, scale not finite (or
                                |scale|*log2(e) past float32 range), causal not
                                0/1, overlapping outputs, num_splits < 1 */
    FA_ERR_UNSUPPORTED = 2,  /* d not in {32, 64, 128}, unknown dtype, a pointer not
                                16-byte aligned (lse: 4-byte), sizes past the index
                                range, or a shape the entry point does not take */
    FA_ERR_HIP = 3,          /* a HIP runtime call or kernel launch failed */
    FA_ERR_WORKSPACE = 4     /* workspace missing, misaligned or too small */
} fa_status;

/*
 * fa_fwd -- the forward pass.
 *
 * q, k, v, out: device pointers as described above; lse: device pointer to
 * [B, H, Nq] float32, or NULL to skip writing LSE.  B, H, Nq, Nk >= 1;
 * d in {32, 64, 128}; causal 0 or 1; dtype an fa_dtype.  scale: the
 * caller's softmax scale (normally 1/sqrt(d); "08. Triton Flash Attention",
 * the exercise's sm_scale), any finite value whose product with log2(e) is
 * a finite float32, negative and zero included (a zero scale gives every
 * visible key the same weight); this holds for every entry point below.
 *
 * Dispatch: Nq == 1 without the mask (single-token decode) runs the split-KV
 * path ("6. FlashAttention 分块逻辑", section 11: K/V split into chunks that
 * are processed independently, then merged by logsumexp weights) with
 * fa_default_num_splits(Nk) chunks and a library-owned workspace kept per
 * (device, stream); any other shape runs the tiled prefill kernel.  Grids of
 * (batch*head, Q block of 128) workgroups too small for the GPU are split
 * along the keys, by the same method at two levels:
 *  - fewer than 512 workgroups whose Q blocks read many K/V tiles (the
 *    causal mask counted: 64 for grids of at most 128 workgroups, 256
 *    above), for 16-bit types: the key range of each Q block is cut into
 *    min(ceil(512 / grid), tiles / 8, 64) chunks of whole tiles (fewer where
 *    whole-tile chunks need fewer), one workgroup each, merged by the same
 *    logsumexp combine through the same library-owned workspace
 *    (B*H*Nq*chunks*(d + 1) float32);
 *  - otherwise, fewer than 256 workgroups whose longest Q block reads at
 *    least 8 tiles: Q blocks of 32 (64 at d = 128 or above 128 workgroups)
 *    queries whose key tiles are shared out between 4 (2) waves of the
 *    workgroup, their partial results merged the same way in shared
 *    memory, with no workspace.
 * The environment variable FA_PREFILL_SPLIT overrides the first choice: 0
 * or 1 never splits, n >= 2 asks for n chunks (capped at the tile count);
 * FA_PREFILL_SHAPE forces a tile shape (sweeps); FA_PREFILL_PIPE=1 runs the
 * 32-key-tile shape with a pipelined schedule (same results bit for bit,
 * slower on this GPU; for measurement).
 * float32 runs the vector-ALU kernel over (batch*head, Q block of 64)
 * workgroups; a grid of fewer than 256 cuts each Q block's key range into
 * min(ceil(512 / grid), 64) chunks of whole 32-key blocks (fewer where
 * whole-block chunks need fewer), merged by the same combine through the
 * same workspace.  FA_F32_SPLIT overrides that choice as FA_PREFILL_SPLIT
 * does.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *out, float *lse,
           int B, int H, int Nq, int Nk, int d, float scale, int causal,
           int dtype, hipStream_t stream);

/*
 * fa_fwd_noalloc -- fa_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, checks and dispatch as fa_fwd, but the
 * split workspace (decode, and prefill grids too small for the GPU, float32
 * included) is a
 * static device array of FA_NOALLOC_SCRATCH_BYTES bytes instead of the
 * library cache, and the call allocates nothing.  Each GPU the library runs
 * on holds its own copy of that array until the process ends; its address is
 * looked up (hipGetSymbolAddress) on the first call on each device.
 *
 * Limit: a split whose workspace (B*H*Nq*chunks*(d + 1) float32) would not
 * fit takes as many chunks as fit (the result then differs from fa_fwd's by
 * rounding only); a prefill that fits fewer than two runs unsplit; a decode
 * (Nq == 1, no mask) whose B*H*(d + 1)*4 bytes exceed the array is rejected
 * with FA_ERR_WORKSPACE before any HIP call.  Where the workspace fits, the
 * chunk count and the result are fa_fwd's, bit for bit.
 *
 * The array keeps the last call's contents; nothing in it needs clearing
 * (every chunk slot is written before it is read).  All calls on one GPU
 * share it: calls that overlap on one GPU (concurrent streams, or threads)
 * race and must be serialised by the caller.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int fa_fwd_noalloc(const void *q, const void *k, const void *v, void *out,
                   float *lse, int B, int H, int Nq, int Nk, int d,
                   float scale, int causal, int dtype, hipStream_t stream);

/*
 * fa_splitkv_workspace_bytes -- bytes of workspace fa_fwd_splitkv needs:
 * B*H*Nq*num_splits*(d + 1) float32 values (each chunk's normalised partial
 * output and its logsumexp), rounded up to 256 bytes.  Returns 0 for
 * arguments outside the accepted ranges.
 */
size_t fa_splitkv_workspace_bytes(int B, int H, int Nq, int d, int num_splits);

/*
 * fa_fwd_splitkv -- single-token decode with an explicit number of K/V
 * chunks ("6. FlashAttention 分块逻辑", section 11.3: stage one computes, per
 * chunk, the local max, local sum and local output; stage two merges them).
 *
 * Chunk c covers keys [c*ceil(Nk/num_splits), min(Nk, (c+1)*ceil(Nk/num_splits))).
 * Stage one stores, per chunk, lse_c = m_c + ln(l_c) and o~_c = o_c / l_c in
 * float32; stage two forms LSE = logsumexp_c(lse_c) and O = sum_c
 * exp(lse_c - LSE) o~_c.  An empty chunk gets weight 0.
 *
 * Nq must be 1 (FA_ERR_UNSUPPORTED otherwise); no causal mask.
 * 1 <= num_splits <= 1024.  workspace: caller-owned device memory of at least
 * fa_splitkv_workspace_bytes(B, H, Nq, d, num_splits) bytes, 16-byte aligned
 * (FA_ERR_WORKSPACE otherwise); it must not be used by other work on the
 * device while this call's kernels run.
 */
int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *out,
                   float *lse, int B, int H, int Nq, int Nk, int d, float scale,
                   int num_splits, void *workspace, size_t workspace_bytes,
                   int dtype, hipStream_t stream);

/*
 * fa_fwd_paged_decode -- single-token decode over a paged K/V cache
 * ("6. FlashAttention 分块逻辑", section 12: the kernel walks a sequence's
 * logical K/V blocks, finds each physical block through the block table and
 * loads it directly, skipping an unallocated block).
 *
 * q: [B, H, 1, d]; k_cache, v_cache: [num_blocks, H, block_size, d] each (the
 * page's [2, num_blocks, num_heads, block_size, head_dim] cache split into its
 * K and V halves); block_table: int32 [B, max_blocks_per_seq], entry j of row
 * b is the physical block holding sequence b's keys [j*block_size,
 * (j+1)*block_size); seq_lens: int32 [B], the number of keys of each
 * sequence.  All device pointers, element type ``dtype`` (fp16 or bf16) for
 * q, the caches and out.  out: [B, H, 1, d]; lse: [B, H] float32 or NULL.
 *
 * A table entry outside [0, num_blocks) marks an unallocated block: its keys
 * are skipped.  seq_lens are clamped to [0, max_blocks_per_seq*block_size];
 * a sequence with no key gets O = 0 and LSE = -inf.  block_size: a power of
 * two in [1, 1024].  The split is as in fa_fwd_splitkv, per sequence: chunks
 * of ceil(len_b / num_splits) keys, 1 <= num_splits <= 1024.  workspace: at
 * least fa_splitkv_workspace_bytes(B, H, 1, d, num_splits) bytes, 16-byte
 * aligned.  Table and lengths must be 4-byte aligned; the other tensors
 * 16-byte aligned.
 */
int fa_fwd_paged_decode(const void *q, const void *k_cache, const void *v_cache,
                        const int *block_table, const int *seq_lens, void *out,
                        float *lse, int B, int H, int d, int block_size,
                        int max_blocks_per_seq, int num_blocks, float scale,
                        int num_splits, void *workspace, size_t workspace_bytes,
                        int dtype, hipStream_t stream);

/*
 * fa_varlen_workspace_bytes -- bytes of workspace fa_fwd_varlen needs for
 * its tile list: 4 * (2 + 2 * (ceil(total_q / 128) + num_seqs)), rounded up
 * to 256.  Returns 0 for arguments outside the accepted ranges.
 */
size_t fa_varlen_workspace_bytes(int num_seqs, int total_q);

/*
 * fa_fwd_varlen -- the forward over a batch of packed sequences of different
 * lengths ("9.4 FlashAttention 与 FlashMLA" section 9.4.6: the work of each
 * workgroup is fixed before the attention kernel starts, and sequences of
 * unequal length are cut into equal tiles for load balance).
 *
 * q: [total_q, H, d]; k, v: [total_k, H, d]; out: [total_q, H, d] (token-
 * major, d fastest), element type ``dtype`` (fp16 or bf16).  lse:
 * [H, total_q] float32 or NULL.  cu_seqlens_q, cu_seqlens_k: device int32
 * [num_seqs + 1] offsets; sequence s is rows [cu_seqlens_q[s],
 * cu_seqlens_q[s+1]) of q attending to rows [cu_seqlens_k[s],
 * cu_seqlens_k[s+1]) of k and v, with the causal mask (if set) top-left
 * within the sequence.  Offsets must start at 0 and not decrease; on the
 * device each sequence's bounds are clamped into [0, total] and the tile
 * list into its bound, so inconsistent offsets give wrong rows, never an
 * access outside the tensors or the workspace.  A query with no key gets O = 0 and
 * LSE = -inf.  1 <= num_seqs <= 4096.  A schedule kernel writes the tile
 * list into ``workspace`` (at least fa_varlen_workspace_bytes(num_seqs,
 * total_q) bytes, 16-byte aligned), then the attention kernel runs over it.
 */
int fa_fwd_varlen(const void *q, const void *k, const void *v, void *out,
                  float *lse, const int *cu_seqlens_q, const int *cu_seqlens_k,
                  int num_seqs, int total_q, int total_k, int H, int d,
                  float scale, int causal, int dtype, void *workspace,
                  size_t workspace_bytes, hipStream_t stream);

/*
 * FP8 forward ("9.4 FlashAttention 与 FlashMLA" section 9.4.4: attention
 * with 8-bit E4M3 inputs; Q and K first multiplied by one random orthogonal
 * matrix so that the quantisation error is spread evenly, "incoherent
 * processing").  Two calls: fa_quantize_fp8 turns fp16/bf16 q, k, v into a
 * "pack" of E4M3 codes, fa_fwd_fp8 runs attention on a pack.  d = 64 or 128.
 *
 * Pack layout (BH = B*H, Nkp = Nk rounded up to a multiple of 64, up(x) = x
 * rounded up to 256; byte offsets from the pack's start):
 *   q8      at 0:                          [BH, Nq, d]  Q M codes
 *   k8      at up(BH*Nq*d):                [BH, Nkp, d] K M codes (rows >= Nk zero)
 *   v8t     at k8 + up(BH*Nkp*d):          [BH, d, Nkp] V codes transposed; within
 *           each group of 64 keys, position p = 32*g + 16*b + r holds key
 *           32*b + 8*(r/4) + 4*g + (r%4) (g, b in {0,1}, r in 0..15), the order
 *           in which the forward kernel holds probabilities; keys >= Nk zero
 *   descale at v8t + up(BH*d*Nkp):         float [3][BH]: amax/448 of Q M, K M, V
 *   scratch at descale + up(3*BH*4):       3*BH words used during quantisation
 *   total   fa_fp8_pack_bytes(B, H, Nq, Nk, d) = scratch + up(3*BH*4).
 * Codes are RNE_E4M3(clamp(x * 448/amax, -448, 448)), amax = max |x| over the
 * (batch, head) (descale 1 for an all-zero head).
 */
size_t fa_fp8_pack_bytes(int B, int H, int Nq, int Nk, int d);

/*
 * fa_quantize_fp8 -- q [B, H, Nq, d], k and v [B, H, Nk, d] (dtype fp16 or
 * bf16) -> pack.  signs: device float [d] of +-1 (the random diagonal of
 * M = diag(signs) H_d / sqrt(d), applied to each row x as x M: the signs
 * first, then H_d, the Sylvester-Hadamard matrix), or NULL for no
 * transform (M = I).  The transform is the fast Walsh-Hadamard
 * butterfly in float32.  pack: at least fa_fp8_pack_bytes bytes, 256-byte
 * aligned, not overlapping the inputs.
 */
int fa_quantize_fp8(const void *q, const void *k, const void *v,
                    const float *signs, int B, int H, int Nq, int Nk, int d,
                    int dtype, void *pack, size_t pack_bytes,
                    hipStream_t stream);

/*
 * fa_fwd_fp8 -- attention on a pack: O = softmax(scale * Q' K'^T [+ mask]) V'
 * with Q' = q8 * descale_q, K' = k8 * descale_k, V' = v8 * descale_v (so
 * Q' K'^T approximates Q K^T; M cancels).  Both products run on the E4M3
 * MFMA with float32 accumulation; P is rounded to E4M3 before P V'.  out:
 * [B, H, Nq, d] in out_dtype (fp16 or bf16); lse: [B, H, Nq] float32 or NULL.
 * The pack must come from fa_quantize_fp8 with the same B, H, Nq, Nk, d.
 */
int fa_fwd_fp8(const void *pack, void *out, float *lse, int B, int H, int Nq,
               int Nk, int d, float scale, int causal, int out_dtype,
               hipStream_t stream);

/*
 * fa_bwd_workspace_bytes -- bytes of workspace fa_bwd needs: two float32
 * values per query row (the statistic LSE*log2(e) and D, see fa_bwd) plus a
 * padding of 64 rows, rounded up to 256 bytes.  Returns 0 for arguments
 * outside the accepted ranges.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int Nq, int d);

/*
 * fa_bwd -- the backward pass by recomputation ("9.4 FlashAttention 与
 * FlashMLA" section 9.4.5: a pre-computed D_i = rowsum(dO_i * O_i), one
 * kernel over K/V blocks for dK and dV, one over Q blocks for dQ; "6.
 * FlashAttention 分块逻辑" section 7.1 for the formulas):
 *
 *     P  = exp(scale * Q K^T [+ mask] - LSE)      (rebuilt per block, never stored)
 *     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
 *     dQ = scale * dS K,  dK = scale * dS^T Q.
 *
 * q, k, v, causal and scale must be those of the forward call that produced
 * ``out`` and ``lse`` (lse is required: [B, H, Nq] float32, natural log).
 * dout: [B, H, Nq, d], the gradient of the loss with respect to out.
 * dq: [B, H, Nq, d]; dk, dv: [B, H, Nk, d]; all in ``dtype`` (fp16 or bf16;
 * fp32 is FA_ERR_UNSUPPORTED), rounded to nearest even from float32
 * accumulators.  P and dS are rounded to ``dtype`` before their products.
 * Keys that no query sees get dK = dV = 0.  The result is bit-for-bit
 * reproducible (no atomics).  workspace: caller-owned device memory of at
 * least fa_bwd_workspace_bytes(B, H, Nq, d) bytes, 16-byte aligned.  dq, dk,
 * dv must not overlap each other, an input or the workspace.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *out,
           const void *dout, const float *lse, void *dq, void *dk, void *dv,
           int B, int H, int Nq, int Nk, int d, float scale, int causal,
           int dtype, void *workspace, size_t workspace_bytes,
           hipStream_t stream);

/*
 * fa_default_num_splits -- chunk count fa_fwd uses for a decode call:
 * ceil(Nk / 256) clamped to [1, 64] (8192 keys -> 32 chunks of 256).
 * Returns 0 if Nk < 1.
 */
int fa_default_num_splits(int Nk);

/*
 * fa_release_workspace -- waits for the devices that used them, then frees
 * every workspace fa_fwd allocated, including those replaced by larger ones
 * (a workspace that grows is never freed in place, since work enqueued
 * earlier may still use it).  Returns FA_OK or FA_ERR_HIP.
 */
int fa_release_workspace(void);

/*
 * fa_map_workgroup -- the prefill kernel's workgroup order, exposed so the
 * host can check it: workgroup ``wg`` of ``BH * Tr`` processes (batch*head
 * index *bh, Q row block *qblock).  Workgroups are spread over the 8 XCDs in
 * dispatch order; the mapping gives each XCD whole heads so their K/V stay
 * in that XCD's L2, and, under the causal mask, the longest (last) Q blocks
 * of a head first.  Returns FA_OK, or FA_ERR_INVALID_ARG for wg out of range.
 */
int fa_map_workgroup(int wg, int BH, int Tr, int causal, int *bh, int *qblock);

/* Static text for a status code. */
const char *fa_status_string(int status);

/* Message for the calling thread's most recent failed call ("" if none). */
const char *fa_last_error(void);

/* ABI version: 1. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* IO_AWARE_AMD_FA_H */
