// fa_internal.h -- launchers shared between the C ABI (fa_api.hip) and the
// kernel translation units.  Every launcher assumes its arguments were
// validated by the ABI layer and only enqueues work on ``stream``.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// The softmax scale with its sign folded into one operand of the score
// product.  scale * (k . q) = |scale| * (k . (-q)) holds exactly: negation
// only flips sign bits, and products and nearest-even rounded sums are odd
// functions.  So the kernels always see a positive exp2 factor (they take
// the row max before scaling) and flip the sign bits of the register-held
// operand (Q in the forward and the dQ kernel, K in the dK/dV kernel) when
// the scale is negative.  A zero scale (either sign) zeroes that operand and
// uses the factor 1: every visible score is then exactly 0, as 0 * (k . q)
// is, while masked scores stay -inf (-inf * 0 would be NaN).
struct FoldedScale {
    float c;        // exp2 factor, > 0
    uint32_t flip;  // XORed into every 32-bit word of the folded operand
    uint32_t keep;  // ANDed into every 32-bit word (0 for a zero scale)
};
constexpr uint32_t kSignBits16 = 0x80008000u;  // two 16-bit elements per word
constexpr uint32_t kSignBits8 = 0x80808080u;   // four E4M3 codes per word
constexpr uint32_t kSignBits32 = 0x80000000u;  // one float32 per word
inline FoldedScale fold_scale(float c, uint32_t sign_bits) {
    if (c > 0.0f) return {c, 0u, ~0u};
    if (c < 0.0f) return {-c, sign_bits, ~0u};
    return {1.0f, 0u, 0u};
}

// Prefill tile shapes the library is built with.  A shape is (waves per
// workgroup, queries per wave, keys per K/V tile); queries per workgroup
// (Br) = waves * queries per wave.
enum PrefillShape {
    kShapeW4Q32 = 0,   // 4 waves x 32 queries = Br 128, Bc 64
    kShapeW4Q64 = 1,   // 4 waves x 64 queries = Br 256, Bc 64
    kShapeW2Q64 = 2,   // 2 waves x 64 queries = Br 128, Bc 64
    kShapeW4Q32B32 = 3,  // 4 waves x 32 queries = Br 128, Bc 32, three waves per SIMD
    kShapeW4Q32K2 = 4,   // 4 waves, 2 query groups of 32, each group's K/V tiles split over 2 waves
                         // (Br 64; Bc 64, d = 128: 32)
    kShapeW4Q32K4 = 5,   // 4 waves on one group of 32 queries, its tiles split over 4 waves
                         // (Br 32; Bc 32, d = 32: 64; d = 128 takes kShapeW4Q32K2)
    kNumPrefillShapes = 6
};

// Queries per workgroup (Br) of a prefill shape.
int prefill_block_rows(int shape);

// The shape a dense launch takes when the grid of ``shape`` would leave
// CUs idle and each Q block's key loop is long: a key-split shape, else
// ``shape``.
int prefill_small_grid_shape(int d, bool causal, int shape, int BH, int Nq, int Nk);

// bf16 / fp16 tiled forward (MFMA).  dtype is FA_F16 or FA_BF16; d in
// {32, 64, 128}.  scale_log2 = scale * log2(e).
hipError_t launch_prefill(int dtype, int d, bool causal, int shape,
                          const void *q, const void *k, const void *v,
                          void *out, float *lse, int BH, int Nq, int Nk,
                          float scale_log2, hipStream_t stream);

// Packed variable-length batch through the same kernel: q [total_q, H, d],
// k and v [total_k, H, d], out like q, lse [H, total_q]; cu_q, cu_k the
// int32 offsets [S + 1] (device).  A schedule kernel first writes the tile
// list into workspace (varlen_workspace_ints ints).
constexpr int kMaxVarlenSeqs = 4096;
long long varlen_max_tiles(int S, int total_q, int block_rows);
hipError_t launch_prefill_varlen(int dtype, int d, bool causal, int shape, const void *q, const void *k,
                                 const void *v, void *out, float *lse, const int *cu_q, const int *cu_k, int S,
                                 int H, int total_q, int total_k, float scale_log2, void *workspace,
                                 hipStream_t stream);

// Split prefill for grids too small to fill the GPU: the key range of every
// (batch*head, Q block) is cut into S chunks of whole K/V tiles, one
// workgroup each; every chunk writes its normalised partial output and its
// logsumexp (the split-KV stage-one layout: o~ [rows, S, d] float32 then
// lse_c [rows, S], rows = BH * Nq) into workspace, and the split-KV combine
// merges them into out and lse.  prefill_split_count chooses S (1: no split;
// FA_PREFILL_SPLIT = 0 disables, a number n >= 2 asks for n chunks).
int prefill_split_count(int d, bool causal, int shape, int BH, int Nq, int Nk);
// At most S chunks of whole tiles, none of them empty: the count a split
// launch of the shape runs with (1: no split).
int prefill_split_normalise(int d, bool causal, int shape, int Nq, int Nk, int S);
hipError_t launch_prefill_split(int dtype, int d, bool causal, int shape, const void *q, const void *k,
                                const void *v, void *out, float *lse, int BH, int Nq, int Nk, float scale_log2,
                                int S, void *workspace, hipStream_t stream);

// The split-KV combine alone: out [rows, d] (dtype) and lse [rows] from the
// chunk partials o~ [rows, S, d] and lse_c [rows, S].
hipError_t launch_combine(int dtype, int d, const float *ws_o, const float *ws_lse, void *out, float *lse,
                          int rows, int S, hipStream_t stream);

// float32 tiled forward (vector ALU), Br = Bc = 64.  With S > 1 the key
// range is cut into S chunks of whole 32-key blocks, one workgroup each,
// written to workspace in the split layout above (S * (d + 1) floats per
// row) and merged by the combine.  f32_split_count chooses S for a grid
// (1: no split; FA_F32_SPLIT = 0 disables, n >= 2 asks for at most n chunks);
// f32_split_normalise gives the count a launch runs with for at most S.
int f32_split_count(bool causal, int BH, int Nq, int Nk);
int f32_split_normalise(bool causal, int Nq, int Nk, int S);
hipError_t launch_prefill_f32(int d, bool causal, const void *q, const void *k,
                              const void *v, void *out, float *lse, int BH,
                              int Nq, int Nk, float scale_log2, int S, void *workspace,
                              hipStream_t stream);

// Split-KV decode: stage one (per chunk partials into the workspace) then
// stage two (logsumexp-weighted combine).  dtype FA_F16 or FA_BF16; Nq == 1.
hipError_t launch_splitkv(int dtype, int d, const void *q, const void *k,
                          const void *v, void *out, float *lse, int BH, int Nk,
                          float scale_log2, int num_splits, void *workspace,
                          hipStream_t stream);

// Split-KV decode over a paged cache: k_cache, v_cache are
// [num_blocks, H, block_size, d]; block_table [B, max_blocks] int32;
// seq_lens [B] int32; block_size = 1 << log2_block.
hipError_t launch_paged_decode(int dtype, int d, const void *q, const void *k_cache, const void *v_cache,
                               const int *block_table, const int *seq_lens, void *out, float *lse, int B, int H,
                               int log2_block, int max_blocks, int num_blocks, float scale_log2, int num_splits,
                               void *workspace, hipStream_t stream);

// FP8 pack (the output of the quantisation step, the input of the FP8
// forward): byte offsets of its parts for BH heads.
struct Fp8Layout {
    size_t q8, k8, v8t, descale, amax, bytes;
    int Nkp;  // keys rounded up to the 64-key group
};
Fp8Layout fp8_layout(int BH, int Nq, int Nk, int d);
hipError_t launch_fp8_quantize(int dtype, int d, const void *q, const void *k, const void *v, const float *signs,
                               void *pack, int BH, int Nq, int Nk, hipStream_t stream);
hipError_t launch_fp8_fwd(int out_dtype, int d, bool causal, const void *pack, void *out, float *lse, int BH,
                          int Nq, int Nk, float scale_log2, hipStream_t stream);

// Backward (bf16 / fp16, MFMA): the dQ kernel (which also writes the
// per-query statistics the second kernel reads) then the dK/dV kernel, in
// stream order.  workspace holds bwd_stats_bytes(BH, Nq) bytes.
size_t bwd_stats_bytes(int BH, int Nq);
hipError_t launch_backward(int dtype, int d, bool causal, const void *q, const void *k, const void *v,
                           const void *out, const void *dout, const float *lse, void *dq, void *dk, void *dv,
                           int BH, int Nq, int Nk, float scale, void *workspace, hipStream_t stream);

}  // namespace fa
