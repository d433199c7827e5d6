// fa_decode.hip -- split-KV forward for single-token decode on gfx950.
//
// Method ("6. FlashAttention 分块逻辑" section 11, FlashDecoding): with one
// query row the Q-block loop has a single block, so the K/V sequence is cut
// into chunks that separate workgroups process in parallel.  Stage one (per
// chunk c): scores s = scale * q K_c^T, local max m_c, p = exp(s - m_c),
// local sum l_c, local output o_c = p V_c; it stores lse_c = m_c + ln l_c and
// the normalised o~_c = o_c / l_c in float32.  Stage two merges the chunks:
// LSE = logsumexp_c lse_c and O = sum_c exp(lse_c - LSE) o~_c, which is the
// same function as the page's sequential (m, l, o) merge.
//
// The same stage one also reads a paged K/V cache (section 12 of the same
// page): keys are found through a per-sequence block table and each sequence
// has its own length, so one launch serves a batch of decode requests of
// different context lengths.
//
// The work is bound by HBM bandwidth (one pass over K and V, about 1 FLOP per
// byte), so the design is about bytes in flight, not arithmetic:
//  * a 256-thread workgroup reads its chunk as 16-byte loads; CH = d/8
//    consecutive lanes cover one key row (256 contiguous bytes at d = 128),
//    so every load instruction reads whole rows;
//  * each thread issues the loads of U = 8 keys of K and of V before it uses
//    any (8 KB per wave in flight per round);
//  * partial dot products are summed across the CH lanes of a row with
//    lane exchanges; each thread keeps an online (m, l, o) over its keys
//    and the workgroup merges the KL = 256/CH key lanes through LDS at the
//    end, so the only HBM traffic besides K and V is the chunk's d + 1
//    floats.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"
#include "fa_layout.h"

namespace fa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2d = 0.693147180559945309417f;
constexpr float kLog2e = 1.442695040888963407360f;
constexpr int kSplitThreads = 256;
// U: keys per thread per round, whose K and V loads are all in flight
// together.  d = 128: 16 (165 VGPRs, three waves per SIMD; 2.9% faster than
// 8 on contiguous B16 H32 Nk8192 in the per-XCD head order, 1% slower on the
// paged decode, which keeps it too so that both paths round alike and agree
// bit for bit under an identity table).  Smaller head dims, whose rounds of
// 256 / (d / 8) * U keys would outgrow common chunks: 8.
template <int D>
constexpr int keys_per_round() { return D >= 128 ? 16 : 8; }
constexpr int kMaxSplits = 1024;

struct SplitArgs {
    const void *q;
    const void *k;
    const void *v;
    float *ws_o;    // [BH, S, D] normalised chunk outputs
    float *ws_lse;  // [BH, S] chunk logsumexp (natural log)
    int BH;         // batch * heads
    int Nk;         // contiguous K/V: keys per (b, h)
    int S;
    int chunk;      // contiguous K/V: keys per chunk = ceil(Nk / S)
    float scale_log2;
    // paged K/V (k, v are caches [num_blocks, H, block_size, D])
    const int *block_table;  // [B, max_blocks]
    const int *seq_lens;     // [B]
    int H;
    int log2_block;
    int max_blocks;
    int num_blocks;
};

struct CombineArgs {
    const float *ws_o;
    const float *ws_lse;
    void *out;
    float *lse;
    int rows;
    int S;
};

// 2-byte element (bf16 or fp16) -> float
template <typename T>
__device__ __forceinline__ float lo_to_f32(uint32_t w);
template <typename T>
__device__ __forceinline__ float hi_to_f32(uint32_t w);

template <>
__device__ __forceinline__ float lo_to_f32<__bf16>(uint32_t w) { return __uint_as_float(w << 16); }
template <>
__device__ __forceinline__ float hi_to_f32<__bf16>(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
template <>
__device__ __forceinline__ float lo_to_f32<_Float16>(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <>
__device__ __forceinline__ float hi_to_f32<_Float16>(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// x plus the value of lane (lane of the same 16-lane row) by a DPP move:
// CTRL is the data-parallel-primitive control of the move.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF,
                                                                      false));
}

// Sum over the N lanes of a key row (N = 4, 8 or 16 consecutive lanes inside
// one 16-lane DPP row), every lane receiving the total: VALU moves within
// the row instead of LDS-crossbar exchanges.  N = 16: rotate by 8, then by 4
// (each lane then holds the sum of its residue class mod 4), then the quad
// exchanges 2 and 1.  N = 8: the half-row mirror pairs lane i with 7 - i,
// leaving each quad with the four pair sums, then the quad exchanges.
template <int N>
__device__ __forceinline__ float row_sum(float x) {
    constexpr int kRor8 = 0x128, kRor4 = 0x124, kHalfMirror = 0x141;
    constexpr int kQuadXor2 = 0x4E, kQuadXor1 = 0xB1;  // quad_perm [2,3,0,1], [1,0,3,2]
    static_assert(N == 4 || N == 8 || N == 16, "a key row spans 4, 8 or 16 lanes");
    if constexpr (N == 16) {
        x = dpp_add<kRor8>(x);
        x = dpp_add<kRor4>(x);
    } else if constexpr (N == 8) {
        x = dpp_add<kHalfMirror>(x);
    }
    x = dpp_add<kQuadXor2>(x);
    return dpp_add<kQuadXor1>(x);
}

// Stage one.  PAGED selects where key j of (b, h) lives: contiguous K/V at
// row (b*H + h)*Nk + j, or, for a paged cache ("6. FlashAttention 分块逻辑"
// section 12), at row (blk*H + h)*block_size + j % block_size of physical
// block blk = block_table[b][j / block_size].  A physical index outside
// [0, num_blocks) marks an unallocated block: its keys are skipped, as the
// page's kernel skips them.
template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(kSplitThreads) void splitkv_partial_kernel(SplitArgs a) {
    constexpr int NT = kSplitThreads;
    constexpr int CH = D / 8;   // lanes per key row (16 bytes each)
    constexpr int KL = NT / CH; // key lanes
    constexpr int U = keys_per_round<D>();
    static_assert(CH <= 64 && (CH & (CH - 1)) == 0, "row lanes must be a power of two within a wave");

    __shared__ float sm_m[KL];
    __shared__ float sm_l[KL];
    __shared__ float sm_o[KL * D];

    const int tid = threadIdx.x;
    const int dc = tid % CH;
    const int kl = tid / CH;
    // Workgroup w goes to XCD w % 8; with the grid a multiple of 8 the
    // prefill's order without the mask gives XCD x a contiguous range of
    // work items.  Contiguous K/V: the items are (head, chunk), so each XCD
    // streams whole heads, chunk after chunk (3-4% faster than consecutive
    // chunks spread over the XCDs).  Paged: a physical block holds every head
    // of its keys, so the items are ((sequence, chunk), head) and each XCD
    // reads whole blocks (1.9% faster than consecutive chunks; the per-head
    // order measured 1.7% slower there).
    int bh, cidx;
    if constexpr (PAGED) {
        int pair, head;
        layout::map_workgroup(blockIdx.x, a.BH / a.H * a.S, a.H, false, pair, head);
        cidx = pair % a.S;
        bh = (pair / a.S) * a.H + head;
    } else {
        layout::map_workgroup(blockIdx.x, a.BH, a.S, false, bh, cidx);
    }
    int len = a.Nk, chunk = a.chunk, b = 0, h = 0;
    if (PAGED) {
        b = bh / a.H;
        h = bh - b * a.H;
        len = min(max(a.seq_lens[b], 0), a.max_blocks << a.log2_block);  // never past the table
        chunk = (len + a.S - 1) / a.S;
    }
    const int kbeg = min(len, cidx * chunk);
    const int kend = min(len, kbeg + chunk);
    const float c = a.scale_log2;
    const int bmask = (1 << a.log2_block) - 1;
    const int *table = a.block_table + (size_t)b * a.max_blocks;
    // element offset of key row j (relative to the K/V base + dc*8), or -1
    auto row_of = [&](int j) -> long long {
        if (!PAGED) return (long long)j * D;
        const int blk = table[j >> a.log2_block];
        if (blk < 0 || blk >= a.num_blocks) return -1;
        return (((long long)blk * a.H + h) * (bmask + 1) + (j & bmask)) * D;
    };

    const size_t base_off = PAGED ? 0 : (size_t)bh * a.Nk * D;
    const T *kp = static_cast<const T *>(a.k) + base_off + dc * 8;
    const T *vp = static_cast<const T *>(a.v) + base_off + dc * 8;
    const u32x4 qraw = *reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.q) + (size_t)bh * D + dc * 8);
    float qv[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        qv[2 * w] = lo_to_f32<T>(qraw[w]);
        qv[2 * w + 1] = hi_to_f32<T>(qraw[w]);
    }

    float m_run = -__builtin_inff();  // exp2 domain
    float l_run = 0.f;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;

    for (int base = kbeg; base < kend; base += KL * U) {
        u32x4 kx[U], vx[U];
        long long roff[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int key = base + kl + KL * i;
            roff[i] = (key < kend) ? row_of(key) : -1;
        }
        // K and V are read once: nontemporal loads keep them from evicting
        // reusable lines and stream faster than plain loads
#pragma unroll
        for (int i = 0; i < U; ++i) {
            kx[i] = u32x4{0u, 0u, 0u, 0u};
            if (roff[i] >= 0) kx[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kp + roff[i]));
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            vx[i] = u32x4{0u, 0u, 0u, 0u};
            if (roff[i] >= 0) vx[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vp + roff[i]));
        }
        float s[U];
        float mx = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < U; ++i) {
            float dot = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                dot = __builtin_fmaf(qv[2 * w], lo_to_f32<T>(kx[i][w]), dot);
                dot = __builtin_fmaf(qv[2 * w + 1], hi_to_f32<T>(kx[i][w]), dot);
            }
            dot = row_sum<CH>(dot);
            s[i] = (roff[i] >= 0) ? dot * c : -__builtin_inff();
            mx = __builtin_fmaxf(mx, s[i]);
        }
        const float m_new = __builtin_fmaxf(m_run, mx);
        const float alpha = (m_new == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        const float msub = (m_new == -__builtin_inff()) ? 0.f : m_new;
        l_run *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const float p = __builtin_amdgcn_exp2f(s[i] - msub);
            l_run += p;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                o[2 * w] = __builtin_fmaf(p, lo_to_f32<T>(vx[i][w]), o[2 * w]);
                o[2 * w + 1] = __builtin_fmaf(p, hi_to_f32<T>(vx[i][w]), o[2 * w + 1]);
            }
        }
        m_run = m_new;
    }

    // merge the KL key lanes of the workgroup
    if (dc == 0) {
        sm_m[kl] = m_run;
        sm_l[kl] = l_run;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_o[kl * D + dc * 8 + e] = o[e];
    __syncthreads();

    const size_t slot = (size_t)bh * a.S + cidx;
    for (int dim = tid; dim < D; dim += NT) {
        float M = -__builtin_inff();
        for (int j = 0; j < KL; ++j) M = __builtin_fmaxf(M, sm_m[j]);
        float L = 0.f, O = 0.f;
        if (M != -__builtin_inff()) {
            for (int j = 0; j < KL; ++j) {
                const float w = __builtin_amdgcn_exp2f(sm_m[j] - M);  // exp2(-inf) = 0 for empty lanes
                L = __builtin_fmaf(sm_l[j], w, L);
                O = __builtin_fmaf(sm_o[j * D + dim], w, O);
            }
        }
        a.ws_o[slot * D + dim] = (L > 0.f) ? O / L : 0.f;
        if (dim == 0) a.ws_lse[slot] = (L > 0.f) ? (M + __builtin_amdgcn_logf(L)) * kLn2d : -__builtin_inff();
    }
}

template <typename T>
__device__ __forceinline__ T from_f32(float x) {
    return (T)x;  // round to nearest even
}

template <typename T, int D>
__global__ __launch_bounds__(256) void splitkv_combine_kernel(CombineArgs a) {
    __shared__ float wts[4][kMaxSplits];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = blockIdx.x * 4 + wave;
    const bool valid = row < a.rows;  // wave-uniform
    const int S = a.S;
    float LSE = 0.f;
    if (valid) {
        const float *lse_c = a.ws_lse + (size_t)row * S;
        float M = -__builtin_inff();
        for (int c = lane; c < S; c += 64) M = __builtin_fmaxf(M, lse_c[c]);
#pragma unroll
        for (int msk = 32; msk > 0; msk >>= 1) M = __builtin_fmaxf(M, __shfl_xor(M, msk));
        if (M == -__builtin_inff()) {  // no visible key in any chunk: O = 0, LSE = -inf
            LSE = M;
            for (int c = lane; c < S; c += 64) wts[wave][c] = 0.f;
        } else {
            float L = 0.f;
            for (int c = lane; c < S; c += 64) L += __builtin_amdgcn_exp2f((lse_c[c] - M) * kLog2e);
#pragma unroll
            for (int msk = 32; msk > 0; msk >>= 1) L += __shfl_xor(L, msk);
            LSE = M + __builtin_amdgcn_logf(L) * kLn2d;
            for (int c = lane; c < S; c += 64) wts[wave][c] = __builtin_amdgcn_exp2f((lse_c[c] - LSE) * kLog2e);
        }
    }
    __syncthreads();  // reached by every wave
    if (!valid) return;

    T *op = static_cast<T *>(a.out) + (size_t)row * D;
    const float *oc = a.ws_o + (size_t)row * S * D;
    for (int dim = lane; dim < D; dim += 64) {
        float acc = 0.f;
        for (int c = 0; c < S; ++c) acc = __builtin_fmaf(wts[wave][c], oc[(size_t)c * D + dim], acc);
        op[dim] = from_f32<T>(acc);
    }
    if (lane == 0 && a.lse != nullptr) a.lse[row] = LSE;
}

template <typename T, int D, bool PAGED>
hipError_t launch_splitkv_typed(const SplitArgs &base, void *out, float *lse, int BH, hipStream_t stream) {
    SplitArgs a = base;
    a.BH = BH;
    float *ws_o = a.ws_o;
    float *ws_lse = ws_o + (size_t)BH * a.S * D;
    a.ws_lse = ws_lse;
    const long long nwg = (long long)BH * a.S;
    if (nwg > 0x7fffffffLL || a.S > kMaxSplits) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((splitkv_partial_kernel<T, D, PAGED>), dim3((unsigned)nwg), dim3(kSplitThreads), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    CombineArgs b;
    b.ws_o = ws_o;
    b.ws_lse = ws_lse;
    b.out = out;
    b.lse = lse;
    b.rows = BH;
    b.S = a.S;
    hipLaunchKernelGGL((splitkv_combine_kernel<T, D>), dim3((BH + 3) / 4), dim3(256), 0, stream, b);
    return hipGetLastError();
}

template <bool PAGED>
hipError_t launch_any(int dtype, int d, const SplitArgs &a, void *out, float *lse, int BH, hipStream_t stream) {
#define FA_CASE(DD)                                                                                 \
    case DD:                                                                                        \
        return dtype == 2 ? launch_splitkv_typed<__bf16, DD, PAGED>(a, out, lse, BH, stream)        \
                          : launch_splitkv_typed<_Float16, DD, PAGED>(a, out, lse, BH, stream);
    if (dtype != 1 && dtype != 2) return hipErrorInvalidValue;
    switch (d) {
        FA_CASE(32)
        FA_CASE(64)
        FA_CASE(128)
        default: return hipErrorInvalidValue;
    }
#undef FA_CASE
}

}  // namespace

hipError_t launch_combine(int dtype, int d, const float *ws_o, const float *ws_lse, void *out, float *lse,
                          int rows, int S, hipStream_t stream) {
    if (S < 1 || S > kMaxSplits || rows < 1) return hipErrorInvalidConfiguration;
    CombineArgs b;
    b.ws_o = ws_o;
    b.ws_lse = ws_lse;
    b.out = out;
    b.lse = lse;
    b.rows = rows;
    b.S = S;
    const dim3 grid((unsigned)((rows + 3) / 4));
#define FA_CASE(DD)                                                                                      \
    case DD:                                                                                             \
        if (dtype == 2) hipLaunchKernelGGL((splitkv_combine_kernel<__bf16, DD>), grid, dim3(256), 0, stream, b); \
        else if (dtype == 1) hipLaunchKernelGGL((splitkv_combine_kernel<_Float16, DD>), grid, dim3(256), 0, stream, b); \
        else hipLaunchKernelGGL((splitkv_combine_kernel<float, DD>), grid, dim3(256), 0, stream, b);             \
        return hipGetLastError();
    if (dtype != 0 && dtype != 1 && dtype != 2) return hipErrorInvalidValue;
    switch (d) {
        FA_CASE(32)
        FA_CASE(64)
        FA_CASE(128)
        default: return hipErrorInvalidValue;
    }
#undef FA_CASE
}

hipError_t launch_splitkv(int dtype, int d, const void *q, const void *k, const void *v, void *out, float *lse,
                          int BH, int Nk, float scale_log2, int num_splits, void *workspace, hipStream_t stream) {
    SplitArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.ws_o = static_cast<float *>(workspace);
    a.Nk = Nk;
    a.S = num_splits;
    a.chunk = (Nk + num_splits - 1) / num_splits;
    a.scale_log2 = scale_log2;
    return launch_any<false>(dtype, d, a, out, lse, BH, stream);
}

hipError_t launch_paged_decode(int dtype, int d, const void *q, const void *k_cache, const void *v_cache,
                               const int *block_table, const int *seq_lens, void *out, float *lse, int B, int H,
                               int log2_block, int max_blocks, int num_blocks, float scale_log2, int num_splits,
                               void *workspace, hipStream_t stream) {
    SplitArgs a = {};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.ws_o = static_cast<float *>(workspace);
    a.S = num_splits;
    a.scale_log2 = scale_log2;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.H = H;
    a.log2_block = log2_block;
    a.max_blocks = max_blocks;
    a.num_blocks = num_blocks;
    return launch_any<true>(dtype, d, a, out, lse, B * H, stream);
}

}  // namespace fa
