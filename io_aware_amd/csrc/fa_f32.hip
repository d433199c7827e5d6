// fa_f32.hip -- tiled FlashAttention forward in float32 (vector ALU).
//
// Same method as the 16-bit path ("6. FlashAttention 分块逻辑" sections 3-6;
// "9.4 FlashAttention 与 FlashMLA" section 9.4.5) with Br = Bc = 64: a
// workgroup owns 64 query rows of one (batch, head), one row per lane of
// each of its NW waves.  K/V blocks of 64 keys are staged in LDS by the whole
// workgroup and read by all lanes of a wave at the same address
// (broadcast); wave w takes keys w*64/NW .. (w+1)*64/NW - 1 of every block,
// so the NW waves split the key loop.  Each lane keeps its query row, its
// float32 output row and its running max / running sum over its wave's keys
// in registers.  Per block: scores, block max, one exact rescale by
// exp(m - m_new), P = exp(S - m_new), l += sum P, O += P V.  At the end the
// NW partial states of a row are merged pairwise through LDS (the split-KV
// combine of section 11 of the first page, inside one workgroup): with
// M = max(m1, m2), l = l1 e^(m1-M) + l2 e^(m2-M), o likewise; then O = o / l
// and LSE = M + ln l.  Every product and sum is a float32 FMA; exp is exp2
// with scale*log2(e) folded in.
//
// A grid of fewer workgroups than the GPU has CUs leaves most of it idle
// while each workgroup walks its whole key range on one CU.  Such grids are
// split along the keys (split-KV, section 11 of the first page): workgroup
// (row block, chunk) walks one chunk of whole 32-key blocks and writes its
// normalised partial o / l and its logsumexp to a workspace, and the
// split-KV combine merges the chunks.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "fa_internal.h"

#ifndef FA_F32_SPLIT_BLOCK
#define FA_F32_SPLIT_BLOCK 32
#endif

namespace fa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2f = 0.693147180559945309417f;

struct F32Args {
    const float *q;
    const float *k;
    const float *v;
    float *out;
    float *lse;
    int Nq;
    int Nk;
    int Tr;  // 64-row Q blocks per (batch, head)
    // split launch: chunk c covers keys [c * chunk, (c + 1) * chunk)
    float *ws_o;    // [BH * Nq, S, D] normalised partials
    float *ws_lse;  // [BH * Nq, S] their logsumexp (natural log)
    int S;
    int chunk;      // keys per chunk, a multiple of the split block
    float scale_log2;  // |scale| * log2(e) (1 for a zero scale; see FoldedScale)
    uint32_t qflip;    // sign bit flipped in Q for a negative scale
    uint32_t qkeep;    // 0 zeroes Q for a zero scale
};

// waves per workgroup: as many as keep q and o (2 D floats per lane) in
// registers at two or more waves per SIMD
template <int D>
constexpr int f32_waves() { return D <= 32 ? 16 : (D <= 64 ? 8 : 4); }

// Keys per K/V block of a split launch: chunks are whole blocks, so a short
// key range still splits over many workgroups (32 measured best against 16
// and 64 on short and long ranges).
constexpr int kSplitBlock = FA_F32_SPLIT_BLOCK;

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(f32_waves<D>() * 64) void prefill_f32_kernel(F32Args a) {
    constexpr int NW = f32_waves<D>();
    constexpr int BR = 64;
    constexpr int BC = SPLIT ? kSplitBlock : 64;
    constexpr int KPW = BC / NW;  // keys of a block per wave
    static_assert(BC % NW == 0, "every wave takes the same number of keys of a block");
    constexpr int C4 = D / 4;     // float4 chunks per row
    constexpr int KV_FLOATS = 2 * BC * D;                 // one K and one V block
    constexpr int MERGE_FLOATS = (NW / 2) * 64 * (D + 2);  // the upper half's (m, l, o) of a merge round
    constexpr int SMEM_FLOATS = KV_FLOATS > MERGE_FLOATS ? KV_FLOATS : MERGE_FLOATS;
    __shared__ __attribute__((aligned(16))) float smem[SMEM_FLOATS];
    f32x4 *ks = reinterpret_cast<f32x4 *>(smem);
    f32x4 *vs = ks + BC * C4;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int wg = blockIdx.x, chunk_idx = 0;
    if constexpr (SPLIT) {  // the chunks of one row block are neighbours
        chunk_idx = wg % a.S;
        wg /= a.S;
    }
    const int bh = wg / a.Tr;
    const int q0 = (wg - bh * a.Tr) * BR;
    const int row = q0 + lane;
    const int Nq = a.Nq;
    const int Nk = a.Nk;
    const float c = a.scale_log2;
    const float *qp = a.q + (size_t)bh * Nq * D;
    const float *kp = a.k + (size_t)bh * Nk * D;
    const float *vp = a.v + (size_t)bh * Nk * D;

    float q[D];
    float o[D];
#pragma unroll
    for (int t = 0; t < D; t += 4) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (row < Nq) x = *reinterpret_cast<const f32x4 *>(qp + (size_t)row * D + t);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __uint_as_float((__float_as_uint(x[e]) ^ a.qflip) & a.qkeep);
        q[t] = x[0];
        q[t + 1] = x[1];
        q[t + 2] = x[2];
        q[t + 3] = x[3];
        o[t] = o[t + 1] = o[t + 2] = o[t + 3] = 0.f;
    }
    float m = -__builtin_inff();  // exp2 domain, over this wave's keys
    float l = 0.f;

    const int kv_end = CAUSAL ? min(Nk, q0 + BR) : Nk;
    // keys [kbeg, kend): all visible ones, or one chunk (workgroup-uniform)
    const int kbeg = SPLIT ? min(kv_end, chunk_idx * a.chunk) : 0;
    const int kend = SPLIT ? min(kv_end, kbeg + a.chunk) : kv_end;
    for (int k0 = kbeg; k0 < kend; k0 += BC) {
        __syncthreads();  // the previous block's reads are done
        for (int idx = tid; idx < BC * C4; idx += NW * 64) {
            const int key = k0 + idx / C4;
            const int c4 = idx % C4;
            f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
            if (key < Nk) {
                kx = *reinterpret_cast<const f32x4 *>(kp + (size_t)key * D + 4 * c4);
                vx = *reinterpret_cast<const f32x4 *>(vp + (size_t)key * D + 4 * c4);
            }
            ks[idx] = kx;
            vs[idx] = vx;
        }
        __syncthreads();

        float s[KPW];
        float mx = -__builtin_inff();
#pragma unroll
        for (int jj = 0; jj < KPW; ++jj) {
            const int j = wave * KPW + jj;
            float dot = 0.f;
#pragma unroll
            for (int t = 0; t < C4; ++t) {
                const f32x4 kx = ks[j * C4 + t];
                dot = __builtin_fmaf(q[4 * t], kx[0], dot);
                dot = __builtin_fmaf(q[4 * t + 1], kx[1], dot);
                dot = __builtin_fmaf(q[4 * t + 2], kx[2], dot);
                dot = __builtin_fmaf(q[4 * t + 3], kx[3], dot);
            }
            const int key = k0 + j;
            const bool visible = key < Nk && (!CAUSAL || key <= row);
            s[jj] = visible ? dot : -__builtin_inff();
            mx = __builtin_fmaxf(mx, s[jj]);
        }
        const float m_new = __builtin_fmaxf(m, mx * c);  // c > 0 (the sign is in Q)
        const float alpha = (m_new == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
        const float msub = (m_new == -__builtin_inff()) ? 0.f : m_new;
        l *= alpha;
#pragma unroll
        for (int t = 0; t < D; ++t) o[t] *= alpha;
#pragma unroll
        for (int jj = 0; jj < KPW; ++jj) {
            const int j = wave * KPW + jj;
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jj], c, -msub));
            l += p;
#pragma unroll
            for (int t = 0; t < C4; ++t) {
                const f32x4 vx = vs[j * C4 + t];
                o[4 * t] = __builtin_fmaf(p, vx[0], o[4 * t]);
                o[4 * t + 1] = __builtin_fmaf(p, vx[1], o[4 * t + 1]);
                o[4 * t + 2] = __builtin_fmaf(p, vx[2], o[4 * t + 2]);
                o[4 * t + 3] = __builtin_fmaf(p, vx[3], o[4 * t + 3]);
            }
        }
        m = m_new;
    }

    // ---- merge the NW partial states of each row, halving the waves per round
#pragma unroll
    for (int half = NW / 2; half >= 1; half >>= 1) {
        __syncthreads();  // LDS is free (block reads or the previous round are done)
        if (wave >= half && wave < 2 * half) {
            float *dst = smem + (size_t)((wave - half) * 64 + lane) * (D + 2);
            dst[0] = m;
            dst[1] = l;
#pragma unroll
            for (int t = 0; t < D; ++t) dst[2 + t] = o[t];
        }
        __syncthreads();
        if (wave < half) {
            const float *src = smem + (size_t)(wave * 64 + lane) * (D + 2);
            const float m2 = src[0], l2 = src[1];
            const float M = __builtin_fmaxf(m, m2);
            // exp2(-inf) = 0 weighs out a side without keys; M = -inf: both empty
            const float a1 = (M == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(m - M);
            const float a2 = (M == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
            l = __builtin_fmaf(l2, a2, l * a1);
#pragma unroll
            for (int t = 0; t < D; ++t) o[t] = __builtin_fmaf(src[2 + t], a2, o[t] * a1);
            m = M;
        }
    }

    // (split launch: this chunk's o / l and logsumexp, -inf with o = 0 where
    // the chunk holds no visible key of the row)
    if (wave == 0 && row < Nq) {
        const float inv = (l > 0.f) ? 1.f / l : 0.f;
        const float lse_row = (l > 0.f) ? (m + __builtin_amdgcn_logf(l)) * kLn2f : -__builtin_inff();
        const size_t slot = SPLIT ? ((size_t)bh * Nq + row) * a.S + chunk_idx : 0;
        float *op = SPLIT ? a.ws_o + slot * D : a.out + (size_t)bh * Nq * D + (size_t)row * D;
#pragma unroll
        for (int t = 0; t < D; t += 4)
            *reinterpret_cast<f32x4 *>(op + t) = f32x4{o[t] * inv, o[t + 1] * inv, o[t + 2] * inv, o[t + 3] * inv};
        if (SPLIT)
            a.ws_lse[slot] = lse_row;
        else if (a.lse != nullptr)
            a.lse[(size_t)bh * Nq + row] = lse_row;
    }
}

// kSplitBlock-key blocks of the key range a split cuts (under the mask, the
// last row block's range; chunks past a row block's range are empty)
int f32_key_blocks(bool causal, int Nq, int Nk) {
    const long long rows = (long long)(Nq + 63) / 64 * 64;
    const int kext = causal && rows < Nk ? (int)rows : Nk;
    return (kext + kSplitBlock - 1) / kSplitBlock;
}

template <int D, bool CAUSAL>
hipError_t launch_f32_one(const void *q, const void *k, const void *v, void *out, float *lse, int BH, int Nq,
                          int Nk, float sl, int S, void *workspace, hipStream_t stream) {
    F32Args a = {};
    a.q = static_cast<const float *>(q);
    a.k = static_cast<const float *>(k);
    a.v = static_cast<const float *>(v);
    a.out = static_cast<float *>(out);
    a.lse = lse;
    a.Nq = Nq;
    a.Nk = Nk;
    a.Tr = (Nq + 63) / 64;
    const FoldedScale fs = fold_scale(sl, kSignBits32);
    a.scale_log2 = fs.c;
    a.qflip = fs.flip;
    a.qkeep = fs.keep;
    if (S > 1) {
        if (S > f32_key_blocks(CAUSAL, Nq, Nk) || workspace == nullptr) return hipErrorInvalidValue;
        a.S = S;
        a.chunk = (f32_key_blocks(CAUSAL, Nq, Nk) + S - 1) / S * kSplitBlock;
        a.ws_o = static_cast<float *>(workspace);
        a.ws_lse = a.ws_o + (size_t)BH * Nq * S * D;
    }
    const long long nwg = (long long)BH * a.Tr * (S > 1 ? S : 1);
    if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (S > 1)
        hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL, true>), dim3((unsigned)nwg), dim3(f32_waves<D>() * 64), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL, false>), dim3((unsigned)nwg), dim3(f32_waves<D>() * 64),
                           0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || S < 2) return err;
    return launch_combine(0, D, a.ws_o, a.ws_lse, out, lse, BH * Nq, S, stream);
}

}  // namespace

int f32_split_normalise(bool causal, int Nq, int Nk, int S) {
    const int blocks = f32_key_blocks(causal, Nq, Nk);
    S = S < blocks ? S : blocks;
    if (S < 2) return 1;
    // whole blocks per chunk; drop chunks that would start past the keys
    const int per = (blocks + S - 1) / S;
    return (blocks + per - 1) / per;
}

int f32_split_count(bool causal, int BH, int Nq, int Nk) {
    if (BH < 1 || Nq < 1 || Nk < 1) return 1;
    const long long grid = (long long)BH * ((Nq + 63) / 64);
    int S;
    const char *env = getenv("FA_F32_SPLIT");
    if (env != nullptr && env[0] != '\0') {
        S = atoi(env);  // 0 or 1: never split; n: at most n chunks
    } else {
        // Split while the grid is below one workgroup per CU: every 64 keys
        // of a workgroup's range cost several microseconds of vector-ALU
        // work on its CU, against a few for the combine launch.  Aim for two
        // workgroups per CU, at most 64 chunks.
        constexpr long long kCUs = 256;
        if (grid >= kCUs) return 1;
        S = (int)((2 * kCUs + grid - 1) / grid);
        S = S < 64 ? S : 64;
    }
    return f32_split_normalise(causal, Nq, Nk, S);
}

hipError_t launch_prefill_f32(int d, bool causal, const void *q, const void *k, const void *v, void *out,
                              float *lse, int BH, int Nq, int Nk, float sl, int S, void *workspace,
                              hipStream_t stream) {
#define FA_CASE(DD)                                                                                             \
    case DD:                                                                                                    \
        return causal ? launch_f32_one<DD, true>(q, k, v, out, lse, BH, Nq, Nk, sl, S, workspace, stream)       \
                      : launch_f32_one<DD, false>(q, k, v, out, lse, BH, Nq, Nk, sl, S, workspace, stream);
    switch (d) {
        FA_CASE(32)
        FA_CASE(64)
        FA_CASE(128)
        default: return hipErrorInvalidValue;
    }
#undef FA_CASE
}

}  // namespace fa
