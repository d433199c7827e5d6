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
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

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
    float scale_log2;  // |scale| * log2(e) (1 for a zero scale; see FoldedScale)
    uint32_t qflip;    // sign bit flipped in Q for a negative scale
    uint32_t qkeep;    // 0 zeroes Q for a zero scale
};

// waves per workgroup: as many as keep q and o (2 D floats per lane) in
// registers at two or more waves per SIMD
template <int D>
constexpr int f32_waves() { return D <= 32 ? 16 : (D <= 64 ? 8 : 4); }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(f32_waves<D>() * 64) void prefill_f32_kernel(F32Args a) {
    constexpr int NW = f32_waves<D>();
    constexpr int BR = 64;
    constexpr int BC = 64;
    constexpr int KPW = BC / NW;  // keys of a block per wave
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
    const int bh = blockIdx.x / a.Tr;
    const int q0 = (blockIdx.x - bh * a.Tr) * BR;
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
    for (int k0 = 0; k0 < kv_end; k0 += BC) {
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

    if (wave == 0 && row < Nq) {
        const float inv = (l > 0.f) ? 1.f / l : 0.f;
        float *op = a.out + (size_t)bh * Nq * D + (size_t)row * D;
#pragma unroll
        for (int t = 0; t < D; t += 4)
            *reinterpret_cast<f32x4 *>(op + t) = f32x4{o[t] * inv, o[t + 1] * inv, o[t + 2] * inv, o[t + 3] * inv};
        if (a.lse != nullptr)
            a.lse[(size_t)bh * Nq + row] = (l > 0.f) ? (m + __builtin_amdgcn_logf(l)) * kLn2f : -__builtin_inff();
    }
}

template <int D, bool CAUSAL>
hipError_t launch_f32_one(const void *q, const void *k, const void *v, void *out, float *lse, int BH, int Nq,
                          int Nk, float sl, hipStream_t stream) {
    F32Args a;
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
    const long long nwg = (long long)BH * a.Tr;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(f32_waves<D>() * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(int d, bool causal, const void *q, const void *k, const void *v, void *out,
                              float *lse, int BH, int Nq, int Nk, float sl, hipStream_t stream) {
#define FA_CASE(DD)                                                                           \
    case DD:                                                                                  \
        return causal ? launch_f32_one<DD, true>(q, k, v, out, lse, BH, Nq, Nk, sl, stream)   \
                      : launch_f32_one<DD, false>(q, k, v, out, lse, BH, Nq, Nk, sl, stream);
    switch (d) {
        FA_CASE(32)
        FA_CASE(64)
        FA_CASE(128)
        default: return hipErrorInvalidValue;
    }
#undef FA_CASE
}

}  // namespace fa
