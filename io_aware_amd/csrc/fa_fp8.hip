// fa_fp8.hip -- FP8 (E4M3) attention forward with incoherent processing, gfx950.
//
// Method ("9.4 FlashAttention 与 FlashMLA" section 9.4.4, the FP8 mode of
// FlashAttention-3): Q, K and V enter the matrix products as 8-bit floats;
// before quantisation Q and K are multiplied by one random orthogonal matrix
// M = diag(s) H_d / sqrt(d) (rows x -> x M: signs, then the Hadamard
// butterfly; the same M for both, so Q K^T is unchanged), which
// spreads large-magnitude channels over all channels and evens out the
// quantisation error.  V is quantised as it is.
//
// Two steps, two entry points:
//  * quantisation (fa_quantize_fp8): a clear kernel, an amax kernel (the
//    transform, then the largest magnitude per (batch, head) and tensor by
//    atomic max) and a quantise kernel (the transform again, x * 448 / amax
//    clamped to +-448, rounded to E4M3 by v_cvt_pk_fp8_f32).  It writes the
//    "pack": Q and K codes row-major, V codes transposed ([d][keys]) with the
//    keys of every 64-key group in the order the attention kernel's P
//    registers hold them, and the per-head descale factors amax / 448.
//  * attention (fa_fwd_fp8): the prefill kernel's structure with the
//    32x32x64 FP8 MFMA (twice the 16-bit rate): S^T = K Q^T from K code rows
//    in LDS and Q code fragments in registers, the online softmax with the
//    lazy rescale (scale * descale_q * descale_k folded into the exp2 FMA),
//    P rounded to E4M3 (P <= 2^8 < 448 under the lazy-rescale bound), and
//    O^T += V^T P^T with V^T rows read straight from the transposed codes --
//    no transposing read is needed, because the pack already holds V^T in
//    the P operand's key order.  O = acc * descale_v / l8, where l8 sums the
//    rounded P that formed acc (so a dominant key keeps weight 1 whatever
//    its rounding), and LSE comes from the float32 sum.
//
// The fast Walsh-Hadamard transform of a row runs in registers: each lane
// holds 8 consecutive elements (three in-lane butterfly stages), the other
// stages pair lanes (lane ^ 1, ^ 2, ...) within the d/8 lanes of the row.
// Every element goes through the same float32 operations in the same order
// as the host reference, so the E4M3 codes are reproducible bit for bit.
#include <cstdint>
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_layout.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;

// D (32x32 float32) += A (32x64) B (64x32), A and B E4M3 (32 codes per lane)
__device__ __forceinline__ f32x16 mfma_e4m3(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// D (16x16 float32) += A (16x128) B (128x16), A and B E4M3 (32 codes per lane)
__device__ __forceinline__ f32x4 mfma16_e4m3(i32x8 a, i32x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
constexpr int kKeyGroup = 64;   // keys per attention tile and per V^T group

struct Fp8Pack {
    uint8_t *q8;      // [BH, Nq, D]
    uint8_t *k8;      // [BH, Nkp, D]
    uint8_t *v8t;     // [BH, D, Nkp], keys permuted within each 64-key group
    float *descale;   // [3][BH]: q, k, v
    uint32_t *amax;   // [3][BH] float bits of max |x| (scratch)
};

template <typename T>
__device__ __forceinline__ void unpack8(u32x4 raw, float x[8]) {
    typedef T t8 __attribute__((ext_vector_type(8)));
    const t8 v = __builtin_bit_cast(t8, raw);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}

// 16 bytes of a row that is read once (nontemporal), or zeros
template <typename T>
__device__ __forceinline__ u32x4 load_once(const T *p, bool ok) {
    return ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)) : u32x4{0u, 0u, 0u, 0u};
}

// Lanes and chunks of a row.  A row of D elements is spread over CH = D/8
// lanes of one DPP row (16 lanes), 8 consecutive elements (a 16-byte chunk)
// per lane.  Lane L of the group holds chunk ck(L) = L ^ (L & 4 ? 3 : 0):
// chunk bit k then sits across the lane exchange L ^ v_k with
// v = (1, 2, 7, 8), and every v_k is one DPP move -- quad permutations for 1
// and 2, the half-row mirror for 7, a row rotation by 8 for 8.
__device__ __forceinline__ int chunk_of_lane(int lc) { return lc ^ ((lc & 4) ? 3 : 0); }

// the value of lane ^ V within each row of 16 lanes
template <int V>
__device__ __forceinline__ float lane_xor(float v) {
    const int b = __float_as_int(v);
    constexpr int ctrl = V == 1 ? 0xB1 : V == 2 ? 0x4E : V == 7 ? 0x141 : 0x128;
    static_assert(V == 1 || V == 2 || V == 7 || V == 8, "one DPP move per exchange");
    return __int_as_float(__builtin_amdgcn_mov_dpp(b, ctrl, 0xF, 0xF, true));
}

// The sign flips of the transform for this lane's chunk, as XOR masks on the
// packed 16-bit elements (bit 15 / 31 of each word): x * (+-1) is exact, so
// flipping the sign bits of the inputs is the same as multiplying.
__device__ __forceinline__ u32x4 sign_masks(const float *signs, int ck) {
    u32x4 m = {0u, 0u, 0u, 0u};
    if (signs != nullptr) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
            m[w] = (signs[8 * ck + 2 * w] < 0.0f ? 0x8000u : 0u) | (signs[8 * ck + 2 * w + 1] < 0.0f ? 0x80000000u : 0u);
    }
    return m;
}

// H_d / sqrt(d) (with NORM; without it the unnormalised butterfly) of the
// row a group of CH = D/8 lanes holds, the signs already applied (nothing if
// there are no signs: M = I).  The butterfly pairs element i with i ^ h; the
// element with bit h clear becomes a + b, the one with it set a - b (a the
// clear one); stages h = 1, 2, 4 run in registers, h = 8, 16, 32, 64 across
// the lanes of the group.
template <int D, bool NORM>
__device__ __forceinline__ void transform_row(float x[8], bool has_signs, int ck) {
    constexpr int CH = D / 8;
    if (!has_signs) return;  // no transform (M = I)
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if ((e & h) == 0) {
                const float a = x[e], b = x[e + h];
                x[e] = a + b;
                x[e + h] = a - b;
            }
        }
    }
    static_assert(CH <= 16, "a row spans at most one 16-lane DPP row");
    auto stage = [&](auto k_tag, auto v_tag) {
        constexpr int K = decltype(k_tag)::value;
        constexpr int V = decltype(v_tag)::value;
        if constexpr ((1 << K) < CH) {
            // lower chunk: x + other; upper chunk: other - x.  Both are
            // fma(x, +-1, other): x * (+-1) is exact, so the one rounding is
            // that of the sum, as in a + b and a - b.
            const float sgn = ((ck >> K) & 1) ? -1.0f : 1.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = __builtin_fmaf(x[e], sgn, lane_xor<V>(x[e]));
        }
    };
    stage(Int<0>{}, Int<1>{});
    stage(Int<1>{}, Int<2>{});
    stage(Int<2>{}, Int<7>{});
    stage(Int<3>{}, Int<8>{});
    if constexpr (NORM) {
        const float norm = (float)(1.0 / __builtin_sqrt((double)D));  // 1/sqrt(d) rounded once to float32
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= norm;
    }
}

// ---------------------------------------------------------------------------
// Quantisation
// ---------------------------------------------------------------------------
__global__ void fp8_clear_kernel(uint32_t *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Rows handled by one workgroup of the amax / quantise kernels: 64 query
// rows, 64 key rows and the 64 value rows of one key group.
constexpr int kQuantRows = 64;
constexpr int kQuantThreads = 256;
// row blocks per amax workgroup: its waves reduce through LDS and it issues
// one atomic per tensor, so each (head, tensor) word sees few atomics
constexpr int kAmaxBlocks = 4;

struct QuantArgs {
    const void *q;
    const void *k;
    const void *v;
    const float *signs;   // [D] or null: no transform
    Fp8Pack pack;
    int BH;
    int Nq;
    int Nk;
    int Nkp;
};

template <typename T, int D>
__global__ __launch_bounds__(kQuantThreads) void fp8_amax_kernel(QuantArgs a) {
    constexpr int CH = D / 8;
    constexpr int RPI = kQuantThreads / CH;   // rows per pass
    constexpr int NP = kQuantRows / RPI;      // passes per row block
    __shared__ float wmax[kQuantThreads / 64][3];
    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int ck = chunk_of_lane(tid % CH);
    const bool has_signs = a.signs != nullptr;
    const u32x4 smask = sign_masks(a.signs, ck);
    // The unnormalised butterfly, then one multiply by 1/sqrt(d) at the end:
    // rounding is monotone and odd, so max_i |fl(x_i / sqrt(d))| equals
    // fl(max_i |x_i| / sqrt(d)), the largest transformed magnitude.
    float m[3] = {0.0f, 0.0f, 0.0f};
    for (int blk = 0; blk < kAmaxBlocks; ++blk) {
        const int r0 = (blockIdx.y * kAmaxBlocks + blk) * kQuantRows;
        // every pass's loads are issued before any is used
        u32x4 rq[NP], rk[NP], rv[NP];
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
            const int row = r0 + pass * RPI + tid / CH;
            rq[pass] = load_once(static_cast<const T *>(a.q) + ((size_t)bh * a.Nq + row) * D + 8 * ck, row < a.Nq);
            rk[pass] = load_once(static_cast<const T *>(a.k) + ((size_t)bh * a.Nk + row) * D + 8 * ck, row < a.Nk);
            rv[pass] = load_once(static_cast<const T *>(a.v) + ((size_t)bh * a.Nk + row) * D + 8 * ck, row < a.Nk);
        }
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
            const int row = r0 + pass * RPI + tid / CH;
            float x[8];
            if (row < a.Nq) {  // CH lanes share the row: the group is uniform, the exchanges stay inside it
                unpack8<T>(rq[pass] ^ smask, x);
                transform_row<D, false>(x, has_signs, ck);
#pragma unroll
                for (int e = 0; e < 8; ++e) m[0] = __builtin_fmaxf(m[0], __builtin_fabsf(x[e]));
            }
            if (row < a.Nk) {
                unpack8<T>(rk[pass] ^ smask, x);
                transform_row<D, false>(x, has_signs, ck);
#pragma unroll
                for (int e = 0; e < 8; ++e) m[1] = __builtin_fmaxf(m[1], __builtin_fabsf(x[e]));
                unpack8<T>(rv[pass], x);
#pragma unroll
                for (int e = 0; e < 8; ++e) m[2] = __builtin_fmaxf(m[2], __builtin_fabsf(x[e]));
            }
        }
    }
    if (has_signs) {
        const float norm = (float)(1.0 / __builtin_sqrt((double)D));
        m[0] *= norm;
        m[1] *= norm;
    }
#pragma unroll
    for (int t = 0; t < 3; ++t) {
#pragma unroll
        for (int msk = 32; msk > 0; msk >>= 1) m[t] = __builtin_fmaxf(m[t], __shfl_xor(m[t], msk));
        if ((tid & 63) == 0) wmax[tid >> 6][t] = m[t];
    }
    __syncthreads();
    if (tid < 3) {
        float r = wmax[0][tid];
#pragma unroll
        for (int w = 1; w < kQuantThreads / 64; ++w) r = __builtin_fmaxf(r, wmax[w][tid]);
        // non-negative floats order like their bit patterns
        atomicMax(&a.pack.amax[tid * a.BH + bh], __float_as_uint(r));
    }
}

__device__ __forceinline__ float inv_scale(uint32_t amax_bits) {
    const float amax = __uint_as_float(amax_bits);
    return amax > 0.0f ? kE4M3Max / amax : 1.0f;
}

// four floats -> four E4M3 codes (round to nearest even), packed little-endian.
// The first conversion writes bytes 0-1 of its "old" operand and keeps bytes
// 2-3, which the second conversion overwrites: any word serves as "old", and
// a's own bits avoid a register clear per word.
__device__ __forceinline__ uint32_t to_e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)__float_as_uint(a), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ float clamp448(float x) {
    return __builtin_fminf(__builtin_fmaxf(x, -kE4M3Max), kE4M3Max);
}

template <typename T, int D>
__global__ __launch_bounds__(kQuantThreads) void fp8_quantize_kernel(QuantArgs a) {
    constexpr int CH = D / 8;
    constexpr int RPI = kQuantThreads / CH;
    __shared__ uint8_t vtile[kQuantRows][D];   // the key group's V codes, key-major
    const int bh = blockIdx.x;
    const int r0 = blockIdx.y * kQuantRows;
    const int tid = threadIdx.x;
    const int ck = chunk_of_lane(tid % CH);
    const bool has_signs = a.signs != nullptr;
    const u32x4 smask = sign_masks(a.signs, ck);
    const float iq = inv_scale(a.pack.amax[bh]);
    const float ik = inv_scale(a.pack.amax[a.BH + bh]);
    const float iv = inv_scale(a.pack.amax[2 * a.BH + bh]);
    if (blockIdx.y == 0 && tid < 3) {
        const float amax = __uint_as_float(a.pack.amax[tid * a.BH + bh]);
        a.pack.descale[tid * a.BH + bh] = amax > 0.0f ? amax / kE4M3Max : 1.0f;
    }
    constexpr int NP = kQuantRows / RPI;      // passes
    // every pass's loads are issued before any is used
    u32x4 rq[NP], rk[NP], rv[NP];
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
        const int row = r0 + pass * RPI + tid / CH;
        rq[pass] = load_once(static_cast<const T *>(a.q) + ((size_t)bh * a.Nq + row) * D + 8 * ck, row < a.Nq);
        rk[pass] = load_once(static_cast<const T *>(a.k) + ((size_t)bh * a.Nk + row) * D + 8 * ck, row < a.Nk);
        rv[pass] = load_once(static_cast<const T *>(a.v) + ((size_t)bh * a.Nk + row) * D + 8 * ck, row < a.Nk);
    }
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
        const int rl = pass * RPI + tid / CH;
        const int row = r0 + rl;
        float x[8];
        if (row < a.Nq) {
            unpack8<T>(rq[pass] ^ smask, x);
            transform_row<D, true>(x, has_signs, ck);
            u32x2 c;
            c[0] = to_e4m3x4(clamp448(x[0] * iq), clamp448(x[1] * iq), clamp448(x[2] * iq), clamp448(x[3] * iq));
            c[1] = to_e4m3x4(clamp448(x[4] * iq), clamp448(x[5] * iq), clamp448(x[6] * iq), clamp448(x[7] * iq));
            *reinterpret_cast<u32x2 *>(a.pack.q8 + ((size_t)bh * a.Nq + row) * D + 8 * ck) = c;
        }
        if (row < a.Nkp) {  // key rows past Nk (padding up to the group) are zero codes
            u32x2 c = {0u, 0u}, cv = {0u, 0u};
            if (row < a.Nk) {
                unpack8<T>(rk[pass] ^ smask, x);
                transform_row<D, true>(x, has_signs, ck);
                c[0] = to_e4m3x4(clamp448(x[0] * ik), clamp448(x[1] * ik), clamp448(x[2] * ik), clamp448(x[3] * ik));
                c[1] = to_e4m3x4(clamp448(x[4] * ik), clamp448(x[5] * ik), clamp448(x[6] * ik), clamp448(x[7] * ik));
                unpack8<T>(rv[pass], x);
                cv[0] = to_e4m3x4(clamp448(x[0] * iv), clamp448(x[1] * iv), clamp448(x[2] * iv), clamp448(x[3] * iv));
                cv[1] = to_e4m3x4(clamp448(x[4] * iv), clamp448(x[5] * iv), clamp448(x[6] * iv), clamp448(x[7] * iv));
            }
            *reinterpret_cast<u32x2 *>(a.pack.k8 + ((size_t)bh * a.Nkp + row) * D + 8 * ck) = c;
            *reinterpret_cast<u32x2 *>(&vtile[rl][8 * ck]) = cv;
        }
    }
    __syncthreads();
    // V^T of the key group: row (dim) j holds the 64 keys at positions
    // p = 32*g + 16*kb + r  <->  key 32*kb + acc_row(r, g)
    if (r0 < a.Nkp) {
        for (int idx = tid; idx < D * 4; idx += kQuantThreads) {
            const int dim = idx >> 2;
            const int p0 = (idx & 3) * 16;  // 16 positions per thread
            uint32_t w[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                uint32_t acc = 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int p = p0 + 4 * q4 + e;
                    const int g = p >> 5, kb = (p >> 4) & 1, r = p & 15;
                    const int key = 32 * kb + layout::acc_row(r, g);
                    acc |= (uint32_t)vtile[key][dim] << (8 * e);
                }
                w[q4] = acc;
            }
            *reinterpret_cast<u32x4 *>(a.pack.v8t + ((size_t)bh * D + dim) * a.Nkp + r0 + p0) =
                u32x4{w[0], w[1], w[2], w[3]};
        }
    }
}

// ---------------------------------------------------------------------------
// Attention on the pack
// ---------------------------------------------------------------------------
struct Fp8Args {
    const uint8_t *q8;
    const uint8_t *k8;
    const uint8_t *v8t;
    const float *descale;
    void *out;
    float *lse;
    int BH;
    int Nq;
    int Nk;
    int Nkp;
    int Tr;
    float scale_log2;  // |scale| * log2(e) (1 for a zero scale; see FoldedScale)
    uint32_t qflip;    // sign bits flipped in the Q codes for a negative scale
    uint32_t qkeep;    // 0 zeroes the Q codes for a zero scale
};

constexpr float kHeldSumBound = 256.0f;
constexpr float kLn2 = 0.693147180559945309417f;

// LDS tile rows of RB bytes, read as 16-byte chunks by 16 consecutive rows:
// chunk c of row r sits at chunk position c ^ ((r / R) & (CHK - 1)) with
// R = 256 / RB rows per bank line, CHK = RB / 16 chunks per row.
template <int RB>
__device__ __forceinline__ int tile_swz(int r) {
    constexpr int R = 256 / RB, CHK = RB / 16;
    return (r / R) & (CHK - 1);
}

template <typename OutT, int D, bool CAUSAL, int NW, int OCC>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC)))
void fp8_fwd_kernel(Fp8Args a) {
    constexpr int NT = NW * 64;
    constexpr int QW = 32;
    constexpr int BR = NW * QW;
    constexpr int BC = kKeyGroup;     // keys per tile
    constexpr int KS = D / 64;        // k-steps of S^T (64 dims each)
    constexpr int DB = D / 32;        // 32-dim blocks of O^T
    constexpr int KROW = D;           // bytes per K code row
    constexpr int VROW = BC;          // bytes per V^T row of a tile
    constexpr int KTILE = BC * KROW;
    constexpr int VTILE = D * VROW;
    constexpr int STAGE = KTILE + VTILE;
    constexpr int KUNITS = KTILE / 16, VUNITS = VTILE / 16;
    static_assert(D == 64 || D == 128, "FP8 head dims");
    static_assert(KUNITS % NT == 0 && VUNITS % NT == 0, "tiles split evenly");
    typedef typename std::conditional<std::is_same<OutT, __bf16>::value, bf16x4, f16x4>::type o4;

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;

    int bh, qblk;
    layout::map_workgroup(blockIdx.x, a.BH, a.Tr, CAUSAL, bh, qblk);
    const int Nq = a.Nq, Nk = a.Nk, Nkp = a.Nkp;
    const int q0 = qblk * BR;
    const int q0w = q0 + wave * QW;
    const float c = a.scale_log2 * a.descale[bh] * a.descale[a.BH + bh];
    const float dv = a.descale[2 * a.BH + bh];

    const uint8_t *kp = a.k8 + (size_t)bh * Nkp * D;
    const uint8_t *vp = a.v8t + (size_t)bh * D * Nkp;
    const __amdgpu_buffer_rsrc_t rsrc_k =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(kp), (short)0, (int)((uint32_t)Nkp * D), kBufferDword3);
    const __amdgpu_buffer_rsrc_t rsrc_v =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(vp), (short)0, (int)((uint32_t)Nkp * D), kBufferDword3);

    // DMA sources: LDS unit u (16 bytes) of the K tile holds row u / (KROW/16),
    // chunk (u % (KROW/16)) ^ swz(row); of the V^T tile, dim u / 4, chunk
    // (u % 4) ^ swz(dim) of the tile's 64 positions.
    uint32_t kdma[KUNITS / NT], vdma[VUNITS / NT];
#pragma unroll
    for (int n = 0; n < KUNITS / NT; ++n) {
        const int u = (n * NW + wave) * 64 + lane;
        const int row = u / (KROW / 16), ch = (u % (KROW / 16)) ^ tile_swz<KROW>(row);
        kdma[n] = (uint32_t)(row * KROW + ch * 16);
    }
#pragma unroll
    for (int n = 0; n < VUNITS / NT; ++n) {
        const int u = (n * NW + wave) * 64 + lane;
        const int dim = u / 4, ch = (u % 4) ^ tile_swz<VROW>(dim);
        vdma[n] = (uint32_t)(dim * Nkp + ch * 16);
    }
    // (the offsets go through named locals: written inline as template-
    // dependent expressions they kept the host pass from emitting the kernel)
    auto issue_tile = [&](int k0, int stage) {
        char *kb = smem + stage * STAGE;
        char *vb = kb + KTILE;
        const uint32_t ks_off = (uint32_t)k0 * KROW;
        const uint32_t vs_off = (uint32_t)k0;
#pragma unroll
        for (int n = 0; n < KUNITS / NT; ++n) {
            const uint32_t o = kdma[n];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_k, (FA_LDS void *)(kb + (n * NW + wave) * 1024), 16, o,
                                                     ks_off, 0, 0);
        }
#pragma unroll
        for (int n = 0; n < VUNITS / NT; ++n) {
            const uint32_t o = vdma[n];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_v, (FA_LDS void *)(vb + (n * NW + wave) * 1024), 16, o,
                                                     vs_off, 0, 0);
        }
    };

    // operand read offsets: K rows (key 32*kb + l32, dims 64*ks + 32*g: two
    // chunks), V^T rows (dim 32*db + l32, positions 32*g: two chunks)
    int koff[2][KS][2], voff[DB][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = 32 * kb + l32, ch = 4 * ks + 2 * g + h;
                koff[kb][ks][h] = row * KROW + ((ch ^ tile_swz<KROW>(row)) * 16);
            }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int dim = 32 * db + l32, ch = 2 * g + h;
            voff[db][h] = KTILE + dim * VROW + ((ch ^ tile_swz<VROW>(dim)) * 16);
        }

    const int kv_end = CAUSAL ? min(Nk, q0 + BR) : Nk;
    const int nt = (kv_end + BC - 1) / BC;
    // the first tile's copy goes out before the Q loads, so that the two
    // wait on memory together
    if (nt > 0) issue_tile(0, 0);

    // Q code fragments (B operand of S^T): lane (query l32, half g) holds
    // dims [64*ks + 32*g, +32).  Every lane loads (rows past the end read
    // the last row, then are zeroed): no branches around the loads.
    const int row = q0w + l32;
    const bool row_ok = row < Nq;  // Nq >= 1
    const uint8_t *qrow = a.q8 + ((size_t)bh * Nq + (row_ok ? row : Nq - 1)) * D;
    i32x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 lo = *reinterpret_cast<const u32x4 *>(qrow + 64 * ks + 32 * g);
        u32x4 hi = *reinterpret_cast<const u32x4 *>(qrow + 64 * ks + 32 * g + 16);
        lo = row_ok ? lo : u32x4{0u, 0u, 0u, 0u};
        hi = row_ok ? hi : u32x4{0u, 0u, 0u, 0u};
        lo = (lo ^ a.qflip) & a.qkeep;  // the sign of the scale, folded into Q
        hi = (hi ^ a.qflip) & a.qkeep;
        qf[ks] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    // two running sums: l_part of the float32 P (for LSE and the lazy-
    // rescale bound) and l8 of the E4M3-rounded P that enters P V (so O is
    // normalised by the weights it was formed with).  l8 is summed on the
    // matrix core: read as the B operand of the 16x16x128 product, the P
    // registers of lanes n and n+32 (query n) form k-quarters 0 and 2 of
    // column n, those of lanes n+16 and n+48 (query n+16) k-quarters 1 and
    // 3.  With A row 0 = ones on quarters 0, 2 and row 1 = ones on quarters
    // 1, 3 (lanes 0, 32 and 17, 49; every other lane zero), lane n < 16 of
    // the accumulator holds the sum of query n in register 0 and of query
    // n+16 in register 1, whatever the byte order inside a lane.
    float m_held = -__builtin_inff();
    float l_part = 0.0f;
    f32x4 l8acc = {0.0f, 0.0f, 0.0f, 0.0f};
    i32x8 ones8;
    {
        const int ones = (lane == 0 || lane == 32 || lane == 17 || lane == 49) ? 0x38383838 : 0;  // E4M3 1.0
#pragma unroll
        for (int w = 0; w < 8; ++w) ones8[w] = ones;
    }

    auto compute_tile = [&](auto stage_tag, int k0) {
        constexpr int S = decltype(stage_tag)::value;
        const char *base = smem + S * STAGE;
        // ---- S^T = K Q^T ------------------------------------------------------
        // (issued at raised wave priority, as in the 16-bit prefill kernel, so
        // that co-resident waves stay out of step)
        __builtin_amdgcn_s_setprio(1);
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 lo = *reinterpret_cast<const u32x4 *>(base + koff[kb][ks][0]);
                const u32x4 hi = *reinterpret_cast<const u32x4 *>(base + koff[kb][ks][1]);
                const i32x8 kf = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                s[kb] = mfma_e4m3(kf, qf[ks], s[kb]);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // ---- mask: key tail and the causal diagonal -----------------------------
        const bool need_mask = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > q0w);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * kb + layout::acc_row(r, g);
                    if (key >= Nk || (CAUSAL && key > row)) s[kb][r] = -__builtin_inff();
                }
        }
        // ---- online softmax with the lazy rescale; P to E4M3 -------------------
        i32x8 pf;
        auto exp_tile = [&](float msub) {
            float lsum = 0.0f;
#pragma unroll
            for (int w = 0; w < 8; ++w) {  // dword w: slots 4w .. 4w+3 = (kb, r) = (w / 4, 4 (w % 4) + e)
                float t[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    t[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[w >> 2][4 * (w & 3) + e], c, -msub));
                    // from the first term: 0 + x does not fold (x = -0), P >= 0
                    lsum = (w == 0 && e == 0) ? t[e] : lsum + t[e];
                }
                pf[w] = (int)to_e4m3x4(t[0], t[1], t[2], t[3]);
            }
            return lsum;
        };
        float lsum = 0.0f;
        bool exact = __ballot(m_held == -__builtin_inff()) != 0ull;
        if (!exact) {
            lsum = exp_tile(m_held);
            exact = __ballot(!(lsum <= kHeldSumBound)) != 0ull;
        }
        if (exact) {
            float mx = -__builtin_inff();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[kb][r]);
            mx = xor32_max(mx);
            const float m_new = __builtin_fmaxf(m_held, mx * c);  // c > 0 (the sign is in Q)
            const float alpha = (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_held - m_new);
            m_held = m_new;
            l_part *= alpha;
            // lane n < 16 keeps queries n (register 0) and n + 16 (register 1)
            const float alpha_hi = __shfl(alpha, (lane + 16) & 63);
            l8acc[0] *= alpha;
            l8acc[1] *= alpha_hi;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            lsum = exp_tile((m_new == -__builtin_inff()) ? 0.0f : m_new);
        }
        l_part += lsum;
        l8acc = mfma16_e4m3(ones8, pf, l8acc);
        // ---- O^T += V^T P^T -------------------------------------------------------
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(base + voff[db][0]);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(base + voff[db][1]);
            const i32x8 vf = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[db] = mfma_e4m3(vf, pf, oacc[db]);
        }
    };

    auto step = [&](auto stage_tag, int jt) {
        constexpr int S = decltype(stage_tag)::value;
        const int k0 = jt * BC;
        if (jt + 1 < nt) issue_tile(k0 + BC, S ^ 1);
        const bool active = (q0w < Nq) && (!CAUSAL || k0 <= q0w + QW - 1);
        if (active) compute_tile(stage_tag, k0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    if (nt > 0) {  // the first tile's copy (issued above) has landed for every thread
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
    for (int jt = 0; jt < nt; jt += 2) {
        step(Int<0>{}, jt);
        if (jt + 1 < nt) step(Int<1>{}, jt + 1);
    }

    // ---- epilogue: O = acc * descale_v / l, LSE = (m + log2 l) ln 2 ------------
    const float l = xor32_sum(l_part);
    const float l8_lo = __shfl(l8acc[0], l32 & 15);
    const float l8_hi = __shfl(l8acc[1], l32 & 15);
    const float l8 = (l32 < 16) ? l8_lo : l8_hi;
    if (row < Nq) {
        OutT *op = static_cast<OutT *>(a.out) + ((size_t)bh * Nq + row) * D;
        const float f = (l8 > 0.0f) ? dv / l8 : 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                f32x4 t;
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = oacc[db][4 * rg + e] * f;
                *reinterpret_cast<o4 *>(op + 32 * db + 8 * rg + 4 * g) = __builtin_convertvector(t, o4);
            }
        if (g == 0 && a.lse != nullptr)
            a.lse[(size_t)bh * Nq + row] = (l > 0.0f) ? (m_held + __builtin_amdgcn_logf(l)) * kLn2 : -__builtin_inff();
    }
}

template <typename T, int D>
hipError_t quantize_typed(const QuantArgs &a, hipStream_t stream) {
    const int n = 3 * a.BH;
    hipLaunchKernelGGL(fp8_clear_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, a.pack.amax, n);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int rows = a.Nq > a.Nkp ? a.Nq : a.Nkp;
    const dim3 grid((unsigned)a.BH, (unsigned)((rows + kQuantRows - 1) / kQuantRows));
    const int amax_rows = kQuantRows * kAmaxBlocks;
    const dim3 agrid((unsigned)a.BH, (unsigned)((rows + amax_rows - 1) / amax_rows));
    hipLaunchKernelGGL((fp8_amax_kernel<T, D>), agrid, dim3(kQuantThreads), 0, stream, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((fp8_quantize_kernel<T, D>), grid, dim3(kQuantThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename OutT, int D, bool CAUSAL>
hipError_t fwd_typed(Fp8Args a, hipStream_t stream) {
    constexpr int NW = 4;
    a.Tr = (a.Nq + NW * 32 - 1) / (NW * 32);
    const long long nwg = (long long)a.BH * a.Tr;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fp8_fwd_kernel<OutT, D, CAUSAL, NW, 3>), dim3((unsigned)nwg), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

Fp8Layout fp8_layout(int BH, int Nq, int Nk, int d) {
    Fp8Layout L;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    L.Nkp = (Nk + kKeyGroup - 1) / kKeyGroup * kKeyGroup;
    L.q8 = 0;
    L.k8 = L.q8 + up((size_t)BH * Nq * d);
    L.v8t = L.k8 + up((size_t)BH * L.Nkp * d);
    L.descale = L.v8t + up((size_t)BH * d * L.Nkp);
    L.amax = L.descale + up((size_t)3 * BH * 4);
    L.bytes = L.amax + up((size_t)3 * BH * 4);
    return L;
}

hipError_t launch_fp8_quantize(int dtype, int d, const void *q, const void *k, const void *v, const float *signs,
                               void *pack, int BH, int Nq, int Nk, hipStream_t stream) {
    const Fp8Layout L = fp8_layout(BH, Nq, Nk, d);
    char *base = static_cast<char *>(pack);
    QuantArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.signs = signs;
    a.pack.q8 = reinterpret_cast<uint8_t *>(base + L.q8);
    a.pack.k8 = reinterpret_cast<uint8_t *>(base + L.k8);
    a.pack.v8t = reinterpret_cast<uint8_t *>(base + L.v8t);
    a.pack.descale = reinterpret_cast<float *>(base + L.descale);
    a.pack.amax = reinterpret_cast<uint32_t *>(base + L.amax);
    a.BH = BH;
    a.Nq = Nq;
    a.Nk = Nk;
    a.Nkp = L.Nkp;
    if (dtype == 2) return d == 128 ? quantize_typed<__bf16, 128>(a, stream) : quantize_typed<__bf16, 64>(a, stream);
    return d == 128 ? quantize_typed<_Float16, 128>(a, stream) : quantize_typed<_Float16, 64>(a, stream);
}

hipError_t launch_fp8_fwd(int out_dtype, int d, bool causal, const void *pack, void *out, float *lse, int BH,
                          int Nq, int Nk, float scale_log2, hipStream_t stream) {
    const Fp8Layout L = fp8_layout(BH, Nq, Nk, d);
    const char *base = static_cast<const char *>(pack);
    Fp8Args a;
    a.q8 = reinterpret_cast<const uint8_t *>(base + L.q8);
    a.k8 = reinterpret_cast<const uint8_t *>(base + L.k8);
    a.v8t = reinterpret_cast<const uint8_t *>(base + L.v8t);
    a.descale = reinterpret_cast<const float *>(base + L.descale);
    a.out = out;
    a.lse = lse;
    a.BH = BH;
    a.Nq = Nq;
    a.Nk = Nk;
    a.Nkp = L.Nkp;
    a.Tr = 0;
    const FoldedScale fs = fold_scale(scale_log2, kSignBits8);
    a.scale_log2 = fs.c;
    a.qflip = fs.flip;
    a.qkeep = fs.keep;
#define FA_FP8_CASE(OT)                                                                         \
    if (d == 128) return causal ? fwd_typed<OT, 128, true>(a, stream) : fwd_typed<OT, 128, false>(a, stream); \
    return causal ? fwd_typed<OT, 64, true>(a, stream) : fwd_typed<OT, 64, false>(a, stream);
    if (out_dtype == 2) {
        FA_FP8_CASE(__bf16)
    }
    FA_FP8_CASE(_Float16)
#undef FA_FP8_CASE
}

}  // namespace fa
