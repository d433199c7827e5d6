// fa_backward.hip -- FlashAttention backward for bf16 / fp16 on gfx950.
//
// Method ("9.4 FlashAttention 与 FlashMLA" section 9.4.5, the two-kernel
// backward; "6. FlashAttention 分块逻辑" section 7, the per-block formulas):
// the probabilities are rebuilt block by block from the saved statistic,
// P = exp(scale * Q K^T - LSE) (masked), never stored, and with
//   D_i = rowsum(dO_i * O_i),  dP = dO V^T,  dS = P * (dP - D),
// the gradients are dV = P^T dO, dK = scale dS^T Q, dQ = scale dS K.  dQ and
// dK/dV accumulate along different directions, so two kernels run, each
// keeping its gradient block in registers for the whole inner loop (no
// atomics, bit-for-bit deterministic):
//
//  * dQ kernel (Q blocks outer, K/V blocks inner).  The structure of the
//    forward kernel: a workgroup of 4 waves owns 128 queries; Q and dO
//    fragments stay in registers; K and V tiles stream through LDS by
//    buffer-to-LDS DMA.  Per tile S^T = K Q^T and dP^T = V dO^T (MFMA, so
//    that each lane's registers belong to one query and LSE and D are
//    per-lane scalars), dS^T = P^T (dP^T - D) in registers, converted in
//    place to the 16-bit operand of dQ^T += K^T dS^T, whose K^T operand is
//    gathered by the transposing LDS read.  The kernel also forms D_i from
//    its O and dO rows and writes (LSE_i log2 e, D_i) for the second kernel.
//  * dK/dV kernel (K/V blocks outer, Q blocks inner).  A workgroup of 4
//    waves owns 128 keys; each wave keeps the K fragments of its 32 keys and
//    its dK, dV accumulators in registers, and reads its V rows from LDS
//    (staged once), which keeps the kernel within two waves per SIMD; Q and
//    dO tiles and their statistics stream through LDS.  Per tile S = Q K^T
//    and dP = dO V^T (each lane's registers belong to one key), P and dS in
//    registers, then dV^T += dO^T P and dK^T += Q^T dS with the dO^T and Q^T
//    operands gathered by the transposing LDS read.
//
// Tiles read both row-wise and transposed (K in the dQ kernel, Q and dO in
// the dK/dV kernel) use the dual XOR swizzle of fa_layout.h, which keeps both
// reads free of LDS bank conflicts.  Masked entries (causal, ragged tails)
// get S = -inf, so P = 0 and, since dP and the statistics are finite,
// dS = 0; tail rows are fetched from the last valid row so no load leaves its
// tensor, and the statistics padding after the last head is zeroed.
#include <cstdlib>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_layout.h"

namespace fa {
namespace {

constexpr float kLog2eF = 1.4426950408889634074f;
constexpr int kStatsPad = 64;  // statistics rows of padding after the last head (one dK/dV query tile)

struct BwdArgs {
    const void *q;
    const void *k;
    const void *v;
    const void *out;
    const void *dout;
    const float *lse;   // [BH, Nq] natural log, from the forward
    void *dq;
    void *dk;
    void *dv;
    f32x2 *stats;       // [BH * Nq + pad] (LSE * log2 e, D), written by the dQ kernel
    int stats_bytes;    // bytes of stats including the padding
    int BH;
    int Nq;
    int Nk;
    int T;              // blocks per (batch, head): Q blocks (dQ kernel) or K blocks (dK/dV kernel)
    float scale;        // the caller's scale (dQ = scale dS K, dK = scale dS^T Q)
    float scale_log2;   // |scale| * log2(e) (1 for a zero scale; see FoldedScale)
    uint32_t sflip;     // sign bits flipped in the register-held score operand (Q in
    uint32_t skeep;     // the dQ kernel, K in the dK/dV kernel); 0 zeroes it
};

// ---------------------------------------------------------------------------
// dQ (and D, and the statistics the dK/dV kernel reads)
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL, int NW, int BC, int OCC>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC)))
void bwd_dq_kernel(BwdArgs a) {
    using M = Mfma<T>;
    using x8 = typename M::x8;
    using x4 = typename M::x4;
    constexpr int NT = NW * 64;
    constexpr int QW = 32;           // queries per wave
    constexpr int BR = NW * QW;      // queries per workgroup
    constexpr int KS = D / 16;       // k-steps over the head dim
    constexpr int DB = D / 32;       // 32-dim blocks of dQ^T
    constexpr int KB = BC / 32;      // 32-key blocks of S^T
    constexpr int KS2 = BC / 16;     // k-steps over keys
    constexpr int CH = D / 8;
    constexpr int ROW = D * 2;
    constexpr int TILE_BYTES = BC * ROW;
    constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K tile + V tile
    constexpr int UNITS = BC * CH;
    constexpr int NDMA = UNITS / NT;
    static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");
    static_assert(UNITS % NT == 0, "a tile must split evenly over the workgroup");
    static_assert(2 * STAGE_BYTES <= 65536, "stage offsets must fit a 16-bit LDS immediate");

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;

    int bh, qblk;
    layout::map_workgroup(blockIdx.x, a.BH, a.T, CAUSAL, bh, qblk);
    const int Nq = a.Nq;
    const int Nk = a.Nk;
    const int q0 = qblk * BR;
    const int q0w = q0 + wave * QW;
    const size_t qbase = (size_t)bh * Nq * D;
    const T *kp = static_cast<const T *>(a.k) + (size_t)bh * Nk * D;
    const T *vp = static_cast<const T *>(a.v) + (size_t)bh * Nk * D;
    const float c = a.scale_log2;
    const uint32_t kv_bytes = (uint32_t)Nk * ROW;
    const __amdgpu_buffer_rsrc_t rsrc_k =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(kp), (short)0, (int)kv_bytes, kBufferDword3);
    const __amdgpu_buffer_rsrc_t rsrc_v =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(vp), (short)0, (int)kv_bytes, kBufferDword3);

    uint32_t kdma[NDMA], vdma[NDMA];
    int dkey[NDMA];
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
        const int u = (n * NW + wave) * 64 + lane;
        kdma[n] = (uint32_t)layout::dual_dma_src_elem<D>(u) * 2;  // K: read row-wise and transposed
        vdma[n] = (uint32_t)layout::k_dma_src_elem<D>(u) * 2;     // V: read row-wise only
        dkey[n] = u / CH;
    }
    int koff[KS], voff[KS], ktoff[DB][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        koff[ks] = layout::dual_row_operand_offset<D>(0, l32, g, ks);
        voff[ks] = layout::k_operand_offset<D>(0, l32, g, ks);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        ktoff[db][0] = layout::dual_tr_operand_offset<D>(db, lane, 0, 0);
        ktoff[db][1] = layout::dual_tr_operand_offset<D>(db, lane, 0, 1);
    }

    auto issue_tile = [&](int k0, int stage) {
        char *kbase = smem + stage * STAGE_BYTES;
        char *vbase = kbase + TILE_BYTES;
        const uint32_t soff = (uint32_t)k0 * ROW;
        const bool tail = k0 + BC > Nk;
#pragma unroll
        for (int n = 0; n < NDMA; ++n) {
            uint32_t ko = kdma[n], vo = vdma[n];
            if (tail) {
                const int over = k0 + dkey[n] - (Nk - 1);  // rows past the end: fetch the last key instead
                if (over > 0) {
                    ko -= (uint32_t)over * ROW;
                    vo -= (uint32_t)over * ROW;
                }
            }
            const int dst = (n * NW + wave) * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_k, (FA_LDS void *)(kbase + dst), 16, ko, soff, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_v, (FA_LDS void *)(vbase + dst), 16, vo, soff, 0, 0);
        }
    };

    const int kv_end = CAUSAL ? min(Nk, q0 + BR) : Nk;
    const int nt = (kv_end + BC - 1) / BC;
    // the first tile's copy goes out before the row loads, so that they wait
    // on memory together
    issue_tile(0, 0);

    // Q and dO fragments (B operands): lane (query l32, half g) holds dims
    // [16*ks + 8*g, +8); the same dims of O give the lane's half of D.
    // Every lane loads (rows past the end read the last row, then are
    // zeroed): no branches around the loads.
    const int row = q0w + l32;
    const bool row_ok = row < Nq;  // Nq >= 1
    const size_t rbase = qbase + (size_t)(row_ok ? row : Nq - 1) * D;
    x8 qf[KS], dof[KS];
    float dpart = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const size_t off = rbase + 16 * ks + 8 * g;
        u32x4 rq = *reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.q) + off);
        u32x4 rdo = *reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.dout) + off);
        u32x4 ro = *reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.out) + off);
        const u32x4 zero = {0u, 0u, 0u, 0u};
        rq = row_ok ? rq : zero;
        rdo = row_ok ? rdo : zero;
        ro = row_ok ? ro : zero;
        qf[ks] = __builtin_bit_cast(x8, (rq ^ a.sflip) & a.skeep);  // the scale's sign, folded into Q
        dof[ks] = __builtin_bit_cast(x8, rdo);
        const x8 of = __builtin_bit_cast(x8, ro);
#pragma unroll
        for (int e = 0; e < 8; ++e) dpart = __builtin_fmaf((float)dof[ks][e], (float)of[e], dpart);
    }
    const float Di = xor32_sum(dpart);
    const float lse2 = row_ok ? a.lse[(size_t)bh * Nq + row] * kLog2eF : 0.0f;
    if (row_ok && g == 0) a.stats[(size_t)bh * Nq + row] = f32x2{lse2, Di};
    // the padding after the last head is read (then masked) by the dK/dV
    // kernel's last tiles: keep it finite
    if (blockIdx.x == 0 && tid < kStatsPad) a.stats[(size_t)a.BH * Nq + tid] = f32x2{0.0f, 0.0f};

    f32x16 dqacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.0f;

    auto compute_tile = [&](auto stage_tag, int k0) {
        constexpr int S = decltype(stage_tag)::value;
        constexpr int KOFF = S * STAGE_BYTES;
        constexpr int VOFF = KOFF + TILE_BYTES;
        // ---- S^T = K Q^T, dP^T = V dO^T ---------------------------------------
        f32x16 s[KB], dp[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[kb][r] = 0.0f;
                dp[kb][r] = 0.0f;
            }
        // step i = (block i / KS, k-step i % KS): at d = 128 its K and V
        // fragments are read PF steps ahead of its two MFMAs (order pinned
        // below; below d = 128 the registers this takes would cost a wave per
        // SIMD, and the compiler schedules)
        constexpr int NK = KB * KS;
        constexpr int PF = D < 128 ? 1 : (NK < 3 ? NK : 3);
        auto read_k = [&](int i) {
            return __builtin_bit_cast(
                x8, *reinterpret_cast<const u32x4 *>(smem + KOFF + (i / KS) * 32 * ROW + koff[i % KS]));
        };
        auto read_v = [&](int i) {
            return __builtin_bit_cast(
                x8, *reinterpret_cast<const u32x4 *>(smem + VOFF + (i / KS) * 32 * ROW + voff[i % KS]));
        };
        x8 kq[PF], vq[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            kq[i] = read_k(i);
            vq[i] = read_v(i);
        }
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const x8 kf = kq[i % PF], vf = vq[i % PF];
            if (i + PF < NK) {
                kq[i % PF] = read_k(i + PF);
                vq[i % PF] = read_v(i + PF);
            }
            s[i / KS] = M::run(kf, qf[i % KS], s[i / KS]);
            dp[i / KS] = M::run(vf, dof[i % KS], dp[i / KS]);
        }
        if constexpr (PF > 1) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                if (i + PF < NK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
        }
        // ---- mask: ragged key tail and the causal diagonal (P = exp2(-inf) = 0;
        // dP is finite, so dS = 0 there too) ---------------------------------------
        const bool need_mask = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > q0w);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * kb + layout::acc_row(r, g);
                    if (key >= Nk || (CAUSAL && key > row)) s[kb][r] = -__builtin_inff();
                }
        }
        // ---- dS^T = P^T (dP^T - D), P^T = exp2(c s - LSE log2 e) -------------------
        x8 dsf[KS2];
#pragma unroll
        for (int ks2 = 0; ks2 < KS2; ++ks2) {
            const int kb = ks2 >> 1;
            const int h = (ks2 & 1) * 8;
            f32x8 t;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][h + e], c, -lse2));
                t[e] = p * (dp[kb][h + e] - Di);
            }
            dsf[ks2] = __builtin_convertvector(t, x8);
        }
        // ---- dQ^T += K^T dS^T ---------------------------------------------------
#pragma unroll
        for (int ks2 = 0; ks2 < KS2; ++ks2)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const char *b0 = smem + KOFF + ktoff[db][0] + 16 * ks2 * ROW;
                const char *b1 = smem + KOFF + ktoff[db][1] + 16 * ks2 * ROW;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4 *)(b0));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4 *)(b1));
                const x8 kt = __builtin_bit_cast(x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                dqacc[db] = M::run(kt, dsf[ks2], dqacc[db]);
            }
    };

    auto step = [&](auto stage_tag, int jt) {
        constexpr int S = decltype(stage_tag)::value;
        const int k0 = jt * BC;
        if (jt + 1 < nt) issue_tile(k0 + BC, S ^ 1);
        const bool active = (q0w < Nq) && (!CAUSAL || k0 <= q0w + QW - 1);  // wave-uniform
        if (active) compute_tile(stage_tag, k0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the first tile (issued above) has landed
    __syncthreads();
    for (int jt = 0; jt < nt; jt += 2) {
        step(Int<0>{}, jt);
        if (jt + 1 < nt) step(Int<1>{}, jt + 1);
    }

    // ---- dQ = scale * acc ----------------------------------------------------
    if (row_ok) {
        T *dqp = static_cast<T *>(a.dq) + qbase + (size_t)row * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                f32x4 t;
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = dqacc[db][4 * rg + e] * a.scale;
                *reinterpret_cast<x4 *>(dqp + 32 * db + 8 * rg + 4 * g) = __builtin_convertvector(t, x4);
            }
    }
}

// ---------------------------------------------------------------------------
// dK and dV
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL, int NW, int BQ, int OCC, bool VLDS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC)))
void bwd_dkdv_kernel(BwdArgs a) {
    using M = Mfma<T>;
    using x8 = typename M::x8;
    using x4 = typename M::x4;
    constexpr int NT = NW * 64;
    constexpr int KW = 32;           // keys per wave
    constexpr int BK = NW * KW;      // keys per workgroup
    constexpr int QB = BQ / 32;      // 32-query blocks per tile
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int KS2 = BQ / 16;     // k-steps over queries
    constexpr int CH = D / 8;
    constexpr int ROW = D * 2;
    constexpr int TILE_BYTES = BQ * ROW;
    constexpr int ST_OFF = 2 * TILE_BYTES;       // (LSE log2 e, D) of the tile's queries
    constexpr int STAGE_BYTES = 2 * TILE_BYTES + 1024;
    constexpr int UNITS = BQ * CH;
    constexpr int NDMA = UNITS / NT;
    constexpr int SUNITS = BQ * 8 / 16;          // 16-byte units of statistics per tile
    static_assert(BQ % 32 == 0 && D % 32 == 0, "tile shape");
    static_assert(UNITS % NT == 0, "a tile must split evenly over the workgroup");
    static_assert(SUNITS <= 64 && BQ * 8 <= 1024, "statistics of a tile: one wave, one slot");
    static_assert(2 * STAGE_BYTES <= 65536, "stage offsets must fit a 16-bit LDS immediate");
    // VLDS: the workgroup's V rows sit in LDS (read per tile) instead of
    // registers, which frees 4*D/8 registers per lane for a second wave per SIMD
    constexpr int VT_OFF = 2 * STAGE_BYTES;
    constexpr int VT_BYTES = VLDS ? BK * ROW : 0;
    constexpr int VUNITS = BK * CH;
    static_assert(!VLDS || VUNITS % NT == 0, "the V rows must split evenly over the workgroup");

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES + VT_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;

    int bh, kr;
    layout::map_workgroup(blockIdx.x, a.BH, a.T, CAUSAL, bh, kr);
    // under the mask the first key blocks see the most queries: map the
    // order's longest-first position onto them
    const int kblk = CAUSAL ? (a.T - 1 - kr) : kr;
    const int Nq = a.Nq;
    const int Nk = a.Nk;
    const int k0 = kblk * BK;
    const int k0w = k0 + wave * KW;
    const T *qp = static_cast<const T *>(a.q) + (size_t)bh * Nq * D;
    const T *dop = static_cast<const T *>(a.dout) + (size_t)bh * Nq * D;
    const float c = a.scale_log2;
    const uint32_t q_bytes = (uint32_t)Nq * ROW;
    const __amdgpu_buffer_rsrc_t rsrc_q =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(qp), (short)0, (int)q_bytes, kBufferDword3);
    const __amdgpu_buffer_rsrc_t rsrc_do =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(dop), (short)0, (int)q_bytes, kBufferDword3);
    // the whole statistics array (padded by a tile past the last head)
    const __amdgpu_buffer_rsrc_t rsrc_st =
        __builtin_amdgcn_make_buffer_rsrc(a.stats, (short)0, a.stats_bytes, kBufferDword3);

    uint32_t qdma[NDMA];
    int dq_row[NDMA];
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
        const int u = (n * NW + wave) * 64 + lane;
        qdma[n] = (uint32_t)layout::dual_dma_src_elem<D>(u) * 2;
        dq_row[n] = u / CH;
    }
    int qoff[KS], qtoff[DB][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qoff[ks] = layout::dual_row_operand_offset<D>(0, l32, g, ks);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        qtoff[db][0] = layout::dual_tr_operand_offset<D>(db, lane, 0, 0);
        qtoff[db][1] = layout::dual_tr_operand_offset<D>(db, lane, 0, 1);
    }

    auto issue_tile = [&](int qt, int stage) {
        char *qbase = smem + stage * STAGE_BYTES;
        char *dobase = qbase + TILE_BYTES;
        const uint32_t soff = (uint32_t)qt * ROW;
        const bool tail = qt + BQ > Nq;
#pragma unroll
        for (int n = 0; n < NDMA; ++n) {
            uint32_t o = qdma[n];
            if (tail) {
                const int over = qt + dq_row[n] - (Nq - 1);  // rows past the end: fetch the last query
                if (over > 0) o -= (uint32_t)over * ROW;
            }
            const int dst = (n * NW + wave) * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_q, (FA_LDS void *)(qbase + dst), 16, o, soff, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_do, (FA_LDS void *)(dobase + dst), 16, o, soff, 0, 0);
        }
        if (wave == 0 && lane < SUNITS) {
            // 16 bytes = the statistics of two queries; past the head's last
            // query this reads the next head's (or the padding): masked below
            const uint32_t st_off = (uint32_t)(((size_t)bh * Nq + qt) * 8);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_st, (FA_LDS void *)(qbase + ST_OFF), 16,
                                                     (uint32_t)lane * 16, st_off, 0, 0);
        }
    };

    auto issue_v_rows = [&]() {
        // the workgroup's BK V rows, K-style swizzle (read row-wise only);
        // rows past the end repeat the last key
        const T *vhead = static_cast<const T *>(a.v) + (size_t)bh * Nk * D;
        const __amdgpu_buffer_rsrc_t rsrc_v = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<T *>(vhead), (short)0, (int)((uint32_t)Nk * ROW), kBufferDword3);
#pragma unroll
        for (int n = 0; n < VUNITS / NT; ++n) {
            const int u = (n * NW + wave) * 64 + lane;
            uint32_t o = (uint32_t)layout::k_dma_src_elem<D>(u) * 2;
            const int over = k0 + u / CH - (Nk - 1);
            if (over > 0) o -= (uint32_t)over * ROW;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_v, (FA_LDS void *)(smem + VT_OFF + (n * NW + wave) * 1024),
                                                     16, o, (uint32_t)k0 * ROW, 0, 0);
        }
    };

    // query tiles: under the mask only queries >= k0 see a key of the block
    const int q_begin = CAUSAL ? (k0 / BQ) * BQ : 0;
    const int nt = q_begin < Nq ? (Nq - q_begin + BQ - 1) / BQ : 0;
    // the V rows and the first query tile go out before the K and V
    // fragment loads, so that they all wait on memory together
    if (nt > 0) {  // workgroup-uniform
        if constexpr (VLDS) issue_v_rows();
        issue_tile(q_begin, 0);
    }


    // K and V fragments (B operands of S = Q K^T and dP = dO V^T): lane (key
    // l32, half g) holds dims [16*ks + 8*g, +8).  Keys past the end repeat
    // the last key; their gradients are not stored.
    const int key = k0w + l32;
    const int key_c = key < Nk ? key : Nk - 1;
    x8 kf[KS], vf[VLDS ? 1 : KS];
    int voff[KS];
    {
        const T *kp = static_cast<const T *>(a.k) + ((size_t)bh * Nk + key_c) * D;
        const T *vp = static_cast<const T *>(a.v) + ((size_t)bh * Nk + key_c) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            // the sign of the scale, folded into K (K serves only S = Q K^T here)
            kf[ks] = __builtin_bit_cast(x8, (*reinterpret_cast<const u32x4 *>(kp + 16 * ks + 8 * g) ^ a.sflip) &
                                                a.skeep);
            if constexpr (!VLDS)
                vf[ks] = __builtin_bit_cast(x8, *reinterpret_cast<const u32x4 *>(vp + 16 * ks + 8 * g));
            voff[ks] = VT_OFF + layout::k_operand_offset<D>(wave, l32, g, ks);
        }
    }
    f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dkacc[db][r] = 0.0f;
            dvacc[db][r] = 0.0f;
        }

    auto compute_tile = [&](auto stage_tag, int qt) {
        constexpr int S = decltype(stage_tag)::value;
        constexpr int QOFF = S * STAGE_BYTES;
        constexpr int DOOFF = QOFF + TILE_BYTES;
        constexpr int SOFF = QOFF + ST_OFF;
        // ---- S = Q K^T, dP = dO V^T ------------------------------------------
        // (issued at raised wave priority so that co-resident waves stay out
        // of step: one wave's exponentials run beside another's MFMAs)
        __builtin_amdgcn_s_setprio(1);
        f32x16 s[QB], dp[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[qb][r] = 0.0f;
                dp[qb][r] = 0.0f;
            }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const x8 qa = __builtin_bit_cast(
                    x8, *reinterpret_cast<const u32x4 *>(smem + QOFF + qb * 32 * ROW + qoff[ks]));
                const x8 da = __builtin_bit_cast(
                    x8, *reinterpret_cast<const u32x4 *>(smem + DOOFF + qb * 32 * ROW + qoff[ks]));
                s[qb] = M::run(qa, kf[ks], s[qb]);
                if constexpr (VLDS) {
                    const x8 vr = __builtin_bit_cast(x8, *reinterpret_cast<const u32x4 *>(smem + voff[ks]));
                    dp[qb] = M::run(da, vr, dp[qb]);
                } else {
                    dp[qb] = M::run(da, vf[ks], dp[qb]);
                }
            }
        __builtin_amdgcn_s_setprio(0);
        // ---- mask: ragged query tail and the causal diagonal (P = exp2(-inf) =
        // 0; dP and the tile's statistics are finite, so dS = 0 there too) ----------
        // register r of query block qb is query qt + 32*qb + acc_row(r, g);
        // registers 4*rg .. 4*rg+3 are four consecutive queries
        const bool need_mask = (qt + BQ > Nq) || (CAUSAL && qt < k0w + KW - 1);
        if (need_mask) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int query = qt + 32 * qb + layout::acc_row(r, g);
                    if (query >= Nq || (CAUSAL && key > query)) s[qb][r] = -__builtin_inff();
                }
        }
        // ---- P = exp2(c s - LSE log2 e), dS = P (dP - D) ------------------------
        x8 pf[KS2], dsf[KS2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            f32x8 tp[2], td[2];
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int qi = 32 * qb + 8 * rg + 4 * g;
                const f32x4 st0 = *reinterpret_cast<const f32x4 *>(smem + SOFF + qi * 8);
                const f32x4 st1 = *reinterpret_cast<const f32x4 *>(smem + SOFF + qi * 8 + 16);
                const float lse2[4] = {st0[0], st0[2], st1[0], st1[2]};
                const float dd[4] = {st0[1], st0[3], st1[1], st1[3]};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * rg + e;
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][r], c, -lse2[e]));
                    tp[r >> 3][r & 7] = p;
                    td[r >> 3][r & 7] = p * (dp[qb][r] - dd[e]);
                }
            }
            pf[2 * qb] = __builtin_convertvector(tp[0], x8);
            pf[2 * qb + 1] = __builtin_convertvector(tp[1], x8);
            dsf[2 * qb] = __builtin_convertvector(td[0], x8);
            dsf[2 * qb + 1] = __builtin_convertvector(td[1], x8);
        }
        // ---- dV^T += dO^T P, dK^T += Q^T dS ---------------------------------------
#pragma unroll
        for (int ks2 = 0; ks2 < KS2; ++ks2)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int o0 = qtoff[db][0] + 16 * ks2 * ROW;
                const int o1 = qtoff[db][1] + 16 * ks2 * ROW;
                const i16x4 dlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4 *)(smem + DOOFF + o0));
                const i16x4 dhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4 *)(smem + DOOFF + o1));
                const i16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4 *)(smem + QOFF + o0));
                const i16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4 *)(smem + QOFF + o1));
                const x8 dot = __builtin_bit_cast(x8, __builtin_shufflevector(dlo, dhi, 0, 1, 2, 3, 4, 5, 6, 7));
                const x8 qtr = __builtin_bit_cast(x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
                dvacc[db] = M::run(dot, pf[ks2], dvacc[db]);
                dkacc[db] = M::run(qtr, dsf[ks2], dkacc[db]);
            }
    };

    auto step = [&](auto stage_tag, int jt) {
        constexpr int S = decltype(stage_tag)::value;
        const int qt = q_begin + jt * BQ;
        if (jt + 1 < nt) issue_tile(qt + BQ, S ^ 1);
        // wave-uniform: the wave has live keys that some query of the tile sees
        const bool active = (k0w < Nk) && (!CAUSAL || qt + BQ - 1 >= k0w);
        if (active) compute_tile(stage_tag, qt);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    if (nt > 0) {  // the V rows and the first tile (issued above) have landed
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        for (int jt = 0; jt < nt; jt += 2) {
            step(Int<0>{}, jt);
            if (jt + 1 < nt) step(Int<1>{}, jt + 1);
        }
    }

    // ---- dK = scale * acc, dV = acc (zero for keys no query sees) -------------
    if (key < Nk) {
        T *dkp = static_cast<T *>(a.dk) + ((size_t)bh * Nk + key) * D;
        T *dvp = static_cast<T *>(a.dv) + ((size_t)bh * Nk + key) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                f32x4 tk, tv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    tk[e] = dkacc[db][4 * rg + e] * a.scale;
                    tv[e] = dvacc[db][4 * rg + e];
                }
                *reinterpret_cast<x4 *>(dkp + 32 * db + 8 * rg + 4 * g) = __builtin_convertvector(tk, x4);
                *reinterpret_cast<x4 *>(dvp + 32 * db + 8 * rg + 4 * g) = __builtin_convertvector(tv, x4);
            }
    }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------
// dK/dV variant: 0 (default) V rows in LDS, two waves per SIMD; 1 V in
// registers, one wave per SIMD.  FA_BWD_DKDV selects one for sweeps.
int bwd_dkdv_variant() {
    const char *env = std::getenv("FA_BWD_DKDV");
    return (env && env[0] == '1' && env[1] == '\0') ? 1 : 0;
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_bwd_typed(BwdArgs a, hipStream_t stream) {
    constexpr int NW = 4;
    constexpr int BC = D >= 128 ? 32 : 64;   // keys per dQ tile
    constexpr int BQ = D >= 128 ? 32 : 64;   // queries per dK/dV tile
    const int BR = NW * 32, BK = NW * 32;
    const int tq = (a.Nq + BR - 1) / BR;
    const int tk = (a.Nk + BK - 1) / BK;
    const long long nq = (long long)a.BH * tq, nk = (long long)a.BH * tk;
    if (nq > 0x7fffffffLL || nk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    a.T = tq;
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, NW, BC, 2>), dim3((unsigned)nq), dim3(NW * 64), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    a.T = tk;
    if (bwd_dkdv_variant() == 1)
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, NW, BQ, 1, false>), dim3((unsigned)nk), dim3(NW * 64), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, NW, BQ, 2, true>), dim3((unsigned)nk), dim3(NW * 64), 0,
                           stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_d(int d, bool causal, const BwdArgs &a, hipStream_t stream) {
#define FA_CASE(DD) \
    case DD: return causal ? launch_bwd_typed<T, DD, true>(a, stream) : launch_bwd_typed<T, DD, false>(a, stream);
    switch (d) {
        FA_CASE(32)
        FA_CASE(64)
        FA_CASE(128)
        default: return hipErrorInvalidValue;
    }
#undef FA_CASE
}

}  // namespace

size_t bwd_stats_bytes(int BH, int Nq) {
    // (LSE log2 e, D) per query, plus one tile of padding read past the last head
    return ((size_t)BH * Nq + kStatsPad) * 8;
}

hipError_t launch_backward(int dtype, int d, bool causal, const void *q, const void *k, const void *v,
                           const void *out, const void *dout, const float *lse, void *dq, void *dk, void *dv,
                           int BH, int Nq, int Nk, float scale, void *workspace, hipStream_t stream) {
    BwdArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.dout = dout;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.stats = static_cast<f32x2 *>(workspace);
    a.stats_bytes = (int)bwd_stats_bytes(BH, Nq);
    a.BH = BH;
    a.Nq = Nq;
    a.Nk = Nk;
    a.scale = scale;
    const FoldedScale fs = fold_scale((float)((double)scale * 1.4426950408889634074), kSignBits16);
    a.scale_log2 = fs.c;
    a.sflip = fs.flip;
    a.skeep = fs.keep;
    if (dtype == 2) return launch_bwd_d<__bf16>(d, causal, a, stream);
    if (dtype == 1) return launch_bwd_d<_Float16>(d, causal, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
