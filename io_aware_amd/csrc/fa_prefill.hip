// fa_prefill.hip -- tiled FlashAttention forward for bf16 / fp16 on gfx950.
//
// Method ("6. FlashAttention 分块逻辑" sections 3-6; "9.4 FlashAttention 与
// FlashMLA" sections 9.4.2-9.4.5; "08. Triton Flash Attention" Steps 1-4):
// one workgroup owns a block of Br query rows of one (batch, head), keeps its
// Q fragments, the float32 accumulator and the running max m / running sum l
// in registers, and streams K/V in blocks of Bc keys through LDS.  Per block:
//   S = scale * Q K^T (MFMA, float32 accumulate), mask, m_new = max(m, rowmax S),
//   rescale acc and l by exp(m - m_new), P = exp(S - m_new) rounded to the
//   input type, l += rowsum P, acc += P V (MFMA);
// after the last block O = acc / l and LSE = m + ln l, with O normalised by
// the sum of the rounded P that formed acc (l itself, in float32, gives the
// LSE).  Score and probability tiles live only in registers.
//
// CDNA4 design (index arithmetic in fa_layout.h, checked on the host):
//  * 32x32x16 bf16/fp16 MFMA in transposed orientation: S^T = K Q^T and
//    O^T = V^T P^T.  Each lane's 16 accumulator registers of a 32x32 block
//    belong to one query, so the row max is 16 in-register maxima plus one
//    exchange between lane halves (v_permlane32_swap), the rescale factor is
//    a per-lane scalar, and the S^T registers convert in place into the P^T
//    operand of the second product (no LDS round trip for P).
//  * Q fragments are loaded once into registers and stay there.
//  * K and V tiles go from device memory straight into LDS by buffer-to-LDS
//    DMA (no staging registers, no staging ALU work; the tile's key offset
//    is a scalar), row-major with XOR swizzles.  The V^T operand is gathered
//    by the gfx950 transposing LDS read, four keys of one head dim per lane.
//  * Two LDS stages: the DMA of block j+1 is issued before block j is
//    computed (one barrier per block).  The block loop is unrolled by two so
//    that stage offsets, like the block and k-step offsets, fold into
//    instruction immediates; per-lane address parts are computed once.
//  * Registers are budgeted for two waves per SIMD: a CU holds two
//    independent workgroups whose MFMA and softmax phases overlap.
//  * exp is computed as exp2 with |scale|*log2(e) folded into one FMA; the
//    sign of the scale is folded into Q (FoldedScale), so the row max can be
//    taken before scaling.
//  * Each wave raises its priority (s_setprio) while it issues the S^T
//    MFMA chain and drops it for the softmax and P V, which keeps the
//    co-resident waves of a SIMD in different phases.  (A pipelined schedule
//    that overlaps inside each wave instead, the next tile's S^T chain
//    interleaved with this tile's softmax as FlashAttention-3 overlaps
//    GEMM and softmax, is kept for measurement: FA_PREFILL_PIPE=1.)
//  * Lazy rescale: P is formed against the max the row is held at; the
//    accumulator is rescaled (and the held max moved to the exact running
//    max) only when some lane's sum of P exceeds the bound: 2^15 over the
//    tile for fp16 (largest finite 65504), 2^30 since the last exact step
//    for bf16 (which also bounds the accumulator).  Until then every P stays
//    within that bound, which the 16-bit type and float32 hold without loss
//    of relative precision, and no per-tile row max is needed;
//    O and LSE are the same function of the inputs because acc, l and m
//    always refer to the same held max.  (With scores of large spread the
//    running max keeps growing; at 2^8 the exact step ran more often: the
//    wave takes it when any of its 32 rows needs it.)
//  * Causal: K/V blocks after a workgroup's last query are never loaded;
//    a wave skips the MFMA work of blocks entirely after its own last query;
//    only blocks that cross the diagonal or the ragged key tail are masked.
//    Rows of the ragged key tail are fetched from the last key (finite data
//    that the mask removes), so no load leaves the tensor.
//  * Workgroup order: whole heads per XCD; under the causal mask the XCD's
//    heads four at a time in two phases (long blocks, then short), longest
//    first, which balances the hardware's in-order dispatch (fa_layout.h).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_layout.h"

namespace fa {
namespace {

struct PrefillArgs {
    const void *q;
    const void *k;
    const void *v;
    void *out;
    float *lse;
    int BH;
    int Nq;
    int Nk;
    int Tr;            // Q row blocks per (batch, head)
    float scale_log2;  // |scale| * log2(e) (1 for a zero scale; see FoldedScale)
    uint32_t qflip;    // sign bits flipped in Q for a negative scale
    uint32_t qkeep;    // 0 zeroes Q for a zero scale
    // packed variable-length batches (q [total_q, H, d], k and v
    // [total_k, H, d], lse [H, total_q]; the tile list from the schedule)
    const int *cu_q;
    const int *cu_k;
    const int *sched;  // [0] = tiles, then (sequence, Q block) pairs from index 2
    int H;
    int total_q;
    int total_k;
    // split prefill: the key range of a Q block is cut into S chunks of
    // `chunk` keys (a multiple of the tile); partials go to ws_o / ws_lse
    float *ws_o;    // [BH * Nq, S, D]
    float *ws_lse;  // [BH * Nq, S]
    int S;
    int chunk;
};

// How a launch maps workgroups to work: dense (batch*head, Q block),
// packed variable-length tiles, or dense with the key range split.
constexpr int kModeDense = 0;
constexpr int kModeVarlen = 1;
constexpr int kModeSplit = 2;

// Bound of the lazy rescale (see the online-softmax step of prefill_kernel).
// fp16: on a lane's sum of P over one tile, which keeps every P within
// 2^15, so P rounded to fp16 stays below its largest finite 65504.  bf16 has
// float32's exponent range, so the bound is on the lane's running sum of P
// since the last exact step: every P, the row sums and the accumulator
// (|acc| <= 2 * 2^30 * max|V| over the two lane halves) stay finite for
// |V| up to 2^96, whatever the length of the key range.
template <typename T>
constexpr float held_sum_bound() { return __is_same(T, _Float16) ? 32768.0f : 0x1p30f; }
template <typename T>
constexpr bool running_sum_bound() { return !__is_same(T, _Float16); }
constexpr float kLn2 = 0.693147180559945309417f;

template <typename T, int D, bool CAUSAL, int NW, int QW, int BC, int OCC, int MODE, int KSPLIT = 1,
          bool PIPE = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC)))
void prefill_kernel(PrefillArgs a) {
    constexpr bool VARLEN = MODE == kModeVarlen;
    constexpr bool SPLIT = MODE == kModeSplit;
    using M = Mfma<T>;
    using x8 = typename M::x8;
    using x4 = typename M::x4;
    // KSPLIT > 1 (grids too small for the GPU): KSPLIT waves share one group
    // of QW queries and take turns over its K/V tiles (wave part p takes
    // tiles p, p + KSPLIT, ...); each step stages KSPLIT consecutive tiles,
    // and at the end the parts' (m, l, acc) are merged through LDS.
    constexpr int NT = NW * 64;      // threads per workgroup
    constexpr int BR = NW / KSPLIT * QW;  // query rows per workgroup
    constexpr int QB = QW / 32;      // 32-query column blocks per wave
    constexpr int KS = D / 16;       // k-steps of S^T = K Q^T
    constexpr int DB = D / 32;       // 32-dim row blocks of O^T
    constexpr int KB = BC / 32;      // 32-key row blocks of S^T
    constexpr int KS2 = BC / 16;     // k-steps of O^T = V^T P^T
    constexpr int CH = D / 8;        // 16-byte chunks per row of K or V
    constexpr int ROW = D * 2;       // bytes per key row
    constexpr int BCS = KSPLIT * BC;             // keys staged per step
    constexpr int TILE_BYTES = BCS * ROW;        // the K (or V) rows of one step
    constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K rows + V rows
    constexpr int UNITS = BCS * CH;              // 16-byte units per step
    constexpr int NDMA = UNITS / NT;             // DMA instructions per thread per step (each of K, V)
    static_assert(QW % 32 == 0 && BC % 32 == 0 && D % 32 == 0, "tile shape");
    static_assert(NW % KSPLIT == 0 && (KSPLIT == 1 || MODE == kModeDense), "key split: dense launches only");
    static_assert(UNITS % NT == 0, "a tile must split evenly over the workgroup");
    static_assert(2 * STAGE_BYTES <= 65536, "stage offsets must fit a 16-bit LDS immediate");

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;

    // Work item: (batch*head, Q block) of a dense launch, or (head, tile of
    // the schedule) of a packed variable-length launch, or (batch*head, Q
    // block, key chunk) of a split launch.  RS is the element stride between
    // consecutive rows of one head.
    int qblk, Nq, Nk, RS, bh = 0, chunk_idx = 0;
    const T *qp, *kp, *vp;
    T *op;
    float *lsep;
    if constexpr (VARLEN) {
        const int t = blockIdx.x / a.H;
        const int h = blockIdx.x - t * a.H;
        if (t >= a.sched[0]) return;  // the grid is an upper bound on the tiles (workgroup-uniform exit)
        const int seq = a.sched[2 + 2 * t];
        qblk = a.sched[3 + 2 * t];
        int qs, qe, ks0, ke;
        layout::varlen_bounds(a.cu_q, seq, a.total_q, qs, qe);
        layout::varlen_bounds(a.cu_k, seq, a.total_k, ks0, ke);
        Nq = qe - qs;
        Nk = ke - ks0;
        RS = a.H * D;
        qp = static_cast<const T *>(a.q) + ((size_t)qs * a.H + h) * D;
        kp = static_cast<const T *>(a.k) + ((size_t)ks0 * a.H + h) * D;
        vp = static_cast<const T *>(a.v) + ((size_t)ks0 * a.H + h) * D;
        op = static_cast<T *>(a.out) + ((size_t)qs * a.H + h) * D;
        lsep = a.lse ? a.lse + (size_t)h * a.total_q + qs : nullptr;
    } else {
        int wg = blockIdx.x;
        if constexpr (SPLIT) {  // the chunks of one Q block are neighbours
            chunk_idx = wg % a.S;
            wg /= a.S;
        }
        layout::map_workgroup(wg, a.BH, a.Tr, CAUSAL, bh, qblk);
        Nq = a.Nq;
        Nk = a.Nk;
        RS = D;
        qp = static_cast<const T *>(a.q) + (size_t)bh * Nq * D;
        kp = static_cast<const T *>(a.k) + (size_t)bh * Nk * D;
        vp = static_cast<const T *>(a.v) + (size_t)bh * Nk * D;
        op = static_cast<T *>(a.out) + (size_t)bh * Nq * D;
        lsep = a.lse ? a.lse + (size_t)bh * Nq : nullptr;
    }
    const int RSB = RS * 2;  // bytes between rows
    const int kpart = KSPLIT > 1 ? wave % KSPLIT : 0;  // the wave's share of the key tiles
    const int q0 = qblk * BR;
    const int q0w = q0 + wave / KSPLIT * QW;
    const float c = a.scale_log2;
    const uint32_t kv_bytes = Nk > 0 ? (uint32_t)(Nk - 1) * RSB + ROW : 0u;
    const __amdgpu_buffer_rsrc_t rsrc_k = __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(kp), (short)0, (int)kv_bytes, kBufferDword3);
    const __amdgpu_buffer_rsrc_t rsrc_v = __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(vp), (short)0, (int)kv_bytes, kBufferDword3);

    // per-lane DMA source offsets (bytes, relative to the tile's first key)
    uint32_t kdma[NDMA], vdma[NDMA];
    int dkey[NDMA];
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
        const int u = (n * NW + wave) * 64 + lane;
        dkey[n] = u / CH;
        kdma[n] = (uint32_t)(layout::k_dma_src_elem<D>(u) + dkey[n] * (RS - D)) * 2;
        vdma[n] = (uint32_t)(layout::v_dma_src_elem<D>(u) + dkey[n] * (RS - D)) * 2;
    }
    // per-lane operand read offsets (bytes within a tile, block / k-step 0)
    int koff[KS], voff[DB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = layout::k_operand_offset<D>(0, l32, g, ks) + kpart * BC * ROW;
#pragma unroll
    for (int db = 0; db < DB; ++db) voff[db] = layout::v_operand_tr_offset<D>(db, lane, 0, 0) + kpart * BC * ROW;

    auto issue_tile = [&](int k0, int stage) {
        char *kbase = smem + stage * STAGE_BYTES;
        char *vbase = kbase + TILE_BYTES;
        const uint32_t soff = (uint32_t)k0 * RSB;
        const bool tail = k0 + BCS > Nk;  // workgroup-uniform
#pragma unroll
        for (int n = 0; n < NDMA; ++n) {
            uint32_t ko = kdma[n], vo = vdma[n];
            if (tail) {
                const int over = k0 + dkey[n] - (Nk - 1);  // rows past the end: fetch the last key instead
                if (over > 0) {
                    ko -= (uint32_t)over * RSB;
                    vo -= (uint32_t)over * RSB;
                }
            }
            const int dst = (n * NW + wave) * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_k, (FA_LDS void *)(kbase + dst), 16, ko, soff, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_v, (FA_LDS void *)(vbase + dst), 16, vo, soff, 0, 0);
        }
    };

    const int kv_end = CAUSAL ? min(Nk, q0 + BR) : Nk;
    // keys [kbeg, kend) of this workgroup: all visible ones, or one chunk
    const int kbeg = SPLIT ? min(kv_end, chunk_idx * a.chunk) : 0;
    const int kend = SPLIT ? min(kv_end, kbeg + a.chunk) : kv_end;
    const int nt = (kend - kbeg + BCS - 1) / BCS;  // steps
    // The first step's K/V copy goes out before the Q loads, so that the two
    // wait on memory together (workgroup-uniform; a sequence or chunk
    // without keys has no step).
    if (nt > 0) issue_tile(kbeg, 0);
    // one K or V tile of BC keys (pipelined schedule: K runs one tile ahead of V)
    auto issue_part = [&](bool is_v, int k0, int stage) {
        char *dbase = smem + stage * STAGE_BYTES + (is_v ? TILE_BYTES : 0);
        const uint32_t soff = (uint32_t)k0 * RSB;
        const bool tail = k0 + BCS > Nk;  // workgroup-uniform
#pragma unroll
        for (int n = 0; n < NDMA; ++n) {
            uint32_t o = is_v ? vdma[n] : kdma[n];
            if (tail) {
                const int over = k0 + dkey[n] - (Nk - 1);
                if (over > 0) o -= (uint32_t)over * RSB;
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_v ? rsrc_v : rsrc_k,
                                                     (FA_LDS void *)(dbase + (n * NW + wave) * 1024), 16, o, soff, 0, 0);
        }
    };
    if constexpr (PIPE) {
        if (nt > 1) issue_part(false, kbeg + BC, 1);
    }

    // Q fragments (B operand of S^T): lane (query l32 of block qb, half g)
    // holds dims [16*ks + 8*g, +8).  Every lane loads (rows past the end
    // read the last row, then are zeroed), so the loads carry no branches
    // and all go out before any of them is waited for.
    x8 qf[QB][KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = q0w + 32 * qb + l32;
        const bool row_ok = row < Nq;  // a workgroup exists only for Nq >= 1
        const T *qrow = qp + (size_t)(row_ok ? row : Nq - 1) * RS;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 raw = *reinterpret_cast<const u32x4 *>(qrow + 16 * ks + 8 * g);
            raw = row_ok ? raw : u32x4{0u, 0u, 0u, 0u};
            raw = (raw ^ a.qflip) & a.qkeep;  // the sign of the scale, folded into Q
            qf[qb][ks] = __builtin_bit_cast(x8, raw);
        }
    }

    f32x16 oacc[QB][DB];
    float m_held[QB];
    float l_part[QB];
    // Two running sums per row: l_part of the float32 P (for LSE and the
    // lazy-rescale test) and lt of the P rounded to the input type, the
    // weights P V is formed with; O is normalised by lt, so O is a convex
    // combination of value rows whatever the rounding of a dominant weight
    // (which is not 1 while the held max lags the row max).  lt is summed
    // on the matrix core: read as the B operand of a 16x16x32 product, the
    // P^T registers of lanes n and n+32 (query n) form K blocks 0 and 2 of
    // column n, those of lanes n+16 and n+48 (query n+16) K blocks 1 and 3.
    // With A row 0 = ones on blocks 0, 2 and row 1 = ones on blocks 1, 3
    // (lanes 0, 32 and 17, 49; every other lane zero), lane n < 16 of the
    // accumulator holds query n's sum in register 0 and query n+16's in
    // register 1.
    f32x4 lt[QB];
    x8 ones8;
    {
        const uint16_t one = (lane == 0 || lane == 32 || lane == 17 || lane == 49) ? M::kOne : (uint16_t)0;
        const uint32_t w2 = (uint32_t)one * 0x10001u;
        ones8 = __builtin_bit_cast(x8, u32x4{w2, w2, w2, w2});
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_held[qb] = -__builtin_inff();
        l_part[qb] = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) lt[qb][r] = 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.0f;
    }

    auto compute_tile = [&](auto stage_tag, int k0) {
        constexpr int S = decltype(stage_tag)::value;
        constexpr int KOFF = S * STAGE_BYTES;
        constexpr int VOFF = KOFF + TILE_BYTES;
        // ---- S^T = K_blk Q^T -------------------------------------------------
        // The wave runs at raised priority while it issues this chain, so
        // that co-resident waves of other workgroups fall out of step with
        // it: one wave's exponentials then run beside another's MFMAs.
        __builtin_amdgcn_s_setprio(1);
        f32x16 s[QB][KB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.0f;
        // K fragments are read KPF steps ahead of the MFMA that takes them
        // (with 64 queries per wave each fragment feeds two MFMAs, which
        // hides the read by itself: the compiler schedules those shapes)
        constexpr int NK = KB * KS;
        constexpr int KPF = QB > 1 ? 1 : (NK < 3 ? NK : 3);
        auto read_k = [&](int i) {
            return __builtin_bit_cast(
                x8, *reinterpret_cast<const u32x4 *>(smem + KOFF + (i / KS) * 32 * ROW + koff[i % KS]));
        };
        x8 kq[KPF];
#pragma unroll
        for (int i = 0; i < KPF; ++i) kq[i] = read_k(i);
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const x8 kf = kq[i % KPF];
            if (i + KPF < NK) kq[i % KPF] = read_k(i + KPF);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb][i / KS] = M::run(kf, qf[qb][i % KS], s[qb][i / KS]);
        }
        // keep that order: KPF reads, then (one MFMA, one read) per step
        if constexpr (QB == 1) {
            __builtin_amdgcn_sched_group_barrier(0x100, KPF, 0);
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i + KPF < NK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }

        __builtin_amdgcn_s_setprio(0);

        // ---- mask: ragged key tail and the causal diagonal ------------------
        // Register r of 32-key block kb holds key base + acc_row(r, 0) with
        // base = k0 + 32 kb + 4 g (acc_row(r, g) = acc_row(r, 0) + 4 g), so
        // one per-lane limit, the last visible offset, decides all 16: a
        // compare with the constant acc_row(r, 0) and a select each.
        const bool need_mask = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > q0w);
        if (need_mask) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int qrow = q0w + 32 * qb + l32;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const int base = k0 + 32 * kb + 4 * g;
                    int lim = Nk - 1 - base;
                    if constexpr (CAUSAL) lim = min(lim, qrow - base);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (layout::acc_row(r, 0) > lim) s[qb][kb][r] = -__builtin_inff();
                }
            }
        }

        // ---- online softmax -------------------------------------------------
        // P = exp2(c*s - m_held) and its row sums are formed first.  A lane's
        // tile sum (bf16: running sum) <= the bound bounds each of its P by it
        // (P >= 0), which is the lazy-rescale invariant, so the row max is only
        // needed when some lane of the wave exceeds it (or has no held max yet).  Then the exact
        // step runs on the untouched scores: m_new = max(m_held, rowmax),
        // rescale acc and l by exp2(m_held - m_new), recompute P.
        x8 pf[QB][KS2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            auto exp_tile = [&](float msub) {
                float lsum = 0.0f;
#pragma unroll
                for (int ks2 = 0; ks2 < KS2; ++ks2) {
                    const int kb = ks2 >> 1;
                    const int h = (ks2 & 1) * 8;
                    f32x8 t;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        t[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb][h + e], c, -msub));
                        // start the sum from the first term: 0 + x cannot be
                        // folded away in IEEE arithmetic (x = -0), and P >= 0
                        lsum = (ks2 == 0 && e == 0) ? t[e] : lsum + t[e];
                    }
                    pf[qb][ks2] = __builtin_convertvector(t, x8);
                }
                return lsum;
            };
            float lsum = 0.0f;
            bool exact = __ballot(m_held[qb] == -__builtin_inff()) != 0ull;
            if (!exact) {
                lsum = exp_tile(m_held[qb]);
                const float held = running_sum_bound<T>() ? l_part[qb] + lsum : lsum;
                exact = __ballot(!(held <= held_sum_bound<T>())) != 0ull;  // also true for inf / NaN
            }
            if (exact) {
                float mx = -__builtin_inff();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[qb][kb][r]);
                mx = xor32_max(mx);
                const float m_new = __builtin_fmaxf(m_held[qb], mx * c);  // c > 0 (the sign is in Q)
                const float alpha =
                    (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_held[qb] - m_new);
                // a wave whose rows have no held max yet (its first block) has
                // nothing accumulated: no rescale
                const bool held_any = __ballot(m_held[qb] != -__builtin_inff()) != 0ull;
                m_held[qb] = m_new;
                if (held_any) {
                    l_part[qb] *= alpha;
                    // lane n < 16 keeps queries n (register 0) and n + 16 (register 1)
                    const float alpha_hi = __shfl(alpha, (lane + 16) & 63);
                    lt[qb][0] *= alpha;
                    lt[qb][1] *= alpha_hi;
#pragma unroll
                    for (int db = 0; db < DB; ++db) oacc[qb][db] *= alpha;
                }
                // a row that has seen no key yet keeps m = -inf: subtract 0
                // there so masked scores give exp2(-inf) = 0, not NaN
                lsum = exp_tile((m_new == -__builtin_inff()) ? 0.0f : m_new);
            }
            l_part[qb] += lsum;
        }

        // ---- O^T += V^T P^T -------------------------------------------------
        // step i = (k-step i / DB, d block i % DB); its V^T fragment (two
        // transposing reads) is read VPF steps ahead of its MFMA (at 32
        // queries per wave, as for K)
        constexpr int NV = KS2 * DB;
        constexpr int VPF = QB > 1 ? 1 : (NV < 3 ? NV : 3);
        auto read_v = [&](int i) {
            const char *base = smem + VOFF + voff[i % DB] + 16 * (i / DB) * ROW;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4 *)(base));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4 *)(base + 8 * ROW));
            return __builtin_bit_cast(x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        x8 vq[VPF];
#pragma unroll
        for (int i = 0; i < VPF; ++i) vq[i] = read_v(i);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const x8 vf = vq[i % VPF];
            if (i + VPF < NV) vq[i % VPF] = read_v(i + VPF);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) oacc[qb][i % DB] = M::run(vf, pf[qb][i / DB], oacc[qb][i % DB]);
        }
        // ---- lt += rowsum of the rounded P (matrix core), after P V -------------
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int ks2 = 0; ks2 < KS2; ++ks2) lt[qb] = M::run16(ones8, pf[qb][ks2], lt[qb]);
        if constexpr (QB == 1) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * VPF, 0);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i + VPF < NV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, KS2, 0);
        }
    };

    auto step = [&](auto stage_tag, int jt) {
        constexpr int S = decltype(stage_tag)::value;
        const int ks0 = kbeg + jt * BCS;
        if (jt + 1 < nt) issue_tile(ks0 + BCS, S ^ 1);
        const int k0 = ks0 + kpart * BC;
        // wave-uniform: the wave has live queries that see some key of its block
        const bool active =
            (q0w < Nq) && (KSPLIT == 1 || k0 < kend) && (!CAUSAL || k0 <= q0w + QW - 1);
        if (active) compute_tile(stage_tag, k0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's DMA of block jt+1 has landed
        __syncthreads();                                    // ... and every thread's; stage S is free
    };

    if constexpr (!PIPE) {
        if (nt > 0) {  // the first step's copy (issued above) has landed for every thread
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
        for (int jt = 0; jt < nt; jt += 2) {
            step(Int<0>{}, jt);
            if (jt + 1 < nt) step(Int<1>{}, jt + 1);
        }
    } else {
        // ---- pipelined schedule: tile j+1's S^T chain beside tile j's softmax --
        // Step j computes S^T of tile j+1 (K in stage (j+1) & 1) while it forms
        // P of tile j, then P V of tile j (V in stage j & 1).  K is copied two
        // tiles ahead and V one: step j issues K of tile j+2 into stage j & 1
        // (last read by step j-1) and V of tile j+1 into stage (j+1) & 1 (last
        // read by step j-1), after the barrier that ends step j-1.  Per element
        // the arithmetic and its order are those of the schedule above.
        static_assert(QB == 1 && KB == 1 && KS2 == 2 && KSPLIT == 1, "pipelined schedule: one 32x32 tile per wave");
        constexpr int NK = KS;
        constexpr int KPF = NK < 3 ? NK : 3;
        auto active_at = [&](int j) {
            return j < nt && q0w < Nq && (!CAUSAL || kbeg + j * BC <= q0w + QW - 1);
        };
        // S^T of the tile in the K stage of kstage_tag into s, each MFMA
        // followed by one K read and NVALU vector instructions of whatever
        // the caller placed in the same block
        auto s_chain = [&](auto kstage_tag, f32x16 &s, auto nvalu_tag) {
            constexpr int KOFF = decltype(kstage_tag)::value * STAGE_BYTES;
            constexpr int NVALU = decltype(nvalu_tag)::value;
            auto read_k = [&](int i) {
                return __builtin_bit_cast(x8, *reinterpret_cast<const u32x4 *>(smem + KOFF + koff[i]));
            };
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = 0.0f;
            x8 kq[KPF];
#pragma unroll
            for (int i = 0; i < KPF; ++i) kq[i] = read_k(i);
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                const x8 kf = kq[i % KPF];
                if (i + KPF < NK) kq[i % KPF] = read_k(i + KPF);
                s = M::run(kf, qf[0][i], s);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, KPF, 0);
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i + KPF < NK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                if constexpr (NVALU > 0) __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);
            }
        };
        auto exp_half = [&](const f32x16 &s, int h, float msub, float &lsum, x8 &p) {
            f32x8 t;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                t[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * h + e], c, -msub));
                lsum = (h == 0 && e == 0) ? t[e] : lsum + t[e];
            }
            p = __builtin_convertvector(t, x8);
        };
        auto tile = [&](auto stage_tag, int j, f32x16 &s_cur, f32x16 &s_next) {
            constexpr int P = decltype(stage_tag)::value;
            constexpr int VOFF = P * STAGE_BYTES + TILE_BYTES;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's copies for this step have landed
            __syncthreads();                                    // ... every thread's; step j-1 is done everywhere
            if (j + 2 < nt) issue_part(false, kbeg + (j + 2) * BC, P);
            if (j + 1 < nt) issue_part(true, kbeg + (j + 1) * BC, P ^ 1);
            if (!active_at(j)) return;  // wave-uniform; no later tile is active either
            const int k0 = kbeg + j * BC;
            const bool need_mask = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > q0w);
            if (need_mask) {
                const int qrow = q0w + l32;
                const int base = k0 + 4 * g;
                int lim = Nk - 1 - base;
                if constexpr (CAUSAL) lim = min(lim, qrow - base);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (layout::acc_row(r, 0) > lim) s_cur[r] = -__builtin_inff();
            }
            // P against the held max (a wave's first tile gives inf or NaN
            // sums there, which the test below sends to the exact step), in
            // one block with the next tile's S^T chain.  After the wave's last
            // active tile that chain reads whatever K stage P^1 holds (in
            // bounds) and its result is never used.
            x8 pf[2];
            float lsum = 0.0f;
            exp_half(s_cur, 0, m_held[0], lsum, pf[0]);
            exp_half(s_cur, 1, m_held[0], lsum, pf[1]);
            s_chain(Int<P ^ 1>{}, s_next, Int<7>{});
            const float held = running_sum_bound<T>() ? l_part[0] + lsum : lsum;
            if (__ballot(!(held <= held_sum_bound<T>())) != 0ull) {
                float mx = -__builtin_inff();
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s_cur[r]);
                mx = xor32_max(mx);
                const float m_new = __builtin_fmaxf(m_held[0], mx * c);  // c > 0 (the sign is in Q)
                const float alpha = (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_held[0] - m_new);
                const bool held_any = __ballot(m_held[0] != -__builtin_inff()) != 0ull;
                m_held[0] = m_new;
                if (held_any) {
                    l_part[0] *= alpha;
                    const float alpha_hi = __shfl(alpha, (lane + 16) & 63);
                    lt[0][0] *= alpha;
                    lt[0][1] *= alpha_hi;
#pragma unroll
                    for (int db = 0; db < DB; ++db) oacc[0][db] *= alpha;
                }
                const float msub = (m_new == -__builtin_inff()) ? 0.0f : m_new;
                exp_half(s_cur, 0, msub, lsum, pf[0]);
                exp_half(s_cur, 1, msub, lsum, pf[1]);
            }
            l_part[0] += lsum;
            // ---- O^T += V^T P^T, then lt += rowsum of the rounded P --------------
            constexpr int NV = KS2 * DB;
            constexpr int VPF = NV < 3 ? NV : 3;
            auto read_v = [&](int i) {
                const char *vb = smem + VOFF + voff[i % DB] + 16 * (i / DB) * ROW;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4 *)(vb));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4 *)(vb + 8 * ROW));
                return __builtin_bit_cast(x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            };
            x8 vq[VPF];
#pragma unroll
            for (int i = 0; i < VPF; ++i) vq[i] = read_v(i);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const x8 vf = vq[i % VPF];
                if (i + VPF < NV) vq[i % VPF] = read_v(i + VPF);
                oacc[0][i % DB] = M::run(vf, pf[i / DB], oacc[0][i % DB]);
            }
#pragma unroll
            for (int ks2 = 0; ks2 < KS2; ++ks2) lt[0] = M::run16(ones8, pf[ks2], lt[0]);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * VPF, 0);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i + VPF < NV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, KS2, 0);
        };
        f32x16 sa, sb;
        if (nt > 0) {  // the prologue's copies (K and V of tile 0, K of tile 1) have landed
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (active_at(0)) s_chain(Int<0>{}, sa, Int<0>{});
        }
        for (int j = 0; j < nt; j += 2) {
            tile(Int<0>{}, j, sa, sb);
            if (j + 1 < nt) tile(Int<1>{}, j + 1, sb, sa);
        }
    }

    // ---- key split: merge the parts of each query group --------------------
    // Parts 1 .. KSPLIT-1 write (m, l, lt, acc) to LDS (free after the last
    // step's barrier, field-major so that lanes hit consecutive banks); part 0
    // merges them as the split-KV combine does: M = max(m, m'), each side
    // weighed by exp2(m - M) (0 for a side without keys).
    if constexpr (KSPLIT > 1) {
        constexpr int NF = QB * (DB * 16 + 6);  // floats per lane per part
        static_assert((NW / KSPLIT) * (KSPLIT - 1) * NF * 64 * 4 <= 2 * STAGE_BYTES, "merge buffer");
        float *mbuf = reinterpret_cast<float *>(smem);
        const int base = (wave / KSPLIT) * (KSPLIT - 1) * NF;
        if (kpart > 0) {
            float *dst = mbuf + (base + (kpart - 1) * NF) * 64 + lane;
            int f = 0;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                dst[64 * f++] = m_held[qb];
                dst[64 * f++] = l_part[qb];
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[64 * f++] = lt[qb][r];
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) dst[64 * f++] = oacc[qb][db][r];
            }
        }
        __syncthreads();
        if (kpart == 0) {
#pragma unroll
            for (int part = 1; part < KSPLIT; ++part) {
                const float *src = mbuf + (base + (part - 1) * NF) * 64 + lane;
                int f = 0;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const float m2 = src[64 * f++];
                    const float l2 = src[64 * f++];
                    const float mm = __builtin_fmaxf(m_held[qb], m2);
                    const bool none = mm == -__builtin_inff();
                    const float a1 = none ? 0.0f : __builtin_amdgcn_exp2f(m_held[qb] - mm);
                    const float a2 = none ? 0.0f : __builtin_amdgcn_exp2f(m2 - mm);
                    m_held[qb] = mm;
                    l_part[qb] = __builtin_fmaf(l2, a2, l_part[qb] * a1);
                    // lane n < 16 keeps the rounded sums of queries n (register
                    // 0) and n + 16 (register 1)
                    const float a1_hi = __shfl(a1, (lane + 16) & 63), a2_hi = __shfl(a2, (lane + 16) & 63);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float lt2 = src[64 * f++];
                        lt[qb][r] = r == 1 ? __builtin_fmaf(lt2, a2_hi, lt[qb][r] * a1_hi)
                                           : __builtin_fmaf(lt2, a2, lt[qb][r] * a1);
                    }
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            oacc[qb][db][r] = __builtin_fmaf(src[64 * f++], a2, oacc[qb][db][r] * a1);
                }
            }
        }
    }

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2 --------------------
    // (split launch: this chunk's normalised partial o~ = acc / l and its
    // logsumexp, -inf with o~ = 0 where the chunk holds no visible key)
    if (kpart != 0) return;  // wave-uniform: the merged state is in part 0
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = xor32_sum(l_part[qb]);
        const float lt_lo = __shfl(lt[qb][0], l32 & 15);
        const float lt_hi = __shfl(lt[qb][1], l32 & 15);
        const float lw = (l32 < 16) ? lt_lo : lt_hi;  // sum of this row's rounded P
        const int row = q0w + 32 * qb + l32;
        if (row < Nq) {
            const float inv = (l > 0.0f && lw > 0.0f) ? 1.0f / lw : 0.0f;
            const float lse_row = (l > 0.0f) ? (m_held[qb] + __builtin_amdgcn_logf(l)) * kLn2 : -__builtin_inff();
            if constexpr (SPLIT) {
                const size_t slot = ((size_t)bh * Nq + row) * a.S + chunk_idx;
                float *wo = a.ws_o + slot * D;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        f32x4 t;
#pragma unroll
                        for (int e = 0; e < 4; ++e) t[e] = oacc[qb][db][4 * rg + e] * inv;
                        *reinterpret_cast<f32x4 *>(wo + 32 * db + 8 * rg + 4 * g) = t;
                    }
                if (g == 0) a.ws_lse[slot] = lse_row;
            } else {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        f32x4 t;
#pragma unroll
                        for (int e = 0; e < 4; ++e) t[e] = oacc[qb][db][4 * rg + e] * inv;
                        const x4 o = __builtin_convertvector(t, x4);
                        *reinterpret_cast<x4 *>(op + (size_t)row * RS + 32 * db + 8 * rg + 4 * g) = o;
                    }
                if (g == 0 && lsep != nullptr) lsep[row] = lse_row;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Tile schedule of a packed variable-length batch ("9.4 FlashAttention 与
// FlashMLA" section 9.4.6: the work of every workgroup is fixed before the
// attention launch, cutting sequences of different lengths into equal
// tiles).  One workgroup orders the sequences by length, longest first (a
// counting sort on 1024 buckets), and lists each sequence's (sequence, Q
// block) tiles of Br queries together, the longest (last, under the mask)
// first.  The attention grid takes tile t for every head h as workgroup
// t*H + h, so all tiles of one (sequence, head) run back to back on one XCD
// (workgroups go to XCD wg % 8; with H a multiple of 8 that is h % 8) and
// its K/V stay in that XCD's L2, while long work starts first and short
// work fills the tail.  Output: sched[0] = number of tiles, then the pairs
// from index 2.
// ---------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;
constexpr int kSchedBuckets = 1024;

template <int BR, int BC, bool CAUSAL>
__global__ __launch_bounds__(kSchedThreads) void varlen_schedule_kernel(const int *cu_q, const int *cu_k, int S,
                                                                         int total_q, int total_k, int max_tiles,
                                                                         int *sched) {
    __shared__ int order[kMaxVarlenSeqs];           // sequences, longest first
    __shared__ int tile_start[kMaxVarlenSeqs + 1];  // first tile of order[i]
    __shared__ int hist[kSchedBuckets];
    __shared__ int scan[kSchedThreads];
    __shared__ int lmax_s;
    static_assert(kSchedBuckets == kSchedThreads, "one bucket per thread");
    const int tid = threadIdx.x;
    auto bounds = [&](int s, int &nb, int &work) {
        int qs, qe, ks, ke;
        layout::varlen_bounds(cu_q, s, total_q, qs, qe);
        layout::varlen_bounds(cu_k, s, total_k, ks, ke);
        nb = (qe - qs + BR - 1) / BR;
        work = nb > 0 ? (ke - ks) : 0;  // key count orders the sequences
    };
    // inclusive block scan of one value per thread (every thread calls it)
    auto block_scan = [&](int v) {
        scan[tid] = v;
        __syncthreads();
        for (int off = 1; off < kSchedThreads; off <<= 1) {
            const int x = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += x;
            __syncthreads();
        }
        const int r = scan[tid];
        const int total = scan[kSchedThreads - 1];
        __syncthreads();
        return make_int2(r, total);
    };

    if (tid == 0) lmax_s = 0;
    hist[tid] = 0;
    __syncthreads();
    for (int s = tid; s < S; s += kSchedThreads) {
        int nb, work;
        bounds(s, nb, work);
        atomicMax(&lmax_s, work);
    }
    __syncthreads();
    const int lmax = lmax_s;
    auto bucket = [&](int work) {  // descending: the longest sequences in bucket 0
        const int b = lmax > 0 ? (int)((long long)work * (kSchedBuckets - 1) / lmax) : 0;
        return kSchedBuckets - 1 - b;
    };
    for (int s = tid; s < S; s += kSchedThreads) {
        int nb, work;
        bounds(s, nb, work);
        atomicAdd(&hist[bucket(work)], 1);
    }
    __syncthreads();
    {
        const int own = hist[tid];
        const int2 r = block_scan(own);
        hist[tid] = r.x - own;  // first position of the bucket
    }
    __syncthreads();
    for (int s = tid; s < S; s += kSchedThreads) {
        int nb, work;
        bounds(s, nb, work);
        order[atomicAdd(&hist[bucket(work)], 1)] = s;
    }
    __syncthreads();
    // first tile of each sequence in that order
    int carry = 0;
    for (int base = 0; base < S; base += kSchedThreads) {
        const int i = base + tid;
        int nb = 0, work;
        if (i < S) bounds(order[i], nb, work);
        const int2 r = block_scan(nb);
        if (i < S) tile_start[i] = carry + r.x - nb;
        carry += r.y;
    }
    const int T = carry;
    if (tid == 0) tile_start[S] = T;
    __syncthreads();
    for (int t = tid; t < T && t < max_tiles; t += kSchedThreads) {
        int lo = 0, hi = S - 1;  // the last position whose first tile is <= t (it has tiles)
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tile_start[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        const int s = order[lo];
        const int r = t - tile_start[lo];
        const int nb = tile_start[lo + 1] - tile_start[lo];
        sched[2 + 2 * t] = s;
        sched[3 + 2 * t] = CAUSAL ? nb - 1 - r : r;  // under the mask the last Q block is the longest
    }
    if (tid == 0) sched[0] = T < max_tiles ? T : max_tiles;  // only decreasing offsets can exceed the bound
}

template <typename T, int D, bool CAUSAL, int NW, int QW, int OCC, int BC = 64, int KSPLIT = 1, bool PIPE = false>
hipError_t launch_one(const PrefillArgs &base, bool varlen, int S, hipStream_t stream) {
    constexpr int BR = NW / KSPLIT * QW;
    PrefillArgs a = base;
    if constexpr (KSPLIT > 1) {  // dense launches only (the host never asks otherwise)
        if (varlen || a.S > 1) return hipErrorInvalidValue;
        a.Tr = (a.Nq + BR - 1) / BR;
        const long long nwg = (long long)a.BH * a.Tr;
        if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((prefill_kernel<T, D, CAUSAL, NW, QW, BC, OCC, kModeDense, KSPLIT>), dim3((unsigned)nwg),
                           dim3(NW * 64), 0, stream, a);
        return hipGetLastError();
    }
    if (!varlen) {
        a.Tr = (a.Nq + BR - 1) / BR;
        const long long nwg = (long long)a.BH * a.Tr;
        if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        if (a.S > 1) {
            const long long nwg_split = nwg * a.S;
            if (nwg_split > 0x7fffffffLL) return hipErrorInvalidConfiguration;
            hipLaunchKernelGGL((prefill_kernel<T, D, CAUSAL, NW, QW, BC, OCC, kModeSplit, 1, PIPE>), dim3((unsigned)nwg_split),
                               dim3(NW * 64), 0, stream, a);
            return hipGetLastError();
        }
        hipLaunchKernelGGL((prefill_kernel<T, D, CAUSAL, NW, QW, BC, OCC, kModeDense, 1, PIPE>), dim3((unsigned)nwg),
                           dim3(NW * 64), 0, stream, a);
        return hipGetLastError();
    }
    const long long tiles = varlen_max_tiles(S, a.total_q, BR);
    const long long nwg = (long long)a.H * tiles;
    if (nwg > 0x7fffffffLL || S < 1 || S > kMaxVarlenSeqs) return hipErrorInvalidConfiguration;
    int *sched = const_cast<int *>(a.sched);
    hipLaunchKernelGGL((varlen_schedule_kernel<BR, BC, CAUSAL>), dim3(1), dim3(kSchedThreads), 0, stream, a.cu_q,
                       a.cu_k, S, a.total_q, a.total_k, (int)tiles, sched);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((prefill_kernel<T, D, CAUSAL, NW, QW, BC, OCC, kModeVarlen, 1, PIPE>), dim3((unsigned)nwg),
                       dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

// FA_PREFILL_PIPE=1 runs shape 3 with the pipelined schedule (next tile's
// S^T chain beside this tile's softmax).  Its results are bit for bit those
// of the default schedule; it needs 204 registers (two waves per SIMD, where
// the default fits three) and measured 12-17% slower, so it is off by default.
bool prefill_pipe() {
    const char *env = getenv("FA_PREFILL_PIPE");
    return env != nullptr && env[0] == '1' && env[1] == '\0';
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_shape(int shape, const PrefillArgs &a, bool varlen, int S, hipStream_t stream) {
    switch (shape) {
        case kShapeW4Q32: return launch_one<T, D, CAUSAL, 4, 32, 2>(a, varlen, S, stream);
        case kShapeW4Q64: return launch_one<T, D, CAUSAL, 4, 64, 1>(a, varlen, S, stream);
        case kShapeW2Q64: return launch_one<T, D, CAUSAL, 2, 64, 1>(a, varlen, S, stream);
        case kShapeW4Q32B32:  // a 32-key tile of d = 32 is too small to split over 256 threads
            if constexpr (D >= 64) {
                if (prefill_pipe()) return launch_one<T, D, CAUSAL, 4, 32, 2, 32, 1, true>(a, varlen, S, stream);
                return launch_one<T, D, CAUSAL, 4, 32, 3, 32>(a, varlen, S, stream);
            }
            else return launch_one<T, D, CAUSAL, 4, 32, 2>(a, varlen, S, stream);
        // key splits: two steps of staged keys must fit 64 KB of LDS
        case kShapeW4Q32K2:
            if constexpr (D >= 128) return launch_one<T, D, CAUSAL, 4, 32, 3, 32, 2>(a, varlen, S, stream);
            else return launch_one<T, D, CAUSAL, 4, 32, 2, 64, 2>(a, varlen, S, stream);
        case kShapeW4Q32K4:
            if constexpr (D >= 128) return launch_one<T, D, CAUSAL, 4, 32, 3, 32, 2>(a, varlen, S, stream);
            else if constexpr (D == 64) return launch_one<T, D, CAUSAL, 4, 32, 2, 32, 4>(a, varlen, S, stream);
            else return launch_one<T, D, CAUSAL, 4, 32, 2, 64, 4>(a, varlen, S, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_typed(int d, bool causal, int shape, const PrefillArgs &a, bool varlen, int S,
                        hipStream_t stream) {
#define FA_CASE(DD)                                                                 \
    case DD:                                                                        \
        return causal ? launch_shape<T, DD, true>(shape, a, varlen, S, stream)      \
                      : launch_shape<T, DD, false>(shape, a, varlen, S, stream);
    switch (d) {
        FA_CASE(32)
        FA_CASE(64)
        FA_CASE(128)
        default: return hipErrorInvalidValue;
    }
#undef FA_CASE
}

void set_scale(PrefillArgs &a, float scale_log2) {
    const FoldedScale fs = fold_scale(scale_log2, kSignBits16);
    a.scale_log2 = fs.c;
    a.qflip = fs.flip;
    a.qkeep = fs.keep;
}

hipError_t launch_any(int dtype, int d, bool causal, int shape, const PrefillArgs &a, bool varlen, int S,
                      hipStream_t stream) {
    if (dtype == 2) return launch_typed<__bf16>(d, causal, shape, a, varlen, S, stream);
    if (dtype == 1) return launch_typed<_Float16>(d, causal, shape, a, varlen, S, stream);
    return hipErrorInvalidValue;
}

}  // namespace

static int prefill_block_cols(int shape, int d);

int prefill_block_rows(int shape) {
    switch (shape) {
        case kShapeW4Q32: return 128;
        case kShapeW4Q64: return 256;
        case kShapeW2Q64: return 128;
        case kShapeW4Q32B32: return 128;
        case kShapeW4Q32K2: return 64;
        case kShapeW4Q32K4: return 32;  // 64 at d = 128, which takes the two-way split
        default: return 0;
    }
}

int prefill_small_grid_shape(int d, bool causal, int shape, int BH, int Nq, int Nk) {
    // Below one workgroup per CU the time is the key loop of the longest Q
    // block, one tile after another in each wave; splitting that loop over
    // KSPLIT waves of the workgroup shortens it KSPLIT-fold for one merge
    // through LDS.  Worth it once the loop holds enough tiles.
    const int br = prefill_block_rows(shape);
    if (br <= 0 || BH < 1 || Nq < 1 || Nk < 1) return shape;
    const long long grid = (long long)BH * ((Nq + br - 1) / br);
    const long long rows = (long long)(Nq + br - 1) / br * br;
    const long long keys = causal && rows < Nk ? rows : Nk;  // the longest Q block's key range
    const int bc = prefill_block_cols(shape, d);
    if (grid >= 256 || keys < 8LL * bc) return shape;
    return (grid <= 128 && d <= 64) ? kShapeW4Q32K4 : kShapeW4Q32K2;
}

// Keys per K/V tile of a shape at head dim d (shape 3 falls back to shape 0
// below d = 64).
static int prefill_block_cols(int shape, int d) { return (shape == kShapeW4Q32B32 && d >= 64) ? 32 : 64; }

// K/V tiles in the longest key range a Q block reads: all Nk keys, or under
// the causal mask (query i sees keys 0..i) at most the rows of the last Q
// block.  Split chunks cover this range only.
static int split_key_tiles(int shape, int d, bool causal, int Nq, int Nk) {
    const int br = prefill_block_rows(shape), bc = prefill_block_cols(shape, d);
    const long long rows = (long long)(Nq + br - 1) / br * br;
    const int kext = causal && rows < Nk ? (int)rows : Nk;
    return (kext + bc - 1) / bc;
}

int prefill_split_count(int d, bool causal, int shape, int BH, int Nq, int Nk) {
    const int br = prefill_block_rows(shape);
    if (br <= 0 || BH < 1 || Nq < 1 || Nk < 1) return 1;
    const long long grid = (long long)BH * ((Nq + br - 1) / br);
    const int key_tiles = split_key_tiles(shape, d, causal, Nq, Nk);
    int S;
    const char *env = getenv("FA_PREFILL_SPLIT");
    if (env != nullptr && env[0] != '\0') {
        S = atoi(env);  // 0 or 1: never split; n: n chunks (at most one tile each)
        if (S < 2) return 1;
        S = S < key_tiles ? S : key_tiles;
    } else {
        // Split only when the grid cannot give every CU two workgroups and
        // the key loop is long enough to pay for the fixed cost of a chunk
        // and of the combine launch (about 6 us together): 64 tiles while
        // at most half the CUs have a workgroup (below that the key loop is
        // split over the waves of each workgroup instead, which needs no
        // second launch: prefill_small_grid_shape), 256 tiles beyond that,
        // where the chunks must share CUs.  Keep at least 8 tiles per chunk.
        constexpr long long kTargetGrid = 512;
        const int min_tiles = grid <= 128 ? 64 : 256;
        if (grid >= kTargetGrid || key_tiles < min_tiles) return 1;
        S = (int)((kTargetGrid + grid - 1) / grid);
        const int by_len = key_tiles / 8;
        S = S < by_len ? S : by_len;
        S = S < 64 ? S : 64;
    }
    return prefill_split_normalise(d, causal, shape, Nq, Nk, S);
}

int prefill_split_normalise(int d, bool causal, int shape, int Nq, int Nk, int S) {
    const int key_tiles = split_key_tiles(shape, d, causal, Nq, Nk);
    S = S < key_tiles ? S : key_tiles;
    if (S < 2) return 1;
    // whole tiles per chunk; drop chunks that would start past the keys
    const int chunk_tiles = (key_tiles + S - 1) / S;
    return (key_tiles + chunk_tiles - 1) / chunk_tiles;
}

hipError_t launch_prefill_split(int dtype, int d, bool causal, int shape, const void *q, const void *k,
                                const void *v, void *out, float *lse, int BH, int Nq, int Nk, float scale_log2,
                                int S, void *workspace, hipStream_t stream) {
    const int bc = prefill_block_cols(shape, d);
    const int key_tiles = split_key_tiles(shape, d, causal, Nq, Nk);
    if (S < 2 || S > key_tiles) return hipErrorInvalidValue;
    PrefillArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.BH = BH;
    a.Nq = Nq;
    a.Nk = Nk;
    set_scale(a, scale_log2);
    a.S = S;
    a.chunk = (key_tiles + S - 1) / S * bc;
    a.ws_o = static_cast<float *>(workspace);
    a.ws_lse = a.ws_o + (size_t)BH * Nq * S * d;
    hipError_t err = launch_any(dtype, d, causal, shape, a, false, 0, stream);
    if (err != hipSuccess) return err;
    return launch_combine(dtype, d, a.ws_o, a.ws_lse, out, lse, BH * Nq, S, stream);
}

long long varlen_max_tiles(int S, int total_q, int block_rows) {
    // sum_s ceil(len_s / Br) <= total_q / Br + S
    return ((long long)total_q + block_rows - 1) / block_rows + S;
}

hipError_t launch_prefill(int dtype, int d, bool causal, int shape, const void *q, const void *k, const void *v,
                          void *out, float *lse, int BH, int Nq, int Nk, float scale_log2, hipStream_t stream) {
    PrefillArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.BH = BH;
    a.Nq = Nq;
    a.Nk = Nk;
    set_scale(a, scale_log2);
    return launch_any(dtype, d, causal, shape, a, false, 0, stream);
}

hipError_t launch_prefill_varlen(int dtype, int d, bool causal, int shape, const void *q, const void *k,
                                 const void *v, void *out, float *lse, const int *cu_q, const int *cu_k, int S,
                                 int H, int total_q, int total_k, float scale_log2, void *workspace,
                                 hipStream_t stream) {
    PrefillArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    set_scale(a, scale_log2);
    a.cu_q = cu_q;
    a.cu_k = cu_k;
    a.sched = static_cast<const int *>(workspace);
    a.H = H;
    a.total_q = total_q;
    a.total_k = total_k;
    return launch_any(dtype, d, causal, shape, a, true, S, stream);
}

}  // namespace fa
