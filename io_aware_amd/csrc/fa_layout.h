// fa_layout.h -- index arithmetic of the prefill kernel, kept free of HIP
// types so that a host program can check it (every LDS write/read pair in
// range, a bijection, and matching the MFMA operand layouts).
//
// Orientation.  The kernel computes the transposed score tile S^T = K Q^T and
// the transposed output O^T = V^T P^T with the 32x32x16 MFMA, so that each
// lane's accumulator registers all belong to one query: for a 32x32 output
// block, lane l holds column n = l % 32 (a query) and rows
//     row(r, g) = 8 * (r / 4) + 4 * g + (r % 4),   r = 0..15, g = l / 32
// (keys for S^T, head dims for O^T).  A row max or a rescale is then a
// per-lane operation plus one exchange between the two lane halves.
//
// MFMA operand convention (A is M x K, B is K x N; 8 elements per lane):
// lane l supplies A[l % 32][kslot(g, s)] and B[kslot(g, s)][l % 32] for
// s = 0..7, with the same kslot function for A and B.  The contraction sums
// over all 16 k, so any kslot assignment that A and B share gives the same
// product; the kernel only relies on that.
//
// Staging.  K and V tiles ([BC keys][D dims] of 2-byte elements, row-major)
// are copied from device memory into LDS by buffer-to-LDS DMA: one
// instruction moves 16 bytes per lane and places lane t's 16 bytes at LDS
// unit (base + t) -- the destination is fixed by the lane, so a layout is
// chosen by picking which source chunk each lane fetches.  LDS unit
// (key, pos) of a tile holds the key's 8-dim chunk pos ^ f(key); the XOR
// swizzles f keep the operand reads free of bank conflicts.
//
// Transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j supplies an address of 4 consecutive 16-bit elements M[j][0..3];
// lane i receives M[4e + i/4][i % 4] for e = 0..3.  Pointing lane j at
// V[k0 + j/4][d0 + 4*(j % 4)] therefore gives lane i the column
// V[k0 .. k0+3][d0 + i]: four consecutive keys of one head dim, which is what
// the A operand of O^T = V^T P^T needs.
#pragma once

#if defined(__HIPCC__)
#define FA_HD __host__ __device__ __forceinline__
#else
#define FA_HD inline
#endif

namespace fa {
namespace layout {

// ---------------------------------------------------------------------------
// Accumulator and P^T layouts
// ---------------------------------------------------------------------------

// Key (within a 32-key block) of S^T register r in lane half g.
FA_HD int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// P^T as the B operand of O^T += V^T P^T: k-step ks2 covers keys
// [16*ks2, 16*ks2 + 16) of the tile; slot s of lane half g holds the key that
// S^T register r = 8*(ks2 % 2) + s of 32-key block ks2 / 2 holds.
FA_HD int pv_key(int ks2, int g, int s) { return 32 * (ks2 >> 1) + acc_row(8 * (ks2 & 1) + s, g); }

// ---------------------------------------------------------------------------
// Swizzles: LDS unit (key, pos) holds 8-dim chunk pos ^ f(key)
//
// Bank model: 64 banks of 4 bytes, 256 bytes served per cycle -- 16 lanes of
// a 16-byte read or 32 lanes of an 8-byte read at a time.  R = 256 / row
// bytes key rows share one 256-byte bank line.
// ---------------------------------------------------------------------------
template <int D>
FA_HD int k_swizzle(int key) {
    // K operand read: 16 lanes = 16 consecutive keys, one chunk column; the
    // XOR puts their 16 chunks at 16 distinct positions of the bank line
    constexpr int CH = D / 8, R = 16 / CH;
    return (key / R) & (CH - 1);
}

template <int D>
FA_HD int v_swizzle(int key) {
    // transposed V read: 32 lanes = 4 consecutive keys x 32 dims (4 chunks);
    // the XOR moves each key's aligned group of 4 chunks to its own quarter
    // of the bank line
    constexpr int CH = D / 8, R = 16 / CH;
    return (4 * ((key / R) & 3)) & (CH - 1);
}

template <int D>
FA_HD int dual_swizzle(int key) {
    // a tile read both ways (the backward's Q, dO and K tiles): row-wise as
    // the K operand (16 consecutive rows, one chunk column) and transposed as
    // the V operand (4 consecutive rows x an aligned group of 4 chunks).  With
    // n = key / R, the low bits of n pick the quarter of the bank line a row's
    // chunk group goes to (4 consecutive rows: 4 quarters), the next bits
    // rotate chunks within the quarter (16 consecutive rows: 16 positions).
    constexpr int CH = D / 8, R = 16 / CH, QC = CH / 4;
    const int n = key / R;
    return (((n % QC) * 4) ^ ((n / QC) & 3)) & (CH - 1);
}

// Byte offset of element (key, dim) of a K or V tile in LDS.
template <int D>
FA_HD int k_elem_offset(int key, int dim) {
    return key * (D * 2) + (((dim >> 3) ^ k_swizzle<D>(key)) << 4) + (dim & 7) * 2;
}
template <int D>
FA_HD int v_elem_offset(int key, int dim) {
    return key * (D * 2) + (((dim >> 3) ^ v_swizzle<D>(key)) << 4) + (dim & 7) * 2;
}

template <int D>
FA_HD int dual_elem_offset(int key, int dim) {
    return key * (D * 2) + (((dim >> 3) ^ dual_swizzle<D>(key)) << 4) + (dim & 7) * 2;
}

// DMA: LDS unit u of a tile (u = 64 * instruction_slot + lane) receives
// source chunk (key, chunk) with key = u / (D/8), chunk = (u % (D/8)) ^ f(key).
// Returned: element offset of that chunk within the tile's rows.
template <int D>
FA_HD int k_dma_src_elem(int u) {
    constexpr int CH = D / 8;
    const int key = u / CH;
    return key * D + (((u % CH) ^ k_swizzle<D>(key)) * 8);
}
template <int D>
FA_HD int v_dma_src_elem(int u) {
    constexpr int CH = D / 8;
    const int key = u / CH;
    return key * D + (((u % CH) ^ v_swizzle<D>(key)) * 8);
}

template <int D>
FA_HD int dual_dma_src_elem(int u) {
    constexpr int CH = D / 8;
    const int key = u / CH;
    return key * D + (((u % CH) ^ dual_swizzle<D>(key)) * 8);
}

// ---------------------------------------------------------------------------
// Operand reads
// ---------------------------------------------------------------------------

// A operand of S^T += K_blk Q^T, k-step ks (dims 16*ks .. 16*ks+15): lane
// (row l32, half g) reads dims [16*ks + 8*g, +8) of key 32*kb + l32 as one
// 16-byte chunk.
template <int D>
FA_HD int k_operand_offset(int kb, int l32, int g, int ks) {
    return k_elem_offset<D>(32 * kb + l32, 16 * ks + 8 * g);
}

// A operand of O^T += V^T P^T for dim block db, k-step ks2 and slot half sh
// (slots 4*sh .. 4*sh+3 = keys 16*ks2 + 8*sh + 4*g + 0..3): the address lane
// (group G = lane / 16, j = lane % 16) hands to the transposed read.  Lane
// half g = G / 2; dims 32*db + 16*(G % 2) + [0, 16) are the group's columns.
template <int D>
FA_HD int v_operand_tr_offset(int db, int lane, int ks2, int sh) {
    const int G = lane >> 4, j = lane & 15;
    const int key = 16 * ks2 + 8 * sh + 4 * (G >> 1) + (j >> 2);
    const int dim = 32 * db + 16 * (G & 1) + 4 * (j & 3);
    return v_elem_offset<D>(key, dim);
}

// The same two reads on a dual-swizzled tile (rows are keys of a K tile, or
// queries of a Q or dO tile).
template <int D>
FA_HD int dual_row_operand_offset(int kb, int l32, int g, int ks) {
    return dual_elem_offset<D>(32 * kb + l32, 16 * ks + 8 * g);
}
template <int D>
FA_HD int dual_tr_operand_offset(int db, int lane, int ks2, int sh) {
    const int G = lane >> 4, j = lane & 15;
    const int key = 16 * ks2 + 8 * sh + 4 * (G >> 1) + (j >> 2);
    const int dim = 32 * db + 16 * (G & 1) + 4 * (j & 3);
    return dual_elem_offset<D>(key, dim);
}

// Model of the transposed read for host checks: the (address owner lane,
// element) that lane i's element e comes from, within its 16-lane group.
FA_HD int tr_src_lane(int i, int e) { return 4 * e + (i >> 2); }
FA_HD int tr_src_elem(int i) { return i & 3; }

// ---------------------------------------------------------------------------
// Workgroup order.  Workgroup wg of nwg = BH * Tr goes to XCD wg % 8 in
// dispatch order, and each XCD starts its workgroups in the order of wg / 8
// as CUs free up (list scheduling).  The map hands each XCD whole heads, so
// the K/V of a head are read through one XCD's L2, and orders the work of an
// XCD so that list scheduling balances it.
//  * Causal, BH a multiple of 8 (XCD x owns heads [x*BH/8, (x+1)*BH/8)):
//    Q blocks have different lengths (block i sees keys up to its last row),
//    and a long block started late leaves a tail.  Two phases: first the
//    blocks of the longest three quarters (i >= Tr/4), then the short ones
//    (i < Tr/4); in each phase the XCD's heads go four at a time, the four
//    heads' blocks interleaved, longest first.  Four heads' K/V are in use at
//    a time; the second phase re-reads only the first quarter of each head's
//    keys.  (Two heads at a time in one phase left the long blocks of the
//    last pairs to the end: 5.5% slower on causal B8 H16 N4096.)
//  * Otherwise (and when nwg is a multiple of 8, XCD x receives the work
//    range [x*nwg/8, (x+1)*nwg/8)): without the mask, one head at a time, so
//    that the blocks running at once on an XCD stream the same K/V through
//    its L2; under the mask (BH not a multiple of 8), heads two at a time,
//    alternating between the pair, each head's Q blocks last-first.
// The map is a bijection of [0, nwg) onto (bh, qblock) pairs; under the
// mask, qblock is the block's position in longest-first order (Tr - 1 is
// the longest for a forward Q block).
// ---------------------------------------------------------------------------
FA_HD void map_workgroup(int wg, int BH, int Tr, bool causal, int &bh, int &qblock) {
    const int nwg = BH * Tr;
    if (causal && (BH & 7) == 0) {
        const int hpx = BH >> 3;            // heads per XCD
        const int x = wg & 7, w = wg >> 3;  // XCD, position in its order
        int gh = hpx < 4 ? hpx : 4;         // heads per group: 4, or a divisor of hpx
        while (hpx % gh) --gh;
        const int split = Tr / 4;           // phase 1: blocks [split, Tr); phase 2: [0, split)
        const int n1 = (Tr - split) * hpx;
        const int lo = w < n1 ? split : 0, hi = w < n1 ? Tr : split;
        const int rem = w < n1 ? w : w - n1;
        const int per_group = (hi - lo) * gh;
        const int grp = rem / per_group, idx = rem - grp * per_group;
        bh = x * hpx + grp * gh + idx % gh;
        qblock = hi - 1 - idx / gh;
        return;
    }
    int work = wg;
    if ((nwg & 7) == 0) {
        const int per_xcd = nwg >> 3;
        work = (wg & 7) * per_xcd + (wg >> 3);
    }
    if (!causal) {  // equal blocks: one head at a time, its blocks sharing its K/V in L2
        bh = work / Tr;
        qblock = work - bh * Tr;
        return;
    }
    const int pair = work / (2 * Tr);
    const int within = work - pair * 2 * Tr;
    int r;
    if (2 * pair + 1 < BH) {  // a full pair of heads: alternate between them
        bh = 2 * pair + (within & 1);
        r = within >> 1;
    } else {                  // the last head of an odd count
        bh = 2 * pair;
        r = within;
    }
    qblock = causal ? (Tr - 1 - r) : r;
}

// ---------------------------------------------------------------------------
// Packed variable-length batches: sequence s covers rows [cu[s], cu[s+1]) of
// a tensor with ``total`` rows.  The offsets are clamped into [0, total] and
// made non-decreasing, so inconsistent offsets give empty or shortened
// sequences, never an access outside the tensor.
// ---------------------------------------------------------------------------
FA_HD void varlen_bounds(const int *cu, int s, int total, int &begin, int &end) {
    int b = cu[s], e = cu[s + 1];
    b = b < 0 ? 0 : (b > total ? total : b);
    e = e < b ? b : (e > total ? total : e);
    begin = b;
    end = e;
}

}  // namespace layout
}  // namespace fa
