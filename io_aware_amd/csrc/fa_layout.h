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
#pragma once

#if defined(__HIPCC__)
#define FA_HD __host__ __device__ __forceinline__
#else
#define FA_HD inline
#endif

namespace fa {
namespace layout {

// ---------------------------------------------------------------------------
// S^T accumulator: key (within the 32-key block) of register r in lane half g
// ---------------------------------------------------------------------------
FA_HD int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// P^T as the B operand of O^T += V^T P^T: k-step ks2 covers keys
// [16*ks2, 16*ks2 + 16) of the tile; slot s of lane half g holds the key that
// S^T register r = 8*(ks2 % 2) + s of 32-key block ks2 / 2 holds.
FA_HD int pv_key(int ks2, int g, int s) {
    return 32 * (ks2 >> 1) + acc_row(8 * (ks2 & 1) + s, g);
}

// ---------------------------------------------------------------------------
// K tile in LDS: row-major [BC keys][D dims] of 2-byte elements, 16-byte
// chunks (8 dims) XOR-swizzled by the key so that the 32 lanes reading one
// chunk column of 32 consecutive keys spread over all banks.
// ---------------------------------------------------------------------------
template <int D>
FA_HD int k_lds_offset(int key, int chunk) {
    constexpr int CH = D / 8;  // 16-byte chunks per key row
    return key * (D * 2) + ((chunk ^ (key & (CH - 1))) * 16);
}

// A operand of S^T += K_blk Q^T for k-step ks (dims 16*ks .. 16*ks+15): lane
// (row l32, half g) reads the 8 dims [16*ks + 8*g, 16*ks + 8*g + 8) of key
// 32*kb + l32 as one 16-byte chunk.
template <int D>
FA_HD int k_operand_offset(int kb, int l32, int g, int ks) {
    return k_lds_offset<D>(32 * kb + l32, 2 * ks + g);
}

// ---------------------------------------------------------------------------
// V tile in LDS, transposed: [D dims][BC keys] of 2-byte elements.  Each dim
// row is cut into 8-byte slots of 4 consecutive keys.  Within every 16 keys
// the slots are ordered (keys 0-3, 8-11, 4-7, 12-15) so that the 8 keys one
// lane half needs for a P^T k-step sit in two adjacent slots; the slot index
// is XOR-swizzled by f(dim) = dim ^ (dim >> 3) so that both the writers
// (8 dims apart) and the readers (consecutive dims) avoid bank conflicts.
// ---------------------------------------------------------------------------
FA_HD int vt_slot_of_group(int u) {           // u: 4-key group, keys 4u..4u+3
    const int u4 = u & 3;
    return 4 * (u >> 2) + (((u4 & 1) << 1) | (u4 >> 1));
}

template <int BC>
FA_HD int vt_lds_offset(int dim, int slot) {
    constexpr int NSLOT = BC / 4;
    return dim * (BC * 2) + ((slot ^ ((dim ^ (dim >> 3)) & (NSLOT - 1))) * 8);
}

// A operand of O^T += V^T P^T for dim block db and k-step ks2: lane
// (dim 32*db + l32, half g) reads slot 4*ks2 + 2*g (keys 16*ks2 + 4g + 0..3)
// and slot 4*ks2 + 2*g + 1 (keys 16*ks2 + 8 + 4g + 0..3).
template <int BC>
FA_HD int v_operand_offset(int db, int l32, int g, int ks2, int half) {
    return vt_lds_offset<BC>(32 * db + l32, 4 * ks2 + 2 * g + half);
}

// ---------------------------------------------------------------------------
// Workgroup order.  Workgroup wg of nwg = BH * Tr goes to XCD wg % 8 in
// dispatch order.  When nwg is a multiple of 8, XCD x receives the
// contiguous work range [x * nwg/8, (x+1) * nwg/8), i.e. whole heads, so the
// K/V of a head are read through one XCD's L2.  Within a head the Q blocks
// run last-first under the causal mask (the last block does the most work).
// The map is a bijection of [0, nwg) onto (bh, qblock) pairs.
// ---------------------------------------------------------------------------
FA_HD void map_workgroup(int wg, int BH, int Tr, bool causal, int &bh, int &qblock) {
    const int nwg = BH * Tr;
    int work = wg;
    if ((nwg & 7) == 0) {
        const int per_xcd = nwg >> 3;
        work = (wg & 7) * per_xcd + (wg >> 3);
    }
    bh = work / Tr;
    const int r = work - bh * Tr;
    qblock = causal ? (Tr - 1 - r) : r;
}

}  // namespace layout
}  // namespace fa
