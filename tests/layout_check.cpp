// layout_check.cpp -- host check of the prefill kernel's index arithmetic
// (io_aware_amd/csrc/fa_layout.h), built with g++ by tests/test_layout.py.
//
// For each tile shape it proves, by enumeration, that
//  * the DMA staging of a K or V tile places every source element exactly
//    once, inside the tile, and where k_elem_offset / v_elem_offset say;
//  * every S^T = K Q^T operand read returns the K elements the MFMA lane
//    contract needs (key 32*kb + l32, dims 16*ks + 8*g .. +7);
//  * every O^T = V^T P^T operand, gathered by the modelled transposed read
//    (lane i of a 16-lane group receives element i%4 of the row that lane
//    4e + i/4 addressed), equals V[key][dim] for the key that the matching
//    P^T slot holds (the S^T accumulator register it came from);
//  * the accumulator row map and the P^T key map are bijections;
//  * the workgroup order is a bijection onto (head, Q block) pairs.
// It also checks that the operand reads are free of LDS bank conflicts under
// a 64-bank, 256-bytes-per-cycle model (d = 64 and 128).
// Exit status 0 and "OK" on success; a message and status 1 otherwise.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "fa_layout.h"

using namespace fa::layout;

static int g_fail = 0;
#define CHECK(cond, ...)                       \
    do {                                       \
        if (!(cond)) {                         \
            std::printf("FAIL: " __VA_ARGS__); \
            std::printf("\n");                 \
            if (++g_fail > 20) std::exit(1);   \
        }                                      \
    } while (0)

// LDS element map after DMA: element index (byte / 2) -> source element key*D + dim
// kind: 0 = K swizzle, 1 = V swizzle, 2 = dual swizzle
template <int D> int src_of(int kind, int u) {
    return kind == 0 ? k_dma_src_elem<D>(u) : kind == 1 ? v_dma_src_elem<D>(u) : dual_dma_src_elem<D>(u);
}
template <int D> int off_of(int kind, int key, int dim) {
    return kind == 0 ? k_elem_offset<D>(key, dim) : kind == 1 ? v_elem_offset<D>(key, dim) : dual_elem_offset<D>(key, dim);
}

template <int D, int BC, int KIND>
std::vector<int> dma_tile() {
    constexpr int CH = D / 8;
    constexpr int TILE = BC * D * 2;
    std::vector<int> lds(TILE / 2, -1), seen(BC * D, 0);
    for (int u = 0; u < BC * CH; ++u) {
        const int src = src_of<D>(KIND, u);
        CHECK(src >= 0 && src + 8 <= BC * D && src % 8 == 0, "DMA source chunk out of the tile");
        if (src < 0 || src + 8 > BC * D) continue;
        for (int e = 0; e < 8; ++e) {
            lds[(16 * u + 2 * e) / 2] = src + e;
            seen[src + e]++;
        }
    }
    for (int i = 0; i < BC * D; ++i) CHECK(seen[i] == 1, "DMA does not place every element exactly once");
    for (int key = 0; key < BC; ++key)
        for (int dim = 0; dim < D; ++dim) {
            const int off = off_of<D>(KIND, key, dim);
            CHECK(off >= 0 && off + 2 <= TILE, "element offset out of the tile");
            if (off >= 0 && off + 2 <= TILE) CHECK(lds[off / 2] == key * D + dim, "element offset disagrees with DMA");
        }
    return lds;
}

// banks: 64 x 4 bytes; conflict degree of a set of (lane, byte range) accesses
int bank_degree(const std::vector<std::pair<int, int>> &acc) {
    std::vector<std::vector<int>> words(64);
    for (auto &a : acc)
        for (int b = a.first; b < a.first + a.second; b += 4) {
            const int word = b / 4, bank = word % 64;
            bool found = false;
            for (int w : words[bank]) found |= (w == word);
            if (!found) words[bank].push_back(word);
        }
    int deg = 0;
    for (auto &w : words) deg = deg > (int)w.size() ? deg : (int)w.size();
    return deg;
}

template <int D, int BC>
void check_tile() {
    constexpr int TILE = BC * D * 2;
    std::vector<int> klds = dma_tile<D, BC, 0>();
    std::vector<int> vlds = dma_tile<D, BC, 1>();
    int kdeg = 0, vdeg = 0;

    for (int kb = 0; kb < BC / 32; ++kb)
        for (int ks = 0; ks < D / 16; ++ks) {
            std::vector<std::pair<int, int>> phase;
            for (int lane = 0; lane < 64; ++lane) {
                const int l32 = lane & 31, g = lane >> 5;
                const int off = k_operand_offset<D>(kb, l32, g, ks);
                CHECK(off >= 0 && off + 16 <= TILE && off % 16 == 0, "K read out of range or misaligned");
                if (off < 0 || off + 16 > TILE) continue;
                for (int e = 0; e < 8; ++e)
                    CHECK(klds[off / 2 + e] == (32 * kb + l32) * D + 16 * ks + 8 * g + e,
                          "K operand fetches the wrong element D=%d", D);
                phase.push_back({off, 16});
                if (phase.size() == 16) {  // 16-byte reads: 16 lanes per 256-byte cycle
                    int d = bank_degree(phase);
                    kdeg = kdeg > d ? kdeg : d;
                    phase.clear();
                }
            }
        }

    for (int db = 0; db < D / 32; ++db)
        for (int ks2 = 0; ks2 < BC / 16; ++ks2)
            for (int sh = 0; sh < 2; ++sh)
                for (int G = 0; G < 4; ++G) {
                    int addr[16];
                    std::vector<std::pair<int, int>> phase;   // 8-byte reads: 32 lanes per 256-byte cycle
                    for (int j = 0; j < 32; ++j) {
                        const int a32 = v_operand_tr_offset<D>(db, 16 * (G & 2) + j, ks2, sh);
                        phase.push_back({a32, 8});
                    }
                    int d = bank_degree(phase);
                    vdeg = vdeg > d ? vdeg : d;
                    for (int j = 0; j < 16; ++j) {
                        addr[j] = v_operand_tr_offset<D>(db, 16 * G + j, ks2, sh);
                        CHECK(addr[j] >= 0 && addr[j] + 8 <= TILE && addr[j] % 8 == 0,
                              "V transposed read out of range or misaligned");
                    }
                    for (int i = 0; i < 16; ++i)
                        for (int e = 0; e < 4; ++e) {
                            const int a = addr[tr_src_lane(i, e)];
                            if (a < 0 || a + 8 > TILE) continue;
                            const int got = vlds[a / 2 + tr_src_elem(i)];
                            const int lane = 16 * G + i, g = lane >> 5, l32 = lane & 31;
                            const int want = pv_key(ks2, g, 4 * sh + e) * D + (32 * db + l32);
                            CHECK(got == want, "V operand fetches the wrong element D=%d BC=%d", D, BC);
                        }
                }
    // the kernel hoists the lane-dependent part of each operand address out of
    // the tile loop and adds the block / k-step part as a constant
    for (int lane = 0; lane < 64; ++lane) {
        const int l32 = lane & 31, g = lane >> 5;
        for (int kb = 0; kb < BC / 32; ++kb)
            for (int ks = 0; ks < D / 16; ++ks)
                CHECK(k_operand_offset<D>(kb, l32, g, ks) == k_operand_offset<D>(0, l32, g, ks) + 32 * kb * D * 2,
                      "K operand offset is not lane part + block constant");
        for (int db = 0; db < D / 32; ++db)
            for (int ks2 = 0; ks2 < BC / 16; ++ks2)
                for (int sh = 0; sh < 2; ++sh)
                    CHECK(v_operand_tr_offset<D>(db, lane, ks2, sh) ==
                              v_operand_tr_offset<D>(db, lane, 0, 0) + (16 * ks2 + 8 * sh) * D * 2,
                          "V operand offset is not lane part + k-step constant");
    }
    std::printf("D=%3d BC=%3d: K-operand bank conflict degree %d, V-operand %d\n", D, BC, kdeg, vdeg);
    if (D >= 64) CHECK(kdeg == 1 && vdeg == 1, "operand reads conflict under the 64-bank model D=%d BC=%d", D, BC);
}

// A dual-swizzled tile: both the row read and the transposed read fetch the
// right elements and are conflict-free (every d).
template <int D, int BC>
void check_dual_tile() {
    constexpr int TILE = BC * D * 2;
    std::vector<int> lds = dma_tile<D, BC, 2>();
    int rdeg = 0, tdeg = 0;
    for (int kb = 0; kb < BC / 32; ++kb)
        for (int ks = 0; ks < D / 16; ++ks) {
            std::vector<std::pair<int, int>> phase;
            for (int lane = 0; lane < 64; ++lane) {
                const int l32 = lane & 31, g = lane >> 5;
                const int off = dual_row_operand_offset<D>(kb, l32, g, ks);
                CHECK(off >= 0 && off + 16 <= TILE && off % 16 == 0, "dual row read out of range");
                if (off < 0 || off + 16 > TILE) continue;
                for (int e = 0; e < 8; ++e)
                    CHECK(lds[off / 2 + e] == (32 * kb + l32) * D + 16 * ks + 8 * g + e, "dual row read wrong D=%d", D);
                CHECK(off == dual_row_operand_offset<D>(0, l32, g, ks) + 32 * kb * D * 2, "dual row offset not lane + const");
                phase.push_back({off, 16});
                if (phase.size() == 16) {
                    int d = bank_degree(phase);
                    rdeg = rdeg > d ? rdeg : d;
                    phase.clear();
                }
            }
        }
    for (int db = 0; db < D / 32; ++db)
        for (int ks2 = 0; ks2 < BC / 16; ++ks2)
            for (int sh = 0; sh < 2; ++sh)
                for (int G = 0; G < 4; ++G) {
                    int addr[16];
                    std::vector<std::pair<int, int>> phase;
                    for (int j = 0; j < 32; ++j) phase.push_back({dual_tr_operand_offset<D>(db, 16 * (G & 2) + j, ks2, sh), 8});
                    int d = bank_degree(phase);
                    tdeg = tdeg > d ? tdeg : d;
                    for (int j = 0; j < 16; ++j) {
                        addr[j] = dual_tr_operand_offset<D>(db, 16 * G + j, ks2, sh);
                        CHECK(addr[j] >= 0 && addr[j] + 8 <= TILE && addr[j] % 8 == 0, "dual tr read out of range");
                        // the slot half changes the swizzle: one lane part per (db, sh), k-steps add a constant
                        CHECK(addr[j] == dual_tr_operand_offset<D>(db, 16 * G + j, 0, sh) + 16 * ks2 * D * 2,
                              "dual tr offset not lane + const");
                    }
                    for (int i = 0; i < 16; ++i)
                        for (int e = 0; e < 4; ++e) {
                            const int a = addr[tr_src_lane(i, e)];
                            if (a < 0 || a + 8 > TILE) continue;
                            const int got = lds[a / 2 + tr_src_elem(i)];
                            const int lane = 16 * G + i, g = lane >> 5, l32 = lane & 31;
                            const int want = pv_key(ks2, g, 4 * sh + e) * D + (32 * db + l32);
                            CHECK(got == want, "dual tr read wrong D=%d BC=%d", D, BC);
                        }
                }
    std::printf("D=%3d BC=%3d: dual tile row-read conflict degree %d, transposed-read %d\n", D, BC, rdeg, tdeg);
    CHECK(rdeg == 1 && tdeg == 1, "dual tile reads conflict D=%d BC=%d", D, BC);
}

void check_maps() {
    std::vector<int> seen(32, 0);
    for (int r = 0; r < 16; ++r)
        for (int g = 0; g < 2; ++g) {
            const int row = acc_row(r, g);
            CHECK(row >= 0 && row < 32, "acc_row out of range");
            if (row >= 0 && row < 32) seen[row]++;
        }
    for (int i = 0; i < 32; ++i) CHECK(seen[i] == 1, "acc_row not a bijection");
    for (int ks2 = 0; ks2 < 8; ++ks2) {
        std::vector<int> cnt(16, 0);
        for (int g = 0; g < 2; ++g)
            for (int s = 0; s < 8; ++s) {
                const int key = pv_key(ks2, g, s) - 16 * ks2;
                CHECK(key >= 0 && key < 16, "pv_key outside its k-step");
                if (key >= 0 && key < 16) cnt[key]++;
            }
        for (int i = 0; i < 16; ++i) CHECK(cnt[i] == 1, "pv_key not a bijection");
    }
    // the transposed-read model is a bijection of the 16 x 4 block
    std::vector<int> hit(64, 0);
    for (int i = 0; i < 16; ++i)
        for (int e = 0; e < 4; ++e) hit[4 * tr_src_lane(i, e) + tr_src_elem(i)]++;
    for (int i = 0; i < 64; ++i) CHECK(hit[i] == 1, "transposed-read model not a bijection");
}

void check_workgroups() {
    const int shapes[][2] = {{1, 1}, {1, 2}, {16, 8}, {128, 32}, {32, 128}, {3, 5}, {7, 9}, {512, 1}, {2, 4}};
    for (auto &sh : shapes)
        for (int causal = 0; causal < 2; ++causal) {
            const int BH = sh[0], Tr = sh[1];
            std::vector<int> seen(BH * Tr, 0);
            for (int wg = 0; wg < BH * Tr; ++wg) {
                int bh = -1, qb = -1;
                map_workgroup(wg, BH, Tr, causal != 0, bh, qb);
                CHECK(bh >= 0 && bh < BH && qb >= 0 && qb < Tr, "map_workgroup out of range");
                if (bh >= 0 && bh < BH && qb >= 0 && qb < Tr) seen[bh * Tr + qb]++;
            }
            for (int i = 0; i < BH * Tr; ++i) CHECK(seen[i] == 1, "map_workgroup not a bijection BH=%d Tr=%d", BH, Tr);
        }
}

int main() {
    check_tile<32, 64>();
    check_tile<64, 64>();
    check_tile<128, 64>();
    check_tile<128, 32>();
    check_tile<128, 128>();
    check_dual_tile<32, 64>();
    check_dual_tile<64, 32>();
    check_dual_tile<64, 64>();
    check_dual_tile<128, 32>();
    check_dual_tile<128, 64>();
    check_maps();
    check_workgroups();
    if (g_fail) return 1;
    std::printf("OK\n");
    return 0;
}
