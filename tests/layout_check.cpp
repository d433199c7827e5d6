// layout_check.cpp -- host check of the prefill kernel's index arithmetic
// (io_aware_amd/csrc/fa_layout.h), built with g++ by tests/test_layout.py.
//
// For each tile shape it proves, by enumeration, that
//  * the K-tile staging writes cover the LDS tile exactly once, in range;
//  * every S^T = K Q^T operand read returns the K element the MFMA lane
//    contract needs (key 32*kb + l32, dims 16*ks + 8*g .. +7);
//  * the transposed V staging writes cover the V^T tile exactly once;
//  * every O^T = V^T P^T operand read returns V[key][dim] for the key that
//    the matching P^T slot holds (the S^T accumulator register it came from);
//  * the accumulator row map and the P^T key map are bijections;
//  * the workgroup order is a bijection onto (head, Q block) pairs.
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

template <int D, int BC>
void check_tile() {
    constexpr int CH = D / 8;
    constexpr int TILE = BC * D * 2;

    // K staging: (key, chunk) -> 16-byte unit
    std::vector<int> kown(TILE / 16, -1);
    for (int key = 0; key < BC; ++key)
        for (int ch = 0; ch < CH; ++ch) {
            const int off = k_lds_offset<D>(key, ch);
            CHECK(off >= 0 && off + 16 <= TILE && off % 16 == 0, "K write out of range D=%d BC=%d", D, BC);
            if (off < 0 || off + 16 > TILE) continue;
            CHECK(kown[off / 16] == -1, "K unit written twice D=%d BC=%d", D, BC);
            kown[off / 16] = key * CH + ch;
        }
    for (int kb = 0; kb < BC / 32; ++kb)
        for (int l32 = 0; l32 < 32; ++l32)
            for (int g = 0; g < 2; ++g)
                for (int ks = 0; ks < D / 16; ++ks) {
                    const int off = k_operand_offset<D>(kb, l32, g, ks);
                    CHECK(off >= 0 && off + 16 <= TILE, "K read out of range");
                    if (off < 0 || off + 16 > TILE) continue;
                    CHECK(kown[off / 16] == (32 * kb + l32) * CH + (2 * ks + g), "K read fetches the wrong chunk");
                }

    // V^T staging: element (key, dim) -> byte
    std::vector<int> vown(TILE / 2, -1);
    for (int u = 0; u < BC / 4; ++u)
        for (int dc = 0; dc < CH; ++dc)
            for (int e = 0; e < 8; ++e) {
                const int dim = 8 * dc + e;
                const int off = vt_lds_offset<BC>(dim, vt_slot_of_group(u));
                CHECK(off >= 0 && off + 8 <= TILE && off % 8 == 0, "V write out of range D=%d BC=%d", D, BC);
                if (off < 0 || off + 8 > TILE) continue;
                for (int j = 0; j < 4; ++j) {
                    const int el = (off + 2 * j) / 2;
                    CHECK(vown[el] == -1, "V element written twice");
                    vown[el] = (4 * u + j) * D + dim;
                }
            }
    for (int i = 0; i < TILE / 2; ++i) CHECK(vown[i] != -1, "V^T tile has a hole");
    for (int db = 0; db < D / 32; ++db)
        for (int l32 = 0; l32 < 32; ++l32)
            for (int g = 0; g < 2; ++g)
                for (int ks2 = 0; ks2 < BC / 16; ++ks2)
                    for (int s = 0; s < 8; ++s) {
                        const int off = v_operand_offset<BC>(db, l32, g, ks2, s >> 2) + 2 * (s & 3);
                        CHECK(off >= 0 && off + 2 <= TILE, "V read out of range");
                        if (off < 0 || off + 2 > TILE) continue;
                        const int want = pv_key(ks2, g, s) * D + (32 * db + l32);
                        CHECK(vown[off / 2] == want, "V read fetches the wrong element D=%d BC=%d", D, BC);
                    }
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
    check_maps();
    check_workgroups();
    if (g_fail) return 1;
    std::printf("OK\n");
    return 0;
}
