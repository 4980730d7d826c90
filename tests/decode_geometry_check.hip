// CPU check of the decode kernels' launch plan and global-memory index
// arithmetic (built for the host only; run by tests/test_geometry.py).
//
// For every shape and head map it enumerates, per workgroup and lane, each
// global address the decode and combine kernels form (Q rows, K/V rows of
// every tile including the prefetch of the last one, K scale indices, partial
// result rows, O and lse rows, the Q scale output) and checks them against the
// buffer sizes; it also checks that every (q-head, query row) is owned by
// exactly one valid slot and that the key splits tile the cache exactly.
// Exit status 0 = clean.
#include "decode_geometry.h"

#include <cstdio>
#include <vector>

using namespace attn::dec;

static long g_errors = 0;
#define REQUIRE(cond, ...)                                                \
    do {                                                                  \
        if (!(cond)) {                                                    \
            if (g_errors < 20) {                                          \
                std::printf("FAIL %s:%d: %s | ", __FILE__, __LINE__, #cond); \
                std::printf(__VA_ARGS__);                                 \
                std::printf("\n");                                        \
            }                                                             \
            ++g_errors;                                                   \
        }                                                                 \
    } while (0)

static void check(int B, int Hq, int Hkv, int Sq, int Sk, int D, const std::vector<int>& kvmap) {
    // group tables as the host builds them
    std::vector<int> horder, gstart(Hkv), gcount(Hkv);
    int max_group = 0;
    for (int k = 0; k < Hkv; ++k) {
        gstart[k] = static_cast<int>(horder.size());
        for (int h = 0; h < Hq; ++h)
            if (kvmap[h] == k) horder.push_back(h);
        gcount[k] = static_cast<int>(horder.size()) - gstart[k];
        if (gcount[k] > max_group) max_group = gcount[k];
    }
    const Plan p = make_plan(B, Hkv, Sq, Sk, max_group);
    REQUIRE(p.hpc >= 1 && p.hpc * Sq <= kSlots, "hpc %d Sq %d", p.hpc, Sq);
    REQUIRE(p.nsplit >= 1 && p.tps >= 1, "nsplit %d tps %d", p.nsplit, p.tps);
    // splits tile [0, ntiles) exactly, none empty
    int covered = 0;
    for (int s = 0; s < p.nsplit; ++s) {
        const int t0 = split_first_tile(s, p.tps), t1 = split_end_tile(s, p.tps, p.ntiles);
        REQUIRE(t0 == covered && t1 > t0, "split %d [%d,%d) covered %d", s, t0, t1, covered);
        covered = t1;
    }
    REQUIRE(covered == p.ntiles, "covered %d of %d tiles", covered, p.ntiles);

    const size_t q_bytes = static_cast<size_t>(B) * Hq * Sq * D * 2;
    const size_t rows_total = partial_rows(B, Hkv, p);
    const int nkblk = (Sk + 63) / 64;
    std::vector<int> owner(static_cast<size_t>(B) * Hq * Sq, 0), written(owner.size(), 0);
    for (int elt = 0; elt < 2; ++elt) {   // INT8 (1-byte K) and FP16 (2-byte K)
        const int kelt = elt ? 2 : 1;
        const size_t kv_k_bytes = static_cast<size_t>(B) * Hkv * Sk * D * kelt;
        const size_t kv_v_bytes = static_cast<size_t>(B) * Hkv * Sk * D * 2;
        const int qsteps = elt ? D / 16 : D / 32;
        const int vcpr = 2 * D / 16, vpt = kTile * vcpr / kThreads;
        for (int bkv = 0; bkv < B * Hkv; ++bkv) {
            const int b = bkv / Hkv, kvh = bkv % Hkv;
            for (int chunk = 0; chunk < p.nchunk; ++chunk)
                for (int split = 0; split < p.nsplit; ++split)
                    for (int lane = 0; lane < kThreads; ++lane) {
                        if (!chunk_has_work(chunk, p.hpc, gcount[kvh])) continue;   // the kernel returns
                        const int n = lane & 31, g = lane >> 5;
                        const Slot sl = slot_of(n, chunk, p.hpc, Sq, gcount[kvh]);
                        REQUIRE(sl.hh >= 0 && sl.hh < gcount[kvh] && sl.i >= 0 && sl.i < Sq,
                                "slot hh %d i %d", sl.hh, sl.i);
                        const int h = horder[gstart[kvh] + sl.hh];
                        const size_t qrow = (static_cast<size_t>(b) * Hq + h) * Sq + sl.i;
                        for (int s = 0; s < D / 32; ++s)
                            for (int hf = 0; hf < 2; ++hf) {
                                const size_t off = qrow * D * 2 + (s * 32 + g * 16 + hf * 8) * 2;
                                REQUIRE(off + 16 <= q_bytes, "q byte %zu", off);
                            }
                        const int first = head_first_slot(n, Sq);
                        if (sl.valid)
                            REQUIRE(first + Sq <= kSlots && first <= n && n < first + Sq, "rowmax %d", first);
                        if (elt == 0 && split == 0 && g == 0 && sl.valid) owner[qrow] += 1;
                        const int t0 = split_first_tile(split, p.tps), t1 = split_end_tile(split, p.tps, p.ntiles);
                        std::vector<int> tiles{t0};
                        for (int t = t0; t < t1; ++t) tiles.push_back(prefetch_tile(t, t1));
                        for (int t : tiles) {
                            REQUIRE(t >= t0 && t < t1, "tile %d of [%d,%d)", t, t0, t1);
                            const int krow = key_row(t * kTile, n, Sk);
                            REQUIRE(krow >= 0 && krow < Sk, "k row %d", krow);
                            for (int s = 0; s < qsteps; ++s) {
                                const int fo = elt ? (s * 16 + g * 8) * 2 : (s * 32 + g * 16);
                                const size_t off = (static_cast<size_t>(bkv) * Sk + krow) * D * kelt + fo;
                                REQUIRE(fo + 16 <= D * kelt && off + 16 <= kv_k_bytes, "k byte %zu", off);
                            }
                            for (int i = 0; i < vpt; ++i) {
                                const int c = lane + kThreads * i;
                                const int vrow = key_row(t * kTile, c / vcpr, Sk);
                                REQUIRE(c / vcpr < kTile, "v tile row %d", c / vcpr);
                                const size_t off = (static_cast<size_t>(bkv) * Sk + vrow) * D * 2 + (c % vcpr) * 16;
                                REQUIRE(vrow >= 0 && vrow < Sk && off + 16 <= kv_v_bytes, "v byte %zu", off);
                            }
                            if (t * kTile < Sk) REQUIRE(((t * kTile) >> 6) < nkblk, "k scale block %d", (t * kTile) >> 6);
                        }
                        if (sl.valid) {
                            const size_t row = partial_row(bkv, chunk, split, n, p);
                            REQUIRE(row < rows_total, "partial row %zu of %zu", row, rows_total);
                            for (int dt = 0; dt < D / 32; ++dt)
                                for (int j4 = 0; j4 < 4; ++j4) {
                                    const int col = dt * 32 + j4 * 8 + g * 4;
                                    REQUIRE(col + 4 <= D, "partial col %d", col);
                                }
                            REQUIRE(static_cast<size_t>(b) * Hq + h < static_cast<size_t>(B) * Hq, "q scale out");
                        }
                    }
            // combine kernel: D/4 threads per slot, 256/(D/4) slots per block,
            // blocks over the first hpc*Sq slots
            const int cg = D / 4, rpb = 256 / cg;
            const int nblk = cdiv(imin(kSlots, p.hpc * Sq), rpb);
            for (int chunk = 0; chunk < p.nchunk; ++chunk)
                for (int bx = 0; bx < nblk; ++bx)
                    for (int tid = 0; tid < 256; ++tid) {
                        const int n = bx * rpb + tid / cg, c4 = tid % cg;
                        REQUIRE(n < kSlots, "combine slot %d", n);
                        const Slot sl = slot_of(n, chunk, p.hpc, Sq, gcount[kvh]);
                        if (!sl.valid) continue;
                        const int h = horder[gstart[kvh] + sl.hh];
                        for (int s = 0; s < p.nsplit; ++s) {
                            const size_t row = partial_row(bkv, chunk, 0, n, p) + static_cast<size_t>(s) * kSlots;
                            REQUIRE(row == partial_row(bkv, chunk, s, n, p), "combine split stride");
                            REQUIRE(row < rows_total && row * D + c4 * 4 + 4 <= rows_total * D, "combine row");
                        }
                        const size_t orow = (static_cast<size_t>(b) * Hq + h) * Sq + sl.i;
                        REQUIRE(orow < static_cast<size_t>(B) * Hq * Sq, "o row %zu", orow);
                        if (elt == 0 && c4 == 0 && orow < written.size()) written[orow] += 1;
                    }
        }
    }
    for (size_t r = 0; r < owner.size(); ++r) REQUIRE(owner[r] == 1, "query row %zu owned %d times", r, owner[r]);
    for (size_t r = 0; r < written.size(); ++r) REQUIRE(written[r] == 1, "output row %zu written %d times", r, written[r]);
    REQUIRE(ws_l_offset(rows_total, D) + rows_total * 4 <= ws_bytes(rows_total, D), "workspace size");
}

int main() {
    long shapes = 0;
    const int sqs[] = {1, 2, 3, 5, 7, 8, 16, 31, 32};
    const int sks[] = {32, 33, 64, 100, 257, 1000, 4096};
    for (int Sq : sqs)
        for (int Sk : sks) {
            if (Sq > Sk) continue;
            std::vector<int> gqa(8), mqa(16, 0), odd{2, 0, 2, 1, 0}, gap{0, 2, 2, 0};   // gap: kv-head 1 unused
            for (int h = 0; h < 8; ++h) gqa[h] = h / 4;
            check(2, 8, 2, Sq, Sk, 64, gqa);
            check(1, 16, 1, Sq, Sk, 128, mqa);
            check(3, 5, 3, Sq, Sk, 64, odd);
            check(2, 4, 3, Sq, Sk, 128, gap);
            shapes += 4;
        }
    std::vector<int> big(32);
    for (int h = 0; h < 32; ++h) big[h] = h / 4;
    check(4, 32, 8, 1, 8192, 128, big);
    check(1, 32, 8, 4, 32768, 128, big);
    std::vector<int> onegroup(40, 0);
    check(1, 40, 1, 32, 2000, 64, onegroup);
    std::vector<int> full(256, 0);   // 256 q-heads on kv-head 0, kv-heads 1..3 unused
    check(1, 256, 4, 1, 100, 64, full);
    shapes += 4;
    std::printf("checked %ld decode shapes, %ld errors\n", shapes, g_errors);
    return g_errors == 0 ? 0 : 1;
}
