// CPU check of the forward kernel's global-memory index arithmetic.
//
// Built for the host only (the shared helpers are __host__ __device__) and
// run by tests/test_geometry.py.  For every shape it enumerates, per
// workgroup, wave and lane, each global address the kernel forms (Q
// fragments, staged K/V tile rows for the whole pipeline schedule including
// the tiles prefetched past the end, scale indices, output columns and the
// score-dump indices) and checks that it lies inside its buffer.  It also
// checks that the work schedule visits every (batch, head, query tile) item
// exactly once, for one item per workgroup and for the two-items-per-
// workgroup grid of causal launches.  Exit status 0 = clean.
#include "fwd_geometry.h"

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <utility>
#include <vector>

using namespace attn::geom;

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

// pv8: the 8-bit P.V variant, whose V tiles come from V^T codes
// [D, 64 * nkblk] per (b, kv-head) instead of row-major fp16 V.
template <int D, bool INT8>
static void check_shape(int B, int Hq, int S, bool causal, bool dump, int tile_lo, int ntiles,
                        bool all_heads, bool pv8 = false, int G = 1) {
    using St = Stage<D, INT8>;
    const int nqt = (S + kTileM - 1) / kTileM;
    if (!dump) {
        tile_lo = 0;
        ntiles = nqt;
    }
    const long nblk = static_cast<long>(B) * Hq * ntiles;
    const size_t qk_head_bytes = static_cast<size_t>(S) * St::KROWG;
    const size_t v_head_bytes = static_cast<size_t>(S) * St::VROWG;
    const int nqblk = (S + 127) / 128, nkblk = (S + 63) / 64;
    // the kernel's item loop: one item per workgroup, or (causal, the score
    // dump included) the schedule over the two-items-per-workgroup grid as well
    const bool persist = causal;
    const int n = static_cast<int>(nblk);
    std::vector<std::pair<int, int>> work;   // (grid, item) in visiting order
    std::vector<char> seen(nblk, 0);
    for (int pass = 0; pass < (persist ? 2 : 1); ++pass) {
        const int grid = pass == 0 ? n : sched_grid(n, (n + 1) / 2);
        std::fill(seen.begin(), seen.end(), 0);
        for (int bid = 0; bid < grid; ++bid) {
            const Sched sc = make_sched(bid, grid, n);
            const int iters = persist ? sched_iters(sc) : 1;
            for (int it = 0; it < iters; ++it) {
                const int item = sched_item(sc, it);
                if (item < 0) continue;
                REQUIRE(item < n && !seen[item], "grid %d bid %d it %d -> item %d", grid, bid, it, item);
                if (item >= n || seen[item]) continue;
                seen[item] = 1;
                if (pass == 0) work.push_back({grid, item});
            }
        }
        for (long i = 0; i < nblk; ++i) REQUIRE(seen[i], "grid %d: item %ld never visited", grid, i);
    }
    std::fill(seen.begin(), seen.end(), 0);
    for (const auto& w : work) {
        const int item = w.second;
        const BlockCoord c = decode_item(item, Hq, ntiles, tile_lo, causal, G);
        REQUIRE(c.b >= 0 && c.b < B && c.pos >= 0 && c.pos < Hq && c.qt >= tile_lo &&
                    c.qt < tile_lo + ntiles && c.qt < nqt,
                "item %d -> b %d pos %d qt %d", item, c.b, c.pos, c.qt);
        if (!(c.b >= 0 && c.b < B && c.pos >= 0 && c.pos < Hq && c.qt >= tile_lo && c.qt < tile_lo + ntiles))
            continue;
        const long slot = (static_cast<long>(c.b) * Hq + c.pos) * ntiles + (c.qt - tile_lo);
        REQUIRE(!seen[slot], "item %d maps to a taken slot", item);
        seen[slot] = 1;
        if (!all_heads && !((c.b == 0 && c.pos == 0) || (c.b == B - 1 && c.pos == Hq - 1))) continue;

        const int q0 = c.qt * kTileM;
        const int nkt = block_key_tiles(S, q0, causal);
        REQUIRE(nkt >= 1 && nkt <= nkblk, "nkt %d nkblk %d", nkt, nkblk);
        REQUIRE(c.qt < nqblk, "q scale index %d of %d", c.qt, nqblk);
        for (int wave = 0; wave < 4; ++wave) {
            const int qw0 = q0 + wave * 32;
            const int nkt_w = wave_key_tiles(nkt, qw0, causal);
            REQUIRE(nkt_w >= 1 && nkt_w <= nkt, "nkt_w %d nkt %d", nkt_w, nkt);
            for (int lane = 0; lane < 64; ++lane) {
                const int qi = qw0 + (lane & 31), g = lane >> 5;
                const int qr = q_row(qi, S);
                REQUIRE(qr >= 0 && qr < S, "q row %d S %d", qr, S);
                for (int s = 0; s < St::QSTEPS; ++s) {
                    const int off = St::q_frag_offset(s, g);
                    REQUIRE(off >= 0 && off + 16 <= St::KROWG, "q frag offset %d", off);
                    if (INT8)
                        for (int hh = 0; hh < 2; ++hh) {
                            const int o16 = St::q16_piece_offset(s, g, hh);
                            REQUIRE(o16 >= 0 && o16 + 16 <= 2 * D, "fp16 q piece offset %d", o16);
                        }
                }
                if (!dump && qi < S)
                    for (int dt = 0; dt < D / 32; ++dt)
                        for (int j4 = 0; j4 < 4; ++j4) {
                            const int col = o_column(dt, j4, g);
                            REQUIRE(col >= 0 && col + 4 <= D, "o column %d", col);
                        }
                if (dump && qi < S)
                    for (int j = 0; j < nkt_w; ++j) {
                        const int n0 = j * kTileN;
                        const int lim = mask_limit(n0, S, qi, g, causal);
                        for (int mt = 0; mt < 2; ++mt)
                            for (int r = 0; r < 16; ++r)
                                if (key_offset(mt, r) < lim) {
                                    const int key = n0 + g * 4 + key_offset(mt, r);
                                    REQUIRE(key >= 0 && key < S && (!causal || key <= qi), "dump key %d", key);
                                    const int row = qi - tile_lo * kTileM;
                                    REQUIRE(row >= 0 && row < ntiles * kTileM, "dump row %d", row);
                                }
                    }
                for (int j = 0; j < nkt_w; ++j) REQUIRE(j < nkblk, "k scale index %d", j);
            }
        }
        // register-staged tiles (the tile-masked kernel's long lists), in the
        // pipeline order of the kernel
        std::vector<int> kn0, vn0;
        if (!dump) {
            const int depth = fwd_prefetch_depth(D, INT8);
            for (int t = 0; t <= depth; ++t) kn0.push_back(t * kTileN);
            for (int t = 0; t < depth; ++t) vn0.push_back(t * kTileN);
            const int iters = depth == 2 ? loop_iterations<2>(nkt) : loop_iterations<1>(nkt);
            for (int j = 0; j < iters; ++j) {
                kn0.push_back(depth == 2 ? k_load_row<2>(j) : k_load_row<1>(j));
                vn0.push_back(depth == 2 ? v_load_row<2>(j) : v_load_row<1>(j));
            }
        }
        // direct-to-LDS staging (every variant; the score dump copies K
        // tiles only): every (wave, instruction, lane) slot of every copied tile
        {
            const int nst = (!INT8 && D == 128) ? 2 : 3;
            std::vector<int> dk, dvv;
            for (int t = 0; t < nst; ++t) dk.push_back(t * kTileN);
            if (!dump)
                for (int t = 0; t + 1 < nst; ++t) dvv.push_back(t * kTileN);
            const int iters = nst == 2 ? dtl_loop_iterations<2>(nkt) : dtl_loop_iterations<3>(nkt);
            REQUIRE(iters >= nkt && iters % nst == 0, "dtl iterations %d", iters);
            for (int j = 0; j < iters; ++j) {
                dk.push_back((j + nst) * kTileN);
                if (!dump) dvv.push_back((j + nst - 1) * kTileN);
                const int ks = j + nst < nkblk ? j + nst : nkblk - 1;   // scale ring index, clamped
                REQUIRE(ks >= 0 && ks < nkblk, "k scale ring %d", ks);
            }
            auto check_tile = [&](int n0, int rb, size_t head_bytes, bool is_v) {
                const int first = tile_first_row(n0, S);
                const int cpr = rb / 16, ni = kTileN * rb / 1024 / 4;
                std::vector<int> seen_slot(static_cast<size_t>(kTileN) * cpr, 0);
                for (int w = 0; w < 4; ++w)
                    for (int i = 0; i < ni; ++i)
                        for (int lane = 0; lane < 64; ++lane) {
                            int r, pc, c;
                            if (rb == 256) {
                                r = Dtl<256>::slot_row(w, i, lane); pc = Dtl<256>::slot_chunk(w, i, lane);
                                c = pc ^ (is_v ? Dtl<256>::v_swz(r) : Dtl<256>::k_swz(r));
                            } else if (rb == 128) {
                                r = Dtl<128>::slot_row(w, i, lane); pc = Dtl<128>::slot_chunk(w, i, lane);
                                c = pc ^ (is_v ? Dtl<128>::v_swz(r) : Dtl<128>::k_swz(r));
                            } else {
                                r = Dtl<64>::slot_row(w, i, lane); pc = Dtl<64>::slot_chunk(w, i, lane);
                                c = pc ^ Dtl<64>::k_swz(r);
                            }
                            REQUIRE(r >= 0 && r < kTileN && pc >= 0 && pc < cpr && c >= 0 && c < cpr,
                                    "dtl slot r %d pc %d c %d", r, pc, c);
                            // the LDS byte the lane writes is the slot's own position
                            REQUIRE((w * ni + i) * 1024 + lane * 16 == r * rb + pc * 16, "dtl lds byte");
                            seen_slot[static_cast<size_t>(r) * cpr + pc] += 1;
                            const int row = tile_lane_row(r, first, S);
                            const size_t off = (static_cast<size_t>(first) + row) * rb + c * 16;
                            REQUIRE(first + row <= S - 1 && off + 16 <= head_bytes, "dtl byte %zu of %zu", off, head_bytes);
                        }
                for (int v : seen_slot) REQUIRE(v == 1, "dtl slot written %d times", v);
            };
            for (int n0 : dk) check_tile(n0, St::KROWG, qk_head_bytes, false);
            if (INT8 && !pv8) {
                // fused-Q kernels: the block's fp16 Q rows q0 .. q0+127 copied
                // as two 64-row halves into V-sized stages (K-style swizzle),
                // then each lane's 16-byte pieces read back from its row
                for (int h = 0; h < 2; ++h) check_tile(q0 + kTileN * h, St::VROWG, v_head_bytes, false);
                const int rb = St::VROWG, cpr = rb / 16;
                for (int h = 0; h < 2; ++h)
                    for (int rq = 0; rq < kTileN; ++rq) {
                        const int first = tile_first_row(q0 + kTileN * h, S);
                        const int row = first + tile_lane_row(rq, first, S);
                        REQUIRE(row == q_row(q0 + kTileN * h + rq, S), "fused q row %d", row);
                        const int sw = rb == 256 ? Dtl<256>::k_swz(rq) : Dtl<128>::k_swz(rq);
                        for (int s = 0; s < St::QSTEPS; ++s)
                            for (int g = 0; g < 2; ++g)
                                for (int hh = 0; hh < 2; ++hh) {
                                    const int c = St::q16_piece_offset(s, g, hh) / 16;
                                    const int pc = c ^ sw;
                                    REQUIRE(c < cpr && pc >= 0 && pc < cpr && rq * rb + pc * 16 + 16 <= kTileN * rb,
                                            "fused q lds read rq %d c %d pc %d", rq, c, pc);
                                }
                    }
            }
            if (!pv8) {
                for (int n0 : dvv) check_tile(n0, St::VROWG, v_head_bytes, true);
            } else {
                // 8-bit V^T tiles: D rows of 64 codes at column v8_tile_col, row stride Sp
                const int Sp = nkblk * kTileN;
                const size_t vt_head_bytes = static_cast<size_t>(D) * Sp;
                for (int n0 : dvv) {
                    const int col = v8_tile_col(n0, nkblk);
                    REQUIRE(col >= 0 && col % kTileN == 0 && col + kTileN <= Sp, "v8 column %d (n0 %d, Sp %d)", col, n0, Sp);
                    std::vector<int> seen(static_cast<size_t>(D) * 4, 0);
                    for (int w = 0; w < 4; ++w)
                        for (int i = 0; i < Dtl8<D>::NI; ++i)
                            for (int lane = 0; lane < 64; ++lane) {
                                const int r = Dtl8<D>::slot_row(w, i, lane), pc = Dtl8<D>::slot_chunk(w, i, lane);
                                const int c = pc ^ Dtl8<D>::swz(r);
                                REQUIRE(r >= 0 && r < D && pc >= 0 && pc < 4 && c >= 0 && c < 4, "v8 slot r %d pc %d c %d", r, pc, c);
                                REQUIRE((w * Dtl8<D>::NI + i) * 1024 + lane * 16 == r * kTileN + pc * 16, "v8 lds byte");
                                seen[static_cast<size_t>(r) * 4 + pc] += 1;
                                const long long off32 = static_cast<long long>(r) * Sp + c * 16;
                                REQUIRE(off32 < (1LL << 32), "v8 lane offset %lld", off32);
                                const size_t off = static_cast<size_t>(col) + static_cast<size_t>(off32);
                                REQUIRE(off + 16 <= vt_head_bytes, "v8 byte %zu of %zu", off, vt_head_bytes);
                            }
                    for (int v : seen) REQUIRE(v == 1, "v8 slot written %d times", v);
                }
            }
        }
        for (int n0 : kn0) {
            const int first = tile_first_row(n0, S);
            REQUIRE(first >= 0 && first <= S - 1, "k first row %d (n0 %d, S %d)", first, n0, S);
            for (int tid = 0; tid < kThreads; ++tid)
                for (int i = 0; i < St::KPT; ++i) {
                    const int cidx = tid + kThreads * i;
                    const int row = tile_lane_row(cidx / St::KCPR, first, S);
                    const long long off32 = static_cast<long long>(row) * St::KROWG + (cidx % St::KCPR) * 16;
                    REQUIRE(row >= 0 && first + row <= S - 1, "k row %d first %d S %d", row, first, S);
                    REQUIRE(off32 >= 0 && off32 < (1LL << 32), "k lane offset %lld", off32);
                    const size_t off = static_cast<size_t>(first) * St::KROWG + static_cast<size_t>(off32);
                    REQUIRE(off + 16 <= qk_head_bytes, "k byte %zu of %zu", off, qk_head_bytes);
                }
        }
        if (pv8) vn0.clear();   // (its V tiles are staged directly, checked above)
        for (int n0 : vn0) {
            const int first = tile_first_row(n0, S);
            REQUIRE(first >= 0 && first <= S - 1, "v first row %d", first);
            for (int tid = 0; tid < kThreads; ++tid)
                for (int i = 0; i < St::VPT; ++i) {
                    const int cidx = tid + kThreads * i;
                    const int row = tile_lane_row(cidx / St::VCPR, first, S);
                    const long long off32 = static_cast<long long>(row) * St::VROWG + (cidx % St::VCPR) * 16;
                    REQUIRE(row >= 0 && first + row <= S - 1, "v row %d first %d S %d", row, first, S);
                    REQUIRE(off32 >= 0 && off32 < (1LL << 32), "v lane offset %lld", off32);
                    const size_t off = static_cast<size_t>(first) * St::VROWG + static_cast<size_t>(off32);
                    REQUIRE(off + 16 <= v_head_bytes, "v byte %zu of %zu", off, v_head_bytes);
                }
        }
    }
    for (long i = 0; i < nblk; ++i) REQUIRE(seen[i], "slot %ld never visited", i);
}

template <int D>
static void check_all_paths(int B, int Hq, int S, bool all_heads) {
    const int nqt = (S + kTileM - 1) / kTileM;
    for (int causal = 0; causal < 2; ++causal) {
        check_shape<D, false>(B, Hq, S, causal, false, 0, 0, all_heads);
        check_shape<D, true>(B, Hq, S, causal, false, 0, 0, all_heads);
        // launch-order groups of q-heads sharing a kv-head (every divisor of Hq)
        for (int G = 2; G <= Hq; ++G)
            if (Hq % G == 0) {
                check_shape<D, false>(B, Hq, S, causal, false, 0, 0, all_heads, false, G);
                check_shape<D, true>(B, Hq, S, causal, true, 0, nqt, all_heads, false, G);
            }
        check_shape<D, true>(B, Hq, S, causal, false, 0, 0, all_heads, true);
        check_shape<D, true>(B, Hq, S, causal, true, 0, nqt, all_heads);
        check_shape<D, true>(B, Hq, S, causal, true, nqt - 1, 1, all_heads);
        check_shape<D, true>(B, Hq, S, causal, true, nqt / 2, (nqt + 1) / 2 - nqt / 2 + 1 > 0 ? 1 : 1, all_heads);
    }
}

// Tile-mask lists: for arbitrary (also malformed) row pointers, entry counts
// and entries, every list index and every key tile stays in bounds.
static void check_mask_lists() {
    unsigned x = 12345u;
    auto rnd = [&](int lo, int hi) {   // inclusive, xorshift
        x ^= x << 13; x ^= x >> 17; x ^= x << 5;
        return lo + static_cast<int>(x % static_cast<unsigned>(hi - lo + 1));
    };
    for (int it = 0; it < 200000; ++it) {
        const int nkblk = rnd(1, 5000), nnz = rnd(0, 3000);
        const int rp0 = rnd(-100, 3100), rp1 = rnd(-100, 3100);
        const MaskRow r = mask_row(rp0, rp1, nnz, nkblk);
        REQUIRE(r.count >= 0 && r.count <= nkblk, "count %d", r.count);
        if (r.count == 0) continue;
        REQUIRE(r.base >= 0 && r.base + r.count <= nnz, "base %d count %d nnz %d", r.base, r.count, nnz);
        for (int pos = 0; pos < r.count + 4; ++pos) {
            const int idx = mask_entry_index(r, pos);
            REQUIRE(idx >= 0 && idx < nnz, "entry index %d of %d", idx, nnz);
        }
        // the LDS copy of a run (launched only while nkblk <= kMaskListMax):
        // copy indices base + i, i < count, and list reads min(pos, count-1)
        if (nkblk <= kMaskListMax) {
            const int n = imin(r.count, kMaskListMax);
            REQUIRE(n == r.count && n <= kMaskListMax && r.base + n <= nnz, "LDS list of %d", n);
            for (int pos = 0; pos < n + 4; ++pos) {
                const int li = imin(pos, n - 1);
                REQUIRE(li >= 0 && li < kMaskListMax, "LDS list index %d", li);
            }
        }
        const int e = static_cast<int>(x);   // any 32-bit entry
        const int kt = mask_entry_tile(e, nkblk);
        REQUIRE(kt >= 0 && kt < nkblk, "key tile %d of %d", kt, nkblk);
        const int ty = mask_entry_type(e);
        REQUIRE(ty >= 0 && ty <= 2, "type %d", ty);
    }
}

// The work schedule alone: for every item count up to 3000 and every grid
// the launch may choose (one item per workgroup, two per workgroup, and any
// grid between min(8, n) and n), each item is visited exactly once.
static void check_schedules() {
    std::vector<int> hits;
    for (int n = 1; n <= 3000; ++n) {
        const int lo = n < 8 ? n : 8;
        std::vector<int> grids{n, sched_grid(n, (n + 1) / 2), sched_grid(n, (n + 2) / 3), sched_grid(n, 1), lo};
        if (n <= 200)
            for (int g = lo; g <= n; ++g) grids.push_back(g);
        for (int grid : grids) {
            REQUIRE(grid >= lo && grid <= n, "n %d grid %d", n, grid);
            hits.assign(n, 0);
            for (int bid = 0; bid < grid; ++bid) {
                const Sched sc = make_sched(bid, grid, n);
                REQUIRE(sc.K >= 1 && sc.k < sc.K, "n %d grid %d bid %d: k %d of %d", n, grid, bid, sc.k, sc.K);
                for (int it = 0; it < sched_iters(sc); ++it) {
                    const int item = sched_item(sc, it);
                    if (item < 0) continue;
                    REQUIRE(item >= sc.first && item < sc.first + sc.count, "item %d outside its XCD range", item);
                    if (item >= 0 && item < n) hits[item] += 1;
                }
            }
            for (int i = 0; i < n; ++i) REQUIRE(hits[i] == 1, "n %d grid %d: item %d visited %d times", n, grid, i, hits[i]);
        }
    }
    // one item per workgroup keeps the plain XCD renumbering
    for (int n = 1; n <= 600; ++n)
        for (int bid = 0; bid < n; ++bid) {
            const Sched sc = make_sched(bid, n, n);
            const int x = bid & 7, per = n >> 3, rem = n & 7;
            REQUIRE(sched_iters(sc) == 1 && sched_item(sc, 0) == x * per + imin(x, rem) + (bid >> 3),
                    "n %d bid %d", n, bid);
        }
}

int main() {
    long shapes = 0;
    check_mask_lists();
    check_schedules();
    for (int S = 1; S <= 300; ++S) {
        check_all_paths<64>(1, 3, S, true);
        check_all_paths<128>(2, 2, S, true);
        shapes += 2;
    }
    const int big[] = {511, 512, 513, 1000, 1023, 1024, 1025, 4095, 4096, 4097, 8192, 16384, 32768};
    for (int S : big) {
        check_all_paths<64>(2, 3, S, S <= 4097);
        check_all_paths<128>(1, 5, S, S <= 4097);
        shapes += 2;
    }
    // many blocks (grid sizes that are not multiples of 8, large batch)
    check_all_paths<128>(64, 16, 1024, false);
    check_all_paths<64>(3, 7, 777, true);
    shapes += 2;
    std::printf("checked %ld shape families, %ld errors\n", shapes, g_errors);
    return g_errors == 0 ? 0 : 1;
}
