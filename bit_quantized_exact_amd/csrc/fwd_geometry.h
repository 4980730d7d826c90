// Launch geometry and global-memory index arithmetic of the forward kernel.
//
// Every global address the forward kernel forms is built from these
// functions, which compile for the host as well, so that a CPU program can
// enumerate them for any shape and check that they stay inside the buffers
// (the geometry check under tests/).
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace attn {
namespace geom {

constexpr int kTileM = 128;   // query rows per workgroup (4 waves x 32)
constexpr int kTileN = 64;    // keys per tile
constexpr int kThreads = 256;

__host__ __device__ inline int imin(int a, int b) { return a < b ? a : b; }

struct BlockCoord {
    int b;    // batch
    int pos;  // position in the kv-grouped head order
    int qt;   // query tile
};

// Logical work item -> (batch, head position, query tile).  Within a batch
// the head positions (q-heads ordered by kv-head) form groups of G
// consecutive positions, the q-heads that share a kv-head (G = 1 when the
// groups are irregular); items run group by group and, inside a group,
// rank-major: the G heads of a group take the same query tile one after the
// other, so their workgroups read the same K/V tiles close together in time
// (and mostly from L2).  Causal launches take the heaviest query tiles of a
// head first.  Bijective on [0, nitems) when Hq is a multiple of G.
__host__ __device__ inline BlockCoord decode_item(int L, int Hq, int ntiles, int tile_lo, bool heavy_first,
                                                  int G = 1) {
    const int per_b = Hq * ntiles;
    BlockCoord c;
    c.b = L / per_b;
    const int rb = L - c.b * per_b;
    const int per_g = G * ntiles;
    const int gi = rb / per_g;
    const int r2 = rb - gi * per_g;
    const int rank = r2 / G;
    c.pos = gi * G + (r2 - rank * G);
    c.qt = tile_lo + (heavy_first ? (ntiles - 1 - rank) : rank);
    return c;
}

// Persistent schedule of the work items over the launch's workgroups.
// Consecutive hardware ids go round-robin over the 8 XCDs: XCD x gets a
// contiguous range of logical items (neighbouring heads share K/V in its
// L2) and its K workgroups walk that range in blocks of K, workgroup k
// taking slot k of even blocks and slot K-1-k of odd ones (a snake, which
// evens out the per-workgroup sums of the heaviest-first causal order).
// Every item is visited exactly once when grid >= min(8, nitems) and
// grid <= nitems; with grid == nitems each workgroup takes one item.
struct Sched {
    int first;   // first logical item of this XCD's range
    int count;   // items in the range
    int k;       // this workgroup's index on its XCD
    int K;       // workgroups on this XCD
};
__host__ __device__ inline Sched make_sched(int bid, int grid, int nitems) {
    const int x = bid & 7;
    const int per = nitems >> 3, rem = nitems & 7;
    Sched s;
    s.first = x * per + imin(x, rem);
    s.count = per + (x < rem ? 1 : 0);
    s.K = (grid >> 3) + (x < (grid & 7) ? 1 : 0);
    s.k = bid >> 3;
    return s;
}
__host__ __device__ inline int sched_iters(const Sched& s) { return (s.count + s.K - 1) / s.K; }
// Logical item of iteration it, or -1 (the last block may be partial).
__host__ __device__ inline int sched_item(const Sched& s, int it) {
    const int slot = it * s.K + ((it & 1) ? s.K - 1 - s.k : s.k);
    return slot < s.count ? s.first + slot : -1;
}
// Workgroups of a launch over nitems items with at most `resident` of them
// on the device at once.
__host__ __device__ inline int sched_grid(int nitems, int resident) {
    const int g = resident < 8 ? 8 : resident;
    return nitems < g ? nitems : g;
}

// Key tiles a workgroup visits, and those a wave needs (causal: the wave's
// last query row bounds its keys).
__host__ __device__ inline int block_key_tiles(int S, int q0, bool causal) {
    const int n_end = causal ? imin(S, q0 + kTileM) : S;
    return (n_end + kTileN - 1) / kTileN;
}
__host__ __device__ inline int wave_key_tiles(int nkt, int qw0, bool causal) {
    return causal ? imin(nkt, (qw0 + 31) / kTileN + 1) : nkt;
}

// Query row read for a lane: rows past the sequence read the last row.
__host__ __device__ inline int q_row(int qi, int S) { return imin(qi, S - 1); }

// Staging of one key tile at n0 (n0 may lie past the sequence end: the
// pipeline prefetches two tiles ahead).  The wave-uniform part is the first
// row of the tile clamped to S-1; each lane adds a row clamped to the rows
// that remain, so every row read lies in [0, S-1].
__host__ __device__ inline int tile_first_row(int n0, int S) { return imin(n0, S - 1); }
__host__ __device__ inline int tile_lane_row(int row, int first_row, int S) {
    return imin(row, S - 1 - first_row);
}

// Global-memory layout of one head's tiles: row bytes, 16-byte chunks per
// row, chunks per thread and per-lane Q fragment bytes.
template <int D, bool INT8>
struct Stage {
    static constexpr int KELT = INT8 ? 1 : 2;          // bytes per Q/K element
    static constexpr int KROWG = D * KELT;             // Q/K row bytes
    static constexpr int VROWG = 2 * D;                // V / O row bytes
    static constexpr int KCPR = KROWG / 16;            // 16-byte chunks per K row
    static constexpr int VCPR = VROWG / 16;
    static constexpr int KPT = kTileN * KCPR / kThreads;
    static constexpr int VPT = kTileN * VCPR / kThreads;
    static constexpr int QSTEPS = INT8 ? D / 32 : D / 16;
    // byte offset within a Q row of the 16-byte fragment for MFMA k-step s, lane half g
    __host__ __device__ static constexpr int q_frag_offset(int s, int g) {
        return INT8 ? (s * 32 + g * 16) : (s * 16 + g * 8) * 2;
    }
    // fused Q quantisation (INT8 path reading fp16 Q): byte offset within an
    // fp16 Q row of 16-byte piece h (0, 1) of the 16 elements behind the
    // int8 fragment of k-step s, lane half g
    __host__ __device__ static constexpr int q16_piece_offset(int s, int g, int h) {
        return (s * 32 + g * 16 + h * 8) * 2;
    }
};

// Direct-to-LDS staging (global_load_lds): one wave instruction moves 64
// lanes x 16 bytes into 1 KB of LDS at a wave-uniform base, lane l writing
// bytes 16 l .. 16 l + 15.  A 64-row tile of RB-byte rows takes 64*RB/1024
// wave instructions, NI per wave (wave w issues w*NI .. w*NI+NI-1).  Rows are
// stored unpadded; the 16-byte chunks of each row are permuted by an XOR with
// a row-dependent value so that the MFMA operand reads of K (16 rows, one
// chunk) and the transposing reads of V (4 rows, 64 bytes) hit 64 distinct
// banks.  Slot (w, i, lane) holds physical chunk pc of row r, i.e. logical
// chunk pc ^ swz(r) of key row r (the XOR is its own inverse).
template <int RB>
struct Dtl {
    static constexpr int CPR = RB / 16;                   // chunks per row
    static constexpr int RPL = RB >= 256 ? 1 : 256 / RB;  // rows per 256-byte bank line
    static constexpr int NI = kTileN * RB / 1024 / 4;     // instructions per wave per tile
    static_assert(kTileN * RB % 4096 == 0 && CPR >= 4, "tile split");
    __host__ __device__ static constexpr int k_swz(int r) { return (r / RPL) % CPR; }
    __host__ __device__ static constexpr int v_swz(int r) { return ((r / RPL) % (4 / RPL)) * 4; }
    __host__ __device__ static constexpr int slot_row(int w, int i, int lane) { return ((w * NI + i) * 64 + lane) / CPR; }
    __host__ __device__ static constexpr int slot_chunk(int w, int i, int lane) { return ((w * NI + i) * 64 + lane) % CPR; }
};

// 8-bit V of the P.V ablation: V^T codes [B*Hkv, D, Sp], Sp = 64 * nkblk.
// A key tile at n0 is D rows of 64 bytes starting at column
// v8_tile_col(n0, nkblk); tiles prefetched past the end are clamped to the
// last tile (always inside the buffer).  It is copied straight into an
// unpadded LDS stage of D rows of 64 bytes whose 16-byte chunks are
// XOR-swizzled by row group (the 32-byte reads of the two lane halves are
// then free of bank conflicts); instruction i of wave w fills stage bytes
// (w*NI + i)*1024 .. +1023.
__host__ __device__ inline int v8_tile_col(int n0, int nkblk) { return imin(n0, (nkblk - 1) * kTileN); }
template <int D>
struct Dtl8 {
    static constexpr int NI = D * kTileN / 1024 / 4;   // instructions per wave per tile
    static_assert(D * kTileN % 4096 == 0, "tile split");
    __host__ __device__ static constexpr int swz(int r) { return (r >> 2) & 3; }
    __host__ __device__ static constexpr int slot_row(int w, int i, int lane) { return ((w * NI + i) * 64 + lane) / 4; }
    __host__ __device__ static constexpr int slot_chunk(int w, int i, int lane) { return ((w * NI + i) * 64 + lane) % 4; }
};

// Tile-mask lists: for each query tile, a run of entries e = (key tile << 2)
// | type in a CSR list (row pointers per query tile); type 1 = every key of
// the tile visible, 2 = key j visible iff j <= query i, 0 = none visible (3 is
// read as 1).  Every index below is clamped, so arbitrary list contents never
// address outside the row-pointer, entry, K, V or scale buffers.
__host__ __device__ inline int imax(int a, int b) { return a > b ? a : b; }
struct MaskRow {
    int base;    // first entry of the query tile
    int count;   // entries used (0 .. nkblk)
};
__host__ __device__ inline MaskRow mask_row(int rp0, int rp1, int nnz, int nkblk) {
    MaskRow r;
    r.base = imin(imax(rp0, 0), imax(nnz, 0));
    r.count = imin(imax(rp1 - r.base, 0), imin(nkblk, imax(nnz, 0) - r.base));
    return r;
}
// Key tiles of a list the tile-masked forward copies into LDS (sequences up
// to 32768 tokens); longer lists are read from global memory.
constexpr int kMaskListMax = 512;
// entry index of list position pos (positions past the end repeat the last; count >= 1)
__host__ __device__ inline int mask_entry_index(const MaskRow& r, int pos) { return r.base + imin(pos, r.count - 1); }
__host__ __device__ inline int mask_entry_tile(int e, int nkblk) { return imin(imax(e >> 2, 0), nkblk - 1); }
__host__ __device__ inline int mask_entry_type(int e) { return (e & 3) == 3 ? 1 : (e & 3); }

// Score register r of 32-key sub-tile mt (32x32 MFMA accumulator layout)
// holds key n0 + g*4 + key_offset(mt, r) of a tile at n0 (g = lane / 32).
__host__ __device__ constexpr int key_offset(int mt, int r) { return mt * 32 + (r >> 2) * 8 + (r & 3); }

// Keys of the tile at n0 visible to query qi satisfy key_offset < mask_limit:
// key < S, and key <= qi when causal.
__host__ __device__ inline int mask_limit(int n0, int S, int qi, int g, bool causal) {
    int lim = S - n0 - g * 4;
    if (causal) lim = imin(lim, qi - n0 - g * 4 + 1);
    return lim;
}

// Output column of accumulator group j4 (4 consecutive registers) of d-tile dt.
__host__ __device__ constexpr int o_column(int dt, int j4, int g) { return dt * 32 + j4 * 8 + g * 4; }

// Pipeline schedule.  K tiles are consumed one iteration before V tiles.
// With prefetch depth DEPTH (1 or 2), iteration j of the main loop issues
// the global loads of K tile j+1+DEPTH and V tile j+DEPTH into registers and
// writes the tiles loaded DEPTH-1 iterations earlier (K tile j+2, V tile
// j+1) to LDS.  The prologue loads K tiles 0..DEPTH and V tiles 0..DEPTH-1.
// At depth 2 the loop runs an even number of iterations (two register sets
// alternate); an iteration past the last tile only stages clamped rows.
// Depth 2 needs a second register set; FP16 at head_dim 128 has no room for it.
__host__ __device__ constexpr int fwd_prefetch_depth(int D, bool int8) { return (!int8 && D == 128) ? 1 : 2; }
template <int DEPTH>
__host__ __device__ inline int k_load_row(int j) { return (j + 1 + DEPTH) * kTileN; }
template <int DEPTH>
__host__ __device__ inline int v_load_row(int j) { return (j + DEPTH) * kTileN; }
template <int DEPTH>
__host__ __device__ inline int loop_iterations(int nkt) { return DEPTH == 2 ? (nkt + 1) & ~1 : nkt; }
// Direct-to-LDS staging with NST stages: the prologue copies K tiles
// 0..NST-1 and V tiles 0..NST-2; iteration j copies K tile j+NST and V tile
// j+NST-1 (tiles past the end copy clamped rows); the loop runs a multiple
// of NST iterations.
template <int NST>
__host__ __device__ inline int dtl_loop_iterations(int nkt) { return (nkt + NST - 1) / NST * NST; }

}  // namespace geom
}  // namespace attn
