// Launch plan and global-memory index arithmetic of the KV-cache (decode)
// attention kernels.
//
// Every global address the decode and combine kernels form is built from
// these functions, which also compile for the host, so that a CPU program can
// enumerate them for any shape and check them against the buffer sizes (the
// geometry check under tests/).
//
// Work decomposition: the queries of all q-heads that share one kv-head are
// packed into the 32 query slots of a wave (whole heads per slot group, so a
// head's queries never straddle two waves); the cached keys are split into
// ranges of 32-key tiles.  One single-wave workgroup handles one
// (batch, kv-head, query chunk, key split) and leaves an unnormalised partial
// result; a combine kernel merges the splits.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace attn {
namespace dec {

constexpr int kSlots = 32;        // query slots per wave (MFMA N dimension)
constexpr int kTile = 32;         // keys per tile
constexpr int kThreads = 64;      // one wave per workgroup
constexpr int kMaxSq = 32;        // queries per head handled in one wave
#ifndef ATTN_DECODE_TARGET_GROUPS
#define ATTN_DECODE_TARGET_GROUPS 1024
#endif
// workgroups a launch aims for: 4 single-wave workgroups per CU keep enough
// of the cache in flight (measured: 2 per CU starve the INT8 path, 8 per CU
// add partial-result traffic and per-workgroup set-up)
constexpr int kTargetGroups = ATTN_DECODE_TARGET_GROUPS;
constexpr int kMinTilesPerSplit = 8;

__host__ __device__ inline int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ inline int imax(int a, int b) { return a > b ? a : b; }
__host__ __device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }

struct Plan {
    int hpc;      // q-heads per query chunk
    int nchunk;   // query chunks per (batch, kv-head)
    int ntiles;   // 32-key tiles of the cache
    int tps;      // tiles per split
    int nsplit;   // key splits
};

// max_group: the largest number of q-heads mapped to one kv-head.
__host__ __device__ inline Plan make_plan(int B, int Hkv, int Sq, int Sk, int max_group) {
    Plan p;
    p.hpc = kSlots / Sq;
    p.nchunk = cdiv(max_group, p.hpc);
    p.ntiles = cdiv(Sk, kTile);
    const long long base = static_cast<long long>(B) * Hkv * p.nchunk;
    const int want = static_cast<int>(imax(1, static_cast<int>((kTargetGroups + base - 1) / base)));
    p.tps = imin(p.ntiles, imax(kMinTilesPerSplit, cdiv(p.ntiles, want)));
    p.nsplit = cdiv(p.ntiles, p.tps);
    return p;
}

// Query slot n (lane % 32) of chunk `chunk`: head index within the kv-head's
// group and query row; valid only if the slot holds a real (head, row).
struct Slot {
    int hh;    // index in the group
    int i;     // query row, 0 .. Sq-1
    bool valid;
};
__host__ __device__ inline Slot slot_of(int n, int chunk, int hpc, int Sq, int group_size) {
    Slot s;
    s.hh = chunk * hpc + n / Sq;
    s.i = n % Sq;
    s.valid = n < hpc * Sq && s.hh < group_size;
    if (!s.valid) {   // read a real row (the group's first head, row 0); never stored
        s.hh = 0;
        s.i = 0;
    }
    return s;
}

// A chunk holds at least one real head (slot 0 is then valid).
__host__ __device__ inline bool chunk_has_work(int chunk, int hpc, int group_size) {
    return chunk * hpc < group_size;
}

// Rows of this slot's head in the 32-slot rowmax table: [first, first + Sq).
__host__ __device__ inline int head_first_slot(int n, int Sq) { return (n / Sq) * Sq; }

// Key row read by a lane for a tile at n0 (rows past the cache read the last row).
__host__ __device__ inline int key_row(int n0, int r, int Sk) { return imin(n0 + r, Sk - 1); }

// Tiles [t0, t1) of split s.
__host__ __device__ inline int split_first_tile(int s, int tps) { return s * tps; }
__host__ __device__ inline int split_end_tile(int s, int tps, int ntiles) { return imin((s + 1) * tps, ntiles); }
// The tile prefetched in the iteration of tile t (the next one, or t itself at the end).
__host__ __device__ inline int prefetch_tile(int t, int t1) { return imin(t + 1, t1 - 1); }

// Visible keys of a tile at n0 for query row i: key_offset < limit, with
// key_offset = (r >> 2) * 8 + (r & 3) for score register r and lane half g.
__host__ __device__ inline int mask_limit(int n0, int Sq, int Sk, int i, int g, bool causal) {
    int lim = Sk - n0 - g * 4;
    if (causal) lim = imin(lim, (Sk - Sq + i) - n0 - g * 4 + 1);
    return lim;
}

// Index of a partial result row: [B*Hkv, nchunk, nsplit, 32].
__host__ __device__ inline size_t partial_row(int bkv, int chunk, int split, int n, const Plan& p) {
    return ((static_cast<size_t>(bkv) * p.nchunk + chunk) * p.nsplit + split) * kSlots + n;
}

// Workspace: partial O [rows, D] fp32, then m and l [rows] fp32, 256-byte aligned pieces.
__host__ __device__ inline size_t partial_rows(int B, int Hkv, const Plan& p) {
    return static_cast<size_t>(B) * Hkv * p.nchunk * p.nsplit * kSlots;
}
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
__host__ __device__ inline size_t ws_m_offset(size_t rows, int D) { return align256(rows * D * 4); }
__host__ __device__ inline size_t ws_l_offset(size_t rows, int D) { return ws_m_offset(rows, D) + align256(rows * 4); }
__host__ __device__ inline size_t ws_bytes(size_t rows, int D) { return ws_l_offset(rows, D) + align256(rows * 4); }

}  // namespace dec
}  // namespace attn
