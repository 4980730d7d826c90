// Internal declarations shared by the host API and the kernel translation
// units of libattn.so.  Not part of the public ABI (that is include/attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "attn.h"

namespace attn {

// Quantisation blocks: rows of Q per scale, rows of (smoothed) K per scale.
constexpr int kBQ = 128;
constexpr int kBK = 64;

// Forward tiling: a workgroup owns BM query rows (4 waves x 32 rows) and walks
// the keys BN at a time.  BM == kBQ and BN == kBK, so one Q scale covers a
// workgroup and one K scale covers a key tile.
constexpr int kBM = 128;
constexpr int kBN = 64;
static_assert(ATTN_MASK_TILE_Q == kBM && ATTN_MASK_TILE_K == kBN, "tile masks use the forward tiles");
constexpr int kFwdThreads = 256;

// K column sums: tokens per partial-sum chunk.
constexpr int kSumChunk = 256;

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

struct QuantWorkspace {
    long long* partial;   // [B*Hkv, <= nchunk, D] exact channel sums, units of 2^-24 (K);
                          // [B*Hkv, nchunk, D] channel maxima as fp32 (the 8-bit V)
    float* mean;          // [B*Hkv, D] (part of the workspace size; no kernel needs it)
    int nchunk;           // chunks of kSumChunk tokens
};

// Offsets of the workspace pieces for a shape (256-byte aligned pieces).
size_t quant_workspace_layout(const attn_shape& s, size_t* mean_offset, int* nchunk);

// The device address of the library's no-allocation scratch (ATTN_NOALLOC_
// SCRATCH_BYTES, one copy per device) on the current device, looked up once
// per device; ATTN_ELAUNCH when the lookup fails.
int noalloc_scratch(void** ptr);

// q may be null (K only): then q_i8 and q_scale are not touched.  fp8
// selects E4M3 codes (stored in the int8 buffers) instead of INT8.
int launch_quantize(const attn_shape& s, const void* q, const void* k, int8_t* q_i8,
                    float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                    const QuantWorkspace& ws, hipStream_t st, bool fp8 = false);

// Per-channel E4M3 V, transposed into [B*Hkv, D, 64*ceil(S/64)] codes, and
// its scales [B*Hkv, D]; uses the partial-sum area of the workspace.
int launch_quantize_v_fp8(const attn_shape& s, const void* v, uint8_t* vt, float* v_scale,
                          const QuantWorkspace& ws, hipStream_t st);

struct FwdParams {
    const void* q;        // fp16 or int8 [B,Hq,S,D]
    const void* k;        // fp16 or int8 [B,Hkv,S,D]
    const void* v;        // fp16 [B,Hkv,S,D]
    void* o;              // fp16 [B,Hq,S,D]
    float* lse;           // fp32 [B,Hq,S] or null
    const float* q_scale; // int8 path: [B,Hq,nqblk]
    const float* k_scale; // int8 path: [B,Hkv,nkblk]
    int32_t* s_out;       // score dump: [B,Hq,ntiles*BM,S] (rows of query tiles tile_lo..)
    float* q_scale_out;   // fused-Q INT8 path: the Q block scales, [B,Hq,nqblk], or null
    const float* v_scale; // 8-bit P.V path: per-channel V scales [B,Hkv,D]
    const int32_t* mask_rowptr;  // tile-mask paths: [nqt + 1] list offsets per query tile
    const int32_t* mask_cols;    // [mask_nnz] entries (key tile << 2) | type
    int mask_nnz;
    int B, Hq, Hkv, S;
    int nqt;              // query tiles in the sequence
    int nqblk, nkblk;     // scale blocks per (b, head)
    int tile_lo, ntiles;  // query tiles handled by this launch
    float scale_log2;     // sm_scale * log2(e)
    int group;            // q-heads per kv-head when every kv-head has the same number, else 1
    uint8_t kvmap[ATTN_MAX_HEADS];   // q-head -> kv-head
    uint8_t horder[ATTN_MAX_HEADS];  // q-heads ordered by kv-head (launch order)
};

// kFp8: E4M3 Q/K codes (v_mfma_f32_32x32x64_f8f6f4), FP16 P.V.
// kInt8Pv8: INT8 Q/K, E4M3 P and per-channel E4M3 V (transposed tiles).
// kFp16Mask / kInt8Mask: the FP16 / INT8 forward under a tile-mask list.
// kDumpInt8 / kDumpInt8FusedQ: the INT8 forward (from INT8 Q, or from fp16 Q
// quantised in the kernel) writing its INT32 score tiles instead of O.
enum class FwdKind { kFp16, kInt8, kDumpInt8, kDumpInt8FusedQ, kInt8FusedQ, kFp8, kInt8Pv8, kFp16Mask, kInt8Mask };

int launch_fwd(FwdKind kind, int head_dim, bool causal, const FwdParams& p, hipStream_t st);

// KV-cache (decode) attention: Sq <= 32 queries per head over Sk cached keys.
struct DecParams {
    const void* q;        // fp16 [B,Hq,Sq,D]
    const void* k;        // int8 or fp16 [B,Hkv,Sk,D]
    const void* v;        // fp16 [B,Hkv,Sk,D]
    void* o;              // fp16 [B,Hq,Sq,D]
    float* lse;           // fp32 [B,Hq,Sq] or null
    const float* k_scale; // INT8 path: [B,Hkv,nkblk]
    float* q_scale_out;   // INT8 path: the per-head Q block scales [B,Hq], or null
    float* ws_o;          // partial results (see decode_geometry.h)
    float* ws_m;
    float* ws_l;
    int B, Hq, Hkv, Sq, Sk, nkblk;
    int hpc, nchunk, ntiles, tps, nsplit;   // the launch plan
    float scale_log2;
    uint16_t gstart[ATTN_MAX_HEADS];  // first position of kv-head k's group in horder
    uint16_t gcount[ATTN_MAX_HEADS];  // size of that group
    uint8_t horder[ATTN_MAX_HEADS];   // q-heads ordered by kv-head
};

int launch_decode(bool int8, int head_dim, bool causal, const DecParams& p, hipStream_t st);

}  // namespace attn
