// Fused attention forward for gfx950: tiled, online softmax; the work items
// are (batch, q-head, 128-row query tile), one or two per workgroup.
//
// What is computed (cited by page title and section):
//   "注意力即一切：从 MHA 到 GQA" §2.2: scores Q K^T, softmax of the scaled
//   scores, weighted sum of V; §2.3: causal mask; §4.1/§5.1: MQA/GQA head
//   sharing; §8.2: tiles of Q and K in on-chip memory plus an online softmax.
//   "FlashAttention" guide (aiunderstanding.org): the online softmax keeps
//   running maxima and sums and rescales partial results as tiles arrive, so
//   the final normalisation is exact and the N x N matrix never reaches HBM.
//   SageAttention article ("又快又准，即插即用！清华8比特量化Attention…"),
//   技术方案: INT8 Q K^T with INT32 accumulation, dequantised with the block
//   scales; P and V stay FP16 for P V.  (The article's FP16 accumulator for
//   P V has no counterpart among the gfx950 FP16 MFMAs, which accumulate in
//   FP32; FP32 is used.)
//
// gfx950 design:
//   * 4 waves, each owning 32 query rows.  Scores are computed transposed,
//     S^T = K Q^T, with v_mfma_f32_32x32x16_f16 (FP16 path) or
//     v_mfma_i32_32x32x32_i8 (INT8 path): Q stays in VGPRs as the B operand
//     for the whole kernel, K tiles are the A operand from LDS.  In the
//     32x32 accumulator layout a lane then holds ONE query column and 16
//     keys, so the row max needs one cross-lane swap (v_permlane32_swap) and
//     the row sum none until the end.
//   * The output is accumulated transposed too, O^T += V^T P^T: P^T is the
//     B operand taken straight from the score registers (no data movement),
//     V^T is the A operand read from a row-major V tile in LDS with
//     ds_read_b64_tr_b16 (a transposing LDS read), and the accumulator rows
//     that a lane rescales all belong to its own query.
//   * Software pipeline: while a wave runs the softmax of key tile j on the
//     VALU, it already issues the MFMAs of the scores of tile j+1, so the
//     matrix and vector pipes overlap inside one wave (and across the two
//     waves that share a SIMD).  K tiles are therefore staged one tile ahead
//     of V tiles, with one barrier per key tile.  The two waves of a SIMD
//     alternate through a raised wave priority over the score MFMAs and
//     exponentials, so one wave's P.V MFMAs and row maxima fill the other's
//     softmax.
//   * Direct-to-LDS staging: K and V tiles go from HBM into LDS with
//     global_load_lds_dwordx4 (no VGPRs, no LDS store instructions) into
//     three (FP16 at D = 128: two) stages per tile kind; the stages are
//     unpadded and XOR-swizzled in 16-byte chunks so that the MFMA operand
//     reads and the transposing reads are free of bank conflicts.  Tiles
//     past an item's last key tile are not copied.  Tile-masked lists longer
//     than the LDS copy of the list holds stage through registers into padded
//     rows instead.  The per-tile K scales are scalar loads, so the stage
//     barriers count copies only.  The INT8 kernel that quantises fp16 Q
//     itself stages Q through LDS too, ahead of the first tiles' copies, and
//     quantises it while they land.
//   * Lazy rescaling: the running maximum is only raised (and O, l rescaled)
//     when a tile's maximum exceeds it by more than 2^8; otherwise the stale
//     maximum is kept, weights stay <= 2^8 (exact in fp16 range), and the
//     final O / l is unchanged mathematically.  This removes the per-tile
//     multiply of the 64 O accumulators per lane in the steady state.
//   * Branch-free tails: K/V rows beyond the sequence are loaded from the
//     last row (clamped index) and masked to -inf, so no load is predicated.
//   * Workgroups are launched XCD-aware: consecutive hardware block ids go
//     round-robin over the 8 XCDs, so work items are numbered such that each
//     XCD receives a contiguous range of (batch, head) pairs ordered by kv
//     head; the q-heads of one GQA group then share K/V in that XCD's L2
//     (where a kv-head's K and V exceed the L2, the group's q-heads at the
//     same query tile are adjacent, so that they read each tile together).
//     Causal launches start with the heaviest (last) query tiles, and with
//     many items they give each workgroup two (a heavy and a light one, in
//     the snake order of geom::make_sched): the workgroups then carry equal
//     work, and the in-order dispatch over the XCDs no longer stalls on an
//     XCD whose slots are still busy.
#include "attn_internal.h"
#include "fwd_geometry.h"

#include <atomic>
#include <cfloat>
#include <type_traits>

namespace attn {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef int i16x __attribute__((ext_vector_type(16)));
typedef int i4x __attribute__((ext_vector_type(4)));
typedef int i8x __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __fp16 tr4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) tr4 lds_tr4;

constexpr float kLn2 = 0.6931471805599453f;
// INT8 scores start their INT32 accumulation at the bit pattern of the fp32
// value 1.5 * 2^23.  While |S32| < 2^22 (it is at most D * 127^2 = 2064512)
// the accumulator bits then read as the fp32 number 1.5 * 2^23 + S32
// exactly, so no integer-to-float conversion is needed; the bias is removed
// inside the fma that scales the score.
constexpr int kI8BiasBits = 0x4B400000;
constexpr float kI8Bias = 12582912.0f;
constexpr float kLazy = 8.0f;   // log2 headroom before the running max is raised

// F8: the 8-bit Q/K codes are E4M3 (FP8 alternative) instead of INT8.
// PV8: the 8-bit P.V ablation (E4M3 P, E4M3 V stored as V^T tiles, staged
// directly into LDS only).
template <int D, bool INT8, bool F8 = false, bool PV8 = false>
struct Cfg : geom::Stage<D, INT8> {
    using G = geom::Stage<D, INT8>;
    using G::KELT, G::KROWG, G::KCPR, G::VCPR, G::KPT, G::QSTEPS;
    static constexpr int KROW = KROWG + 16;                    // K row bytes in LDS
    static constexpr int VROW = 2 * D + 64;                    // V row bytes in LDS (register staging)
    static constexpr int VPT = G::VPT;
    static constexpr int KBYTES = kBN * KROW;
    static constexpr int VBYTES = kBN * VROW;
    static constexpr int KSTAGE = kBN * KROWG;                 // unpadded tiles (direct-to-LDS staging)
    static constexpr int VSTAGE = PV8 ? D * kBN : kBN * 2 * D; // (PV8: D rows of 64 key codes)
    static constexpr int DT = D / 32;                          // 32-row d tiles of O^T
    static_assert(kBN * KCPR % kFwdThreads == 0 && kBN * VCPR % kFwdThreads == 0, "tile split");
    static_assert(geom::kTileM == kBM && geom::kTileN == kBN && geom::kThreads == kFwdThreads, "geometry");
    static_assert(!F8 || (INT8 && QSTEPS % 2 == 0), "FP8 scores pair two 16-byte k-steps");
    typedef std::conditional_t<INT8, i4x, h8> qfrag_t;         // B operand fragment of Q
    typedef std::conditional_t<INT8 && !F8, i16x, f16x> acc_t; // 32x32 score accumulator
};

__device__ __forceinline__ h8 join(tr4 a, tr4 b) {
    h8 r;
    __builtin_memcpy(&r, &a, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &b, 8);
    return r;
}

__device__ __forceinline__ h8 pack8(float a0, float a1, float a2, float a3, float a4, float a5,
                                    float a6, float a7) {
    const h2 p0 = __builtin_convertvector((f2){a0, a1}, h2);
    const h2 p1 = __builtin_convertvector((f2){a2, a3}, h2);
    const h2 p2 = __builtin_convertvector((f2){a4, a5}, h2);
    const h2 p3 = __builtin_convertvector((f2){a6, a7}, h2);
    const h4 lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
    const h4 hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// x combined with the same register of lane ^ 32 (the other half of this
// lane's query row), without an LDS round trip.
__device__ __forceinline__ float row_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
    return a > b ? a : b;
}
__device__ __forceinline__ int row_max_i(int x) {
    const auto r = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(x), static_cast<unsigned>(x), false, false);
    return max(static_cast<int>(r[0]), static_cast<int>(r[1]));
}
// Maximum of the non-negative values v over the 64 lanes of the wave, read
// from lane 63: prefix maxima within each 16-lane row by the DPP row shifts
// 1, 2, 4, 8, then the row broadcasts of lanes 15 and 31 into the rows above
// (lanes shifted in from outside a row, and rows outside a broadcast's row
// mask, take 0, which leaves a maximum of non-negative values unchanged).
// All VALU: no LDS round trip per step as with cross-lane shuffles.
__device__ __forceinline__ unsigned wave_max_nonneg(unsigned v) {
    v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, true)));
    v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, true)));
    v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, true)));
    v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, true)));
    v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xa, 0xf, false)));
    v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xc, 0xf, false)));
    return static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}
__device__ __forceinline__ float row_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Direct-to-LDS staging synchronisation: wait until at most VM vector-memory
// operations of this wave are outstanding (its earlier tile copies have
// landed in LDS) and its own LDS reads are done, then a workgroup barrier.
// A bare s_barrier, because __syncthreads also waits for every outstanding
// copy, which would drain the prefetch; the empty asm statements keep the
// compiler from moving memory operations across the wait and the barrier.
template <int VM>
__device__ __forceinline__ void lds_stage_barrier() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((VM & 0xF) | (0x7 << 4) | (0x0 << 8) | ((VM >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Direct-to-LDS copies: 16 bytes per lane from base + off[i] into the LDS
// block at lds + 1024 i + 16 * lane (global_load_lds_dwordx4, saddr form),
// N of them in one inline-asm block.  Issued with the builtin, the
// compiler's wait counting treats every LDS read as unordered while such a
// copy is in flight and drains all LDS reads (lgkmcnt(0)) wherever it waits
// for one; the copies' completion is tracked by the explicit waits of
// lds_stage_barrier in any case.  The copies take their LDS address from
// M0, which the compiler reserves (it ignores M0 in a clobber list), so each
// block saves M0 into an SGPR of its own at its head and restores it at its
// tail: no value the compiler keeps in M0 is changed.  The s_nop 4 covers
// the wait states after a vector instruction that wrote an SGPR the copies
// read (every input is written before the block; the hazard recognizer does
// not look at asm inputs), each s_nop 0 the M0 write before an LDS DMA.
template <int N>
__device__ __forceinline__ void dtl_copies(const char* base, const uint32_t (&off)[N], const char* lds) {
    static_assert(N == 1 || N == 2 || N == 4, "copies per block");
    const uint32_t l0 = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)lds));
    uint32_t saved_m0;
    if constexpr (N == 1) {
        asm volatile("s_mov_b32 %0, m0\n\ts_nop 4\n\t"
                     "s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(saved_m0) : "v"(off[0]), "s"(base), "s"(l0) : "memory");
    } else if constexpr (N == 2) {
        const uint32_t l1 = l0 + 1024;
        asm volatile("s_mov_b32 %0, m0\n\ts_nop 4\n\t"
                     "s_mov_b32 m0, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %3\n\t"
                     "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(saved_m0) : "v"(off[0]), "v"(off[1]), "s"(base), "s"(l0), "s"(l1) : "memory");
    } else {
        const uint32_t l1 = l0 + 1024, l2 = l0 + 2048, l3 = l0 + 3072;
        asm volatile("s_mov_b32 %0, m0\n\ts_nop 4\n\t"
                     "s_mov_b32 m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %5\n\t"
                     "s_mov_b32 m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %5\n\t"
                     "s_mov_b32 m0, %8\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %5\n\t"
                     "s_mov_b32 m0, %9\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, %5\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(saved_m0)
                     : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(base), "s"(l0), "s"(l1),
                       "s"(l2), "s"(l3)
                     : "memory");
    }
}

#ifndef ATTN_FWD_DTL
#define ATTN_FWD_DTL 1
#endif

typedef const __attribute__((address_space(3))) char* lds_cptr;

// Scores of one 64-key tile (FP16 or INT8) as score_tile computes them (same
// MFMAs in the same order), from per-lane LDS addresses of the K chunks the
// wave reads at each k-step, given for query-row block 0 (block 1 lies 32
// rows further: the swizzle repeats every 32 rows at these row sizes).
template <int D, bool INT8, bool BIASED, int N, typename QF, typename ACC>
__device__ __forceinline__ void score_tile_at(const lds_cptr (&ka)[N], const QF* qf, ACC* acc,
                                              const ACC* init = nullptr) {
    using C = Cfg<D, INT8, false>;
    static_assert(N == C::QSTEPS, "one address per k-step");
    static_assert(32 % geom::Dtl<C::KROWG>::RPL == 0 && (32 / geom::Dtl<C::KROWG>::RPL) % geom::Dtl<C::KROWG>::CPR == 0,
                  "the K swizzle must repeat every 32 rows");
    static_assert(!BIASED || INT8, "the bias applies to INT32 accumulators");
    if (init) {
        acc[0] = *init;
        acc[1] = *init;
    } else if constexpr (BIASED) {
        acc[0] = kI8BiasBits;
        acc[1] = kI8BiasBits;
    } else {
        acc[0] = ACC{};
        acc[1] = ACC{};
    }
#pragma unroll
    for (int s = 0; s < C::QSTEPS; ++s)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            if constexpr (INT8) {
                typedef const __attribute__((address_space(3))) i4x lds_i4x;
                const i4x a = *(lds_i4x*)(ka[s] + mt * 32 * C::KROWG);
                acc[mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[s], acc[mt], 0, 0, 0);
            } else {
                typedef const __attribute__((address_space(3))) h8 lds_h8;
                const h8 a = *(lds_h8*)(ka[s] + mt * 32 * C::KROWG);
                acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[s], acc[mt], 0, 0, 0);
            }
        }
}

// Transposed scores of one 64-key tile for this wave's 32 queries:
// acc[mt] holds keys mt*32 + (r/4)*8 + (lane/32)*4 + r%4 (register r) of query
// lane%32.  The same code feeds the forward and the INT32 score dump.
// For F8 two consecutive 16-byte k-steps form one 32-byte operand of
// v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32 accumulation); A and B take
// their bytes from the same k positions, so the products pair up as in the
// INT8 form.
template <int D, bool INT8, bool F8 = false, bool BIASED = false, bool SWZ = false>
__device__ __forceinline__ void score_tile(const char* ks, const typename Cfg<D, INT8, F8>::qfrag_t* qf,
                                           int l32, int g, typename Cfg<D, INT8, F8>::acc_t acc[2]) {
    using C = Cfg<D, INT8, F8>;
    // 16-byte chunk `chunk` of K row `row`: padded rows, or the swizzled
    // unpadded rows of direct-to-LDS staging
    auto kchunk = [&](int row, int chunk) -> const char* {
        if constexpr (SWZ) return ks + row * C::KROWG + ((chunk ^ geom::Dtl<C::KROWG>::k_swz(row)) << 4);
        else return ks + row * C::KROW + (chunk << 4);
    };
    static_assert(!BIASED || (INT8 && !F8), "the bias applies to INT32 accumulators");
    if constexpr (BIASED) {
        acc[0] = kI8BiasBits;
        acc[1] = kI8BiasBits;
    } else {
        acc[0] = typename C::acc_t{};
        acc[1] = typename C::acc_t{};
    }
    if constexpr (F8) {
#pragma unroll
        for (int s2 = 0; s2 < C::QSTEPS / 2; ++s2) {
            const i8x b = __builtin_shufflevector(qf[2 * s2], qf[2 * s2 + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const i4x a0 = *reinterpret_cast<const i4x*>(kchunk(mt * 32 + l32, 2 * (2 * s2) + g));
                const i4x a1 = *reinterpret_cast<const i4x*>(kchunk(mt * 32 + l32, 2 * (2 * s2 + 1) + g));
                const i8x a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
                acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[mt], 0, 0, 0, 0, 0, 0);
            }
        }
        return;
    }
#pragma unroll
    for (int s = 0; s < C::QSTEPS; ++s) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            if constexpr (INT8) {
                const i4x a = *reinterpret_cast<const i4x*>(kchunk(mt * 32 + l32, 2 * s + g));
                acc[mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[s], acc[mt], 0, 0, 0);
            } else {
                const h8 a = *reinterpret_cast<const h8*>(kchunk(mt * 32 + l32, 2 * s + g));
                acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[s], acc[mt], 0, 0, 0);
            }
        }
    }
}

using geom::key_offset;

// Waves per SIMD the register allocation targets: two (up to 256 registers
// a lane), or three (168) at head_dim 64 where that fits without spilling
// (INT8, and the unmasked non-causal FP16 kernel): same-run A/B on the
// head_dim-64 video workload +4 % INT8, +2 % FP16.
constexpr int fwd_waves(int D, bool INT8, bool CAUSAL, bool BMASK) {
    return D == 64 && (INT8 || (!CAUSAL && !BMASK)) ? 3 : 2;
}

template <int D, bool INT8, bool CAUSAL, bool DUMP, bool QF16 = false, bool F8 = false, bool PV8 = false,
          bool BMASK = false, bool MLDS = false>
__global__ __launch_bounds__(kFwdThreads)
__attribute__((amdgpu_waves_per_eu(fwd_waves(D, INT8, CAUSAL, BMASK), fwd_waves(D, INT8, CAUSAL, BMASK))))
void fwd_kernel(const FwdParams p_in) {
    static_assert(!QF16 || INT8, "in-kernel Q quantisation is an INT8 forward variant");
    static_assert(!F8 || (INT8 && !DUMP && !QF16 && !PV8), "FP8 scores: standalone-quantised Q/K");
    static_assert(!PV8 || (INT8 && !DUMP && !QF16 && !F8), "8-bit P.V: INT8 Q/K");
    static_assert(!BMASK || (!CAUSAL && !DUMP && !QF16 && !F8 && !PV8), "tile masks: FP16 or two-call INT8");
    static_assert(!MLDS || BMASK, "the LDS copy of the key-tile list belongs to the tile-masked forward");
    using C = Cfg<D, INT8, F8, PV8>;
    typedef typename C::qfrag_t qfrag_t;
    typedef typename C::acc_t acc_t;
    // Staging: direct-to-LDS copies into unpadded swizzled stages (NST of
    // them, one array each so that the compiler can tell the copies of
    // different stages apart), or the register path into padded tiles
    // (tile-mask lists too long for their LDS copy).  The INT32 score dump
    // (DUMP) runs the direct-to-LDS INT8 pipeline of the forward itself --
    // the same K copies, stages, swizzle and score MFMAs, with or without
    // the in-kernel Q quantisation -- and writes each tile's INT32 scores
    // instead of running the softmax and P.V (it copies no V tiles).
    // (the tile-masked variant stages directly only with its key-tile list
    // copied into LDS first (MLDS): read per iteration from global memory, the
    // wave-uniform entry loads would become vector loads queued behind the
    // copies into LDS; lists too long for the LDS copy keep the register path)
    constexpr bool DTL = ATTN_FWD_DTL && (!BMASK || MLDS);
    static_assert(!DUMP || (DTL && INT8 && !F8 && !PV8), "the score dump runs the direct-to-LDS INT8 forward");
    static_assert(!PV8 || DTL, "the 8-bit P.V variant stages its V^T tiles directly into LDS");
    __shared__ int mlist[MLDS ? geom::kMaskListMax : 1];
#ifndef ATTN_FWD_NST_F16_D128
#define ATTN_FWD_NST_F16_D128 2
#endif
    constexpr int NST = (!INT8 && D == 128) ? ATTN_FWD_NST_F16_D128 : 3;
    __shared__ __attribute__((aligned(16))) char smem[DTL ? 16 : 2 * C::KBYTES + 2 * C::VBYTES];
    __shared__ __attribute__((aligned(16))) char dk0[DTL ? C::KSTAGE : 16], dk1[DTL ? C::KSTAGE : 16],
        dk2[DTL && NST == 3 ? C::KSTAGE : 16];
    __shared__ __attribute__((aligned(16))) char dv0[DTL ? C::VSTAGE : 16], dv1[DTL ? C::VSTAGE : 16],
        dv2[DTL && NST == 3 ? C::VSTAGE : 16];
    auto kbuf = [&](int i) { return smem + i * C::KBYTES; };
    auto vbuf = [&](int i) { return smem + 2 * C::KBYTES + i * C::VBYTES; };

    // ---- this workgroup's work items (batch, q-head, query tile) ----
    // One item per workgroup, or (causal launches with many items) several
    // per workgroup in the snake order of geom::make_sched: the dispatch gap
    // between workgroups then recurs per several items, and the heaviest-
    // first query tiles pair up with light ones.
    constexpr bool PERSIST = CAUSAL && !BMASK;
    const geom::Sched sched = geom::make_sched(blockIdx.x, gridDim.x, p_in.B * p_in.Hq * p_in.ntiles);
    const int n_iter = PERSIST ? geom::sched_iters(sched) : 1;
    for (int it = 0; it < n_iter; ++it) {
    const int item = geom::sched_item(sched, it);
    if (item < 0) continue;
    // The parameters are read through the kernel-argument pointer, made
    // opaque per item, and the thread id likewise: otherwise the compiler
    // hoists every parameter load and the per-lane address arithmetic out of
    // the item loop and keeps them live across the body, which spills and
    // costs the P.V loads their read-ahead.  (p_in is the only argument.)
    typedef const __attribute__((address_space(4))) FwdParams KParams;
    KParams* pk = (KParams*)__builtin_amdgcn_kernarg_segment_ptr();   // (address-space cast)
    int tid = threadIdx.x;
    if constexpr (PERSIST) {
        asm volatile("" : "+s"(pk));
        asm volatile("" : "+v"(tid));
    }
    KParams& p = *pk;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int S = p.S;
    // The softmax scale, read once per item into a register the compiler
    // cannot re-derive: read through p inside the key loop it becomes a
    // scalar load per tile whose wait (lgkmcnt) also drains the LDS reads.
    float scale_log2 = p.scale_log2;
    if constexpr (PERSIST) asm volatile("" : "+s"(scale_log2));
    // (tile masks are mostly causal-like too, heavier for later query tiles)
    const geom::BlockCoord bc = geom::decode_item(item, p.Hq, p.ntiles, p.tile_lo, CAUSAL || BMASK, p.group);
    const int b = bc.b;
    const int h = p.horder[bc.pos];
    const int kvh = p.kvmap[h];
    const int qt = bc.qt;

    const int q0 = qt * kBM;
    const int qw0 = q0 + wave * 32;      // first query row of this wave
    const int qi = qw0 + l32;            // this lane's query row
    const size_t bhq = static_cast<size_t>(b) * p.Hq + h;
    const size_t bhk = static_cast<size_t>(b) * p.Hkv + kvh;

    // Tile-mask variant (the APB page's FlashAttention kernel with a changed
    // mask shape): the key tiles of this query tile come from its run of the
    // mask list, in list order; a query tile with an empty run has no visible
    // key (O = 0, lse = -inf).
    geom::MaskRow mrow{0, 0};
    if constexpr (BMASK) {
        mrow = geom::mask_row(p.mask_rowptr[qt], p.mask_rowptr[qt + 1], p.mask_nnz, p.nkblk);
        if (mrow.count == 0) {
            if (qi < S) {
                _Float16* orow = static_cast<_Float16*>(p.o) + (bhq * S + static_cast<size_t>(qi)) * D;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) *reinterpret_cast<h4*>(orow + geom::o_column(dt, j4, g)) = h4{};
                if (p.lse && g == 0) p.lse[bhq * S + qi] = -INFINITY;
            }
            continue;
        }
        if constexpr (MLDS) {
            // the workgroup's run of the list into LDS (count <= nkblk <= kMaskListMax,
            // which the launch checks; clamped again here)
            const int n = geom::imin(mrow.count, geom::kMaskListMax);
            for (int i = tid; i < n; i += kFwdThreads) mlist[i] = p.mask_cols[mrow.base + i];
            mrow.count = n;
            __syncthreads();
        }
    }
    // list entry at position pos (positions past the end repeat the last one)
    auto mask_entry = [&](int pos) -> int {
        if constexpr (MLDS) return mlist[geom::imin(pos, mrow.count - 1)];
        else return p.mask_cols[geom::mask_entry_index(mrow, pos)];
    };
    // first key of the tile at list position pos (BMASK), else tile pos itself
    auto tile_row = [&](int pos) -> int {
        if constexpr (BMASK) return geom::mask_entry_tile(mask_entry(pos), p.nkblk) * kBN;
        else return pos * kBN;
    };
    auto tile_type = [&](int pos) -> int {
        if constexpr (BMASK) return geom::mask_entry_type(mask_entry(pos));
        else return CAUSAL ? 2 : 1;
    };
    const int nkt = BMASK ? mrow.count : geom::block_key_tiles(S, q0, CAUSAL);      // key tiles of the block
    const int nkt_w = BMASK ? nkt : geom::wave_key_tiles(nkt, qw0, CAUSAL);         // key tiles this wave needs

    // ---- K / V staging: each thread moves KPT (VPT) 16-byte chunks per tile.
    // Rows past the sequence are read from row S-1 (always in bounds) and
    // masked out of the softmax.
    const char* kg = static_cast<const char*>(p.k) + bhk * S * C::KROWG;
    const int vt_stride = p.nkblk * kBN;   // PV8: key columns per V^T row
    const char* vg = static_cast<const char*>(p.v) +
                     (PV8 ? bhk * static_cast<size_t>(D) * vt_stride : bhk * S * C::VROWG);
    // Addresses: a wave-uniform tile base plus a 32-bit per-lane offset
    // (row clamped to the sequence), so the loads use the scalar-base form.
    // Register sets for staging (a second set when prefetching two tiles ahead).
    constexpr int DEPTH = geom::fwd_prefetch_depth(D, INT8);
    i4x kreg[DEPTH][C::KPT], vreg[DEPTH][C::VPT];
    auto gload_k = [&](int n0, i4x (&dst)[C::KPT]) {
        const int first = geom::tile_first_row(n0, S);
        const char* base = kg + static_cast<size_t>(first) * C::KROWG;
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) {
            const int c = tid + kFwdThreads * i;
            const uint32_t off = static_cast<uint32_t>(geom::tile_lane_row(c / C::KCPR, first, S)) * C::KROWG +
                                 (c % C::KCPR) * 16;
            dst[i] = *reinterpret_cast<const i4x*>(base + off);
        }
    };
    auto gload_v = [&](int n0, i4x (&dst)[C::VPT]) {
        const int first = geom::tile_first_row(n0, S);
        const char* base = vg + static_cast<size_t>(first) * C::VROWG;
#pragma unroll
        for (int i = 0; i < C::VPT; ++i) {
            const int c = tid + kFwdThreads * i;
            const uint32_t off = static_cast<uint32_t>(geom::tile_lane_row(c / C::VCPR, first, S)) * C::VROWG +
                                 (c % C::VCPR) * 16;
            dst[i] = *reinterpret_cast<const i4x*>(base + off);
        }
    };
    auto sstore_k = [&](int stage, const i4x (&src)[C::KPT]) {
        char* ks = kbuf(stage);
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) {
            const int c = tid + kFwdThreads * i;
            *reinterpret_cast<i4x*>(ks + (c / C::KCPR) * C::KROW + (c % C::KCPR) * 16) = src[i];
        }
    };
    auto sstore_v = [&](int stage, const i4x (&src)[C::VPT]) {
        char* vs = vbuf(stage);
#pragma unroll
        for (int i = 0; i < C::VPT; ++i) {
            const int c = tid + kFwdThreads * i;
            *reinterpret_cast<i4x*>(vs + (c / C::VCPR) * C::VROW + (c % C::VCPR) * 16) = src[i];
        }
    };

    // direct-to-LDS copies of one tile into a stage: instruction i of this
    // wave fills bytes (wave*NI + i)*1024 .. +1023 of the stage; each lane
    // fetches the logical chunk its slot holds (row clamped to the sequence)
    using DK = geom::Dtl<C::KROWG>;
    using DV = geom::Dtl<2 * D>;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    // Per-lane offsets of a whole tile (no row clamped), the same for every
    // tile.  Made opaque so that the compiler keeps them as they are rather
    // than folding them into the clamped form it computes per tile.  (Not in
    // the one-item head_dim-64 kernels: there the extra registers spill.)
    constexpr bool WHOLE = PERSIST || D == 128;
    uint32_t koff_whole[DK::NI], voff_whole[DV::NI];
    if constexpr (WHOLE) {
#pragma unroll
        for (int i = 0; i < DK::NI; ++i) {
            const int r = DK::slot_row(wave, i, lane);
            koff_whole[i] = static_cast<uint32_t>(r) * C::KROWG + (DK::slot_chunk(wave, i, lane) ^ DK::k_swz(r)) * 16;
            asm volatile("" : "+v"(koff_whole[i]));
        }
#pragma unroll
        for (int i = 0; i < DV::NI; ++i) {
            const int r = DV::slot_row(wave, i, lane);
            voff_whole[i] = static_cast<uint32_t>(r) * C::VROWG + (DV::slot_chunk(wave, i, lane) ^ DV::v_swz(r)) * 16;
            asm volatile("" : "+v"(voff_whole[i]));
        }
    }
    auto dtl_k = [&](int n0, char* st) __attribute__((always_inline)) {
        const int first = geom::tile_first_row(n0, S);
        const char* base = kg + static_cast<size_t>(first) * C::KROWG;
        // A whole tile (every row inside the sequence: all but the last)
        // takes the unclamped offsets computed once per item.
        if (WHOLE && n0 + kBN <= S) {
            dtl_copies<DK::NI>(base, koff_whole, st + wave_s * DK::NI * 1024);
            return;
        }
        uint32_t off[DK::NI];
#pragma unroll
        for (int i = 0; i < DK::NI; ++i) {
            const int r = DK::slot_row(wave, i, lane);
            const int c = DK::slot_chunk(wave, i, lane) ^ DK::k_swz(r);
            off[i] = static_cast<uint32_t>(geom::tile_lane_row(r, first, S)) * C::KROWG + c * 16;
        }
        dtl_copies<DK::NI>(base, off, st + wave_s * DK::NI * 1024);
    };
    using D8 = geom::Dtl8<D>;
    constexpr int VNI = DUMP ? 0 : PV8 ? D8::NI : DV::NI;   // V copy instructions per wave per tile
    auto dtl_v = [&](int n0, char* st) __attribute__((always_inline)) {
        if constexpr (DUMP) return;   // (the score dump needs no V)
        if constexpr (PV8) {
            // D rows of 64 key codes of the V^T tile at column v8_tile_col
            const char* base = vg + geom::v8_tile_col(n0, p.nkblk);
            uint32_t off[D8::NI];
#pragma unroll
            for (int i = 0; i < D8::NI; ++i) {
                const int r = D8::slot_row(wave, i, lane);
                const int c = D8::slot_chunk(wave, i, lane) ^ D8::swz(r);
                off[i] = static_cast<uint32_t>(r) * vt_stride + c * 16;
            }
            dtl_copies<D8::NI>(base, off, st + wave_s * D8::NI * 1024);
            return;
        }
        const int first = geom::tile_first_row(n0, S);
        const char* base = vg + static_cast<size_t>(first) * C::VROWG;
        if (WHOLE && n0 + kBN <= S) {   // (a whole tile, as for K)
            dtl_copies<DV::NI>(base, voff_whole, st + wave_s * DV::NI * 1024);
            return;
        }
        uint32_t off[DV::NI];
#pragma unroll
        for (int i = 0; i < DV::NI; ++i) {
            const int r = DV::slot_row(wave, i, lane);
            const int c = DV::slot_chunk(wave, i, lane) ^ DV::v_swz(r);
            off[i] = static_cast<uint32_t>(geom::tile_lane_row(r, first, S)) * C::VROWG + c * 16;
        }
        dtl_copies<DV::NI>(base, off, st + wave_s * DV::NI * 1024);
    };
    char* dks[3] = {dk0, dk1, dk2};
    char* dvs[3] = {dv0, dv1, dv2};
    // head_dim 128, FP16 or INT8 codes: the K read addresses of every stage,
    // computed once per item and kept in registers (opaque to the compiler,
    // which otherwise re-adds the stage base to each lane offset per tile).
    constexpr bool KADDR = DTL && !F8 && D == 128;
    lds_cptr kaddr[3][C::QSTEPS];
    if constexpr (KADDR) {
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
            for (int s = 0; s < C::QSTEPS; ++s) {
                kaddr[st][s] = (lds_cptr)(dks[st] + l32 * C::KROWG + (((2 * s + g) ^ DK::k_swz(l32)) << 4));
                asm volatile("" : "+v"(kaddr[st][s]));
            }
    }
    // K scale of key tile t (clamped to the last block; tiles past the end are
    // never used).  The base and the block count are read once per item into
    // registers: read through p per tile, they are reloaded after every copy
    // block (whose memory clobber invalidates them).  The scales are read
    // through a constant-address-space pointer at a wave-uniform index, i.e.
    // with scalar loads: they count against neither the copies' wait counter
    // (a vector load would, and the compiler's wait for it would drain the
    // copies) nor, issued right before a stage barrier (which waits for the
    // LDS and scalar counter anyway), the LDS reads' waits inside a tile.
    // (The scales are written by the K quantiser before this kernel starts
    // and are read-only while it runs.)
    typedef const __attribute__((address_space(4))) float cfloat;
    cfloat* ks_base = (cfloat*)(p.k_scale + (INT8 && !DUMP ? bhk * p.nkblk : 0));
    int ks_last = p.nkblk - 1;
    if constexpr (PERSIST) {
        asm volatile("" : "+s"(ks_base));
        asm volatile("" : "+s"(ks_last));
    }
    auto kscale_at = [&](int t) -> float {
        if constexpr (BMASK) t = tile_row(t) / kBN;   // (list position -> key tile)
        return ks_base[__builtin_amdgcn_readfirstlane(geom::imin(t, ks_last))];
    };
    float ksring[3] = {1.0f, 1.0f, 1.0f};

    // The prologue's copies into LDS (K_0 .. K_{NST-1}, V_0 .. V_{NST-2})
    // and Q's loads overlap.  The FP16 kernels load Q first, so that the
    // first score tile waits for Q and K_0 only, not for the whole copy queue;
    // the INT8 kernel on INT8 Q issues the copies first.  The INT8 kernel
    // that quantises fp16 Q itself copies Q into LDS first, into the stages
    // of V_1 and V_2 (free until V_1's copies, which go out once every wave
    // has read its Q rows), then K_0, K_1, V_0 and K_2: it waits for Q's
    // copies alone (an explicit count of the copies after them), quantises Q
    // while the tiles land, and only then issues V_1.  (Loaded into
    // registers, Q would be waited for by the compiler, whose wait also
    // covers every copy issued after the loads.)  (Register staging: K_0's
    // loads go out before Q.)
    constexpr bool QFIRST = DTL && !INT8;
    constexpr bool QLDS = DTL && QF16;
    static_assert(!QLDS || NST == 3, "Q staging uses the stages of V_1 and V_2");
    // copies of the query block's fp16 rows q0 + 64 h .. q0 + 64 h + 63 (rows
    // past the sequence read row S-1) into a V-sized stage, 16-byte chunks
    // XOR-swizzled by row as in the K stages (row-wise reads below)
    auto dtl_q = [&](int h, char* st) __attribute__((always_inline)) {
        const int first = geom::tile_first_row(q0 + kBN * h, S);
        const char* base = static_cast<const char*>(p.q) + (bhq * S + static_cast<size_t>(first)) * C::VROWG;
        uint32_t off[DV::NI];
#pragma unroll
        for (int i = 0; i < DV::NI; ++i) {
            const int r = DV::slot_row(wave, i, lane);
            const int c = DV::slot_chunk(wave, i, lane) ^ DV::k_swz(r);
            off[i] = static_cast<uint32_t>(geom::tile_lane_row(r, first, S)) * C::VROWG + c * 16;
        }
        dtl_copies<DV::NI>(base, off, st + wave_s * DV::NI * 1024);
    };
    auto dtl_prologue = [&]() __attribute__((always_inline)) {
        dtl_k(tile_row(0), dks[0]);
        dtl_k(tile_row(1), dks[1]);
        dtl_v(tile_row(0), dvs[0]);
        if constexpr (NST == 3) {
            dtl_k(tile_row(2), dks[2]);
            dtl_v(tile_row(1), dvs[1]);
        }
    };
    if constexpr (DTL && !QFIRST) {
        if constexpr (QLDS) {
            dtl_q(0, dvs[1]);
            dtl_q(1, dvs[2]);
            dtl_k(tile_row(0), dks[0]);
            dtl_k(tile_row(1), dks[1]);
            dtl_v(tile_row(0), dvs[0]);
            dtl_k(tile_row(2), dks[2]);
        } else {
            dtl_prologue();
        }
        if constexpr (INT8 && !DUMP) {
#pragma unroll
            for (int t = 0; t < NST; ++t) ksring[t] = kscale_at(t);
        }
    } else if constexpr (!DTL) {
        gload_k(tile_row(0), kreg[0]);
    }

    // ---- Q fragment (B operand of S^T = K Q^T), kept in VGPRs.  Rows past
    // the sequence read the last row; they are never stored.
    qfrag_t qf[C::QSTEPS];
    float qscale_fused = 0.0f;
    if constexpr (!QF16) {
        const char* qrow = static_cast<const char*>(p.q) +
                           (bhq * S + static_cast<size_t>(geom::q_row(qi, S))) * (D * C::KELT);
#pragma unroll
        for (int s = 0; s < C::QSTEPS; ++s) {
            // 16 bytes per lane: int8 elements s*32 + g*16.., or fp16 elements s*16 + g*8..
            qf[s] = *reinterpret_cast<const qfrag_t*>(qrow + C::q_frag_offset(s, g));
        }
        if constexpr (QFIRST) dtl_prologue();
    } else {
        // In-kernel per-block quantisation of Q (SageAttention article,
        // 技术方案: INT8 Q with one scale per FlashAttention-sized block).  The
        // workgroup's 128 rows are exactly one Q block, so the block absmax is
        // a workgroup reduction and INT8 Q never goes through HBM.  Same rule
        // as the standalone quantiser: a = max|x|, r = 127/a, delta = a/127
        // (correctly rounded), q = clamp(rint(x * r), -127, 127); a == 0 gives
        // q = 0 and delta = 0.  Rows past the sequence repeat row S-1, which
        // leaves the maximum unchanged.
        h8 qraw[C::QSTEPS][2];
        if constexpr (QLDS) {
            // Q's copies have landed (those of K_0, K_1, V_0 and K_2 may not)
            lds_stage_barrier<3 * DK::NI + VNI>();
            const int rq = (wave & 1) * 32 + l32;   // row in the stage of this wave's half
            const char* qs = ((wave >> 1) ? dvs[2] : dvs[1]) + rq * C::VROWG;
#pragma unroll
            for (int s = 0; s < C::QSTEPS; ++s)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int c = C::q16_piece_offset(s, g, hh) / 16;
                    qraw[s][hh] = *reinterpret_cast<const h8*>(qs + ((c ^ DV::k_swz(rq)) << 4));
                }
        } else {
            const char* qrow = static_cast<const char*>(p.q) +
                               (bhq * S + static_cast<size_t>(geom::q_row(qi, S))) * (2 * D);
#pragma unroll
            for (int s = 0; s < C::QSTEPS; ++s)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    qraw[s][hh] = *reinterpret_cast<const h8*>(qrow + C::q16_piece_offset(s, g, hh));
        }
        // |x| max on the fp16 bit patterns: with the sign bit cleared, the
        // integer order of finite values' patterns is the order of their
        // magnitudes (two per 32-bit word, packed 16-bit maxima)
        u16x2 mx2 = {0, 0};
#pragma unroll
        for (int s = 0; s < C::QSTEPS; ++s)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const i4x w = __builtin_bit_cast(i4x, qraw[s][hh]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(u16x2, static_cast<unsigned>(w[e]) & 0x7fff7fffu));
            }
        // (the wave's maximum pattern, then its value: the same order)
        const unsigned mxw = wave_max_nonneg(mx2[0] > mx2[1] ? mx2[0] : mx2[1]);
        const float amax = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(mxw)));
        __shared__ float qmax[4];
        if (lane == 0) qmax[wave] = amax;
        // (LDS only: a full __syncthreads would also wait for the copies)
        if constexpr (QLDS) lds_stage_barrier<63>();
        else __syncthreads();
        const float a = __builtin_fmaxf(__builtin_fmaxf(qmax[0], qmax[1]), __builtin_fmaxf(qmax[2], qmax[3]));
        const float r = a == 0.0f ? 0.0f : __fdiv_rn(127.0f, a);
        qscale_fused = a == 0.0f ? 0.0f : __fdiv_rn(a, 127.0f);
        // q = rint(x * r): |x * r| <= 127 (1 + 2^-23) here, so the clamp to
        // [-127, 127] never acts, and adding 1.5 * 2^23 rounds x * r to an
        // integer (nearest, ties to even, as rint) whose two's-complement low
        // byte is the code.  The product is rounded on its own, as
        // fma(x, r, 0) (one rounding of the exact product, i.e. the fp32
        // product, which lets the fp16 x feed a mixed-precision FMA
        // directly), and the sum separately.
#pragma unroll
        for (int s = 0; s < C::QSTEPS; ++s) {
            uint32_t w[4];
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                uint32_t b[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
#pragma clang fp contract(off)
                    const float t = __builtin_fmaf(static_cast<float>(qraw[s][e4 >> 1][(e4 & 1) * 4 + e]), r, 0.0f);
                    b[e] = __float_as_uint(t + 12582912.0f);
                }
                const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);
                const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u);
                w[e4] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
            }
            __builtin_memcpy(&qf[s], w, 16);
        }
    }
    // V_1 into the stage Q has left (every wave read its Q rows before the
    // workgroup barrier of the block maximum)
    if constexpr (QLDS) dtl_v(tile_row(1), dvs[1]);

    // Visible keys of a tile at n0 satisfy key_offset(mt, r) < lim for this lane.
    auto mask_limit = [&](int n0) { return geom::mask_limit(n0, S, qi, g, CAUSAL); };
    auto tile_needs_mask = [&](int n0) { return (n0 + kBN > S) || (CAUSAL && n0 + kBN - 1 > qw0); };

    {
        float m_run = -INFINITY;   // running row max (log2 units); equal in lanes l and l^32
        float l_run = 0.0f;        // this lane's partial row sum
        f16x oacc[C::DT];
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) oacc[dt] = f16x{};
        // INT8: the per-tile score scale is (dQ sm_scale log2 e) dK_j
        float qscale_log2 = scale_log2;
        if constexpr (INT8 && !DUMP) qscale_log2 *= QF16 ? qscale_fused : p.q_scale[bhq * p.nqblk + qt];
        float m_thr = -INFINITY;   // m_run plus the lazy headroom: a tile max above it raises m_run
        const float* kscale = p.k_scale;

        // ---- prologue: K_0 -> LDS, S_0, then K_1 and V_0 -> LDS (and, at
        // depth 2, K_2 and V_1 into the second register set) ----
        constexpr bool kBiased = INT8 && !F8;   // INT32 scores read as biased fp32
        acc_t sc[2];
        // The accumulators' starting block (the bias bits), held in registers
        // for the whole item and opaque to the compiler, which would otherwise
        // re-create it with eight 64-bit moves per tile.
        acc_t bias_blk{};
        if constexpr (kBiased && KADDR) {
            bias_blk = kI8BiasBits;
            asm volatile("" : "+v"(bias_blk));
        }
        if constexpr (DTL) {
            // K_0 has landed (the INT8 kernel on INT8 Q: every prologue copy; the
            // others leave the later copies in flight)
            lds_stage_barrier<(QFIRST || QLDS) ? (NST == 3 ? 2 * DK::NI + 2 * VNI : DK::NI + VNI) : 0>();
            score_tile<D, INT8, F8, kBiased, true>(dks[0], qf, l32, g, sc);
        } else {
            sstore_k(0, kreg[0]);
            __syncthreads();
            score_tile<D, INT8, F8, kBiased>(kbuf(0), qf, l32, g, sc);
            gload_k(tile_row(1), kreg[0]);
            gload_v(tile_row(0), vreg[0]);
            sstore_k(1, kreg[0]);
            sstore_v(0, vreg[0]);
            if constexpr (DEPTH == 2) {
                gload_k(tile_row(2), kreg[DEPTH - 1]);
                gload_v(tile_row(1), vreg[DEPTH - 1]);
            }
            __syncthreads();
        }

        // ---- main loop: at entry sc holds S_j; LDS holds K_{j+1} and V_j.
        // Loads and stores run unconditionally (tiles past the end read the
        // clamped last row into buffers nobody reads): conditional memory ops
        // make the compiler wait for every outstanding load at the loop head.
        // Iteration j loads into set LS and writes set SS to LDS (the same set
        // at depth 1; the set loaded one iteration earlier at depth 2).
        // One key tile: the softmax of S_j, the scores S_{j+1} from the K tile
        // at ksn and O^T += V_j^T P_j^T from the V tile at vsc (padded rows,
        // or the swizzled unpadded rows of direct-to-LDS staging when SWZ).
        auto compute = [&](int j, const char* ksn, int kst, const char* vsc, float kscale_j, auto swz_tag)
                           __attribute__((always_inline)) {
            constexpr bool SWZ = decltype(swz_tag)::value;
            const int n0 = tile_row(j);
            if constexpr (DUMP) {
                // the INT32 scores of tile j (accumulator bits minus the bias
                // bits: the accumulation started at 0x4B400000 and |S32| < 2^22)
                // for the visible keys of this lane's query row, then the next
                // tile's scores exactly as the forward computes them
                if (qi < S) {
                    int32_t* orow = p.s_out + (bhq * p.ntiles * kBM + (qi - p.tile_lo * kBM)) * static_cast<size_t>(S);
                    const int lim = mask_limit(n0);
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            if (key_offset(mt, r) < lim)
                                orow[n0 + g * 4 + key_offset(mt, r)] = static_cast<int>(sc[mt][r]) - kI8BiasBits;
                }
                acc_t sn[2];
                if constexpr (KADDR && SWZ) score_tile_at<D, INT8, kBiased>(kaddr[kst], qf, sn);
                else score_tile<D, INT8, F8, kBiased, SWZ>(ksn, qf, l32, g, sn);
                sc[0] = sn[0];
                sc[1] = sn[1];
            } else {
                // scores in log2 units: s * c with c = (dQ dK) sm_scale log2(e)
                float c = scale_log2;
                if constexpr (INT8) c = fmaxf(qscale_log2 * kscale_j, FLT_MIN);
                float sv[2][16];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        // (through a scalar: __builtin_bit_cast of a vector element
                        // reads the vector's first element)
                        if constexpr (kBiased) sv[mt][r] = __int_as_float(static_cast<int>(sc[mt][r]));
                        else sv[mt][r] = static_cast<float>(sc[mt][r]);
                    }
                const int ty = tile_type(j);
                const bool needs = BMASK ? (n0 + kBN > S || ty == 0 || (ty == 2 && n0 + kBN - 1 > qw0))
                                         : tile_needs_mask(n0);
                if (needs) {
                    const int lim = !BMASK ? mask_limit(n0)
                                           : ty == 0 ? -kBN : geom::mask_limit(n0, S, qi, g, ty == 2);
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            if (!(key_offset(mt, r) < lim)) sv[mt][r] = -INFINITY;
                }
                float m_tile;
                if constexpr (kBiased) {
                    // biased scores are positive floats (masked ones -inf), so
                    // they order as their bit patterns do as signed integers
                    int mi = __float_as_int(sv[0][0]);
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) mi = max(mi, __float_as_int(sv[mt][r]));
                    // (the biased maximum minus the bias is exact: both lie in [2^23, 2^24))
                    m_tile = (__int_as_float(row_max_i(mi)) - kI8Bias) * c;
                } else {
                    float mx = sv[0][0];
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, sv[mt][r]);
                    m_tile = row_max(mx) * c;
                }
                const bool raise = m_tile > m_thr;
                if (__ballot(raise)) {
                    // (each row decides for itself: a row's result never depends on
                    // the scores of the other rows of the wave)
                    const float m_new = raise ? m_tile : m_run;
                    // (with tile masks a row may have seen no key yet: its state is
                    // empty, alpha = 0 avoids exp2(-inf - -inf))
                    const float alpha = BMASK && m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
                    m_run = m_new;
                    // (8-bit P needs p <= 1: no lazy headroom there)
                    m_thr = m_new + (PV8 ? 0.0f : kLazy);
                    l_run *= alpha;
#pragma unroll
                    for (int dt = 0; dt < C::DT; ++dt) oacc[dt] *= alpha;
                }

                // scores of the next tile (MFMA) overlap the exponentials (VALU)
                // The two waves of a SIMD alternate: the one issuing the next
                // tile's score MFMAs and this tile's exponentials runs at the
                // raised priority, the other fills in with its P.V MFMAs and
                // row maxima (same-run A/B: +3-4 % on the 8192-token prefill).
                __builtin_amdgcn_s_setprio(1);
                acc_t sn[2];
                if constexpr (KADDR && SWZ)
                    score_tile_at<D, INT8, kBiased>(kaddr[kst], qf, sn, kBiased ? &bias_blk : nullptr);
                else score_tile<D, INT8, F8, kBiased, SWZ>(ksn, qf, l32, g, sn);

                const float m_eff = BMASK && m_run == -INFINITY ? 0.0f : m_run;   // (masked rows: weights 0)
                const float negm = kBiased ? -__builtin_fmaf(kI8Bias, c, m_eff) : -m_eff;
                float pv[2][16];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        pv[mt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[mt][r], c, negm));
                float psum = 0.0f;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) psum += pv[mt][r];
                l_run += psum;
                if constexpr (PV8) {
                    // ---- O^T += V8^T P8^T (one MFMA per d tile).  Dword k of
                    // the E4M3(448 p) codes of lane half g holds the tile's
                    // 4-key group (k >> 2) * 8 + (k & 3) * 2 + g (the score
                    // layout); exchanging dwords 4..7 of half 0 with dwords
                    // 0..3 of half 1 leaves half g the groups 8g .. 8g+7 in
                    // order, i.e. keys 32g .. 32g+31, which is what it reads
                    // from the natural V^T row.
                    int pw[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const float* q = &pv[k >> 2][(k & 3) * 4];
                        int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0] * 448.0f, q[1] * 448.0f, 0, false);
                        w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2] * 448.0f, q[3] * 448.0f, w, true);
                        pw[k] = w;
                    }
                    i8x pb8;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const auto x = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(pw[i]),
                                                                        static_cast<unsigned>(pw[4 + i]), false, false);
                        pb8[2 * i] = static_cast<int>(x[0]);
                        pb8[2 * i + 1] = static_cast<int>(x[1]);
                    }
                    const char* vs = vsc;
#pragma unroll
                    for (int dt = 0; dt < C::DT; ++dt) {
                        const int r = dt * 32 + l32;
                        const char* row = vs + r * kBN;
                        const i4x a0 = *reinterpret_cast<const i4x*>(row + (((2 * g) ^ D8::swz(r)) << 4));
                        const i4x a1 = *reinterpret_cast<const i4x*>(row + (((2 * g + 1) ^ D8::swz(r)) << 4));
                        const i8x a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
                        oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb8, oacc[dt], 0, 0, 0, 0, 0, 0);
                    }
                    sc[0] = sn[0];
                    sc[1] = sn[1];
                } else {
                h8 pb[4];
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) {
                    const float* q = &pv[k4 >> 1][(k4 & 1) * 8];
                    pb[k4] = pack8(q[0], q[1], q[2], q[3], q[4], q[5], q[6], q[7]);
                }

                __builtin_amdgcn_s_setprio(0);
                // ---- O^T += V^T P^T ----
                const char* vs = vsc;
                const int grp = lane >> 4, li = lane & 15;
                // byte b of V row `row` (padded rows, or swizzled 16-byte chunks)
                auto vbyte = [&](int row, int b) -> const char* {
                    if constexpr (SWZ) return vs + row * (2 * D) + (((b >> 4) ^ DV::v_swz(row)) << 4) + (b & 15);
                    else return vs + row * C::VROW + b;
                };
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) {
                    const int vb = (dt * 32 + (grp & 1) * 16 + (li & 3) * 4) * 2;
#pragma unroll
                    for (int k4 = 0; k4 < 4; ++k4) {
                        const int krow = k4 * 16 + g * 4 + (li >> 2);
                        const tr4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_tr4*)vbyte(krow, vb));
                        const tr4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_tr4*)vbyte(krow + 8, vb));
                        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(join(lo, hi), pb[k4], oacc[dt], 0, 0, 0);
                    }
                }
                // keep the transposing reads ahead of their consumers (4 MFMAs,
                // or 2 where the FP16 D=128 register budget is tight)
                __builtin_amdgcn_sched_group_barrier(0x100, (!INT8 && D == 128) ? 4 : 8, 0);
#pragma unroll
                for (int i = 0; i < 4 * C::DT; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                sc[0] = sn[0];
                sc[1] = sn[1];
                }
            }
        };
        // register staging: iteration j loads into set LS and writes set SS
        // to LDS (the same set at depth 1; the set loaded one iteration earlier
        // at depth 2)
        auto step = [&](int j, auto ls_tag) __attribute__((always_inline)) {
            constexpr int LS = decltype(ls_tag)::value;
            constexpr int SS = DEPTH == 2 ? 1 - LS : LS;
            gload_k(BMASK ? tile_row(j + 1 + DEPTH) : geom::k_load_row<DEPTH>(j), kreg[LS]);
            gload_v(BMASK ? tile_row(j + DEPTH) : geom::v_load_row<DEPTH>(j), vreg[LS]);
            if (j < nkt_w) {
                float ksj = 1.0f;
                if constexpr (INT8) ksj = kscale[bhk * p.nkblk + (BMASK ? tile_row(j) / kBN : j)];
                compute(j, kbuf((j + 1) & 1), 0, vbuf(j & 1), ksj, std::false_type{});
            }
            sstore_k(j & 1, kreg[SS]);
            sstore_v((j + 1) & 1, vreg[SS]);
            __syncthreads();
        };
        // direct-to-LDS staging, iteration j (J = j mod NST): K_{j+1} and V_j
        // must have landed (the copies of the last iteration may stay in
        // flight at NST = 3), then after the barrier K_{j+NST} goes into the
        // stage K_j left and V_{j+NST-1} into the stage V_{j-1} left.
        // The K scale of tile j is loaded NST iterations ahead into slot J of a
        // small register ring, at the end of an iteration: the next stage
        // barrier's wait covers the scalar load, so no wait inside a tile does.
        // (The barrier waits for the copies only: a K scale read with a
        // vector load instead would just make it wait for one more copy.)
        // Tiles past the item's last one are not copied; the barrier after an
        // iteration that skipped a copy waits for every copy (its count
        // assumes the full set of copies after the awaited ones).
        auto dstep = [&](int j, auto j_tag) __attribute__((always_inline)) {
            constexpr int J = decltype(j_tag)::value;
            const float ksj = ksring[J];
            // (the score dump drains every copy: its global stores share the
            // vector-memory counter with the copies)
            if constexpr (NST == 3 && !DUMP) {
                if (j + NST <= nkt) lds_stage_barrier<DK::NI + VNI>();
                else lds_stage_barrier<0>();
            } else {
                lds_stage_barrier<0>();
            }
            if (j + NST < nkt) dtl_k(tile_row(j + NST), dks[J]);
            if (j + NST - 1 < nkt) dtl_v(tile_row(j + NST - 1), dvs[(J + NST - 1) % NST]);
            if (j < nkt_w) compute(j, dks[(J + 1) % NST], (J + 1) % NST, dvs[J], ksj, std::true_type{});
            if constexpr (INT8 && !DUMP) ksring[J] = kscale_at(j + NST);
        };
        if constexpr (DTL) {
            const int iters = geom::dtl_loop_iterations<NST>(nkt);
            for (int j = 0; j < iters; j += NST) {
                dstep(j, std::integral_constant<int, 0>{});
                dstep(j + 1, std::integral_constant<int, 1>{});
                if constexpr (NST == 3) dstep(j + 2, std::integral_constant<int, 2>{});
            }
        } else if constexpr (DEPTH == 2) {
            const int iters = geom::loop_iterations<2>(nkt);
            for (int j = 0; j < iters; j += 2) {
                step(j, std::integral_constant<int, 0>{});
                step(j + 1, std::integral_constant<int, 1>{});
            }
        } else {
            for (int j = 0; j < nkt; ++j) step(j, std::integral_constant<int, 0>{});
        }

        // No copy into LDS may still be landing when the workgroup ends or its
        // next item's copies go out, and every wave must be done with the
        // stages: drained here, before the output stores, so that nothing
        // waits for the stores (the next item's loads go out behind them).
        if constexpr (DTL) lds_stage_barrier<0>();
        // (stored after the loop: a global store ahead of it would keep the
        // compiler from using scalar loads for the per-tile K scales)
        if constexpr (QF16)
            if (p.q_scale_out && tid == 0) p.q_scale_out[bhq * p.nqblk + qt] = qscale_fused;
        if constexpr (!DUMP) {
            const float l_tot = row_sum(l_run);
            // (a row of a tile-masked query tile may see no key: O = 0, lse = -inf)
            const float inv = BMASK && !(l_tot > 0.0f) ? 0.0f : 1.0f / l_tot;
            if (qi < S) {
                _Float16* orow = static_cast<_Float16*>(p.o) + (bhq * S + static_cast<size_t>(qi)) * D;
                if constexpr (PV8) {
                    // undo the 448 of P8 and apply the per-channel V scales
                    const float* vsc = p.v_scale + bhk * D;
#pragma unroll
                    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                        for (int j4 = 0; j4 < 4; ++j4) {
                            const int col = geom::o_column(dt, j4, g);
#pragma unroll
                            for (int e = 0; e < 4; ++e) oacc[dt][j4 * 4 + e] *= vsc[col + e] * (1.0f / 448.0f);
                        }
                }
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        const h2 a = __builtin_convertvector((f2){oacc[dt][j4 * 4 + 0] * inv, oacc[dt][j4 * 4 + 1] * inv}, h2);
                        const h2 bb = __builtin_convertvector((f2){oacc[dt][j4 * 4 + 2] * inv, oacc[dt][j4 * 4 + 3] * inv}, h2);
                        *reinterpret_cast<h4*>(orow + geom::o_column(dt, j4, g)) = __builtin_shufflevector(a, bb, 0, 1, 2, 3);
                    }
                if (p.lse && g == 0) p.lse[bhq * S + qi] = (m_run + __builtin_log2f(l_tot)) * kLn2;
            }
        }
    }
    }   // work items
}

// Compute units of the current device (cached per device; 256 if unknown).
int device_compute_units() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int D, bool INT8, bool CAUSAL, bool DUMP, bool QF16 = false, bool F8 = false, bool PV8 = false,
          bool BMASK = false, bool MLDS = false>
void launch_one(const FwdParams& p, hipStream_t st) {
    const int items = p.B * p.Hq * p.ntiles;
    // causal launches with at least 8 items per compute unit: two items per
    // workgroup (measured on the prefill shapes from 512 to 32768 tokens:
    // +5 to +20 %; three or more per workgroup, or non-causal launches, gain
    // nothing or lose to the slower tail)
    const bool two = CAUSAL && !BMASK && items >= 8 * device_compute_units();
    const int grid = two ? geom::sched_grid(items, (items + 1) / 2) : items;
    hipLaunchKernelGGL((fwd_kernel<D, INT8, CAUSAL, DUMP, QF16, F8, PV8, BMASK, MLDS>), dim3(grid),
                       dim3(kFwdThreads), 0, st, p);
}

template <int D>
void launch_d(FwdKind kind, bool causal, const FwdParams& p, hipStream_t st) {
    switch (kind) {
        case FwdKind::kFp16:
            causal ? launch_one<D, false, true, false>(p, st) : launch_one<D, false, false, false>(p, st);
            break;
        case FwdKind::kInt8:
            causal ? launch_one<D, true, true, false>(p, st) : launch_one<D, true, false, false>(p, st);
            break;
        case FwdKind::kDumpInt8:
            causal ? launch_one<D, true, true, true>(p, st) : launch_one<D, true, false, true>(p, st);
            break;
        case FwdKind::kDumpInt8FusedQ:
            causal ? launch_one<D, true, true, true, true>(p, st) : launch_one<D, true, false, true, true>(p, st);
            break;
        case FwdKind::kInt8FusedQ:
            causal ? launch_one<D, true, true, false, true>(p, st) : launch_one<D, true, false, false, true>(p, st);
            break;
        case FwdKind::kFp8:
            causal ? launch_one<D, true, true, false, false, true>(p, st)
                   : launch_one<D, true, false, false, false, true>(p, st);
            break;
        case FwdKind::kInt8Pv8:
            causal ? launch_one<D, true, true, false, false, false, true>(p, st)
                   : launch_one<D, true, false, false, false, false, true>(p, st);
            break;
        case FwdKind::kFp16Mask:
            p.nkblk <= geom::kMaskListMax ? launch_one<D, false, false, false, false, false, false, true, true>(p, st)
                                          : launch_one<D, false, false, false, false, false, false, true>(p, st);
            break;
        case FwdKind::kInt8Mask:
            p.nkblk <= geom::kMaskListMax ? launch_one<D, true, false, false, false, false, false, true, true>(p, st)
                                          : launch_one<D, true, false, false, false, false, false, true>(p, st);
            break;
    }
}

}  // namespace

int launch_fwd(FwdKind kind, int head_dim, bool causal, const FwdParams& p, hipStream_t st) {
    if (head_dim == 64)
        launch_d<64>(kind, causal, p, st);
    else
        launch_d<128>(kind, causal, p, st);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ELAUNCH;
}

}  // namespace attn
