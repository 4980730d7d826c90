// Fused attention forward for gfx950: tiled, online softmax, one workgroup per
// (batch, q-head, 128-row query tile).
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
//     keys, so the row max needs a single cross-lane exchange (lane ^ 32) and
//     the row sum none until the end.
//   * The output is accumulated transposed too, O^T += V^T P^T: P^T is the
//     B operand taken straight from the score registers (no data movement),
//     V^T is the A operand read from a row-major V tile in LDS with
//     ds_read_b64_tr_b16 (a transposing LDS read), and the accumulator rows
//     that a lane rescales by alpha all belong to its own query.
//   * K and V tiles of 64 keys are double-buffered in LDS through registers;
//     one barrier per key tile.  Row padding keeps the MFMA operand reads and
//     the transposing reads free of bank conflicts.
//   * Workgroups are launched XCD-aware: consecutive hardware block ids go
//     round-robin over the 8 XCDs, so blocks are renumbered such that each
//     XCD receives a contiguous range of (batch, head) pairs ordered by kv
//     head; the q-heads of one GQA group then share K/V in that XCD's L2.
//     Causal launches start with the heaviest (last) query tiles.
#include "attn_internal.h"

#include <cfloat>

namespace attn {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef int i16x __attribute__((ext_vector_type(16)));
typedef int i4x __attribute__((ext_vector_type(4)));
typedef __fp16 tr4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) tr4 lds_tr4;

constexpr float kLn2 = 0.6931471805599453f;

template <int D, bool INT8>
struct Cfg {
    static constexpr int KELT = INT8 ? 1 : 2;                 // bytes per K element
    static constexpr int KROWG = D * KELT;                     // K row bytes in HBM
    static constexpr int KROW = KROWG + 16;                    // K row bytes in LDS
    static constexpr int VROW = 2 * D + 64;                    // V row bytes in LDS
    static constexpr int KBYTES = kBN * KROW;
    static constexpr int VBYTES = kBN * VROW;
    static constexpr int STAGE = KBYTES + VBYTES;
    static constexpr int KCPR = KROWG / 16;                    // 16-byte chunks per K row
    static constexpr int VCPR = 2 * D / 16;
    static constexpr int KPT = kBN * KCPR / kFwdThreads;       // K chunks per thread
    static constexpr int VPT = kBN * VCPR / kFwdThreads;
    static constexpr int QSTEPS = INT8 ? D / 32 : D / 16;      // MFMA k-steps over head_dim
    static constexpr int DT = D / 32;                          // 32-row d tiles of O^T
    static_assert(kBN * KCPR % kFwdThreads == 0 && kBN * VCPR % kFwdThreads == 0, "tile split");
};

template <bool INT8>
struct QFrag;
template <>
struct QFrag<false> { typedef h8 type; };
template <>
struct QFrag<true> { typedef i4x type; };

__device__ __forceinline__ h8 join(tr4 a, tr4 b) {
    h8 r;
    __builtin_memcpy(&r, &a, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &b, 8);
    return r;
}

template <int D, bool INT8, bool CAUSAL, bool DUMP>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(const FwdParams p) {
    using C = Cfg<D, INT8>;
    typedef typename QFrag<INT8>::type qfrag_t;
    __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int S = p.S;

    // ---- block id -> (batch, q-head, query tile), XCD-aware ----
    const int nblk = gridDim.x;
    const int bid = blockIdx.x;
    const int per = nblk >> 3, rem = nblk & 7, xcd = bid & 7;
    const int L = xcd * per + min(xcd, rem) + (bid >> 3);
    const int per_b = p.Hq * p.ntiles;
    const int b = L / per_b;
    const int rb = L - b * per_b;
    const int pos = rb / p.ntiles;
    const int rank = rb - pos * p.ntiles;
    const int h = p.horder[pos];
    const int kvh = p.kvmap[h];
    const int qt = p.tile_lo + ((CAUSAL && !DUMP) ? (p.ntiles - 1 - rank) : rank);

    const int q0 = qt * kBM;
    const int qw0 = q0 + wave * 32;      // first query row of this wave
    const int qi = qw0 + l32;            // this lane's query row
    const size_t bhq = static_cast<size_t>(b) * p.Hq + h;
    const size_t bhk = static_cast<size_t>(b) * p.Hkv + kvh;

    const int n_end = CAUSAL ? min(S, q0 + kBM) : S;
    const int nkt = (n_end + kBN - 1) / kBN;

    // ---- Q fragment (B operand of S^T = K Q^T), kept in VGPRs ----
    qfrag_t qf[C::QSTEPS];
    {
        const char* qrow = static_cast<const char*>(p.q) +
                           (bhq * S + static_cast<size_t>(qi)) * (D * C::KELT);
#pragma unroll
        for (int s = 0; s < C::QSTEPS; ++s) {
            // 16 bytes per lane: int8 elements s*32 + g*16.., or fp16 elements s*16 + g*8..
            const int off = INT8 ? (s * 32 + g * 16) : (s * 16 + g * 8) * 2;
            qf[s] = qi < S ? *reinterpret_cast<const qfrag_t*>(qrow + off) : qfrag_t{};
        }
    }

    const char* kg = static_cast<const char*>(p.k) + bhk * S * C::KROWG;
    const char* vg = static_cast<const char*>(p.v) + bhk * S * (2 * D);

    i4x kreg[C::KPT], vreg[C::VPT];
    auto gload = [&](int n0) {
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) {
            const int c = tid + kFwdThreads * i;
            const int row = c / C::KCPR, col = c % C::KCPR;
            const int key = n0 + row;
            kreg[i] = key < S ? *reinterpret_cast<const i4x*>(kg + static_cast<size_t>(key) * C::KROWG + col * 16)
                              : i4x{0, 0, 0, 0};
        }
        if constexpr (!DUMP) {   // the score dump reads no V (p.v is null there)
#pragma unroll
            for (int i = 0; i < C::VPT; ++i) {
                const int c = tid + kFwdThreads * i;
                const int row = c / C::VCPR, col = c % C::VCPR;
                const int key = n0 + row;
                vreg[i] = key < S ? *reinterpret_cast<const i4x*>(vg + static_cast<size_t>(key) * (2 * D) + col * 16)
                                  : i4x{0, 0, 0, 0};
            }
        }
    };
    auto sstore = [&](int stage) {
        char* ks = smem + stage * C::STAGE;
        char* vs = ks + C::KBYTES;
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) {
            const int c = tid + kFwdThreads * i;
            *reinterpret_cast<i4x*>(ks + (c / C::KCPR) * C::KROW + (c % C::KCPR) * 16) = kreg[i];
        }
        if constexpr (!DUMP) {
#pragma unroll
            for (int i = 0; i < C::VPT; ++i) {
                const int c = tid + kFwdThreads * i;
                *reinterpret_cast<i4x*>(vs + (c / C::VCPR) * C::VROW + (c % C::VCPR) * 16) = vreg[i];
            }
        }
    };

    float m_run = -INFINITY;   // running row max (log2 units), same in lanes l and l^32
    float l_run = 0.0f;        // this lane's partial row sum
    f16x oacc[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) oacc[dt] = f16x{};

    float qscale = 0.0f;   // the score dump has no scales (p.q_scale is null there)
    if constexpr (INT8 && !DUMP) qscale = p.q_scale[bhq * p.nqblk + qt];

    gload(0);
    sstore(0);
    __syncthreads();

    for (int it = 0; it < nkt; ++it) {
        const int n0 = it * kBN;
        if (it + 1 < nkt) gload(n0 + kBN);
        const char* ks = smem + (it & 1) * C::STAGE;
        const char* vs = ks + C::KBYTES;
        const bool active = !CAUSAL || n0 <= qw0 + 31;
        if (active) {
            // ---- S^T tile: 64 keys x 32 queries, two 32x32 MFMA tiles ----
            float sv[2][16];
            if constexpr (INT8) {
                i16x acc[2] = {i16x{}, i16x{}};
#pragma unroll
                for (int s = 0; s < C::QSTEPS; ++s) {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        const i4x a = *reinterpret_cast<const i4x*>(ks + (mt * 32 + l32) * C::KROW + s * 32 + g * 16);
                        acc[mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[s], acc[mt], 0, 0, 0);
                    }
                }
                if constexpr (DUMP) {
                    if (qi < S) {
                        int32_t* orow = p.s_out + (bhq * p.ntiles * kBM + (qi - p.tile_lo * kBM)) * static_cast<size_t>(S);
#pragma unroll
                        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int key = n0 + mt * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
                                if (key < S && (!CAUSAL || key <= qi)) orow[key] = acc[mt][r];
                            }
                    }
                }
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sv[mt][r] = static_cast<float>(acc[mt][r]);
            } else {
                f16x acc[2] = {f16x{}, f16x{}};
#pragma unroll
                for (int s = 0; s < C::QSTEPS; ++s) {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        const h8 a = *reinterpret_cast<const h8*>(ks + (mt * 32 + l32) * C::KROW + (s * 16 + g * 8) * 2);
                        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[s], acc[mt], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sv[mt][r] = acc[mt][r];
            }

            if constexpr (!DUMP) {
                // scores in log2 units: s * c, c = (dQ dK) sm_scale log2(e)
                float c = p.scale_log2;
                if (INT8) c = fmaxf(qscale * p.k_scale[bhk * p.nkblk + it] * p.scale_log2, FLT_MIN);
                const bool need_mask = (n0 + kBN > S) || (CAUSAL && n0 + kBN - 1 > qw0);
                if (need_mask) {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = n0 + mt * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
                            if (key >= S || (CAUSAL && key > qi)) sv[mt][r] = -INFINITY;
                        }
                }
                float mx = sv[0][0];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[mt][r]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float m_new = fmaxf(m_run, mx * c);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                float psum = 0.0f;
                h8 pb[4];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[mt][r], c, -m_new));
                        psum += pv;
                        pb[mt * 2 + (r >> 3)][r & 7] = static_cast<_Float16>(pv);
                    }
                l_run = l_run * alpha + psum;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) oacc[dt] *= alpha;

                // ---- O^T += V^T P^T ----
                const int grp = lane >> 4, li = lane & 15;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) {
                    const char* vb = vs + (dt * 32 + (grp & 1) * 16 + (li & 3) * 4) * 2;
#pragma unroll
                    for (int k4 = 0; k4 < 4; ++k4) {
                        const int krow = k4 * 16 + g * 4 + (li >> 2);
                        const tr4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                            (lds_tr4*)(vb + krow * C::VROW));
                        const tr4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                            (lds_tr4*)(vb + (krow + 8) * C::VROW));
                        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(join(lo, hi), pb[k4], oacc[dt], 0, 0, 0);
                    }
                }
            }
        }
        if (it + 1 < nkt) sstore((it + 1) & 1);
        __syncthreads();
    }

    if constexpr (!DUMP) {
        const float l_tot = l_run + __shfl_xor(l_run, 32);
        const float inv = 1.0f / l_tot;
        if (qi < S) {
            _Float16* orow = static_cast<_Float16*>(p.o) + (bhq * S + static_cast<size_t>(qi)) * D;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    h4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = static_cast<_Float16>(oacc[dt][j * 4 + e] * inv);
                    *reinterpret_cast<h4*>(orow + dt * 32 + j * 8 + g * 4) = v;
                }
            if (p.lse && g == 0) p.lse[bhq * S + qi] = (m_run + __builtin_log2f(l_tot)) * kLn2;
        }
    }
}

template <int D, bool INT8, bool CAUSAL, bool DUMP>
void launch_one(const FwdParams& p, hipStream_t st) {
    const int blocks = p.B * p.Hq * p.ntiles;
    hipLaunchKernelGGL((fwd_kernel<D, INT8, CAUSAL, DUMP>), dim3(blocks), dim3(kFwdThreads), 0, st, p);
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
