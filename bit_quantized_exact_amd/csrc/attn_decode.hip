// KV-cache (decode) attention for gfx950: a few queries per head over a long
// key/value cache, split over the keys, then merged.
//
// What is computed (cited by page title and section):
//   "注意力即一切：从 MHA 到 GQA" §3.4: the keys and values of all earlier
//   tokens are cached and the current token's queries attend over them;
//   §4.1/§5.1: with MQA/GQA the q-heads of a group share one cached K/V;
//   §2.3: under the causal mask the queries are the last Sq positions, so
//   query i sees cached keys j <= Sk - Sq + i.
//   SageAttention article (技术方案): INT8 Q K^T (K smoothed by its channel
//   mean over the cached tokens and quantised per 64-key block), dequantised
//   with the block scales; P and V in FP16.  The Sq <= 32 queries of one head
//   form one Q quantisation block, quantised here in the kernel.
//   "FlashAttention" guide (FAQ): per key range, a running maximum and sum;
//   ranges are merged exactly by rescaling with the maxima.
//
// gfx950 design.  Decode reads every cached byte once and does little
// arithmetic per byte, so the bound is HBM bandwidth:
//   * the queries of all q-heads of one kv-head are packed into the 32 query
//     slots of one wave, so a K/V byte is read once per group, not per head;
//   * the cache is split into ranges of 32-key tiles, one single-wave
//     workgroup per (batch, kv-head, query chunk, range), a few thousand
//     workgroups per launch, each streaming its range with the next tile's
//     loads in flight while the current tile is computed;
//   * K tiles go straight from HBM into the MFMA operand registers (the
//     transposed form S^T = K Q^T takes K rows as the A operand); V tiles pass
//     through padded LDS for the transposing reads of O^T += V^T P^T, loaded
//     with the non-temporal (streaming) cache policy;
//   * each workgroup leaves its unnormalised partial O, running maximum and
//     sum; a combine kernel rescales and sums the ranges (exactly as the
//     online softmax merges tiles) and writes O and the log-sum-exp.
#include "attn_internal.h"
#include "decode_geometry.h"

#include <cfloat>
#include <type_traits>

namespace attn {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef int i16x __attribute__((ext_vector_type(16)));
typedef int i4x __attribute__((ext_vector_type(4)));
typedef __fp16 tr4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) tr4 lds_tr4;

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;
constexpr int kI8BiasBits = 0x4B400000;   // fp32 1.5 * 2^23: INT32 scores read as biased fp32
constexpr float kI8Bias = 12582912.0f;

template <int D, bool INT8>
struct DecCfg {
    static constexpr int KELT = INT8 ? 1 : 2;
    static constexpr int KROWG = D * KELT;                 // cached K row bytes
    static constexpr int QSTEPS = INT8 ? D / 32 : D / 16;  // 16-byte MFMA k-steps
    static constexpr int VROWG = 2 * D;                    // V row bytes
    static constexpr int VCPR = VROWG / 16;                // 16-byte chunks per V row
    static constexpr int VPT = dec::kTile * VCPR / dec::kThreads;   // V chunks per lane per tile
    static constexpr int VROW = 2 * D + 64;                // padded V row in LDS
    static constexpr int DT = D / 32;
    static_assert(dec::kTile * VCPR % dec::kThreads == 0, "V tile split");
    typedef std::conditional_t<INT8, i4x, h8> frag_t;
    typedef std::conditional_t<INT8, i16x, f16x> acc_t;
    __host__ __device__ static constexpr int frag_offset(int s, int g) {
        return INT8 ? (s * 32 + g * 16) : (s * 16 + g * 8) * 2;
    }
};

__device__ __forceinline__ h8 join(tr4 a, tr4 b) {
    h8 r;
    __builtin_memcpy(&r, &a, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &b, 8);
    return r;
}

__device__ __forceinline__ h8 pack8(const float* a) {
    const h2 p0 = __builtin_convertvector((f2){a[0], a[1]}, h2);
    const h2 p1 = __builtin_convertvector((f2){a[2], a[3]}, h2);
    const h2 p2 = __builtin_convertvector((f2){a[4], a[5]}, h2);
    const h2 p3 = __builtin_convertvector((f2){a[6], a[7]}, h2);
    const h4 lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
    const h4 hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float row_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Score register r of the 32x32 accumulator holds key n0 + g*4 + key_off(r).
__host__ __device__ constexpr int key_off(int r) { return (r >> 2) * 8 + (r & 3); }

template <int D, bool INT8, bool CAUSAL>
__global__ __launch_bounds__(dec::kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_kernel(const DecParams p) {
    using C = DecCfg<D, INT8>;
    typedef typename C::frag_t frag_t;
    typedef typename C::acc_t acc_t;
    __shared__ __attribute__((aligned(16))) char vs[dec::kTile * C::VROW];
    __shared__ float rowmax[dec::kSlots];

    const int lane = threadIdx.x;
    const int n = lane & 31;           // query slot
    const int g = lane >> 5;           // lane half (key subset / k-slot half)
    const int split = blockIdx.x, chunk = blockIdx.y, bkv = blockIdx.z;
    const int b = bkv / p.Hkv, kvh = bkv - b * p.Hkv;
    const int Sq = p.Sq, Sk = p.Sk;
    // chunks past this kv-head's group (or a kv-head no q-head reads) have nothing to do
    if (!dec::chunk_has_work(chunk, p.hpc, p.gcount[kvh])) return;
    const dec::Plan plan{p.hpc, p.nchunk, p.ntiles, p.tps, p.nsplit};
    const dec::Slot sl = dec::slot_of(n, chunk, p.hpc, Sq, p.gcount[kvh]);
    const int h = p.horder[p.gstart[kvh] + sl.hh];
    const size_t qrow = (static_cast<size_t>(b) * p.Hq + h) * Sq + sl.i;

    const char* kg = static_cast<const char*>(p.k) + static_cast<size_t>(bkv) * Sk * C::KROWG;
    const char* vg = static_cast<const char*>(p.v) + static_cast<size_t>(bkv) * Sk * C::VROWG;
    const int t0 = dec::split_first_tile(split, p.tps);
    const int t1 = dec::split_end_tile(split, p.tps, p.ntiles);

    frag_t kc[C::QSTEPS], kn[C::QSTEPS];
    i4x vr[C::VPT];
    auto gload_k = [&](int t, frag_t (&dst)[C::QSTEPS]) {
        const char* row = kg + static_cast<size_t>(dec::key_row(t * dec::kTile, n, Sk)) * C::KROWG;
#pragma unroll
        for (int s = 0; s < C::QSTEPS; ++s) dst[s] = *reinterpret_cast<const frag_t*>(row + C::frag_offset(s, g));
    };
    // V rows are read whole by consecutive lanes and never again: non-temporal
    // loads (the streaming cache policy).  K keeps the default policy: each
    // K load instruction touches 32 bytes of 32 different rows, and the rows'
    // other bytes come with the next k-steps' loads, which the default policy
    // serves from the cache lines the first one brought in.
    auto gload_v = [&](int t) {
#pragma unroll
        for (int i = 0; i < C::VPT; ++i) {
            const int c = lane + dec::kThreads * i;
            const int r = c / C::VCPR;
            const char* src = vg + static_cast<size_t>(dec::key_row(t * dec::kTile, r, Sk)) * C::VROWG + (c % C::VCPR) * 16;
            vr[i] = __builtin_nontemporal_load(reinterpret_cast<const i4x*>(src));
        }
    };
    auto sstore_v = [&]() {
#pragma unroll
        for (int i = 0; i < C::VPT; ++i) {
            const int c = lane + dec::kThreads * i;
            *reinterpret_cast<i4x*>(vs + (c / C::VCPR) * C::VROW + (c % C::VCPR) * 16) = vr[i];
        }
    };

    gload_k(t0, kc);
    gload_v(t0);

    // ---- Q fragment (B operand): fp16 as is, or one INT8 block per head
    // (the head's Sq <= 32 rows) with the rule of the standalone quantiser:
    // a = max|x|, r = 127/a, delta = a/127 (correctly rounded),
    // q = clamp(rint(x r), -127, 127); a == 0 gives q = 0, delta = 0.
    frag_t qf[C::QSTEPS];
    float qscale = 1.0f;
    if constexpr (!INT8) {
        const char* qp = static_cast<const char*>(p.q) + qrow * (2 * D);
#pragma unroll
        for (int s = 0; s < C::QSTEPS; ++s) qf[s] = *reinterpret_cast<const h8*>(qp + C::frag_offset(s, g));
    } else {
        const char* qp = static_cast<const char*>(p.q) + qrow * (2 * D);
        float xq[C::QSTEPS][16];
        float amax = 0.0f;
#pragma unroll
        for (int s = 0; s < C::QSTEPS; ++s)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                // the 16 int8 slots s*32 + g*16 .. +15 come from fp16 elements at the same indices
                const h8 v = *reinterpret_cast<const h8*>(qp + (s * 32 + g * 16 + hf * 8) * 2);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    xq[s][hf * 8 + e] = static_cast<float>(v[e]);
                    amax = __builtin_fmaxf(amax, __builtin_fabsf(xq[s][hf * 8 + e]));
                }
            }
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));   // whole row
        if (g == 0) rowmax[n] = amax;
        __syncthreads();
        float a = 0.0f;
        const int first = dec::head_first_slot(n, Sq);
        for (int r = 0; r < Sq && first + r < dec::kSlots; ++r) a = __builtin_fmaxf(a, rowmax[first + r]);
        const float rq = a == 0.0f ? 0.0f : __fdiv_rn(127.0f, a);
        qscale = a == 0.0f ? 0.0f : __fdiv_rn(a, 127.0f);
#pragma unroll
        for (int s = 0; s < C::QSTEPS; ++s) {
            uint32_t w[4];
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                uint32_t packed = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float t = __builtin_rintf(xq[s][e4 * 4 + e] * rq);
                    t = __builtin_fminf(__builtin_fmaxf(t, -127.0f), 127.0f);
                    packed |= (static_cast<uint32_t>(static_cast<int>(t)) & 0xffu) << (8 * e);
                }
                w[e4] = packed;
            }
            __builtin_memcpy(&qf[s], w, 16);
        }
        if (p.q_scale_out && split == 0 && g == 0 && sl.valid && sl.i == 0)
            p.q_scale_out[static_cast<size_t>(b) * p.Hq + h] = qscale;
    }

    float m_run = -INFINITY;   // running maximum (log2 units), equal in lanes n and n+32
    float l_run = 0.0f;        // this lane's partial sum
    f16x oacc[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) oacc[dt] = f16x{};

    for (int t = t0; t < t1; ++t) {
        const int n0 = t * dec::kTile;
        sstore_v();
        const int tn = dec::prefetch_tile(t, t1);
        gload_k(tn, kn);
        gload_v(tn);
        __syncthreads();

        // ---- scores S^T = K Q^T of the tile (one 32x32 block) ----
        acc_t acc;
        if constexpr (INT8) acc = kI8BiasBits;
        else acc = acc_t{};
#pragma unroll
        for (int s = 0; s < C::QSTEPS; ++s) {
            if constexpr (INT8) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kc[s], qf[s], acc, 0, 0, 0);
            else acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kc[s], qf[s], acc, 0, 0, 0);
        }
        float c = p.scale_log2;
        if constexpr (INT8) c = __builtin_fmaxf(qscale * p.k_scale[static_cast<size_t>(bkv) * p.nkblk + (n0 >> 6)] * p.scale_log2, FLT_MIN);
        float sv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if constexpr (INT8) sv[r] = __int_as_float(static_cast<int>(acc[r]));
            else sv[r] = acc[r];
        }
        if (n0 + dec::kTile > Sk || (CAUSAL && n0 + dec::kTile - 1 > Sk - Sq)) {
            const int lim = dec::mask_limit(n0, Sq, Sk, sl.i, g, CAUSAL);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (!(key_off(r) < lim)) sv[r] = -INFINITY;
        }
        float mx = sv[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = __builtin_fmaxf(mx, sv[r]);
        const float m_tile = (INT8 ? row_max(mx) - kI8Bias : row_max(mx)) * c;
        const bool raise = m_tile > m_run + kLazy;
        if (__ballot(raise)) {
            // (each row decides for itself: a row's result never depends on the
            // scores of the other rows of the wave)
            const float m_new = raise ? m_tile : m_run;
            // (a row that has seen no key yet has an empty state: alpha = 0 avoids
            // exp2(-inf - -inf) when the other rows of the wave raise their maximum)
            const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) oacc[dt] *= alpha;
        }
        // a row with no visible key so far keeps m = -inf: its weights are 0
        const float m_eff = m_run == -INFINITY ? 0.0f : m_run;
        const float negm = INT8 ? -__builtin_fmaf(kI8Bias, c, m_eff) : -m_eff;
        float pv[16];
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], c, negm));
            psum += pv[r];
        }
        l_run += psum;
        const h8 pb0 = pack8(&pv[0]);
        const h8 pb1 = pack8(&pv[8]);

        // ---- O^T += V^T P^T (V^T by transposing LDS reads) ----
        const int grp = lane >> 4, li = lane & 15;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            const char* vb = vs + (dt * 32 + (grp & 1) * 16 + (li & 3) * 4) * 2;
#pragma unroll
            for (int k4 = 0; k4 < 2; ++k4) {
                const int krow = k4 * 16 + g * 4 + (li >> 2);
                const tr4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_tr4*)(vb + krow * C::VROW));
                const tr4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_tr4*)(vb + (krow + 8) * C::VROW));
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(join(lo, hi), k4 ? pb1 : pb0, oacc[dt], 0, 0, 0);
            }
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < C::QSTEPS; ++s) kc[s] = kn[s];
    }

    // ---- partial result of this key range ----
    const float l_tot = row_sum(l_run);
    if (sl.valid) {
        const size_t row = dec::partial_row(bkv, chunk, split, n, plan);
        float* orow = p.ws_o + row * D;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const int col = dt * 32 + j4 * 8 + g * 4;
                *reinterpret_cast<f4*>(orow + col) = f4{oacc[dt][j4 * 4 + 0], oacc[dt][j4 * 4 + 1],
                                                        oacc[dt][j4 * 4 + 2], oacc[dt][j4 * 4 + 3]};
            }
        if (g == 0) {
            p.ws_m[row] = m_run;
            p.ws_l[row] = l_tot;
        }
    }
}

// Merge the key ranges: m = max_s m_s, w_s = 2^(m_s - m), l = sum_s w_s l_s,
// O = sum_s w_s O_s / l (ranges with no visible key have m_s = -inf, w_s = 0).
// Thread (r, c4): query slot 8 * blockIdx.x + r of one (batch, kv-head,
// chunk), output columns 4 c4 .. 4 c4 + 3; blocks without a valid slot exit.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const DecParams p) {
    constexpr int CG = D / 4;            // 4-column groups per row
    constexpr int RPB = 256 / CG;        // slots per block
    const int chunk = blockIdx.y, bkv = blockIdx.z;
    const int b = bkv / p.Hkv, kvh = bkv - b * p.Hkv;
    const int c4 = threadIdx.x % CG;
    const int n = blockIdx.x * RPB + threadIdx.x / CG;
    const dec::Plan plan{p.hpc, p.nchunk, p.ntiles, p.tps, p.nsplit};
    const dec::Slot sl = dec::slot_of(n, chunk, p.hpc, p.Sq, p.gcount[kvh]);
    if (!sl.valid) return;
    const int h = p.horder[p.gstart[kvh] + sl.hh];
    const size_t row0 = dec::partial_row(bkv, chunk, 0, n, plan);
    const size_t stride = dec::kSlots;   // rows between consecutive splits of one slot
    float m = -INFINITY;
#pragma unroll 8
    for (int s = 0; s < p.nsplit; ++s) m = __builtin_fmaxf(m, p.ws_m[row0 + s * stride]);
    float l = 0.0f;
    f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
    for (int s = 0; s < p.nsplit; ++s) {
        const size_t row = row0 + s * stride;
        const float ms = p.ws_m[row];
        const float w = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - m);
        l += w * p.ws_l[row];
        acc += w * *reinterpret_cast<const f4*>(p.ws_o + row * D + c4 * 4);
    }
    const float inv = 1.0f / l;
    _Float16* out = static_cast<_Float16*>(p.o) + ((static_cast<size_t>(b) * p.Hq + h) * p.Sq + sl.i) * D + c4 * 4;
    const h2 lo = __builtin_convertvector((f2){acc[0] * inv, acc[1] * inv}, h2);
    const h2 hi = __builtin_convertvector((f2){acc[2] * inv, acc[3] * inv}, h2);
    *reinterpret_cast<h4*>(out) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
    if (p.lse && c4 == 0) p.lse[(static_cast<size_t>(b) * p.Hq + h) * p.Sq + sl.i] = (m + __builtin_log2f(l)) * kLn2;
}

template <int D, bool INT8>
void launch_decode_d(bool causal, const DecParams& p, hipStream_t st) {
    const dim3 grid(p.nsplit, p.nchunk, p.B * p.Hkv);
    if (causal)
        hipLaunchKernelGGL((decode_kernel<D, INT8, true>), grid, dim3(dec::kThreads), 0, st, p);
    else
        hipLaunchKernelGGL((decode_kernel<D, INT8, false>), grid, dim3(dec::kThreads), 0, st, p);
    // only the blocks holding the first hpc*Sq slots can have valid slots
    const int rpb = 256 / (D / 4);
    const int used = dec::imin(dec::kSlots, p.hpc * p.Sq);
    hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(dec::cdiv(used, rpb), p.nchunk, p.B * p.Hkv), dim3(256), 0,
                       st, p);
}

}  // namespace

int launch_decode(bool int8, int head_dim, bool causal, const DecParams& p, hipStream_t st) {
    if (head_dim == 64)
        int8 ? launch_decode_d<64, true>(causal, p, st) : launch_decode_d<64, false>(causal, p, st);
    else
        int8 ? launch_decode_d<128, true>(causal, p, st) : launch_decode_d<128, false>(causal, p, st);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ELAUNCH;
}

}  // namespace attn
