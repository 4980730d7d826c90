// K smoothing and per-block INT8 quantisation of Q and K for gfx950.
//
// SageAttention article ("又快又准，即插即用！清华8比特量化Attention…"), section
// 技术方案: K <- K - mean(K) removes K's channel outliers and leaves softmax
// unchanged; Q and K are then quantised to INT8 with one scale per
// FlashAttention-sized block.  The pages print neither the scale formula nor
// the rounding; this file implements the symmetric absmax reading
// (delta = max|x| / 127, q = rint(x * (127 / max|x|)) saturated to +-127,
// ties to even) with the mean taken per channel over all tokens.
//
// Every result here is bit-exact by construction and independent of launch
// order and reduction order:
//   * the channel sum is exact (every fp16 value is an integer multiple of
//     2^-24, below 2^40 in those units): fp64 within a chunk of tokens, then
//     int64 in those units across chunks, so any summation order gives the
//     same integer (finite inputs);
//   * maxima are exact;
//   * the remaining fp32 operations (subtract, two correctly rounded
//     divisions, one product, rint) are single IEEE operations.  This file is
//     compiled with -ffp-contract=off so that no product is fused.
//
// The kernels stream HBM: each reads its inputs once (K twice: sums, then
// quantisation) with 16-byte loads and writes int8 with 8-byte stores.  The K
// quantiser adds the (at most 32) partial sums of its (b, kv-head) itself, so
// K takes two launches (sums, quantisation) at any length.
#include "attn_internal.h"

#include <algorithm>
#include <cfloat>
#include <mutex>

namespace attn {
namespace {

typedef int i4x __attribute__((ext_vector_type(4)));
typedef int i2x __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float half_bits_to_float(unsigned h) {
    _Float16 x;
    const unsigned short s = static_cast<unsigned short>(h);
    __builtin_memcpy(&x, &s, 2);
    return static_cast<float>(x);
}

// Per (b, kv-head, group of cps chunks of kSumChunk tokens): exact column
// sums of K.  Thread t owns one 16-byte column chunk (8 channels) and every
// RG-th row of each chunk; per chunk all of its row loads are issued before
// the first add (rows past the sequence read the last row and are dropped).
// Each thread sums in fp64, which is exact here: every fp16 value is an
// integer multiple of 2^-24 below 2^40 in those units, and a thread adds at
// most cps * kSumChunk / RG <= 4096 of them (cps <= 512 for S <= 2^22), so
// its sum is such a multiple below 2^52 < 2^53.  It is converted to that
// integer (int64) before the threads of a column are added, so the group
// total (below 2^57) and any later total are exact in any order.  Grouping
// chunks keeps the partials per (b, kv-head) at kMaxPartials, few enough for
// the K quantiser to add them itself (no mean launch).
constexpr int kColsumThreads = 512;
constexpr int kMaxPartials = 32;
// The columns are split over NCS workgroups (blockIdx.z: columns
// z*D/NCS .. +D/NCS), so that a group of chunks spreads over NCS workgroups.
template <int D, int NCS = 1>
__global__ __launch_bounds__(kColsumThreads) void k_colsum_kernel(const uint16_t* __restrict__ k, int S,
                                                                  int cps, int npart,
                                                                  long long* __restrict__ partial) {
    constexpr int DW = D / NCS;                 // columns of this workgroup
    constexpr int CPR = DW / 8;                 // 16-byte chunks per row
    constexpr int RG = kColsumThreads / CPR;    // row groups
    constexpr int RPT = kSumChunk / RG;         // rows per thread per chunk
    static_assert(kSumChunk % RG == 0 && 512 * RPT <= 4096 && 4096.0 * 65536.0 * 16777216.0 < 9007199254740992.0,
                  "exact fp64 thread sums");
    __shared__ long long red[RG][DW];
    const int t = threadIdx.x;
    const int cc = t % CPR, rg = t / CPR;
    const int grp = blockIdx.x;
    const size_t bk = blockIdx.y;
    const int col0 = static_cast<int>(blockIdx.z) * DW;
    const uint16_t* base = k + bk * static_cast<size_t>(S) * D + col0 + cc * 8;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // the rows of chunk c of the group (rows past the sequence read the last row)
    auto load = [&](int c, i4x (&v)[RPT]) __attribute__((always_inline)) {
        const int r0 = (grp * cps + c) * kSumChunk + rg;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = r0 + i * RG;
            v[i] = *reinterpret_cast<const i4x*>(base + static_cast<size_t>(r < S ? r : S - 1) * D);
        }
    };
    auto add = [&](int c, const i4x (&v)[RPT]) __attribute__((always_inline)) {
        const int r0 = (grp * cps + c) * kSumChunk + rg;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            if (r0 + i * RG >= S) break;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const unsigned w = static_cast<unsigned>(v[i][e]);
                acc[2 * e] += static_cast<double>(half_bits_to_float(w & 0xffffu));
                acc[2 * e + 1] += static_cast<double>(half_bits_to_float(w >> 16));
            }
        }
    };
    // the chunks of the group (those starting inside the sequence), with the
    // next chunk's loads in flight while the current one is added
    const int nc = min(cps, (S + kSumChunk - 1) / kSumChunk - grp * cps);
    i4x va[RPT], vb[RPT];
    if (nc > 0) load(0, va);
    for (int c = 0; c < nc; c += 2) {
        if (c + 1 < nc) load(c + 1, vb);
        add(c, va);
        if (c + 1 < nc) {
            if (c + 2 < nc) load(c + 2, va);
            add(c + 1, vb);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rg][cc * 8 + e] = static_cast<long long>(__builtin_ldexp(acc[e], 24));
    __syncthreads();
    if (t < DW) {
        long long s = 0;
#pragma unroll
        for (int g = 0; g < RG; ++g) s += red[g][t];
        partial[(bk * npart + grp) * D + col0 + t] = s;
    }
}

// Maximum of the non-negative values v over the 64 lanes of the wave, read
// from lane 63: prefix maxima within each 16-lane row by the DPP row shifts
// 1, 2, 4, 8, then the row broadcasts of lanes 15 and 31 into the rows above
// (lanes shifted in from outside a row, and rows outside a broadcast's row
// mask, take 0, which leaves a maximum of non-negative values unchanged).
// Non-negative floats order as their bit patterns do as unsigned integers.
__device__ __forceinline__ float wave_max_nonneg(float x) {
    unsigned v = __float_as_uint(x);
    v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, true)));
    v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, true)));
    v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, true)));
    v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, true)));
    v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xa, 0xf, false)));
    v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xc, 0xf, false)));
    return __uint_as_float(static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(v), 63)));
}

// Maximum of the non-negative v over the 256-thread workgroup (through red[4]).
__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max_nonneg(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// INT8 code of x with r = 127 / a, |x| <= a: clamp(rint(x r), -127, 127) as
// the low byte of fp32(fp32(x r) + 1.5 * 2^23).  |x r| <= 127 (1 + 2^-24)^2
// < 127.5, so the clamp never acts, and adding 1.5 * 2^23 rounds x r to an
// integer (to nearest, ties to even, as rint) held in the low mantissa bits.
// (The product and the sum are rounded separately: this file is compiled
// without contraction.)
__device__ __forceinline__ unsigned quant_byte(float x, float r) {
    return __float_as_uint(x * r + 12582912.0f) & 0xffu;
}

// E4M3 codes of x0*r, x1*r (saturated to +-448 first) in bytes 0 and 1 of
// the result, v_cvt_pk_fp8_f32 rounding to nearest even.
__device__ __forceinline__ unsigned e4m3_pair(float x0, float x1, float r) {
    const float t0 = fminf(fmaxf(x0 * r, -448.0f), 448.0f);
    const float t1 = fminf(fmaxf(x1 * r, -448.0f), 448.0f);
    return static_cast<unsigned>(__builtin_amdgcn_cvt_pk_fp8_f32(t0, t1, 0, false)) & 0xffffu;
}

// One block of ROWS rows of one (b, head) matrix: absmax, scale, 8-bit codes.
// SMOOTH subtracts the channel mean first (K); Q is quantised as is.  FP8
// selects the E4M3 grid (448 in place of 127, E4M3 rounding in place of
// rint + clamp): the FP8 alternative the SageAttention article compares with.
// MEANP (with SMOOTH, the form the K path uses): the workgroup adds the
// exact partial channel sums of its (b, kv-head) itself (at most
// kMaxPartials int64 values per channel) and divides once, mu =
// fp32(fp64(sum) / S), instead of reading means from `mean`; every
// workgroup of a (b, kv-head) forms the same integer total, so the same
// means.  The block with blk == 0 writes the means to mean_out when it is
// not null.
template <int D, int ROWS, bool SMOOTH, bool FP8 = false, bool MEANP = false>
__global__ __launch_bounds__(256) void quant_block_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ mean,
                                                          int8_t* __restrict__ q,
                                                          float* __restrict__ scale, int H,
                                                          int S, int nblk,
                                                          const long long* __restrict__ partial,
                                                          int nchunk, float* __restrict__ mean_out,
                                                          int bpw) {
    constexpr float kTop = FP8 ? 448.0f : 127.0f;
    constexpr int CPR = D / 8;
    constexpr int CHUNKS = ROWS * CPR;
    constexpr int PER = CHUNKS / 256;
    static_assert(CHUNKS % 256 == 0, "chunks must split evenly");
    __shared__ float red[2][4];
    const int t = threadIdx.x;
    const int cc = t % CPR;   // 256 % CPR == 0: the column chunk is fixed per thread
    const size_t mat = static_cast<size_t>(blockIdx.z) * H + blockIdx.y;
    const uint16_t* xb = x + mat * static_cast<size_t>(S) * D;
    int8_t* qb = q + mat * static_cast<size_t>(S) * D;

    float mu[8];
    if constexpr (MEANP) {
        static_assert(SMOOTH && 256 % D == 0, "means from chunk sums: smoothed K");
        constexpr int G = 256 / D;   // threads per channel
        __shared__ long long red[G][D];
        __shared__ float smu[D];
        const int c = t % D, grp = t / D;
        const long long* src = partial + mat * static_cast<size_t>(nchunk) * D + c;
        long long s4[4] = {0, 0, 0, 0};
        int i = grp;
        for (; i + 3 * G < nchunk; i += 4 * G) {
#pragma unroll
            for (int u = 0; u < 4; ++u) s4[u] += src[static_cast<size_t>(i + u * G) * D];
        }
        for (; i < nchunk; i += G) s4[0] += src[static_cast<size_t>(i) * D];
        red[grp][c] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        __syncthreads();
        if (grp == 0) {
            long long tot = 0;
#pragma unroll
            for (int g2 = 0; g2 < G; ++g2) tot += red[g2][c];
            const double total = __builtin_ldexp(static_cast<double>(tot), -24);
            const float m = static_cast<float>(total / static_cast<double>(S));
            smu[c] = m;
            if (mean_out && blockIdx.x == 0) mean_out[mat * D + c] = m;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e) mu[e] = smu[cc * 8 + e];
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) mu[e] = SMOOTH ? mean[mat * D + cc * 8 + e] : 0.0f;
    }

    // bpw consecutive blocks per workgroup (the means above are formed once
    // for all of them); the block maxima alternate between two LDS slots
    for (int bi = 0; bi < bpw; ++bi) {
    const int blk = blockIdx.x * bpw + bi;
    if (blk >= nblk) break;   // (workgroup-uniform)
    const int r0 = blk * ROWS;
    float v[PER][8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int row = r0 + (t + 256 * i) / CPR;
        if (row < S) {
            const i4x w = *reinterpret_cast<const i4x*>(xb + static_cast<size_t>(row) * D + cc * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const unsigned u = static_cast<unsigned>(w[e]);
                float lo = half_bits_to_float(u & 0xffffu);
                float hi = half_bits_to_float(u >> 16);
                if (SMOOTH) {
                    lo = lo - mu[2 * e];
                    hi = hi - mu[2 * e + 1];
                }
                v[i][2 * e] = lo;
                v[i][2 * e + 1] = hi;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[i][e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
    }
    const float a = block_max(amax, red[bi & 1]);
    const float r = (a == 0.0f) ? 0.0f : __fdiv_rn(kTop, a);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int row = r0 + (t + 256 * i) / CPR;
        if (row < S) {
            unsigned packed[2] = {0u, 0u};
            if constexpr (FP8) {
#pragma unroll
                for (int e = 0; e < 8; e += 2) packed[e / 4] |= e4m3_pair(v[i][e], v[i][e + 1], r) << (8 * (e % 4));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const unsigned b8 = quant_byte(v[i][e], r);
                    packed[e / 4] |= b8 << (8 * (e % 4));
                }
            }
            i2x out;
            out[0] = static_cast<int>(packed[0]);
            out[1] = static_cast<int>(packed[1]);
            *reinterpret_cast<i2x*>(qb + static_cast<size_t>(row) * D + cc * 8) = out;
        }
    }
    if (t == 0) scale[mat * nblk + blk] = (a == 0.0f) ? 0.0f : __fdiv_rn(a, kTop);
    }
}

// 8-bit V of the P.V ablation, pass 1: per (b, kv-head, chunk of kSumChunk
// tokens) the column maxima of |V| (exact, any order).
template <int D>
__global__ __launch_bounds__(256) void v_colmax_kernel(const uint16_t* __restrict__ v, int S,
                                                       int nchunk, float* __restrict__ partial) {
    constexpr int CPR = D / 8;
    constexpr int RG = 256 / CPR;
    __shared__ float red[RG][D];
    const int t = threadIdx.x;
    const int cc = t % CPR, rg = t / CPR;
    const int chunk = blockIdx.x;
    const size_t bk = blockIdx.y;
    constexpr int RPT = kSumChunk / RG;
    const uint16_t* base = v + bk * static_cast<size_t>(S) * D + cc * 8;
    const int r0 = chunk * kSumChunk + rg;
    // every row load in flight before the first max (rows past the sequence
    // read the last row, which leaves the maxima unchanged)
    i4x w[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = r0 + i * RG;
        w[i] = *reinterpret_cast<const i4x*>(base + static_cast<size_t>(r < S ? r : S - 1) * D);
    }
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < RPT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const unsigned u = static_cast<unsigned>(w[i][e]);
            m[2 * e] = fmaxf(m[2 * e], fabsf(half_bits_to_float(u & 0xffffu)));
            m[2 * e + 1] = fmaxf(m[2 * e + 1], fabsf(half_bits_to_float(u >> 16)));
        }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rg][cc * 8 + e] = m[e];
    __syncthreads();
    if (t < D) {
        float a = 0.0f;
        for (int g = 0; g < RG; ++g) a = fmaxf(a, red[g][t]);
        partial[(bk * nchunk + chunk) * D + t] = a;
    }
}

// Pass 2, per (b, kv-head, 64-key tile): a_c = max over the chunks,
// r_c = 448/a_c, code = E4M3(clamp(v r_c)), written TRANSPOSED: vt is
// [B*Hkv, D, Sp] with Sp = 64 * ceil(S/64) and zero codes for keys >= S.
// Tile 0 also writes delta_c = a_c/448.
template <int D>
__global__ __launch_bounds__(256) void v_quant_kernel(const uint16_t* __restrict__ v, int S,
                                                      int nchunk, const float* __restrict__ partial,
                                                      uint8_t* __restrict__ vt,
                                                      float* __restrict__ v_scale) {
    constexpr int CPR = D / 8;                 // 16-byte chunks per V row
    constexpr int OUT_PER = D * 4 / 256;       // 16-byte output chunks per thread
    constexpr int TROW = 64 + 16;              // transposed tile row bytes in LDS
    __shared__ float rs[D];
    __shared__ __attribute__((aligned(16))) uint8_t tile[D * TROW];
    const int t = threadIdx.x;
    const int n0 = blockIdx.x * 64;
    const size_t bk = blockIdx.y;
    const int Sp = gridDim.x * 64;
    {
        // the chunk maxima: 256 / D threads per channel, loads unrolled so
        // they are in flight together
        constexpr int G = 256 / D;
        __shared__ float gmax[G][D];
        const int c = t % D, grp = t / D;
        const float* src = partial + bk * static_cast<size_t>(nchunk) * D + c;
        float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        int i = grp;
        for (; i + 3 * G < nchunk; i += 4 * G) {
#pragma unroll
            for (int u = 0; u < 4; ++u) a4[u] = fmaxf(a4[u], src[static_cast<size_t>(i + u * G) * D]);
        }
        for (; i < nchunk; i += G) a4[0] = fmaxf(a4[0], src[static_cast<size_t>(i) * D]);
        gmax[grp][c] = fmaxf(fmaxf(a4[0], a4[1]), fmaxf(a4[2], a4[3]));
        __syncthreads();
        if (t < D) {
            float a = 0.0f;
#pragma unroll
            for (int g = 0; g < G; ++g) a = fmaxf(a, gmax[g][t]);
            rs[t] = a == 0.0f ? 0.0f : __fdiv_rn(448.0f, a);
            if (blockIdx.x == 0) v_scale[bk * D + t] = a == 0.0f ? 0.0f : __fdiv_rn(a, 448.0f);
        }
    }
    __syncthreads();
    // Codes into the transposed tile: a unit is 4 consecutive rows x one
    // 16-byte column chunk (8 channels); the 4 codes of a channel are one
    // dword of its tile row (the 16 units of a chunk column write 16
    // consecutive dwords: no LDS bank conflicts).  Rows past the sequence
    // give code 0.
    const uint16_t* base = v + bk * static_cast<size_t>(S) * D;
    for (int u = t; u < 16 * CPR; u += 256) {
        const int r0 = (u % 16) * 4, cc = u / 16;
        i4x w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            w[j] = i4x{0, 0, 0, 0};
            if (n0 + r0 + j < S) w[j] = *reinterpret_cast<const i4x*>(base + static_cast<size_t>(n0 + r0 + j) * D + cc * 8);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int ch = cc * 8 + e;
            float x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned word = static_cast<unsigned>(w[j][e >> 1]);
                x[j] = half_bits_to_float((e & 1) ? (word >> 16) : (word & 0xffffu));
            }
            const unsigned code = e4m3_pair(x[0], x[1], rs[ch]) | (e4m3_pair(x[2], x[3], rs[ch]) << 16);
            *reinterpret_cast<unsigned*>(tile + ch * TROW + r0) = code;
        }
    }
    __syncthreads();
    uint8_t* out = vt + bk * static_cast<size_t>(D) * Sp + n0;
#pragma unroll
    for (int i = 0; i < OUT_PER; ++i) {
        const int c = t + 256 * i;
        const int d = c / 4, part = c % 4;
        *reinterpret_cast<i4x*>(out + static_cast<size_t>(d) * Sp + part * 16) =
            *reinterpret_cast<const i4x*>(tile + d * TROW + part * 16);
    }
}

template <int D, bool FP8>
int launch_quantize_d(const attn_shape& s, const void* q, const void* k, int8_t* q_i8,
                      float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                      const QuantWorkspace& ws, hipStream_t st) {
    const int S = s.seq;
    const int BH_kv = s.batch * s.heads_kv;
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    // chunks per column-sum workgroup, so that at most kMaxPartials partial
    // sums per (b, kv-head) remain for the K quantiser to add
    const int cps = ceil_div(ws.nchunk, kMaxPartials);
    const int npart = ceil_div(ws.nchunk, cps);
    // (head_dim 128: the columns in two halves, two workgroups per group of chunks)
    constexpr int NCS = D == 128 ? 2 : 1;
    hipLaunchKernelGGL((k_colsum_kernel<D, NCS>), dim3(npart, BH_kv, NCS), dim3(kColsumThreads), 0, st, kk, S, cps,
                       npart, ws.partial);
    const int nkb = ceil_div(S, kBK), nqb = ceil_div(S, kBQ);
    // K blocks per quantiser workgroup: one while that leaves at most 1024
    // workgroups, else up to 8 (each workgroup adds the partial sums once
    // for all of its blocks)
    const int bpw = std::min(8, std::max(1, nkb * BH_kv / 1024));
    hipLaunchKernelGGL((quant_block_kernel<D, kBK, true, FP8, true>), dim3(ceil_div(nkb, bpw), s.heads_kv, s.batch),
                       dim3(256), 0, st, kk, static_cast<const float*>(nullptr), k_i8, k_scale, s.heads_kv,
                       S, nkb, ws.partial, npart, k_mean, bpw);
    if (qq)
        hipLaunchKernelGGL((quant_block_kernel<D, kBQ, false, FP8>), dim3(nqb, s.heads_q, s.batch),
                           dim3(256), 0, st, qq, static_cast<const float*>(nullptr), q_i8, q_scale,
                           s.heads_q, S, nqb, static_cast<const long long*>(nullptr), 0,
                           static_cast<float*>(nullptr), 1);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ELAUNCH;
}

}  // namespace

// The workspace of attn_quantize_k_noalloc: a file-scope device array.  In
// host code its name is only a stand-in for the symbol; the device address is
// looked up per device with hipGetSymbolAddress (each device holds its own
// copy at its own address) and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

int noalloc_scratch(void** ptr) {
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ATTN_ELAUNCH;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_ELAUNCH;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return ATTN_OK;
}

size_t quant_workspace_layout(const attn_shape& s, size_t* mean_offset, int* nchunk) {
    const int nc = ceil_div(s.seq, kSumChunk);
    const size_t bh = static_cast<size_t>(s.batch) * s.heads_kv;
    const size_t part = bh * nc * s.head_dim * sizeof(long long);
    const size_t off = (part + 255) & ~static_cast<size_t>(255);
    const size_t total = off + bh * s.head_dim * sizeof(float);
    if (mean_offset) *mean_offset = off;
    if (nchunk) *nchunk = nc;
    return (total + 255) & ~static_cast<size_t>(255);
}

int launch_quantize(const attn_shape& s, const void* q, const void* k, int8_t* q_i8,
                    float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                    const QuantWorkspace& ws, hipStream_t st, bool fp8) {
    if (s.head_dim == 64)
        return fp8 ? launch_quantize_d<64, true>(s, q, k, q_i8, q_scale, k_i8, k_scale, k_mean, ws, st)
                   : launch_quantize_d<64, false>(s, q, k, q_i8, q_scale, k_i8, k_scale, k_mean, ws, st);
    return fp8 ? launch_quantize_d<128, true>(s, q, k, q_i8, q_scale, k_i8, k_scale, k_mean, ws, st)
               : launch_quantize_d<128, false>(s, q, k, q_i8, q_scale, k_i8, k_scale, k_mean, ws, st);
}

int launch_quantize_v_fp8(const attn_shape& s, const void* v, uint8_t* vt, float* v_scale,
                          const QuantWorkspace& ws, hipStream_t st) {
    const int S = s.seq;
    const int BH_kv = s.batch * s.heads_kv;
    const uint16_t* vv = static_cast<const uint16_t*>(v);
    // the column maxima reuse the partial-sum area of the workspace (4 of its 8 bytes per entry)
    float* part = reinterpret_cast<float*>(ws.partial);
    const int ntile = ceil_div(S, 64);
    if (s.head_dim == 64) {
        hipLaunchKernelGGL(v_colmax_kernel<64>, dim3(ws.nchunk, BH_kv), dim3(256), 0, st, vv, S, ws.nchunk, part);
        hipLaunchKernelGGL(v_quant_kernel<64>, dim3(ntile, BH_kv), dim3(256), 0, st, vv, S, ws.nchunk, part, vt, v_scale);
    } else {
        hipLaunchKernelGGL(v_colmax_kernel<128>, dim3(ws.nchunk, BH_kv), dim3(256), 0, st, vv, S, ws.nchunk, part);
        hipLaunchKernelGGL(v_quant_kernel<128>, dim3(ntile, BH_kv), dim3(256), 0, st, vv, S, ws.nchunk, part, vt, v_scale);
    }
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ELAUNCH;
}

}  // namespace attn
