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
// quantisation) with 16-byte loads and writes int8 with 8-byte stores.  Up to
// 8192 tokens the K quantiser adds the chunk sums of its (b, kv-head) itself,
// so K takes two launches (sums, quantisation) instead of three.
#include "attn_internal.h"

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

// Per (b, kv-head, chunk of kSumChunk tokens): exact column sums of K.
// Thread t owns one 16-byte column chunk (8 channels) and every RG-th row of
// the chunk; all of its row loads are issued before the first add (rows past
// the sequence read the last row and are dropped).  The sums are taken in
// fp64, which is exact here: every fp16 value is an integer multiple of 2^-24
// below 2^40 in those units, so any sum of at most kSumChunk of them is such
// a multiple below 2^48 < 2^53.  The chunk total is then stored as that
// integer (int64), which keeps the cross-chunk total exact in any order.
constexpr int kColsumThreads = 512;
template <int D>
__global__ __launch_bounds__(kColsumThreads) void k_colsum_kernel(const uint16_t* __restrict__ k, int S,
                                                                  int nchunk,
                                                                  long long* __restrict__ partial) {
    constexpr int CPR = D / 8;                  // 16-byte chunks per row
    constexpr int RG = kColsumThreads / CPR;    // row groups
    constexpr int RPT = kSumChunk / RG;         // rows per thread
    static_assert(kSumChunk % RG == 0 && kSumChunk * 65536.0 * 16777216.0 < 9007199254740992.0,
                  "exact fp64 chunk sums");
    __shared__ double red[RG][D];
    const int t = threadIdx.x;
    const int cc = t % CPR, rg = t / CPR;
    const int chunk = blockIdx.x;
    const size_t bk = blockIdx.y;
    const uint16_t* base = k + bk * static_cast<size_t>(S) * D + cc * 8;
    const int r0 = chunk * kSumChunk + rg;
    i4x v[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = r0 + i * RG;
        v[i] = *reinterpret_cast<const i4x*>(base + static_cast<size_t>(r < S ? r : S - 1) * D);
    }
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
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
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rg][cc * 8 + e] = acc[e];
    __syncthreads();
    if (t < D) {
        double s = 0.0;
#pragma unroll
        for (int g = 0; g < RG; ++g) s += red[g][t];
        partial[(bk * nchunk + chunk) * D + t] = static_cast<long long>(__builtin_ldexp(s, 24));
    }
}

// Per (b, kv-head): total over chunks, mu = fp32(fp64(sum) / S).  kMeanGroups
// threads per channel each add every kMeanGroups-th chunk (loads unrolled so
// they are in flight together), then LDS combines the groups.
constexpr int kMeanGroups = 4;
template <int D>
__global__ __launch_bounds__(D * kMeanGroups) void k_mean_kernel(const long long* __restrict__ partial, int S,
                                                                 int nchunk, float* __restrict__ mean,
                                                                 float* __restrict__ mean_out) {
    __shared__ long long red[kMeanGroups][D];
    const size_t bk = blockIdx.x;
    const int c = threadIdx.x % D, grp = threadIdx.x / D;
    const long long* src = partial + bk * static_cast<size_t>(nchunk) * D + c;
    long long s[4] = {0, 0, 0, 0};
    int i = grp;
    for (; i + 3 * kMeanGroups < nchunk; i += 4 * kMeanGroups) {
#pragma unroll
        for (int u = 0; u < 4; ++u) s[u] += src[static_cast<size_t>(i + u * kMeanGroups) * D];
    }
    for (; i < nchunk; i += kMeanGroups) s[0] += src[static_cast<size_t>(i) * D];
    red[grp][c] = (s[0] + s[1]) + (s[2] + s[3]);
    __syncthreads();
    if (grp == 0) {
        long long tot = 0;
#pragma unroll
        for (int g = 0; g < kMeanGroups; ++g) tot += red[g][c];
        // (double)tot is exact below 2^53 and correctly rounded above; the
        // 2^-24 scaling is exact; the division and the narrowing are IEEE
        // operations.
        const double total = __builtin_ldexp(static_cast<double>(tot), -24);
        const float mu = static_cast<float>(total / static_cast<double>(S));
        mean[bk * D + c] = mu;
        if (mean_out) mean_out[bk * D + c] = mu;
    }
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ int quant_one(float x, float r) {
    float t = __builtin_rintf(x * r);
    t = fminf(fmaxf(t, -127.0f), 127.0f);
    return static_cast<int>(t);
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
// MEANP (with SMOOTH): the workgroup adds the per-chunk exact channel sums of
// its (b, kv-head) itself - the same integer totals and the same division as
// k_mean_kernel, so the same means - instead of reading them from `mean`;
// for short sequences this saves the separate mean launch.  The block with
// blk == 0 writes the means to mean_out when it is not null.
template <int D, int ROWS, bool SMOOTH, bool FP8 = false, bool MEANP = false>
__global__ __launch_bounds__(256) void quant_block_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ mean,
                                                          int8_t* __restrict__ q,
                                                          float* __restrict__ scale, int H,
                                                          int S, int nblk,
                                                          const long long* __restrict__ partial,
                                                          int nchunk, float* __restrict__ mean_out) {
    constexpr float kTop = FP8 ? 448.0f : 127.0f;
    constexpr int CPR = D / 8;
    constexpr int CHUNKS = ROWS * CPR;
    constexpr int PER = CHUNKS / 256;
    static_assert(CHUNKS % 256 == 0, "chunks must split evenly");
    __shared__ float red[4];
    const int t = threadIdx.x;
    const int cc = t % CPR;   // 256 % CPR == 0: the column chunk is fixed per thread
    const int blk = blockIdx.x;
    const size_t mat = static_cast<size_t>(blockIdx.z) * H + blockIdx.y;
    const uint16_t* xb = x + mat * static_cast<size_t>(S) * D;
    int8_t* qb = q + mat * static_cast<size_t>(S) * D;
    const int r0 = blk * ROWS;

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
            if (mean_out && blk == 0) mean_out[mat * D + c] = m;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e) mu[e] = smu[cc * 8 + e];
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) mu[e] = SMOOTH ? mean[mat * D + cc * 8 + e] : 0.0f;
    }

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
    const float a = block_max(amax, red);
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
                    const unsigned b8 = static_cast<unsigned>(quant_one(v[i][e], r)) & 0xffu;
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

// Up to this many chunk sums per (b, kv-head) (sequences up to 8192 tokens)
// the K quantiser adds them itself; longer sequences keep the mean kernel,
// whose one reduction per (b, kv-head) is cheaper than one per K block.
constexpr int kMeanInQuantMaxChunks = 32;

template <int D, bool FP8>
int launch_quantize_d(const attn_shape& s, const void* q, const void* k, int8_t* q_i8,
                      float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                      const QuantWorkspace& ws, hipStream_t st) {
    const int S = s.seq;
    const int BH_kv = s.batch * s.heads_kv;
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    hipLaunchKernelGGL(k_colsum_kernel<D>, dim3(ws.nchunk, BH_kv), dim3(kColsumThreads), 0, st, kk, S,
                       ws.nchunk, ws.partial);
    const int nkb = ceil_div(S, kBK), nqb = ceil_div(S, kBQ);
    if (ws.nchunk <= kMeanInQuantMaxChunks) {
        hipLaunchKernelGGL((quant_block_kernel<D, kBK, true, FP8, true>), dim3(nkb, s.heads_kv, s.batch),
                           dim3(256), 0, st, kk, static_cast<const float*>(nullptr), k_i8, k_scale, s.heads_kv,
                           S, nkb, ws.partial, ws.nchunk, k_mean);
    } else {
        hipLaunchKernelGGL(k_mean_kernel<D>, dim3(BH_kv), dim3(D * kMeanGroups), 0, st, ws.partial, S, ws.nchunk,
                           ws.mean, k_mean);
        hipLaunchKernelGGL((quant_block_kernel<D, kBK, true, FP8>), dim3(nkb, s.heads_kv, s.batch),
                           dim3(256), 0, st, kk, ws.mean, k_i8, k_scale, s.heads_kv, S, nkb,
                           static_cast<const long long*>(nullptr), 0, static_cast<float*>(nullptr));
    }
    if (qq)
        hipLaunchKernelGGL((quant_block_kernel<D, kBQ, false, FP8>), dim3(nqb, s.heads_q, s.batch),
                           dim3(256), 0, st, qq, static_cast<const float*>(nullptr), q_i8, q_scale,
                           s.heads_q, S, nqb, static_cast<const long long*>(nullptr), 0,
                           static_cast<float*>(nullptr));
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
