// C ABI of libattn.so: argument validation, launch geometry and dispatch.
//
// Validation is plain host code that runs before any HIP call, so every
// rejected argument is observable without a GPU.  The library allocates
// nothing: the caller passes every buffer, including the quantisation
// workspace.
#include "attn_internal.h"
#include "decode_geometry.h"

#include <algorithm>
#include <cmath>
#include <cstring>

namespace attn {
namespace {

constexpr double kLog2e = 1.4426950408889634;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_shape(const attn_shape* s) {
    if (!s) return ATTN_EINVAL;
    if (s->batch <= 0 || s->heads_q <= 0 || s->heads_kv <= 0 || s->seq <= 0 || s->head_dim <= 0)
        return ATTN_EINVAL;
    if (s->head_dim != 64 && s->head_dim != 128) return ATTN_EUNSUPPORTED;
    if (s->heads_q > ATTN_MAX_HEADS || s->heads_kv > ATTN_MAX_HEADS) return ATTN_EUNSUPPORTED;
    if (s->seq > ATTN_MAX_SEQ) return ATTN_EUNSUPPORTED;
    // the (batch, q-head, 128-row tile) work items are counted in an int and
    // launched on a 1-D grid (one or two per workgroup)
    const long long blocks = static_cast<long long>(s->batch) * s->heads_q * ceil_div(s->seq, kBM);
    if (blocks > 0x7fffffffLL) return ATTN_EUNSUPPORTED;
    // the quantisation grids put batch*heads_kv (and batch) in grid dimension y/z
    if (static_cast<long long>(s->batch) * s->heads_kv > 65535LL) return ATTN_EUNSUPPORTED;
    return ATTN_OK;
}

// Builds the q-head -> kv-head map and the launch order of q-heads (stable
// sort by kv-head, so heads that share K/V are launched next to each other).
int build_map(const attn_shape& s, const int32_t* user_map, FwdParams* p) {
    if (!user_map) {
        if (s.heads_q % s.heads_kv != 0) return ATTN_EINVAL;
        const int grp = s.heads_q / s.heads_kv;
        for (int h = 0; h < s.heads_q; ++h) p->kvmap[h] = static_cast<uint8_t>(h / grp);
    } else {
        for (int h = 0; h < s.heads_q; ++h) {
            if (user_map[h] < 0 || user_map[h] >= s.heads_kv) return ATTN_ERANGE;
            p->kvmap[h] = static_cast<uint8_t>(user_map[h]);
        }
    }
    int n = 0;
    bool uniform = s.heads_q % s.heads_kv == 0;
    for (int k = 0; k < s.heads_kv; ++k) {
        const int n0 = n;
        for (int h = 0; h < s.heads_q; ++h)
            if (p->kvmap[h] == k) p->horder[n++] = static_cast<uint8_t>(h);
        if (n - n0 != s.heads_q / s.heads_kv) uniform = false;
    }
    // Launch-order groups (the q-heads of one kv-head, when all are the same
    // size): only when one kv-head's K and V exceed the 4 MB L2 of an XCD.
    // Smaller ones stay L2-resident in any order, and there the per-head order
    // pairs heavy and light causal tiles better (measured: the 1024-token
    // batched MQA workload runs 4 % slower grouped).
    const bool big_kv = 4.0 * s.seq * s.head_dim > 4.0 * 1024 * 1024;
    p->group = uniform && big_kv ? s.heads_q / s.heads_kv : 1;
    return ATTN_OK;
}

int check_scale(float sm_scale, int head_dim, float* scale_log2) {
    if (std::isnan(sm_scale) || std::isinf(sm_scale)) return ATTN_EINVAL;
    const double sc = sm_scale > 0.0f ? static_cast<double>(sm_scale) : 1.0 / std::sqrt(static_cast<double>(head_dim));
    *scale_log2 = static_cast<float>(sc * kLog2e);
    return ATTN_OK;
}

void fill_common(const attn_shape& s, FwdParams* p) {
    p->B = s.batch;
    p->Hq = s.heads_q;
    p->Hkv = s.heads_kv;
    p->S = s.seq;
    p->nqt = ceil_div(s.seq, kBM);
    p->nqblk = ceil_div(s.seq, kBQ);
    p->nkblk = ceil_div(s.seq, kBK);
    p->tile_lo = 0;
    p->ntiles = p->nqt;
}

int check_kv_shape(const attn_kv_shape* s) {
    if (!s) return ATTN_EINVAL;
    if (s->batch <= 0 || s->heads_q <= 0 || s->heads_kv <= 0 || s->seq_q <= 0 || s->seq_kv <= 0 ||
        s->head_dim <= 0)
        return ATTN_EINVAL;
    if (s->seq_q > s->seq_kv) return ATTN_EINVAL;
    if (s->head_dim != 64 && s->head_dim != 128) return ATTN_EUNSUPPORTED;
    if (s->heads_q > ATTN_MAX_HEADS || s->heads_kv > ATTN_MAX_HEADS) return ATTN_EUNSUPPORTED;
    if (s->seq_kv > ATTN_MAX_SEQ || s->seq_q > ATTN_DECODE_MAX_SEQ_Q) return ATTN_EUNSUPPORTED;
    if (static_cast<long long>(s->batch) * s->heads_kv > 65535LL) return ATTN_EUNSUPPORTED;
    return ATTN_OK;
}

// Group tables of the decode launch: q-heads ordered by kv-head, each
// kv-head's first position and count; returns the largest group.
int build_groups(const attn_kv_shape& s, const int32_t* user_map, DecParams* p, int* max_group) {
    uint8_t kvmap[ATTN_MAX_HEADS];
    if (!user_map) {
        if (s.heads_q % s.heads_kv != 0) return ATTN_EINVAL;
        const int grp = s.heads_q / s.heads_kv;
        for (int h = 0; h < s.heads_q; ++h) kvmap[h] = static_cast<uint8_t>(h / grp);
    } else {
        for (int h = 0; h < s.heads_q; ++h) {
            if (user_map[h] < 0 || user_map[h] >= s.heads_kv) return ATTN_ERANGE;
            kvmap[h] = static_cast<uint8_t>(user_map[h]);
        }
    }
    int n = 0, mg = 0;
    for (int k = 0; k < s.heads_kv; ++k) {
        p->gstart[k] = static_cast<uint16_t>(n);
        for (int h = 0; h < s.heads_q; ++h)
            if (kvmap[h] == k) p->horder[n++] = static_cast<uint8_t>(h);
        p->gcount[k] = static_cast<uint16_t>(n - p->gstart[k]);
        if (p->gcount[k] > mg) mg = p->gcount[k];
    }
    *max_group = mg;
    return ATTN_OK;
}

// Validates a decode call and fills everything but the tensor pointers.
int prepare_decode(const attn_kv_shape* shape, const int32_t* kv_head_map, float sm_scale, DecParams* p,
                   size_t* ws_bytes) {
    int st = check_kv_shape(shape);
    if (st != ATTN_OK) return st;
    std::memset(p, 0, sizeof(*p));
    int max_group = 0;
    if ((st = build_groups(*shape, kv_head_map, p, &max_group)) != ATTN_OK) return st;
    if ((st = check_scale(sm_scale, shape->head_dim, &p->scale_log2)) != ATTN_OK) return st;
    const dec::Plan plan = dec::make_plan(shape->batch, shape->heads_kv, shape->seq_q, shape->seq_kv, max_group);
    if (plan.nchunk > 65535) return ATTN_EUNSUPPORTED;
    p->B = shape->batch;
    p->Hq = shape->heads_q;
    p->Hkv = shape->heads_kv;
    p->Sq = shape->seq_q;
    p->Sk = shape->seq_kv;
    p->nkblk = ceil_div(shape->seq_kv, kBK);
    p->hpc = plan.hpc;
    p->nchunk = plan.nchunk;
    p->ntiles = plan.ntiles;
    p->tps = plan.tps;
    p->nsplit = plan.nsplit;
    *ws_bytes = dec::ws_bytes(dec::partial_rows(shape->batch, shape->heads_kv, plan), shape->head_dim);
    return ATTN_OK;
}

void set_workspace(DecParams* p, void* workspace, int D) {
    const dec::Plan plan{p->hpc, p->nchunk, p->ntiles, p->tps, p->nsplit};
    const size_t rows = dec::partial_rows(p->B, p->Hkv, plan);
    char* w = static_cast<char*>(workspace);
    p->ws_o = reinterpret_cast<float*>(w);
    p->ws_m = reinterpret_cast<float*>(w + dec::ws_m_offset(rows, D));
    p->ws_l = reinterpret_cast<float*>(w + dec::ws_l_offset(rows, D));
}

// The INT32 score dump of the INT8 forward (from INT8 Q, or fp16 Q quantised
// in the kernel) for query tiles q_tile_lo..q_tile_hi.
int debug_dump(const attn_shape* shape, const void* q, bool fused_q, const int8_t* k_i8,
               const int32_t* kv_head_map, int causal, int32_t q_tile_lo, int32_t q_tile_hi,
               int32_t* s_out, float* q_scale_out, void* stream) {
    int st = check_shape(shape);
    if (st != ATTN_OK) return st;
    if (!q || !k_i8 || !s_out) return ATTN_EINVAL;
    if (!aligned(q, 16) || !aligned(k_i8, 16) || !aligned(s_out, 4) || (q_scale_out && !aligned(q_scale_out, 4)))
        return ATTN_EINVAL;
    const int nqt = ceil_div(shape->seq, kBM);
    if (q_tile_lo < 0 || q_tile_hi < q_tile_lo || q_tile_hi >= nqt) return ATTN_EINVAL;
    FwdParams p;
    std::memset(&p, 0, sizeof(p));
    if ((st = build_map(*shape, kv_head_map, &p)) != ATTN_OK) return st;
    fill_common(*shape, &p);
    p.q = q;
    p.k = k_i8;
    p.s_out = s_out;
    p.q_scale_out = q_scale_out;
    p.tile_lo = q_tile_lo;
    p.ntiles = q_tile_hi - q_tile_lo + 1;
    return launch_fwd(fused_q ? FwdKind::kDumpInt8FusedQ : FwdKind::kDumpInt8, shape->head_dim, causal != 0, p,
                      static_cast<hipStream_t>(stream));
}

}  // namespace
}  // namespace attn

using namespace attn;

extern "C" {

int attn_quant_blocks(int32_t* bq, int32_t* bk) {
    if (bq) *bq = kBQ;
    if (bk) *bk = kBK;
    return ATTN_OK;
}

size_t attn_quantize_workspace_bytes(const attn_shape* shape) {
    if (check_shape(shape) != ATTN_OK) return 0;
    return quant_workspace_layout(*shape, nullptr, nullptr);
}

int attn_quantize_qk(const attn_shape* shape, const void* q_f16, const void* k_f16, int8_t* q_i8,
                     float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean, void* workspace,
                     void* stream) {
    int st = check_shape(shape);
    if (st != ATTN_OK) return st;
    if (!q_f16 || !k_f16 || !q_i8 || !q_scale || !k_i8 || !k_scale || !workspace) return ATTN_EINVAL;
    if (!aligned(q_f16, 16) || !aligned(k_f16, 16) || !aligned(q_i8, 16) || !aligned(k_i8, 16) ||
        !aligned(workspace, 16) || !aligned(q_scale, 4) || !aligned(k_scale, 4) ||
        (k_mean && !aligned(k_mean, 4)))
        return ATTN_EINVAL;
    size_t mean_off = 0;
    QuantWorkspace ws;
    quant_workspace_layout(*shape, &mean_off, &ws.nchunk);
    ws.partial = static_cast<long long*>(workspace);
    ws.mean = reinterpret_cast<float*>(static_cast<char*>(workspace) + mean_off);
    return launch_quantize(*shape, q_f16, k_f16, q_i8, q_scale, k_i8, k_scale, k_mean, ws,
                           static_cast<hipStream_t>(stream));
}

int attn_quantize_k(const attn_shape* shape, const void* k_f16, int8_t* k_i8, float* k_scale,
                    float* k_mean, void* workspace, void* stream) {
    int st = check_shape(shape);
    if (st != ATTN_OK) return st;
    if (!k_f16 || !k_i8 || !k_scale || !workspace) return ATTN_EINVAL;
    if (!aligned(k_f16, 16) || !aligned(k_i8, 16) || !aligned(workspace, 16) || !aligned(k_scale, 4) ||
        (k_mean && !aligned(k_mean, 4)))
        return ATTN_EINVAL;
    size_t mean_off = 0;
    QuantWorkspace ws;
    quant_workspace_layout(*shape, &mean_off, &ws.nchunk);
    ws.partial = static_cast<long long*>(workspace);
    ws.mean = reinterpret_cast<float*>(static_cast<char*>(workspace) + mean_off);
    return launch_quantize(*shape, nullptr, k_f16, nullptr, nullptr, k_i8, k_scale, k_mean, ws,
                           static_cast<hipStream_t>(stream));
}

int attn_quantize_k_noalloc(const attn_shape* shape, const void* k_f16, int8_t* k_i8, float* k_scale,
                            float* k_mean, void* stream) {
    int st = check_shape(shape);
    if (st != ATTN_OK) return st;
    if (!k_f16 || !k_i8 || !k_scale) return ATTN_EINVAL;
    if (!aligned(k_f16, 16) || !aligned(k_i8, 16) || !aligned(k_scale, 4) || (k_mean && !aligned(k_mean, 4)))
        return ATTN_EINVAL;
    size_t mean_off = 0;
    QuantWorkspace ws;
    if (quant_workspace_layout(*shape, &mean_off, &ws.nchunk) > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ESCRATCH;
    void* scratch = nullptr;
    if ((st = noalloc_scratch(&scratch)) != ATTN_OK) return st;
    ws.partial = static_cast<long long*>(scratch);
    ws.mean = reinterpret_cast<float*>(static_cast<char*>(scratch) + mean_off);
    return launch_quantize(*shape, nullptr, k_f16, nullptr, nullptr, k_i8, k_scale, k_mean, ws,
                           static_cast<hipStream_t>(stream));
}

int attn_fwd_int8_fused_q(const attn_shape* shape, const void* q_f16, const int8_t* k_i8,
                          const float* k_scale, const void* v_f16, void* o_f16, float* lse,
                          float* q_scale_out, const int32_t* kv_head_map, int causal,
                          float sm_scale, void* stream) {
    int st = check_shape(shape);
    if (st != ATTN_OK) return st;
    if (!q_f16 || !k_i8 || !k_scale || !v_f16 || !o_f16) return ATTN_EINVAL;
    if (!aligned(q_f16, 16) || !aligned(k_i8, 16) || !aligned(v_f16, 16) || !aligned(o_f16, 16) ||
        !aligned(k_scale, 4) || (lse && !aligned(lse, 4)) || (q_scale_out && !aligned(q_scale_out, 4)))
        return ATTN_EINVAL;
    FwdParams p;
    std::memset(&p, 0, sizeof(p));
    if ((st = build_map(*shape, kv_head_map, &p)) != ATTN_OK) return st;
    if ((st = check_scale(sm_scale, shape->head_dim, &p.scale_log2)) != ATTN_OK) return st;
    fill_common(*shape, &p);
    p.q = q_f16;
    p.k = k_i8;
    p.v = v_f16;
    p.o = o_f16;
    p.lse = lse;
    p.k_scale = k_scale;
    p.q_scale_out = q_scale_out;
    return launch_fwd(FwdKind::kInt8FusedQ, shape->head_dim, causal != 0, p, static_cast<hipStream_t>(stream));
}

int attn_fwd_int8(const attn_shape* shape, const int8_t* q_i8, const float* q_scale,
                  const int8_t* k_i8, const float* k_scale, const void* v_f16, void* o_f16,
                  float* lse, const int32_t* kv_head_map, int causal, float sm_scale,
                  void* stream) {
    int st = check_shape(shape);
    if (st != ATTN_OK) return st;
    if (!q_i8 || !q_scale || !k_i8 || !k_scale || !v_f16 || !o_f16) return ATTN_EINVAL;
    if (!aligned(q_i8, 16) || !aligned(k_i8, 16) || !aligned(v_f16, 16) || !aligned(o_f16, 16) ||
        !aligned(q_scale, 4) || !aligned(k_scale, 4) || (lse && !aligned(lse, 4)))
        return ATTN_EINVAL;
    FwdParams p;
    std::memset(&p, 0, sizeof(p));
    if ((st = build_map(*shape, kv_head_map, &p)) != ATTN_OK) return st;
    if ((st = check_scale(sm_scale, shape->head_dim, &p.scale_log2)) != ATTN_OK) return st;
    fill_common(*shape, &p);
    p.q = q_i8;
    p.k = k_i8;
    p.v = v_f16;
    p.o = o_f16;
    p.lse = lse;
    p.q_scale = q_scale;
    p.k_scale = k_scale;
    return launch_fwd(FwdKind::kInt8, shape->head_dim, causal != 0, p, static_cast<hipStream_t>(stream));
}

int attn_fwd_fp16(const attn_shape* shape, const void* q_f16, const void* k_f16, const void* v_f16,
                  void* o_f16, float* lse, const int32_t* kv_head_map, int causal, float sm_scale,
                  void* stream) {
    int st = check_shape(shape);
    if (st != ATTN_OK) return st;
    if (!q_f16 || !k_f16 || !v_f16 || !o_f16) return ATTN_EINVAL;
    if (!aligned(q_f16, 16) || !aligned(k_f16, 16) || !aligned(v_f16, 16) || !aligned(o_f16, 16) ||
        (lse && !aligned(lse, 4)))
        return ATTN_EINVAL;
    FwdParams p;
    std::memset(&p, 0, sizeof(p));
    if ((st = build_map(*shape, kv_head_map, &p)) != ATTN_OK) return st;
    if ((st = check_scale(sm_scale, shape->head_dim, &p.scale_log2)) != ATTN_OK) return st;
    fill_common(*shape, &p);
    p.q = q_f16;
    p.k = k_f16;
    p.v = v_f16;
    p.o = o_f16;
    p.lse = lse;
    return launch_fwd(FwdKind::kFp16, shape->head_dim, causal != 0, p, static_cast<hipStream_t>(stream));
}

int attn_debug_qk_int32(const attn_shape* shape, const int8_t* q_i8, const int8_t* k_i8,
                        const int32_t* kv_head_map, int causal, int32_t q_tile_lo,
                        int32_t q_tile_hi, int32_t* s_out, void* stream) {
    return debug_dump(shape, q_i8, false, k_i8, kv_head_map, causal, q_tile_lo, q_tile_hi, s_out, nullptr,
                      stream);
}

int attn_debug_qk_int32_fused_q(const attn_shape* shape, const void* q_f16, const int8_t* k_i8,
                                const int32_t* kv_head_map, int causal, int32_t q_tile_lo,
                                int32_t q_tile_hi, int32_t* s_out, float* q_scale_out,
                                void* stream) {
    return debug_dump(shape, q_f16, true, k_i8, kv_head_map, causal, q_tile_lo, q_tile_hi, s_out, q_scale_out,
                      stream);
}

int attn_quantize_qk_fp8(const attn_shape* shape, const void* q_f16, const void* k_f16,
                         uint8_t* q_f8, float* q_scale, uint8_t* k_f8, float* k_scale,
                         float* k_mean, void* workspace, void* stream) {
    int st = check_shape(shape);
    if (st != ATTN_OK) return st;
    if (!q_f16 || !k_f16 || !q_f8 || !q_scale || !k_f8 || !k_scale || !workspace) return ATTN_EINVAL;
    if (!aligned(q_f16, 16) || !aligned(k_f16, 16) || !aligned(q_f8, 16) || !aligned(k_f8, 16) ||
        !aligned(workspace, 16) || !aligned(q_scale, 4) || !aligned(k_scale, 4) ||
        (k_mean && !aligned(k_mean, 4)))
        return ATTN_EINVAL;
    size_t mean_off = 0;
    QuantWorkspace ws;
    quant_workspace_layout(*shape, &mean_off, &ws.nchunk);
    ws.partial = static_cast<long long*>(workspace);
    ws.mean = reinterpret_cast<float*>(static_cast<char*>(workspace) + mean_off);
    return launch_quantize(*shape, q_f16, k_f16, reinterpret_cast<int8_t*>(q_f8), q_scale,
                           reinterpret_cast<int8_t*>(k_f8), k_scale, k_mean, ws,
                           static_cast<hipStream_t>(stream), true);
}

int attn_fwd_fp8(const attn_shape* shape, const uint8_t* q_f8, const float* q_scale,
                 const uint8_t* k_f8, const float* k_scale, const void* v_f16, void* o_f16,
                 float* lse, const int32_t* kv_head_map, int causal, float sm_scale, void* stream) {
    int st = check_shape(shape);
    if (st != ATTN_OK) return st;
    if (!q_f8 || !q_scale || !k_f8 || !k_scale || !v_f16 || !o_f16) return ATTN_EINVAL;
    if (!aligned(q_f8, 16) || !aligned(k_f8, 16) || !aligned(v_f16, 16) || !aligned(o_f16, 16) ||
        !aligned(q_scale, 4) || !aligned(k_scale, 4) || (lse && !aligned(lse, 4)))
        return ATTN_EINVAL;
    FwdParams p;
    std::memset(&p, 0, sizeof(p));
    if ((st = build_map(*shape, kv_head_map, &p)) != ATTN_OK) return st;
    if ((st = check_scale(sm_scale, shape->head_dim, &p.scale_log2)) != ATTN_OK) return st;
    fill_common(*shape, &p);
    p.q = q_f8;
    p.k = k_f8;
    p.v = v_f16;
    p.o = o_f16;
    p.lse = lse;
    p.q_scale = q_scale;
    p.k_scale = k_scale;
    return launch_fwd(FwdKind::kFp8, shape->head_dim, causal != 0, p, static_cast<hipStream_t>(stream));
}

int64_t attn_v_fp8_stride(const attn_shape* shape) {
    if (check_shape(shape) != ATTN_OK) return 0;
    return static_cast<int64_t>(ceil_div(shape->seq, kBK)) * kBK;
}

int attn_quantize_v_fp8(const attn_shape* shape, const void* v_f16, uint8_t* v_f8t, float* v_scale,
                        void* workspace, void* stream) {
    int st = check_shape(shape);
    if (st != ATTN_OK) return st;
    if (!v_f16 || !v_f8t || !v_scale || !workspace) return ATTN_EINVAL;
    if (!aligned(v_f16, 16) || !aligned(v_f8t, 16) || !aligned(workspace, 16) || !aligned(v_scale, 4))
        return ATTN_EINVAL;
    size_t mean_off = 0;
    QuantWorkspace ws;
    quant_workspace_layout(*shape, &mean_off, &ws.nchunk);
    ws.partial = static_cast<long long*>(workspace);
    ws.mean = reinterpret_cast<float*>(static_cast<char*>(workspace) + mean_off);
    return launch_quantize_v_fp8(*shape, v_f16, v_f8t, v_scale, ws, static_cast<hipStream_t>(stream));
}

int attn_fwd_int8_pv8(const attn_shape* shape, const int8_t* q_i8, const float* q_scale,
                      const int8_t* k_i8, const float* k_scale, const uint8_t* v_f8t,
                      const float* v_scale, void* o_f16, float* lse, const int32_t* kv_head_map,
                      int causal, float sm_scale, void* stream) {
    int st = check_shape(shape);
    if (st != ATTN_OK) return st;
    if (!q_i8 || !q_scale || !k_i8 || !k_scale || !v_f8t || !v_scale || !o_f16) return ATTN_EINVAL;
    if (!aligned(q_i8, 16) || !aligned(k_i8, 16) || !aligned(v_f8t, 16) || !aligned(o_f16, 16) ||
        !aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4) || (lse && !aligned(lse, 4)))
        return ATTN_EINVAL;
    FwdParams p;
    std::memset(&p, 0, sizeof(p));
    if ((st = build_map(*shape, kv_head_map, &p)) != ATTN_OK) return st;
    if ((st = check_scale(sm_scale, shape->head_dim, &p.scale_log2)) != ATTN_OK) return st;
    fill_common(*shape, &p);
    p.q = q_i8;
    p.k = k_i8;
    p.v = v_f8t;
    p.o = o_f16;
    p.lse = lse;
    p.q_scale = q_scale;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    return launch_fwd(FwdKind::kInt8Pv8, shape->head_dim, causal != 0, p, static_cast<hipStream_t>(stream));
}

size_t attn_decode_workspace_bytes(const attn_kv_shape* shape, const int32_t* kv_head_map) {
    DecParams p;
    size_t bytes = 0;
    if (prepare_decode(shape, kv_head_map, 0.0f, &p, &bytes) != ATTN_OK) return 0;
    return bytes;
}

int attn_decode_int8(const attn_kv_shape* shape, const void* q_f16, const int8_t* k_i8,
                     const float* k_scale, const void* v_f16, void* o_f16, float* lse,
                     float* q_scale_out, const int32_t* kv_head_map, int causal, float sm_scale,
                     void* workspace, void* stream) {
    DecParams p;
    size_t bytes = 0;
    int st = prepare_decode(shape, kv_head_map, sm_scale, &p, &bytes);
    if (st != ATTN_OK) return st;
    if (!q_f16 || !k_i8 || !k_scale || !v_f16 || !o_f16 || !workspace) return ATTN_EINVAL;
    if (!aligned(q_f16, 16) || !aligned(k_i8, 16) || !aligned(v_f16, 16) || !aligned(o_f16, 16) ||
        !aligned(workspace, 16) || !aligned(k_scale, 4) || (lse && !aligned(lse, 4)) ||
        (q_scale_out && !aligned(q_scale_out, 4)))
        return ATTN_EINVAL;
    p.q = q_f16;
    p.k = k_i8;
    p.v = v_f16;
    p.o = o_f16;
    p.lse = lse;
    p.k_scale = k_scale;
    p.q_scale_out = q_scale_out;
    set_workspace(&p, workspace, shape->head_dim);
    return launch_decode(true, shape->head_dim, causal != 0, p, static_cast<hipStream_t>(stream));
}

int attn_decode_fp16(const attn_kv_shape* shape, const void* q_f16, const void* k_f16,
                     const void* v_f16, void* o_f16, float* lse, const int32_t* kv_head_map,
                     int causal, float sm_scale, void* workspace, void* stream) {
    DecParams p;
    size_t bytes = 0;
    int st = prepare_decode(shape, kv_head_map, sm_scale, &p, &bytes);
    if (st != ATTN_OK) return st;
    if (!q_f16 || !k_f16 || !v_f16 || !o_f16 || !workspace) return ATTN_EINVAL;
    if (!aligned(q_f16, 16) || !aligned(k_f16, 16) || !aligned(v_f16, 16) || !aligned(o_f16, 16) ||
        !aligned(workspace, 16) || (lse && !aligned(lse, 4)))
        return ATTN_EINVAL;
    p.q = q_f16;
    p.k = k_f16;
    p.v = v_f16;
    p.o = o_f16;
    p.lse = lse;
    set_workspace(&p, workspace, shape->head_dim);
    return launch_decode(false, shape->head_dim, causal != 0, p, static_cast<hipStream_t>(stream));
}

int attn_block_mask_tiles(int32_t seq, int32_t* q_tiles, int32_t* k_tiles) {
    if (seq <= 0 || seq > ATTN_MAX_SEQ) return ATTN_EINVAL;
    if (q_tiles) *q_tiles = ceil_div(seq, ATTN_MASK_TILE_Q);
    if (k_tiles) *k_tiles = ceil_div(seq, ATTN_MASK_TILE_K);
    return ATTN_OK;
}

int attn_block_mask_apb(int32_t seq, int32_t anchor, int32_t passing, uint8_t* mask) {
    if (!mask || seq <= 0 || seq > ATTN_MAX_SEQ || anchor < 0 || passing < 0) return ATTN_EINVAL;
    if (anchor % ATTN_MASK_TILE_Q || passing % ATTN_MASK_TILE_Q || anchor + passing > seq) return ATTN_EINVAL;
    const int nqt = ceil_div(seq, ATTN_MASK_TILE_Q), nkt = ceil_div(seq, ATTN_MASK_TILE_K);
    for (int qt = 0; qt < nqt; ++qt) {
        const int i0 = qt * ATTN_MASK_TILE_Q, i1 = std::min(seq, i0 + ATTN_MASK_TILE_Q) - 1;
        const bool passing_rows = i0 >= anchor && i0 < anchor + passing;
        for (int kt = 0; kt < nkt; ++kt) {
            const int j0 = kt * ATTN_MASK_TILE_K, j1 = std::min(seq, j0 + ATTN_MASK_TILE_K) - 1;
            uint8_t m = 0;
            if (!passing_rows) m = j1 <= i0 ? 1 : (j0 <= i1 ? 2 : 0);   // causal over [anchor|passing|local]
            mask[static_cast<size_t>(qt) * nkt + kt] = m;
        }
    }
    return ATTN_OK;
}

int attn_block_mask_csr(int32_t seq, const uint8_t* mask, int32_t* row_ptr, int32_t* cols, int32_t* nnz) {
    if (!mask || !row_ptr || !cols || !nnz || seq <= 0 || seq > ATTN_MAX_SEQ) return ATTN_EINVAL;
    const int nqt = ceil_div(seq, ATTN_MASK_TILE_Q), nkt = ceil_div(seq, ATTN_MASK_TILE_K);
    for (size_t e = 0; e < static_cast<size_t>(nqt) * nkt; ++e)
        if (mask[e] > 2) return ATTN_EINVAL;
    int n = 0;
    for (int qt = 0; qt < nqt; ++qt) {
        row_ptr[qt] = n;
        const int i0 = qt * ATTN_MASK_TILE_Q, i1 = std::min(seq, i0 + ATTN_MASK_TILE_Q) - 1;
        for (int kt = 0; kt < nkt; ++kt) {
            int m = mask[static_cast<size_t>(qt) * nkt + kt];
            const int j0 = kt * ATTN_MASK_TILE_K, j1 = std::min(seq, j0 + ATTN_MASK_TILE_K) - 1;
            if (m == 2 && j1 <= i0) m = 1;   // every key precedes every query of the tile
            if (m == 2 && j0 > i1) m = 0;    // no key precedes any query of the tile
            if (m) cols[n++] = (kt << 2) | m;
        }
    }
    row_ptr[nqt] = n;
    *nnz = n;
    return ATTN_OK;
}

int attn_fwd_fp16_masked(const attn_shape* shape, const void* q_f16, const void* k_f16, const void* v_f16,
                         void* o_f16, float* lse, const int32_t* kv_head_map, const int32_t* mask_row_ptr,
                         const int32_t* mask_cols, int32_t mask_nnz, float sm_scale, void* stream) {
    int st = check_shape(shape);
    if (st != ATTN_OK) return st;
    if (!q_f16 || !k_f16 || !v_f16 || !o_f16 || !mask_row_ptr || mask_nnz < 0 || (mask_nnz > 0 && !mask_cols))
        return ATTN_EINVAL;
    if (!aligned(q_f16, 16) || !aligned(k_f16, 16) || !aligned(v_f16, 16) || !aligned(o_f16, 16) ||
        (lse && !aligned(lse, 4)) || !aligned(mask_row_ptr, 4) || !aligned(mask_cols, 4))
        return ATTN_EINVAL;
    FwdParams p;
    std::memset(&p, 0, sizeof(p));
    if ((st = build_map(*shape, kv_head_map, &p)) != ATTN_OK) return st;
    if ((st = check_scale(sm_scale, shape->head_dim, &p.scale_log2)) != ATTN_OK) return st;
    fill_common(*shape, &p);
    p.q = q_f16;
    p.k = k_f16;
    p.v = v_f16;
    p.o = o_f16;
    p.lse = lse;
    p.mask_rowptr = mask_row_ptr;
    p.mask_cols = mask_cols;
    p.mask_nnz = mask_nnz;
    return launch_fwd(FwdKind::kFp16Mask, shape->head_dim, false, p, static_cast<hipStream_t>(stream));
}

int attn_fwd_int8_masked(const attn_shape* shape, const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                         const float* k_scale, const void* v_f16, void* o_f16, float* lse,
                         const int32_t* kv_head_map, const int32_t* mask_row_ptr, const int32_t* mask_cols,
                         int32_t mask_nnz, float sm_scale, void* stream) {
    int st = check_shape(shape);
    if (st != ATTN_OK) return st;
    if (!q_i8 || !q_scale || !k_i8 || !k_scale || !v_f16 || !o_f16 || !mask_row_ptr || mask_nnz < 0 ||
        (mask_nnz > 0 && !mask_cols))
        return ATTN_EINVAL;
    if (!aligned(q_i8, 16) || !aligned(k_i8, 16) || !aligned(v_f16, 16) || !aligned(o_f16, 16) ||
        !aligned(q_scale, 4) || !aligned(k_scale, 4) || (lse && !aligned(lse, 4)) || !aligned(mask_row_ptr, 4) ||
        !aligned(mask_cols, 4))
        return ATTN_EINVAL;
    FwdParams p;
    std::memset(&p, 0, sizeof(p));
    if ((st = build_map(*shape, kv_head_map, &p)) != ATTN_OK) return st;
    if ((st = check_scale(sm_scale, shape->head_dim, &p.scale_log2)) != ATTN_OK) return st;
    fill_common(*shape, &p);
    p.q = q_i8;
    p.k = k_i8;
    p.v = v_f16;
    p.o = o_f16;
    p.lse = lse;
    p.q_scale = q_scale;
    p.k_scale = k_scale;
    p.mask_rowptr = mask_row_ptr;
    p.mask_cols = mask_cols;
    p.mask_nnz = mask_nnz;
    return launch_fwd(FwdKind::kInt8Mask, shape->head_dim, false, p, static_cast<hipStream_t>(stream));
}

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_EINVAL: return "invalid argument";
        case ATTN_EUNSUPPORTED: return "unsupported shape";
        case ATTN_ELAUNCH: return "kernel launch failed";
        case ATTN_ERANGE: return "kv_head_map entry out of range";
        case ATTN_ESCRATCH: return "shape exceeds the no-allocation scratch buffer (ATTN_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

}  // extern "C"
