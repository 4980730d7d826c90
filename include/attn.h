/*
 * attn.h - C ABI of the MI355X (gfx950) 8-bit attention forward library
 * (libattn.so).
 *
 * The library computes the attention forward pass O = softmax(Q K^T * scale) V
 * in two forms:
 *   - the 8-bit SageAttention form: K is smoothed by subtracting its
 *     per-channel mean over tokens, Q and K are quantised per block to INT8,
 *     Q K^T runs as an INT8 contraction with INT32 accumulation and is
 *     dequantised with the block scales, and P V runs with P and V in FP16;
 *   - an exact FP16 FlashAttention-style form (tiled, online softmax).
 *
 * Sources (web pages; cited by title and section):
 *   [SA]       "又快又准，即插即用！清华8比特量化Attention，两倍加速于
 *              FlashAttention2，各端到端任务均不掉点！" (SageAttention article,
 *              17aitech reprint), section 技术方案 (technical approach) and its
 *              plug-and-play example (a drop-in for scaled_dot_product_attention).
 *   [MHA-GQA]  "注意力即一切：从 MHA 到 GQA" (bojinhu.xyz), §2.2 (the four steps),
 *              §2.3 (causal mask), §4.1 (MQA), §5.1 (GQA), §8.2 (tiling and
 *              online softmax).
 *   [FA-guide] "FlashAttention" guide (aiunderstanding.org): tiling in on-chip
 *              memory, online softmax, exactness.
 *
 * Conventions shared by every call
 * --------------------------------
 * Layout.  Q, O: [batch, heads_q, seq, head_dim]; K, V: [batch, heads_kv, seq,
 *   head_dim]; all contiguous, row-major, head_dim innermost.  Q and K share
 *   one sequence length.  head_dim must be 64 or 128.
 * Memory.  Every tensor pointer is DEVICE memory owned by the caller, 16-byte
 *   aligned.  The library allocates and frees nothing and keeps no mutable
 *   global state beyond per-device caches of the compute-unit count (which
 *   sizes the forward launches) and of the address of its no-allocation
 *   scratch array (attn_quantize_k_noalloc); calls are thread-safe.
 *   kv_head_map is a HOST pointer.
 * Execution.  Every call enqueues its kernels on `stream` (a hipStream_t; NULL
 *   means the null stream) and returns without synchronising.
 * Errors.  Calls return a status code and never throw.  All argument checks run
 *   on the host before any HIP call, so a rejected call touches no device
 *   state.  A failed launch returns ATTN_ELAUNCH.  Input values must be finite;
 *   results for inf/nan inputs are unspecified.
 * GQA/MQA ([MHA-GQA] §4.1, §5.1).  Query head h reads K/V of kv-head map[h].
 *   kv_head_map == NULL selects map[h] = h / (heads_q / heads_kv), which needs
 *   heads_q % heads_kv == 0.  An explicit map has heads_q entries in
 *   [0, heads_kv).  heads_q and heads_kv are at most ATTN_MAX_HEADS.
 * Scale.  sm_scale <= 0 selects 1/sqrt(head_dim) ([MHA-GQA] §2.2).
 * Causal ([MHA-GQA] §2.3).  causal != 0 gives key j weight 0 for query i when
 *   j > i.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct attn_shape {
    int32_t batch;
    int32_t heads_q;
    int32_t heads_kv;
    int32_t seq;       /* 1 .. ATTN_MAX_SEQ */
    int32_t head_dim;  /* 64 or 128 */
} attn_shape;

enum {
    ATTN_OK = 0,
    ATTN_EINVAL = -1,       /* null pointer, non-positive size, misalignment, bad argument */
    ATTN_EUNSUPPORTED = -2, /* head_dim not 64/128, too many heads, sequence too long */
    ATTN_ELAUNCH = -3,      /* a kernel launch failed */
    ATTN_ERANGE = -4,       /* kv_head_map entry outside [0, heads_kv) */
    ATTN_ESCRATCH = -5      /* the shape needs more than the no-allocation scratch holds */
};

#define ATTN_MAX_HEADS 256
#define ATTN_MAX_SEQ (1 << 22)

/* Quantisation block sizes: rows per Q block (BQ) and per K block (BK).
 * [SA] 技术方案 sets the granularity to the FlashAttention tile; the pages
 * print no number, the library uses BQ = 128, BK = 64.  Either pointer may be
 * NULL.  Returns ATTN_OK. */
int attn_quant_blocks(int32_t* bq, int32_t* bk);

/* Bytes of device workspace attn_quantize_qk needs for `shape` (the per-chunk
 * exact channel sums of K and the fp32 channel means).  0 for an invalid
 * shape. */
size_t attn_quantize_workspace_bytes(const attn_shape* shape);

/* K smoothing and per-block INT8 quantisation of Q and K ([SA] 技术方案).
 *
 * mean: mu[b,k,c] = fp32( fp64(sum_j K[b,k,j,c]) / S ), the sum over all S
 *       tokens taken exactly (fp16 values are integer multiples of 2^-24),
 *       rounded once to fp64, divided by S in fp64, rounded to fp32.  The mean
 *       runs over all tokens also for causal attention: the shift q_i . mu is
 *       constant along each score row, so softmax is unchanged.  K must be
 *       finite (with an inf or NaN in a channel its mean is unspecified).
 * smooth: ks = fp32(K) - mu (one fp32 subtraction).  Q is not smoothed.
 * quantise, per block X of BQ rows of one (b,h) of Q, or BK rows of one
 *       (b,k) of ks (the last block of a sequence may be partial):
 *       a = max|x|; a == 0 gives q = 0, delta = 0; otherwise r = 127/a and
 *       delta = a/127 (fp32, correctly rounded), q = clamp(rint(x*r), -127, 127)
 *       with x*r one fp32 product and rint ties-to-even.
 *
 * q_f16   in   fp16 [B,Hq,S,D]
 * k_f16   in   fp16 [B,Hkv,S,D]
 * q_i8    out  int8 [B,Hq,S,D]
 * q_scale out  fp32 [B,Hq,ceil(S/BQ)]
 * k_i8    out  int8 [B,Hkv,S,D]   (quantised smoothed K)
 * k_scale out  fp32 [B,Hkv,ceil(S/BK)]
 * k_mean  out  fp32 [B,Hkv,D] or NULL
 * workspace    device scratch of attn_quantize_workspace_bytes(shape) bytes,
 *              16-byte aligned; its contents on entry are ignored.
 * Results are bit-exact and independent of launch order. */
int attn_quantize_qk(const attn_shape* shape, const void* q_f16, const void* k_f16,
                     int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                     float* k_mean, void* workspace, void* stream);

/* 8-bit attention forward ([SA] 技术方案; tiling and online softmax per
 * [FA-guide] and [MHA-GQA] §8.2).
 *   S32[i,j] = sum_c q_i8[i,c] * k_i8[j,c]            (INT8 MFMA, exact INT32)
 *   s[i,j]   = S32[i,j] * q_scale[i/BQ] * k_scale[j/BK] * sm_scale
 *   P        = online softmax of s over the visible keys, rounded to fp16
 *   O        = (P V) / rowsum   (FP16 MFMA, fp32 accumulation), stored fp16
 * Inputs are the outputs of attn_quantize_qk plus V fp16 [B,Hkv,S,D].
 * o_f16 out fp16 [B,Hq,S,D]; lse out fp32 [B,Hq,S] (natural-log
 * log-sum-exp of s per row) or NULL. */
int attn_fwd_int8(const attn_shape* shape, const int8_t* q_i8, const float* q_scale,
                  const int8_t* k_i8, const float* k_scale, const void* v_f16,
                  void* o_f16, float* lse, const int32_t* kv_head_map, int causal,
                  float sm_scale, void* stream);

/* K smoothing and per-block INT8 quantisation of K only: the K half of
 * attn_quantize_qk (same outputs, same rules, same workspace size), for use
 * with attn_fwd_int8_fused_q. */
int attn_quantize_k(const attn_shape* shape, const void* k_f16, int8_t* k_i8, float* k_scale,
                    float* k_mean, void* workspace, void* stream);

/* attn_quantize_k for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels, outputs and bit-exact results, with the workspace taken
 * from a scratch array of ATTN_NOALLOC_SCRATCH_BYTES that the library keeps
 * in device memory (one per GPU it runs on, held until the process ends)
 * instead of a caller buffer.  The call allocates nothing (no hipMalloc, no
 * allocating library routine); the caller still passes K and the outputs.
 * Shapes whose attn_quantize_workspace_bytes exceed the scratch are rejected
 * with ATTN_ESCRATCH before anything is launched (the scratch holds, e.g., 32
 * (batch, kv-head) pairs of 65536 tokens at head_dim 128).  The scratch needs
 * no initial contents (every byte is written before it is read), but it is
 * shared by every call on one GPU: calls that overlap on one GPU (other
 * streams, other host threads) race and must be ordered by the caller.
 * ATTN_ELAUNCH also reports a failed lookup of the scratch's device address. */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
int attn_quantize_k_noalloc(const attn_shape* shape, const void* k_f16, int8_t* k_i8, float* k_scale,
                            float* k_mean, void* stream);

/* 8-bit attention forward that quantises Q itself: Q is read as fp16 and
 * each BQ-row block is quantised inside the forward kernel with exactly the
 * rule of attn_quantize_qk (the kernel's query tile is one Q block), so INT8
 * Q never travels through HBM.  Otherwise identical to attn_fwd_int8: for the
 * same inputs it returns bitwise the same O and lse as attn_quantize_qk
 * followed by attn_fwd_int8.
 * q_f16 in fp16 [B,Hq,S,D]; k_i8, k_scale from attn_quantize_k (or
 * attn_quantize_qk); v_f16 fp16 [B,Hkv,S,D]; o_f16 out fp16 [B,Hq,S,D];
 * lse out fp32 [B,Hq,S] or NULL; q_scale_out out fp32 [B,Hq,ceil(S/BQ)] (the
 * Q block scales) or NULL. */
int attn_fwd_int8_fused_q(const attn_shape* shape, const void* q_f16, const int8_t* k_i8,
                          const float* k_scale, const void* v_f16, void* o_f16, float* lse,
                          float* q_scale_out, const int32_t* kv_head_map, int causal,
                          float sm_scale, void* stream);

/* Exact FP16 attention forward (the FlashAttention-style baseline,
 * [FA-guide]: exact values, tiles in on-chip memory, online softmax).
 *   s = (Q K^T) * sm_scale with FP16 MFMA and fp32 accumulation, online
 *   softmax in fp32, P rounded to fp16 for P V (FP16 MFMA, fp32 accumulation),
 *   O = (P V) / rowsum stored as fp16; lse as for attn_fwd_int8. */
int attn_fwd_fp16(const attn_shape* shape, const void* q_f16, const void* k_f16,
                  const void* v_f16, void* o_f16, float* lse,
                  const int32_t* kv_head_map, int causal, float sm_scale, void* stream);

/* Test hook for [SA] 技术方案's INT8 Q K^T with INT32 accumulation: the INT32
 * score tiles exactly as attn_fwd_int8 computes them -- the same kernel, with
 * the same copies of K into LDS, the same LDS layout and the same matrix
 * instructions, launched on the same work schedule -- written out in place of
 * the softmax and P V (no V is read).  For every (b, h) and every query row i
 * in q-tiles q_tile_lo..q_tile_hi (tiles of BQ rows, inclusive;
 * 0 <= q_tile_lo <= q_tile_hi < ceil(S/BQ), else ATTN_EINVAL), writes
 * S32[i, j] = sum_c q_i8[b,h,i,c] * k_i8[b,map[h],j,c] for every visible key
 * j to s_out[b, h, i - q_tile_lo*BQ, j]; s_out is int32 device memory
 * [B, Hq, (q_tile_hi - q_tile_lo + 1) * BQ, S].  Entries of masked keys
 * (j > i when causal) and of rows beyond S are left untouched. */
int attn_debug_qk_int32(const attn_shape* shape, const int8_t* q_i8, const int8_t* k_i8,
                        const int32_t* kv_head_map, int causal, int32_t q_tile_lo,
                        int32_t q_tile_hi, int32_t* s_out, void* stream);

/* Test hook: as attn_debug_qk_int32, for the kernel of attn_fwd_int8_fused_q,
 * which reads fp16 Q and quantises each BQ-row block itself ([SA] 技术方案:
 * per-block INT8 Q).  q_f16 fp16 [B,Hq,S,D]; the scores are those of the INT8
 * Q codes the kernel forms (the rule of attn_quantize_qk); q_scale_out out
 * fp32 [B,Hq,ceil(S/BQ)] or NULL receives the Q block scales of the dumped
 * tiles (other entries untouched).  Same errors as attn_debug_qk_int32. */
int attn_debug_qk_int32_fused_q(const attn_shape* shape, const void* q_f16, const int8_t* k_i8,
                                const int32_t* kv_head_map, int causal, int32_t q_tile_lo,
                                int32_t q_tile_hi, int32_t* s_out, float* q_scale_out,
                                void* stream);

/* ---- FP8 alternative and 8-bit P.V ablation ------------------------------
 * [SA] 技术方案 chooses INT8 for Q and K because it is more accurate than FP8,
 * and keeps P and V in FP16 because 8-bit P and V (INT8, E4M3 or E5M2) lose
 * accuracy in some layers.  These calls provide both alternatives on the
 * gfx950 FP8 matrix cores so the claims can be measured.  FP8 means OCP E4M3
 * (bias 7, largest magnitude 448, no infinities); codes are stored one byte per
 * element and converted with round-to-nearest-even. */

/* As attn_quantize_qk (same mean, smoothing, blocks and workspace), but with
 * the E4M3 grid: per block a = max|x|; a == 0 gives r = 0 (codes of +-0) and
 * delta = 0; otherwise r = 448/a and delta = a/448 (fp32, correctly rounded)
 * and the code is E4M3(clamp(x*r, -448, 448)), x*r one fp32 product, the sign
 * of a zero product kept.  q_f8 [B,Hq,S,D], k_f8 [B,Hkv,S,D] E4M3 codes. */
int attn_quantize_qk_fp8(const attn_shape* shape, const void* q_f16, const void* k_f16,
                         uint8_t* q_f8, float* q_scale, uint8_t* k_f8, float* k_scale,
                         float* k_mean, void* workspace, void* stream);

/* Attention forward with E4M3 Q/K: as attn_fwd_int8, with
 *   s[i,j] = (sum_c dec(q_f8[i,c]) dec(k_f8[j,c])) * q_scale * k_scale * sm_scale,
 * the sum on the FP8 matrix cores with fp32 accumulation (products are exact;
 * the accumulation order is the hardware's).  P and V as attn_fwd_int8. */
int attn_fwd_fp8(const attn_shape* shape, const uint8_t* q_f8, const float* q_scale,
                 const uint8_t* k_f8, const float* k_scale, const void* v_f16, void* o_f16,
                 float* lse, const int32_t* kv_head_map, int causal, float sm_scale, void* stream);

/* Row stride, in bytes (= keys), of the transposed 8-bit V that
 * attn_quantize_v_fp8 writes: 64 * ceil(seq / 64).  0 for an invalid shape. */
int64_t attn_v_fp8_stride(const attn_shape* shape);

/* 8-bit V for the P.V ablation: one E4M3 scale per (b, kv-head, channel) over
 * all tokens: a_c = max_j |V[b,k,j,c]|, r = 448/a_c, delta_c = a_c/448 (fp32,
 * correctly rounded; a_c == 0 gives r = 0, delta_c = 0), code =
 * E4M3(clamp(v*r, -448, 448)).  The codes are written TRANSPOSED, the layout
 * the P.V matrix-core operand wants:
 *   v_f8t [B, Hkv, D, stride] with v_f8t[b,k,c,j] = code of V[b,k,j,c] for
 *   j < seq and 0 for seq <= j < stride (stride = attn_v_fp8_stride).
 * v_scale out fp32 [B,Hkv,D].  workspace: attn_quantize_workspace_bytes(shape)
 * bytes, 16-byte aligned, contents ignored. */
int attn_quantize_v_fp8(const attn_shape* shape, const void* v_f16, uint8_t* v_f8t,
                        float* v_scale, void* workspace, void* stream);

/* Attention forward with INT8 Q/K (as attn_fwd_int8) and 8-bit P and V: the
 * online softmax (running maximum raised whenever a key tile exceeds it, so
 * every weight p <= 1) rounds each weight to E4M3(448 p) against the running
 * maximum of its 64-key tile; P.V runs on the FP8 matrix cores with fp32
 * accumulation; the row sum uses the unrounded weights;
 *   O[i,c] = delta_c / 448 * (sum_j E4M3(448 p_ij) dec(v_f8t[c,j])) / rowsum.
 * v_f8t, v_scale from attn_quantize_v_fp8.  Other arguments as attn_fwd_int8. */
int attn_fwd_int8_pv8(const attn_shape* shape, const int8_t* q_i8, const float* q_scale,
                      const int8_t* k_i8, const float* k_scale, const uint8_t* v_f8t,
                      const float* v_scale, void* o_f16, float* lse, const int32_t* kv_head_map,
                      int causal, float sm_scale, void* stream);

/* ---- KV-cache (decode) attention ------------------------------------------
 * [MHA-GQA] §3.4: during generation the keys and values of all earlier tokens
 * are cached; the queries of the current token(s) attend over the cache.
 * seq_q queries per head (the LAST seq_q positions of the sequence) attend
 * over seq_kv >= seq_q cached keys; under the causal mask query i sees keys
 * j <= seq_kv - seq_q + i (bottom-right alignment).  Layout: Q, O
 * [batch, heads_q, seq_q, head_dim]; K, V [batch, heads_kv, seq_kv, head_dim];
 * other conventions as above.  seq_q is at most ATTN_DECODE_MAX_SEQ_Q. */
#define ATTN_DECODE_MAX_SEQ_Q 32

typedef struct attn_kv_shape {
    int32_t batch;
    int32_t heads_q;
    int32_t heads_kv;
    int32_t seq_q;     /* 1 .. min(seq_kv, ATTN_DECODE_MAX_SEQ_Q) */
    int32_t seq_kv;    /* 1 .. ATTN_MAX_SEQ */
    int32_t head_dim;  /* 64 or 128 */
} attn_kv_shape;

/* Bytes of device workspace the decode calls need for `shape` and the head map
 * (per-split partial results: the cache is split over many workgroups whose
 * partial maxima, sums and outputs are then merged).  0 if the arguments are
 * invalid. */
size_t attn_decode_workspace_bytes(const attn_kv_shape* shape, const int32_t* kv_head_map);

/* 8-bit decode ([SA] 技术方案 on a KV cache).  The cached K is smoothed and
 * quantised by attn_quantize_k called with seq = seq_kv (mean over all cached
 * tokens, BK-key blocks).  Each head's seq_q query rows form one Q block and
 * are quantised inside the kernel with the rule of attn_quantize_qk
 * (a = max|x| over the block, delta = a/127, q = clamp(rint(x*127/a))).
 *   s[i,j] = (sum_c q_i8[i,c] k_i8[j,c]) * delta_q * k_scale[j/BK] * sm_scale
 * then the online softmax, P rounded to fp16, P V in FP16 with fp32
 * accumulation, O stored fp16.
 * q_scale_out out fp32 [batch, heads_q] (the Q block scales) or NULL;
 * lse out fp32 [batch, heads_q, seq_q] or NULL; workspace of
 * attn_decode_workspace_bytes(shape, kv_head_map) bytes, 16-byte aligned. */
int attn_decode_int8(const attn_kv_shape* shape, const void* q_f16, const int8_t* k_i8,
                     const float* k_scale, const void* v_f16, void* o_f16, float* lse,
                     float* q_scale_out, const int32_t* kv_head_map, int causal, float sm_scale,
                     void* workspace, void* stream);

/* Exact FP16 decode: as attn_fwd_fp16 for seq_q queries over the cache. */
int attn_decode_fp16(const attn_kv_shape* shape, const void* q_f16, const void* k_f16,
                     const void* v_f16, void* o_f16, float* lse, const int32_t* kv_head_map,
                     int causal, float sm_scale, void* workspace, void* stream);

/* ---- Tile-level attention masks (APB-style anchor / passing / local) ------
 * The APB page computes attention with a FlashAttention kernel whose mask has
 * a changed shape: on one device the keys are an anchor block (the first
 * tokens), a passing block (keys and values handed over from earlier devices)
 * and the local context.  These calls run the forward kernels under any mask
 * given per tile pair: query tile qt (ATTN_MASK_TILE_Q rows) x key tile kt
 * (ATTN_MASK_TILE_K keys) with a dense host mask of ceil(seq/TILE_Q) x
 * ceil(seq/TILE_K) bytes, row-major:
 *   0  no key of the tile is visible to any query of the query tile;
 *   1  every key of the tile is visible;
 *   2  key j is visible to query i iff j <= i (causal within the tile pair).
 * A query row with no visible key gets O = 0 and lse = -inf.  Q and K share
 * one sequence length; one mask serves every batch entry and head. */
#define ATTN_MASK_TILE_Q 128
#define ATTN_MASK_TILE_K 64

/* Mask dimensions for a sequence length (either pointer may be NULL). */
int attn_block_mask_tiles(int32_t seq, int32_t* q_tiles, int32_t* k_tiles);

/* Host helper: the APB layout as a tile mask.  Keys (and query positions) are
 * [anchor | passing | local], local = seq - anchor - passing; anchor and
 * passing are multiples of ATTN_MASK_TILE_Q.  Anchor queries attend causally
 * within the anchor; local queries attend to the anchor and passing blocks and
 * causally to the local block (causal over the concatenation); queries at
 * passing positions attend to nothing (the passing block only lends keys and
 * values).  mask: host buffer of q_tiles * k_tiles bytes. */
int attn_block_mask_apb(int32_t seq, int32_t anchor, int32_t passing, uint8_t* mask);

/* Host helper: the dense tile mask as the list the kernels read.  row_ptr
 * [q_tiles + 1] and cols [q_tiles * k_tiles] are host buffers; cols[e] =
 * (kt << 2) | type for the visible tiles of each query tile in key order,
 * row_ptr[qt] .. row_ptr[qt+1] delimiting query tile qt; *nnz = entries
 * written.  Type-2 tiles wholly below the diagonal become type 1 and those
 * wholly above it are dropped (same mask).  Mask values above 2: ATTN_EINVAL. */
int attn_block_mask_csr(int32_t seq, const uint8_t* mask, int32_t* row_ptr, int32_t* cols, int32_t* nnz);

/* The FP16 and the INT8 forward under a tile mask.  mask_row_ptr and
 * mask_cols are DEVICE copies of attn_block_mask_csr's output (mask_cols may be
 * NULL when mask_nnz == 0).  The kernels clamp every list index, so a
 * malformed list gives unspecified results but never an access outside the
 * buffers.  Other arguments as attn_fwd_fp16 / attn_fwd_int8 (no causal flag:
 * the mask says it). */
int attn_fwd_fp16_masked(const attn_shape* shape, const void* q_f16, const void* k_f16, const void* v_f16,
                         void* o_f16, float* lse, const int32_t* kv_head_map, const int32_t* mask_row_ptr,
                         const int32_t* mask_cols, int32_t mask_nnz, float sm_scale, void* stream);
int attn_fwd_int8_masked(const attn_shape* shape, const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                         const float* k_scale, const void* v_f16, void* o_f16, float* lse,
                         const int32_t* kv_head_map, const int32_t* mask_row_ptr, const int32_t* mask_cols,
                         int32_t mask_nnz, float sm_scale, void* stream);

/* Static text for a status code. */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
