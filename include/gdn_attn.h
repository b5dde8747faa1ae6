/*
 * gdn_attn.h -- C ABI of the full-attention layer that the hybrid stack puts
 * beside its Gated DeltaNet layers, in libgdn (AMD Instinct MI355X, gfx950).
 *
 * The operations follow "L'attention hybride" (Qwen3.8-27B architecture
 * chapter, mkdocs.reaper.mx), section "Les 16 couches d'attention complete":
 *   - its configuration block: 24 query heads, 4 key/value heads, head width
 *     256, an output gate, a partial rotary factor of 0.25, no bias, RoPE base
 *     1e7;
 *   - "Le facteur 2 sur W_Q": the query projection also yields the output
 *     gate, so each query head comes with a gate vector of the same width;
 *   - the parameter table ("Le decompte"): q and k each have a normalisation
 *     weight of 256 entries;
 *   - "GQA a 6:1": each key/value head serves six query heads, and the cache
 *     holds keys and values of the 4 key/value heads per token;
 *   - "Le RoPE partiel": only 64 of the 256 dimensions of each head are
 *     rotated by position.
 * RMSNorm follows "Les briques d'un reseau de neurones" (Kimi K3
 * foundations), section 4.  What is computed, per sequence b, token t at
 * position p (prefill: p = t; decode: p = cache_len[b]):
 *   q = RoPE_p(RMSNorm(qg[t, h, 0, :]) * q_norm_w),  g = qg[t, h, 1, :]
 *   k = RoPE_p(RMSNorm(k[t, j, :]) * k_norm_w)      (stored in k_cache)
 *   o[t, h, :] = sigmoid(g) * softmax_{u <= p}(scale * q . k_u) v_u
 * with key/value head j = h / (Hq/Hkv); RMSNorm(x) = x / sqrt(mean(x^2) +
 * norm_eps); RoPE_p turns dimension pairs (i, i + rot_dim/2), i < rot_dim/2,
 * by p * rope_theta^(-2i/rot_dim) (the rotate-half pairing) and leaves
 * dimensions >= rot_dim as they are.
 *
 * Conventions are those of gdn.h: device pointers owned by the caller, work
 * enqueued on `stream`, host-side argument checks returning a gdn_status,
 * strides in elements, bf16 as uint16 bit patterns.  Arithmetic is fp32 with
 * bf16 MFMA operands (q, k and the softmax weights are rounded to bf16 for
 * the products).
 */
#ifndef GDN_ATTN_H
#define GDN_ATTN_H

#include "gdn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t B;          /* sequences */
  int32_t T;          /* tokens per sequence: prefill >= 0 (from position 0); decode 1 */
  int32_t Hq, Hkv;    /* query heads, key/value heads; Hq % Hkv == 0 */
  int32_t D;          /* head width: 256 */
  int32_t rot_dim;    /* rotated dimensions: a multiple of 8, 0 <= rot_dim <= D (64) */
  int32_t S_max;      /* cache capacity in tokens per sequence: a positive multiple of 64 */
  float rope_theta;   /* RoPE base (1e7) */
  float norm_eps;     /* RMSNorm epsilon of q and k */
  float scale;        /* softmax scale, normally 1/sqrt(D) */
  int64_t stride_qg;  /* elements between consecutive tokens of qg (>= 2 Hq D) */
  int64_t stride_k, stride_v;  /* of k and v (>= Hkv D) */
  int64_t stride_o;   /* of o (>= Hq D); every stride a multiple of 4 */
} gdn_attn_dims;

/*
 * Cache layout (bf16), per sequence b and key/value head j:
 *   k_cache [B][Hkv][S_max][D]: the rotated, normalised key of position p at
 *           ((b Hkv + j) S_max + p) D + d;
 *   v_cache [B][Hkv][S_max/64][D][64]: values in blocks of 64 positions, each
 *           block transposed: element (p, d) at
 *           ((b Hkv + j) S_max/64 + p/64) 64 D + 64 d + p % 64.
 * Both are 16-byte aligned.
 */

/*
 * gdn_attn_prefill -- causal attention over T new tokens of each of B
 * sequences, starting at position 0 (the prompt of a request).
 *   qg [B, T, Hq, 2, D]: per query head the query (D) then its gate (D);
 *      token stride stride_qg, sequence stride T stride_qg
 *   k, v [B, T, Hkv, D] (token strides stride_k, stride_v)
 *   q_norm_w, k_norm_w [D]
 *   k_cache, v_cache: positions [0, T) of each sequence are written
 *   o [B, T, Hq D] (token stride stride_o): the gated outputs
 *   workspace: gdn_attn_prefill_workspace_size bytes, 256-byte aligned (the
 *      normalised, rotated queries)
 * D must be 256 and T <= S_max.  All bf16; qg, k, v, o and the weights
 * 8-byte aligned, the caches 16-byte aligned.
 */
gdn_status gdn_attn_prefill(const gdn_attn_dims* dims, const void* qg, const void* k, const void* v,
                            const void* q_norm_w, const void* k_norm_w, void* k_cache, void* v_cache, void* o,
                            void* workspace, size_t workspace_bytes, void* stream);
size_t gdn_attn_prefill_workspace_size(const gdn_attn_dims* dims);

/*
 * gdn_attn_decode -- one new token per sequence (dims->T == 1): its key and
 * value are written at position cache_len[b] of the caches, and its query
 * attends to positions [0, cache_len[b]].
 *   qg [B, Hq, 2, D], k, v [B, Hkv, D] (sequence strides stride_qg, stride_k,
 *      stride_v); o [B, Hq D] (stride_o)
 * Hq/Hkv must be at most 16 (the query heads of a group are the 16 columns of
 * the decode kernel's matrix products).
 *   cache_len [B] int32 DEVICE memory: tokens already cached per sequence,
 *      0 <= cache_len[b] < S_max (device data: not checked on the host; the
 *      kernels clamp it into that range); not modified -- the caller advances
 *      it after the call
 *   workspace: gdn_attn_decode_workspace_size bytes, 256-byte aligned
 * The keys are split into blocks of 256 positions, each handled by its own
 * workgroup, and the partial softmax sums are combined by a second kernel.
 */
gdn_status gdn_attn_decode(const gdn_attn_dims* dims, const void* qg, const void* k, const void* v,
                           const void* q_norm_w, const void* k_norm_w, const int32_t* cache_len, void* k_cache,
                           void* v_cache, void* o, void* workspace, size_t workspace_bytes, void* stream);
size_t gdn_attn_decode_workspace_size(const gdn_attn_dims* dims);

#ifdef __cplusplus
}
#endif

#endif /* GDN_ATTN_H */
