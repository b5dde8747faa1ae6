/*
 * gdn.h -- C ABI of libgdn, the Gated DeltaNet sequence mixer on AMD
 * Instinct MI355X (gfx950).
 *
 * The operations follow these pages:
 *   "L'attention hybride" (Qwen3.8-27B architecture chapter, mkdocs.reaper.mx)
 *     - config block "Les 48 couches Gated DeltaNet": 16 key heads, 48 value
 *       heads, head width 128, conv kernel 4, swish output gate, float32
 *       recurrent state;
 *     - table "Le decompte": the q | k | v | z channel split of the input
 *       projection, one beta and one alpha per value head, a depthwise causal
 *       conv of kernel 4 over q, k, v without bias, a 128-weight output norm;
 *     - section "La dissymetrie 16 / 48": one key head serves Hv/Hk value
 *       heads (3 here, 8 in the larger variant); each value head keeps a
 *       d_k x d_v state;
 *     - section "La recurrence": alpha_t in (0,1) decays the whole state,
 *       beta_t in (0,1) rewrites the association of k_t (the update formula
 *       is missing from the page text; the gated delta rule
 *       S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *       o_t = S_t q_t, read after the update, is what is computed);
 *     - sections "L'etat, en memoire" and "Le float32 n'est pas un detail":
 *       the state has a fixed size whatever the length and is kept in fp32.
 *   "Chapitre 16 - Assembler un systeme de type Kimi K3" (course page,
 *   cours.spawnkit.ai), sections 16.2 and 16.3: prefill processes a prompt
 *   block by block and hands the state from block to block; decode reads the
 *   fixed state, produces the token's output and updates the state.
 *   "Les briques d'un reseau de neurones" (Kimi K3 foundations), section 2
 *   (SiLU = x sigmoid(x)) and section 4 (RMSNorm with epsilon under the root
 *   and a per-coordinate gain).
 *
 * Conventions common to every call
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates no device memory and keeps no state between calls; scratch
 *     space comes from the caller (gdn_prefill_workspace_size).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs asynchronously; the library never synchronises.
 *   - Argument errors are detected on the host before any device work and
 *     return a status; the thread-local message is in gdn_last_error().
 *     A failed kernel launch returns GDN_ERR_DEVICE.  Nothing throws.
 *   - Element strides are counted in elements of the tensor's own dtype.
 *   - bf16 tensors hold IEEE bfloat16 bit patterns (uint16 storage).
 *   - Gate values are data and are not checked: the domain is
 *     log_alpha <= 0 and 0 <= beta <= 1 (the closed ends are allowed).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,        /* a required pointer is NULL */
  GDN_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes / strides */
  GDN_ERR_UNSUPPORTED = 3, /* valid request that no kernel here implements */
  GDN_ERR_ALIGN = 4,       /* pointer or stride not aligned as required */
  GDN_ERR_DEVICE = 5       /* HIP runtime error (launch failure, no device) */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Flag: divide q and k of each (token, key head) by sqrt(sum of squares +
 * l2_eps) before use (per-head L2 normalisation). */
#define GDN_FLAG_QK_L2NORM 1u
/* Flag (gdn_prefill): run the token-by-token kernel, fp32 arithmetic
 * throughout, instead of the chunked one; it needs no workspace.  The chunked
 * kernel multiplies fp16 operands with fp32 accumulation.  It scales v and the
 * state into fp16's range by powers of two (per chunk and 16-column value
 * tile), so their magnitudes are not bounded; the key-side products assume
 * keys and queries of norm about 1 or less (GDN_FLAG_QK_L2NORM gives that).
 * Use this flag for keys far from unit norm without the L2 flag. */
#define GDN_FLAG_TOKEN_SERIAL 2u
/* gdn_prefill_gated only: apply the norm inside the chunked kernels whatever the
 * batch (without it they do when B * Hv is at least the GPU's CU count). */
#define GDN_FLAG_NORM_IN_CHAIN 4u

/*
 * Shapes of one recurrence call.
 *   B, T        batch and tokens per sequence (T >= 1)
 *   Hk, Hv      key heads and value heads; Hv % Hk == 0; value head h uses
 *               key head h / (Hv / Hk)  (consecutive groups)
 *   Dk, Dv      head widths; the kernels implement Dk == Dv in {16,32,64,128}
 *   io          gdn_dtype of q, k, v and o (gates and state are fp32)
 *   flags       GDN_FLAG_* bits
 *   stride_*    elements between consecutive tokens of q, k, v, o; heads are
 *               packed inside a token (q: Hk*Dk, v and o: Hv*Dv) so each
 *               stride is at least that width; the batch stride is
 *               T * stride.  Strides larger than the width let q, k, v be
 *               views into one [B, T, C] conv output.
 *   q_scale     multiplies q after normalisation (1.0 reads S_t q_t as is)
 *   l2_eps      epsilon of the L2 normalisation (used with the flag only)
 */
typedef struct {
  int32_t B, T, Hk, Hv, Dk, Dv;
  int32_t io;
  uint32_t flags;
  int64_t stride_q, stride_k, stride_v, stride_o;
  float q_scale;
  float l2_eps;
} gdn_dims;

/*
 * gdn_prefill -- the gated delta rule over T tokens for every (b, value head),
 * chunkwise ("Chapitre 16", 16.2; "L'attention hybride", "La recurrence").
 *   q, k       [B, T, Hk, Dk]  io dtype, token strides stride_q / stride_k
 *   v          [B, T, Hv, Dv]  io dtype, token stride stride_v
 *   log_alpha  [B, T, Hv] fp32 contiguous (log of the decay, <= 0)
 *   beta       [B, T, Hv] fp32 contiguous (write strength)
 *   state_in   [B, Hv, Dk, Dv] fp32 contiguous, M = S^T (row i = key
 *              coordinate, column j = value coordinate); NULL = zero state
 *   state_out  [B, Hv, Dk, Dv] fp32, final state; NULL = not written; may be
 *              the same pointer as state_in (updated in place)
 *   o          [B, T, Hv, Dv]  io dtype, token stride stride_o;
 *              o_t = S_t q_t with S_t after token t's update
 *   workspace, workspace_bytes  device scratch, see gdn_prefill_workspace_size
 * The bf16, Dk == Dv == 128 case with at most 64 value heads per key head
 * runs the chunked MFMA kernels (chunks of 64 tokens); other supported shapes
 * run the token-serial kernel.
 * Alignment: bf16 with D == 128 needs q, k, v, o 16-byte aligned and strides
 * multiples of 8; states need 16-byte alignment.
 * o must not overlap q, k or v.
 */
gdn_status gdn_prefill(const gdn_dims* dims, const void* q, const void* k, const void* v,
                       const float* log_alpha, const float* beta, const float* state_in,
                       float* state_out, void* o, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * gdn_prefill_gated -- gdn_prefill followed by the layer's gated RMSNorm of
 * every output row ("L'attention hybride", config block: swish output gate;
 * table "Le decompte": one 128-weight norm per layer; the prefill as for
 * gdn_prefill):
 *     y[b,t,h,:] = o / sqrt(mean(o^2) + norm_eps) * norm_w * z * sigmoid(z)
 * with o[b,t,h,:] the row gdn_prefill would write; o itself is not written.
 *   dims, q, k, v, log_alpha, beta, state_in, state_out, workspace: as for
 *               gdn_prefill (same workspace size query); dims->Dv in {64, 128}
 *   z           [B, T, Hv, Dv] io dtype, token stride stride_z >= Hv*Dv (the
 *               gate half of the projection output, a view is fine)
 *   norm_w      [Dv] io dtype, shared by all heads
 *   y           [B, T, Hv, Dv] io dtype, token stride dims->stride_o
 * z, norm_w and y 16-byte aligned, stride_z and stride_o multiples of 8.
 * Where the chunked kernels run and B * Hv is at least the GPU's CU count (or
 * with GDN_FLAG_NORM_IN_CHAIN), the norm is applied in the chain kernel's
 * output epilogue (one workgroup per value head holds whole rows) and o never
 * reaches memory; otherwise the prefill writes o into y and the norm runs over
 * y in place (two launches, the same results up to o's bf16 rounding).
 * Errors as for gdn_prefill and gdn_gated_rmsnorm.
 */
gdn_status gdn_prefill_gated(const gdn_dims* dims, const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta, const float* state_in,
                             float* state_out, const void* z, int64_t stride_z, const void* norm_w,
                             float norm_eps, void* y, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * gdn_prefill_static -- gdn_prefill with no workspace argument and no
 * allocation, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * chunked kernels run in a fixed 64 MiB device array that the library holds
 * on each GPU it runs on until the process ends; the call allocates nothing
 * and frees nothing.  Arguments, layouts and results are gdn_prefill's (the
 * results are the same bits as gdn_prefill's with any workspace).  Dims
 * whose smallest workspace (one chunk of operands, see
 * gdn_prefill_workspace_size, plus the state carry when state_out is NULL)
 * exceeds 64 MiB fail with GDN_ERR_SHAPE before anything runs.  Nothing in
 * the array has to start at any value.  All calls on one GPU share its
 * array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and give wrong results; serialise them.
 */
gdn_status gdn_prefill_static(const gdn_dims* dims, const void* q, const void* k, const void* v,
                              const float* log_alpha, const float* beta, const float* state_in,
                              float* state_out, void* o, void* stream);

/*
 * gdn_prefill_workspace_size -- bytes of device workspace gdn_prefill wants
 * for these dims (0 when the call needs none).  The chunked kernel keeps, per
 * (sequence, value head, chunk of a window), the per-chunk matrices that do
 * not depend on the state (55 KiB: the -W, K^T, U0 and P operands and the
 * row scalings, plus 16 KiB per key head for the scaled Q).  A window is a
 * whole number of rounds of resident prep workgroups (512 (chunk, key head)
 * pairs at up to 19 value heads per key head, 256 beyond): as many rounds as keep it
 * within about 96 MiB, so that the chain kernel finds its operands in the
 * GPU's last-level cache, or, when one round alone is larger, as many as fit
 * in 2 GiB; windows are then balanced.  The state is carried between windows
 * through state_out, or through a carry area inside the workspace when
 * state_out is NULL.  A smaller workspace is accepted down to one chunk per
 * window (plus the carry when needed); GDN_ERR_SHAPE below that.  The
 * workspace is caller-owned device memory, 256-byte aligned, used only during
 * the call's kernels on `stream`.
 */
size_t gdn_prefill_workspace_size(const gdn_dims* dims);

/*
 * gdn_prefill_varlen -- prefill of dims->B sequences of different lengths
 * packed along the token axis (a continuous-batching prefill; "Chapitre 16",
 * 16.2: each request's prompt is processed block by block and its state is
 * handed from block to block; "L'etat, en memoire": one fixed-size state per
 * request).  Sequence s holds tokens [cu_seqlens[s], cu_seqlens[s+1]) of the
 * packed tensors; dims->T is the total token count.
 *   cu_seqlens  [B+1] int32 DEVICE memory: cu_seqlens[0] = 0, non-decreasing,
 *               cu_seqlens[B] = T (device data: not checked on the host; the
 *               kernels clamp every range into [0, T], so a malformed table
 *               gives unspecified results but no access outside the arrays);
 *               empty sequences are allowed and pass their state through
 *   q, k [T, Hk, Dk]; v, o [T, Hv, Dv]; log_alpha, beta [T, Hv]: as gdn_prefill
 *               with B = 1 (token strides stride_q/k/v/o)
 *   state_in / state_out [B, Hv, Dk, Dv] fp32 per sequence, as gdn_prefill
 *   workspace   gdn_prefill_varlen_workspace_size bytes (or fewer, down to the
 *               chunk maps, one chunk per window and the state carry).  Its
 *               head holds the chunk maps, (B + 1 + ceil(T/64) + B) int32
 *               rounded up to 256 bytes, written by the call's first kernel
 * Chunks never span two sequences; every other rule is gdn_prefill's.
 */
gdn_status gdn_prefill_varlen(const gdn_dims* dims, const int32_t* cu_seqlens, const void* q, const void* k,
                              const void* v, const float* log_alpha, const float* beta, const float* state_in,
                              float* state_out, void* o, void* workspace, size_t workspace_bytes, void* stream);

/* gdn_prefill_varlen_workspace_size -- workspace bytes gdn_prefill_varlen wants
 * for these dims (B sequences, T tokens in all), whatever the lengths. */
size_t gdn_prefill_varlen_workspace_size(const gdn_dims* dims);

/*
 * gdn_decode_step -- one token per sequence from a resident state
 * ("Chapitre 16", 16.3).  dims->T must be 1.
 *   q, k [B, Hk, Dk]; v, o [B, Hv, Dv] (io dtype, per-sequence strides
 *   stride_q/k/v/o); log_alpha, beta [B, Hv] fp32;
 *   state [B, Hv, Dk, Dv] fp32, read once and overwritten in place.
 * Computes u = M^T k, w = M^T q in one pass over M, then
 * d = beta (v - alpha u), M <- alpha M + k d^T, o = alpha w + (k . q) d.
 * The state is loaded and stored with non-temporal hints: a step leaves
 * none of it in the caches for the next kernel.
 */
gdn_status gdn_decode_step(const gdn_dims* dims, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, float* state, void* o,
                           void* stream);

/*
 * gdn_conv1d_silu -- depthwise causal conv of K taps over C channels, then
 * SiLU ("L'attention hybride", table "Le decompte": kernel 4 over the q|k|v
 * channels, K weights per channel, no bias; "Les briques", section 2):
 *     y[b,t,c] = silu( sum_{j<K} w[c][j] * x[b, t-(K-1)+j, c] )
 *   x     [B, T, C] dtype, token stride stride_x (>= C), batch stride T*stride_x
 *   w     [C, K] dtype, contiguous
 *   conv_state_in  [B, C, K-1] dtype: the inputs at t = -(K-1) .. -1, oldest
 *                  first; NULL = zeros
 *   conv_state_out [B, C, K-1] dtype: the last K-1 inputs of this call
 *                  (taken from conv_state_in when T < K-1); NULL = not written;
 *                  must not alias conv_state_in
 *   y     [B, T, C] dtype, token stride stride_y (>= C); must not overlap x
 * Arithmetic is fp32; y is rounded once to the dtype.  K must be 4; C a
 * multiple of 8 and, for bf16, pointers 16-byte aligned with strides
 * multiples of 8.
 */
gdn_status gdn_conv1d_silu(int32_t B, int32_t T, int32_t C, int32_t K, int32_t dtype,
                           const void* x, int64_t stride_x, const void* w,
                           const void* conv_state_in, void* conv_state_out, void* y,
                           int64_t stride_y, void* stream);

/*
 * gdn_conv1d_silu_l2 -- gdn_conv1d_silu with the per-head L2 normalisation of
 * q and k in the same pass (the L2 flag of gdn_prefill / gdn_decode_step,
 * moved into the conv's epilogue; the layer's q and k lead the q|k|v channels,
 * "L'attention hybride", table "Le decompte"):
 *     y[b,t,c] as gdn_conv1d_silu, then for each head of 128 channels
 *     h < l2_channels / 128:  y_h <- y_h / sqrt(sum(y_h^2) + l2_eps)
 * in fp32 before y is rounded once.  The prefill then runs without the L2 flag.
 *   l2_channels  multiple of 128 in [0, C] (2 * Hk * Dk for the layer); when it
 *                is above 0, C must be a multiple of 128
 *   l2_eps       >= 0
 * Other arguments, layouts and errors as gdn_conv1d_silu.
 */
gdn_status gdn_conv1d_silu_l2(int32_t B, int32_t T, int32_t C, int32_t K, int32_t dtype, const void* x,
                              int64_t stride_x, const void* w, const void* conv_state_in, void* conv_state_out,
                              void* y, int64_t stride_y, int32_t l2_channels, float l2_eps, void* stream);

/*
 * gdn_gated_rmsnorm -- per-head RMSNorm with one shared D-weight, times
 * swish(z) ("L'attention hybride", config block: swish output gate; table
 * "Le decompte": 128 norm weights per layer; "Les briques", section 4):
 *     y = x / sqrt(mean(x^2) + eps) * w * z * sigmoid(z)      per D-row
 * Rows are (token, head) pairs: row (t, h) of x starts at x + t*stride_x +
 * h*D (likewise z and y), so x can be the prefill output [n_tok, H*D] and z
 * a view into the projection output.
 *   n_tok >= 0, H >= 1, D in {64, 128}; x, z, w, y dtype; w is [D];
 *   y may alias x (in place).  bf16 needs 16-byte aligned pointers and
 *   strides multiples of 8.
 */
gdn_status gdn_gated_rmsnorm(int64_t n_tok, int32_t H, int32_t D, int32_t dtype, const void* x,
                             int64_t stride_x, const void* z, int64_t stride_z, const void* w,
                             float eps, void* y, int64_t stride_y, void* stream);

/*
 * gdn_gates -- beta and log alpha of every (token, value head) from the raw
 * outputs of the in_proj_ba projection ("L'attention hybride", table "Le
 * decompte": one beta and one alpha per value head, 2*Hv outputs per token,
 * beta first; "Les briques", section 2 table: sigmoid, softplus(x) =
 * log(1 + e^x)).  The pages leave alpha's activation open; the layer recipe
 * log alpha = -exp(A_log) * softplus(a + dt_bias) is used:
 *     beta[t][h]      = sigmoid(ba[t][h])
 *     log_alpha[t][h] = -exp(A_log[h]) * softplus(ba[t][Hv + h] + dt_bias[h])
 *   ba        [n_tok, stride_ba] dtype (stride_ba >= 2*Hv), element-aligned
 *   A_log, dt_bias [Hv] fp32 (per-head parameters of the layer)
 *   log_alpha, beta [n_tok, Hv] fp32, contiguous: the gate inputs of
 *                   gdn_prefill and gdn_decode_step
 * fp32 arithmetic; softplus and sigmoid are evaluated without overflow for
 * any finite input.  n_tok == 0 is a no-op.
 */
gdn_status gdn_gates(int64_t n_tok, int32_t Hv, int32_t dtype, const void* ba, int64_t stride_ba,
                     const float* A_log, const float* dt_bias, float* log_alpha, float* beta, void* stream);

/*
 * gdn_decode_token -- one decode token per sequence, for a serving loop
 * ("Chapitre 16", 16.3: decode reads the fixed per-request state, produces
 * the token's output and updates the state; 16.2 and "L'etat, en memoire":
 * the state is per request and has a fixed size).  Same step as
 * gdn_decode_step, with two differences:
 *   - the gates are formed in the kernel from the raw in_proj_ba outputs
 *     exactly as gdn_gates does: ba [B, stride_ba] in ba_dtype (bf16 or
 *     fp32), A_log and dt_bias [Hv] fp32;
 *   - the states live in a caller-owned pool state_pool [S, Hv, Dk, Dv] fp32
 *     (16-byte aligned): sequence b uses entry slots[b] (slots: [B] int32,
 *     device memory), or entry b when slots is NULL.  A negative slot skips
 *     the sequence: neither its state nor its output row is touched, and so
 *     does a slot >= n_slots (n_slots = S, the pool's entry count; slot values
 *     are device data, so the kernel checks them, not the host).  Two
 *     sequences of one call must not share a slot (their updates would race).
 *     Without slots the pool needs n_slots >= B (GDN_ERR_SHAPE otherwise).
 * dims->T must be 1; q, k, v, o and flags (GDN_FLAG_QK_L2NORM) as for
 * gdn_decode_step.
 */
gdn_status gdn_decode_token(const gdn_dims* dims, const void* q, const void* k, const void* v, int32_t ba_dtype,
                            const void* ba, int64_t stride_ba, const float* A_log, const float* dt_bias,
                            float* state_pool, int32_t n_slots, const int32_t* slots, void* o, void* stream);

/*
 * gdn_decode_layer -- one decode token of a whole Gated DeltaNet mixer layer,
 * fused into one kernel per (sequence, value head): depthwise causal conv +
 * SiLU of the token's q | k | v channels against their rolling window, L2
 * norm of q and k (GDN_FLAG_QK_L2NORM), gates from the raw in_proj_ba outputs
 * (as gdn_gates), the gated delta rule on the pooled state (as
 * gdn_decode_token), and the gated RMSNorm x swish(z) of the head's output
 * (as gdn_gated_rmsnorm).  ("L'attention hybride", table "Le decompte": the
 * q|k|v|z split of the projection, kernel-4 conv over q, k, v, one beta and
 * one alpha per value head, the 128-weight norm; config block: swish output
 * gate; "Chapitre 16", 16.3: a decode step reads the per-request state,
 * emits the token's output and updates the state.)  bf16 I/O, Dk = Dv = D = 128.
 * With C = (2*Hk + Hv)*D channels and S pool entries:
 *   x [B, >= C] (row stride stride_x): the token's channels before the conv
 *   conv_w [C, 4]; conv_state_in / conv_state_out [S, C, 3]: the window pool,
 *     read from _in and written to _out (distinct buffers; a serving loop
 *     swaps them each step); the key head's q and k windows are written once
 *   ba [B, >= 2*Hv] (stride_ba); A_log, dt_bias [Hv] fp32
 *   state_pool [S, Hv, D, D] fp32, updated in place; n_slots = S, the entry
 *     count of both pools
 *   slots [B] int32 device memory or NULL (entry b; then n_slots >= B); a
 *     negative slot, or one >= n_slots, skips the sequence (nothing of it is
 *     read or written; the kernel checks, since slots are device data); slots
 *     must be distinct
 *   z [B, >= Hv*D] (stride_z); norm_w [D]; out [B, >= Hv*D] (stride_out)
 *   o [B, >= Hv*D] (stride_o) receives the output before the norm, or NULL
 * Alignment: state_pool and conv_w 16 bytes; x, conv_state_in and
 * conv_state_out 4 bytes with stride_x even; the rest their element size.
 */
typedef struct {
  int32_t B, Hk, Hv, D;
  uint32_t flags;               /* GDN_FLAG_QK_L2NORM or 0 */
  float q_scale, l2_eps, norm_eps;
  int32_t n_slots;              /* entries S of state_pool and of the window pools */
  const void* x;
  int64_t stride_x;
  const void* conv_w;
  const void* conv_state_in;
  void* conv_state_out;
  const void* ba;
  int64_t stride_ba;
  const float* A_log;
  const float* dt_bias;
  float* state_pool;
  const int32_t* slots;
  const void* z;
  int64_t stride_z;
  const void* norm_w;
  void* out;
  int64_t stride_out;
  void* o;
  int64_t stride_o;
} gdn_decode_layer_args;

gdn_status gdn_decode_layer(const gdn_decode_layer_args* args, void* stream);

/* Message of the last failed call on this thread ("" if none).  The string
 * is owned by the library and valid until the next call on this thread. */
const char* gdn_last_error(void);

/* ABI version: major * 10000 + minor * 100 + patch. */
int32_t gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
