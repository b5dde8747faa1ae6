// gdn_internal.h -- parameter blocks and kernel launchers shared between the
// host API (gdn_api.cpp) and the HIP kernel translation units.  Host-visible
// only; no device code here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace gdn {

// One-time set-up of a launcher (kernel attributes such as the dynamic LDS
// size), which HIP keeps per device: runs `f` on the first call on each device,
// or on every call for a device index past the table.  Concurrent first calls
// may both run `f`, which must be idempotent.
struct PerDeviceOnce {
  std::atomic<bool> done[64] = {};
  template <typename F>
  hipError_t run(F&& f) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool tracked = dev >= 0 && dev < 64;
    if (tracked && done[dev].load(std::memory_order_acquire)) return hipSuccess;
    e = f();
    if (e == hipSuccess && tracked) done[dev].store(true, std::memory_order_release);
    return e;
  }
};

// Compute units of the current device (hipDeviceProp_t::multiProcessorCount),
// read once per device; 256 (MI355X) when no device is visible, so that size
// queries answer on a host without a GPU.
int device_cu_count();

// Arguments of the recurrence kernels (prefill and decode share them).
struct RecArgs {
  int32_t B, T, Hk, Hv, G, D;
  uint32_t flags;
  float q_scale, l2_eps;
  int64_t sq, sk, sv, so;  // token strides (elements)
  const void* q;
  const void* k;
  const void* v;
  const float* la;
  const float* beta;
  const float* state_in;   // may be null (zero state)
  float* state_out;        // may be null
  void* o;
  // Token-serial kernel only.  When ba is set, the gates are formed from the raw
  // in_proj_ba outputs ([token][sba], beta logits at [0, Hv), alpha inputs at
  // [Hv, 2 Hv), dtype ba_io) with A_log and dt_bias [Hv], instead of read from
  // la / beta.  When slots is set, row b of the batch keeps its state in entry
  // slots[b] of state_in / state_out (a pool); a negative slot skips the row.
  const void* ba = nullptr;
  int64_t sba = 0;
  int32_t ba_io = 0;
  const float* A_log = nullptr;
  const float* dt_bias = nullptr;
  const int32_t* slots = nullptr;
  int32_t nslots = 0;      // pool entries: slots outside [0, nslots) skip the row
  // Variable-length batch: nseq sequences packed along the token axis, sequence s
  // holding tokens [cu_seqlens[s], cu_seqlens[s+1]).  The chunked kernels then see
  // B == 1 (one packed token stream); chunks never span two sequences.
  const int32_t* cu_seqlens = nullptr;
  int32_t nseq = 0;
  // Chunked kernels on a packed batch: chunk_start[s] is the first chunk of
  // sequence s in the window numbering ([nseq + 1] entries), chunk_seq[c] the
  // sequence of chunk c (nseq past the last chunk).  Written into the workspace
  // by the launcher's map kernel.
  const int32_t* chunk_start = nullptr;
  const int32_t* chunk_seq = nullptr;
  // Chunked prefill with the gated RMSNorm applied in the chain (bf16 I/O): o then
  // receives y = o_row / sqrt(mean(o_row^2) + geps) * w * z * sigmoid(z) per (token,
  // value head) row instead of o; z is [token][sz] bf16 (head h at h*D), w [D] bf16.
  const void* gz = nullptr;
  int64_t sz = 0;
  const void* gw = nullptr;
  float geps = 0.f;
};

// io: 0 = fp32, 1 = bf16 (same codes as gdn_dtype).
hipError_t launch_recurrent(const RecArgs& a, int io, hipStream_t s);

// One decode token of a whole layer's mixer (bf16 I/O, head width 128): conv +
// SiLU of the token's q|k|v channels against a window pool, L2 norm of q and k,
// gates from raw in_proj_ba outputs, the recurrence on a state pool, and the
// gated RMSNorm of the output.  Pools are indexed by slots[b] (or b).
struct LayerArgs {
  int32_t B, Hk, Hv, G;
  uint32_t flags;
  float q_scale, l2_eps, norm_eps;
  const uint16_t* x;          // [B][sx]: the token's pre-conv q | k | v channels
  int64_t sx;
  const uint16_t* conv_w;     // [C][4]
  const uint16_t* cs_in;      // [S][C][3] window pool read
  uint16_t* cs_out;           // [S][C][3] window pool written (distinct from cs_in)
  const uint16_t* ba;         // [B][sba] raw beta logits | alpha inputs
  int64_t sba;
  const float* A_log;
  const float* dt_bias;
  float* pool;                // [S][Hv][128][128]
  const int32_t* slots;       // [B] or null
  int32_t nslots;             // S: slots outside [0, S) skip the sequence
  const uint16_t* z;          // [B][sz]
  int64_t sz;
  const uint16_t* norm_w;     // [128]
  uint16_t* out;              // [B][sout]
  int64_t sout;
  uint16_t* o;                // [B][so] pre-norm output, or null
  int64_t so;
};
hipError_t launch_decode_layer(const LayerArgs& a, hipStream_t s);
// Chunked prefill: a prep kernel and a chain kernel per window of chunks.
// The workspace holds the chunk maps of a packed batch, then, per (b, value
// head, chunk of the window), the fragments and row scalings the prep kernel
// produces; when the sequence needs several windows and there is no state_out,
// a state carry follows.
size_t chunk_ws_bytes_per_chunk(const RecArgs& a);
size_t chunk_ws_carry_bytes(const RecArgs& a);
// packed batches: the chunk maps at the workspace start (a multiple of 256 bytes; 0 otherwise)
size_t chunk_map_bytes(const RecArgs& a);
// chunks the windows run over, and the preferred number per window (balanced)
int chunk_count(const RecArgs& a);
int chunk_window_chunks(const RecArgs& a);
// With a.gz set the chain applies the gated RMSNorm to every output row (one
// workgroup per head); fixed-length batches only.
hipError_t launch_chunk_prefill(const RecArgs& a, void* ws, size_t ws_bytes, hipStream_t s);

struct ConvArgs {
  int32_t B, T, C, K;
  int64_t sx, sy;
  const void* x;
  const void* w;
  const void* cs_in;
  void* cs_out;
  void* y;
  // channels [0, l2c) are L2-normalised per 128-channel head after the SiLU:
  // y <- y / sqrt(sum(y^2) + l2_eps) (l2c and C multiples of 128 when l2c > 0)
  int32_t l2c = 0;
  float l2_eps = 0.f;
};
hipError_t launch_conv1d_silu(const ConvArgs& a, int io, hipStream_t s);

struct NormArgs {
  int64_t n_tok;
  int32_t H, D;
  int64_t sx, sz, sy;
  const void* x;
  const void* z;
  const void* w;
  float eps;
  void* y;
};
hipError_t launch_gated_rmsnorm(const NormArgs& a, int io, hipStream_t s);

struct GateArgs {
  int64_t n_tok;
  int32_t Hv;
  int64_t sba;
  const void* ba;
  const float* A_log;
  const float* dt_bias;
  float* la;
  float* beta;
};
hipError_t launch_gates(const GateArgs& a, int io, hipStream_t s);

// Full-attention layer (gdn_attn.hip).  Prefill: tokens [0, T) of B sequences;
// decode: T == 1 at position cache_len[b].  qrot is the normalised, rotated
// queries [B*T][Hq][256] bf16; part the decode partials.
struct AttnArgs {
  int32_t B, T, Hq, Hkv, rot_dim, S_max;
  float theta, eps, scale;
  int64_t sqg, sk, sv, so;
  const uint16_t* qg;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* qw;
  const uint16_t* kw;
  const int32_t* cache_len;   // decode only
  uint16_t* kc;
  uint16_t* vc;
  uint16_t* o;
  uint16_t* qrot;
  float* part;                // decode only
  int32_t split = 256;        // decode only: cached positions per wave, 256 or 512
};
// RoPE inverse frequencies theta^(-2f/rot_dim), f < rot_dim/2, computed on the host in fp64
struct RopeTable {
  double inv_freq[128];
};
// Decode splits: the workspace holds partial results for ceil(S_max / kAttnSplit) splits,
// the most a call uses (a wave takes kAttnSplit or 2 kAttnSplit positions); floats per
// partial result
constexpr int kAttnSplit = 256;
constexpr int kAttnPartFloats = 260;
__host__ __device__ inline int attn_splits(int S_max) { return (S_max + kAttnSplit - 1) / kAttnSplit; }
hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t s);

// Measurement probes (gdn_probe.hip): n_workgroups x 4 waves of MFMA rounds, and
// a device copy in blocks of kProbeCopyBlockBytes.
constexpr size_t kProbeCopyBlockBytes = 256 * 8 * 16;
hipError_t launch_probe_mfma(int n_workgroups, int iters, float* sink, hipStream_t s);
hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t s);

}  // namespace gdn
