// Kernel parameter block shared by the host runtime and the gfx950 kernels.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kie {

constexpr int kThreads = 512;              // one workgroup per CU: 8 wave64s
constexpr int kWaves = kThreads / 64;
constexpr int kMaxGroup = 4;               // query heads per KV head
constexpr int kMaxHeadDim = 128;           // 16 lanes x 8 fp16 per K/V row
constexpr int kMaxActiveExperts = 16;      // top_k + shared
constexpr int kBatch = 4;                  // GEMV: 16-byte loads per lane per batch
constexpr int kPartCap = 2048;             // GEMV: per-block task partials in LDS (floats)
constexpr int kMaxTopK = 256;              // top-k / top-p candidate pool, at most
constexpr int kGroups = 8;                 // grid barrier: arrival groups (one per XCD)
constexpr int kGroupStride = 64;           // grid barrier: words between counters (256 B)
constexpr int kBarrierWords = kGroupStride * (1 + kGroups);
constexpr int kTraceEvents = 1024;         // trace slots per workgroup

// Status codes written by the device into Params::err (same values as kie_status).
constexpr int kErrTimeout = -7;

struct LayerPtrs {
  const __half *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm;
  const __half *w_gate, *w_up, *w_down;
  const __half *router, *e_gate, *e_up, *e_down;
};

enum Mode : int { kPrefill = 0, kDecode = 1 };

struct Params {
  // ---- shapes
  int L, d, H, nkv, hd, F, Vin, Vout, cap;
  int E, topk, nshared, Fe;     // MoE (E == 0: dense)
  int moe_renorm;               // MoE: routed weights rescaled to sum to 1
  float eps;
  int n_wg;                     // workgroups in the grid
  int splits;                   // attention position splits per KV head
  // ---- weights (caller-owned, fp16)
  const __half* tok_emb;        // [Vin][d]
  const __half* final_norm;     // [d]
  const __half* lm_head;        // [Vout][d]
  const LayerPtrs* layers;      // device array [L]
  // ---- library-owned device state
  __half* kc;                   // [L][nkv][cap][hd]
  __half* vc;                   // [L][nkv][cap][hd]
  const float* rope_cos;        // [cap][hd/2]
  const float* rope_sin;        // [cap][hd/2]
  unsigned long long* act;      // activation arena of 64-bit words: plain (epoch << 32 | fp32
                                // bits) or pair (two 24-bit-rounded fp32 values + epoch tag)
  int act_words;
  int off_x;                    // [d]            residual stream, plain (read by its owners,
                                //                the router and lm_head)
  int off_xh;                   // [d/2]          residual stream, pairs (GEMV inputs)
  int off_qkv;                  // [H*hd + 2*nkv*hd]  plain
  int off_o;                    // [H*hd/2]       attention output (head-major), pairs
  int off_u;                    // [max(F, (topk+nshared)*Fe)/2]  FFN hidden, pairs
  int off_router;               // [E]            router logits
  int off_part;                 // [nkv][splits][G][hd+2]  split-K partials (acc, m, l)
  unsigned epoch0;              // epoch of (step 0, layer 0, slot 0) of this launch
  unsigned* bar;                // grid barrier counters [kBarrierWords]
  unsigned long long* amax;     // [2] packed (logit, index) argmax slots
  int* err;                     // device error word (0 = ok)
  int* state;                   // [0] pending token, [1] graph-mode step counter
  int* expert_log;              // [cap][L][topk] MoE routing record, by position
  // ---- per call
  int mode;                     // kPrefill / kDecode
  int n_steps;
  int pos0;                     // position of step 0
  const int* prompt;            // prefill: tokens [n_steps + 1]
  int* out_tokens;              // decode: [n_steps]
  float* out_logits;            // decode: [n_steps][Vout] or nullptr
  long long timeout_ticks;      // barrier watchdog in wall-clock ticks
  int spin_limit;               // > 0: cap on polls per wait (forced-watchdog tests)
  unsigned long long* trace;    // [n_wg][kTraceEvents] barrier clock stamps, or nullptr
  int trace_step;               // the decode step that is traced
  // ---- per call: how a decode step picks its token
  int sample;                   // 0: greedy argmax; 1: temperature sampling (Gumbel-max);
                                // 2: the same draw restricted by top-k / top-p
  float temperature;            // > 0 when sampling
  unsigned long long seed;      // sampling key (Philox4x64 key word 0)
  int top_k;                    // sample == 2: candidates kept, 1..kMaxTopK (0: the whole pool)
  float top_p;                  // sample == 2: nucleus mass, (0, 1]
  float* zbuf;                  // [Vout] the step's logits, for the top-k / top-p selection
};

// Host-visible launchers implemented next to the kernels.
int max_blocks_per_cu(int group, bool moe, size_t lds_bytes);
// p_dev: a device copy of p (the persistent kernel re-reads it per stage)
hipError_t launch_mono(const Params& p, const Params* p_dev, size_t lds_bytes, bool plain,
                       hipStream_t s);
hipError_t launch_staged_step(const Params& p, size_t lds_bytes, hipStream_t s);
// stage: the staged mode's stage numbering (kSQkv = 0, kSAttn, kSMerge, kSO, kSGateUp, kSDown,
// kSRouter, kSMoeGateUp, kSMoeDown, kSLm); kSAttn also runs the merge
hipError_t launch_stage(const Params& p, size_t lds_bytes, int stage, int l, hipStream_t s);
hipError_t launch_gemv(const __half* w, const float* x, float* y, int rows, int cols, int n_wg,
                       hipStream_t s);
size_t gemv_lds_bytes(int cols);
hipError_t launch_barrier_test(unsigned* bar, unsigned* slots, int* violations, int* err, int n_wg,
                               int rounds, long long timeout_ticks, int spin_limit,
                               hipStream_t s);
// kind: 0 non-temporal global loads, 1 plain global loads, 2 the decode
// kernel's non-temporal buffer loads (bytes < 4 GiB); depth 1, 2, 4, 8 or 16
hipError_t launch_stream(const void* src, void* dst, size_t bytes, int n_wg, int depth, int kind,
                         unsigned* sink, hipStream_t s);
// Batched prefill (kie_prefill.hip)
hipError_t launch_split(const float* x, int ldx, __half* hi, __half* lo, int M, int K, hipStream_t s);
hipError_t launch_gemm(const __half* ahi, const __half* alo, int lda, const __half* w, int ldw, float* c,
                       int ldc, int M, int N, int K, bool accumulate, hipStream_t s);
// tiles: device int[3 * ntiles] of (first row, end row, weight index), at most 64 rows each
hipError_t launch_gemm_grouped(const __half* ahi, const __half* alo, int lda, const __half* w, size_t wstride,
                               int ldw, float* c, int ldc, const int* tiles, int ntiles, int N, int K,
                               hipStream_t s);
hipError_t launch_embed(const __half* emb, const int* tok, int d, float* X, int T, hipStream_t s);
hipError_t launch_rmsnorm_split(const float* X, const __half* gain, int d, float eps, __half* hi, __half* lo,
                                int T, hipStream_t s);
hipError_t launch_rope_kv(float* QKV, int ldq, int H, int nkv, int hd, int pos0, const float* cosT,
                          const float* sinT, __half* kc, __half* vc, int cap, int T, hipStream_t s);
hipError_t launch_attn_prefill(const float* QKV, int ldq, const __half* kc, const __half* vc, int cap, int H,
                               int nkv, int hd, int pos0, float* O, int T, hipStream_t s);
hipError_t launch_swiglu_split(const float* G, const float* U, size_t n, __half* hi, __half* lo,
                               hipStream_t s);
// Groups `rows` compact rows by expert on the device: fill (int[E]) and
// tiles (int[3 * max_tiles]) are workspace; perm/inv as the grouped products
// and the combine read them.  E must be at most 1024.
hipError_t launch_moe_group(const int* ids, int rows, int E, int* fill, int* tiles, int max_tiles, int* perm,
                            int* inv, hipStream_t s);
hipError_t launch_route(const float* R, int E, int topk, int renorm, int* ids, float* wts, int* log, int L, int l,
                        int pos0, int T, hipStream_t s);
hipError_t launch_gather_rows(const __half* hi, const __half* lo, int d, const int* perm, int topk, __half* ch,
                              __half* cl, int rows, hipStream_t s);
hipError_t launch_swiglu_w_split(const float* G, const float* U, int F, int rows, const int* perm, const float* wts,
                                 __half* hi, __half* lo, hipStream_t s);
hipError_t launch_combine(float* X, int d, const float* Y, const int* inv, int topk, int T, hipStream_t s);

// Dynamic LDS layout (in floats) shared by host and device:
//   [0, hcap)               GEMV input vector (largest GEMV input length) or
//                           the attention unit's q / new K,V / per-wave state
//                           / the split partials it merges
//   [part_off, +kPartCap)   GEMV per-task partials of one row block
//   [sums_off, +kPartCap)   GEMV row sums of one row block; MoE router logits
//   [xown_off, +kPartCap)   this workgroup's rows of the residual stream
//   [red_off, +kRedFloats)  reductions, argmax keys, MoE routing
struct LdsLayout {
  int hcap;
  int part_off;
  int sums_off;
  int xown_off;
  int red_off;
  int total;
};
constexpr int kRedIdsOff = 2 * kWaves;                       // int[kMaxActiveExperts]
constexpr int kRedWtsOff = kRedIdsOff + kMaxActiveExperts;   // float[kMaxActiveExperts]
constexpr int kRedFloats = kRedWtsOff + kMaxActiveExperts;

__host__ __device__ inline LdsLayout lds_layout(const Params& p) {
  int v = p.d;
  v = v > p.H * p.hd ? v : p.H * p.hd;
  const int moe_in = (p.topk + p.nshared) * p.Fe;
  if (p.E == 0) v = v > p.F ? v : p.F;
  else v = v > moe_in ? v : moe_in;
  const int G = p.H / p.nkv;
  const int gpad = G <= 1 ? 1 : G <= 2 ? 2 : 4;
  const int S = p.splits > 1 ? p.splits : 1;
  const int attn = gpad * p.hd + 2 * p.hd + (kWaves + S) * gpad * (p.hd + 2);
  v = v > attn ? v : attn;
  if (G >= 2 && p.hd % 16 == 0 && p.hd <= 80) {
    // the matrix-core attention unit: q high/low, and per wave a transposed
    // V tile (32 positions x the head dimension rounded up to 32) and P
    // high/low, all fp16, above the wave states
    const int cols = 32 * ((p.hd / 16 + 1) / 2);
    const int halves = 2 * gpad * p.hd + kWaves * cols * 40 + 2 * kWaves * gpad * 40;
    const int mm = gpad * p.hd + 2 * p.hd + ((kWaves * gpad * (p.hd + 2) + 3) & ~3) + (halves + 1) / 2;
    v = v > mm ? v : mm;
  }
  LdsLayout L;
  L.hcap = (v + 63) & ~63;
  L.part_off = L.hcap;
  L.sums_off = L.part_off + kPartCap;
  L.xown_off = L.sums_off + kPartCap;
  L.red_off = L.xown_off + kPartCap;
  L.total = L.red_off + kRedFloats;
  return L;
}

}  // namespace kie
