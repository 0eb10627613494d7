/*
 * kie.h — C ABI of libkie.so: batch-1 decode of an fp16 decoder-only
 * transformer as one GPU-resident persistent kernel on MI355X (gfx950).
 *
 * What the library does
 *   The pages describe a "persistent monokernel": one GPU-resident program
 *   that runs the whole decode path (matrix multiplies, attention,
 *   normalisation and sampling) and never hands control back to the CPU
 *   between tokens (page "Breaking the memory wall: 3,000 tokens/s
 *   inference on standard GPUs", agentlenshq.com, section "1. The Monokernel
 *   Runtime").
 *   They name the overheads it removes: ~4.5 us per kernel launch,
 *   host-side scheduling and CPU sampling, and grid-wide synchronisation
 *   (same page, section "Where the microseconds are lost").  kie_decode()
 *   runs n_steps tokens in ONE kernel launch; token feedback (greedy argmax)
 *   stays on the device.
 *
 * Model (the pages give no layer equations; the plain pre-norm reading):
 *   x = E[tok];  per layer:  x += Wo·Attn(RoPE(Wq·rms(x)), RoPE(Wk·rms(x)), Wv·rms(x))
 *                            x += FFN(rms(x))        (SwiGLU, or MoE below)
 *   logits = Wlm·rms(x);  next token = argmax (lowest index on ties).
 *   RMSNorm: x / sqrt(mean(x^2) + eps) * gain.  RoPE: rotate-half pairs
 *   (j, j + head_dim/2), theta_j = base^(-2j/head_dim).  Attention scale
 *   1/sqrt(head_dim), causal, query head i reads KV head i / (H / n_kv).
 *   MoE FFN: p = softmax(Wr·h); the top_k largest p (lower id on ties) mix
 *   with weights p (not renormalised), plus n_shared_experts always-on
 *   experts with weight 1.  Only active experts are read, as the pages
 *   stress that bandwidth follows active parameters (same page, section
 *   "Scaling to frontier MoE models").
 *
 * Conventions
 *   - All weights are fp16, row-major [out][in], in device memory owned by
 *     the caller; they must outlive the handle.  The library never writes
 *     or frees them.  Every GEMV input length (d_model, n_heads*head_dim,
 *     ffn_hidden, expert_hidden) must be a multiple of 8 (16-byte rows).
 *   - Activations are fp32; the KV cache is fp16 (round to nearest even).
 *   - Prefill/decode split: after kie_prefill(t, P) the cache holds
 *     positions 0..P-2 and t[P-1] is pending at position P-1.  Decode step
 *     i runs the model on the pending token at position P-1+i, writes
 *     out_tokens[i] = its greedy token g_i (and its logits) and makes g_i
 *     pending.  decode(a) followed by decode(b) equals decode(a+b).
 *   - Every call is synchronous: it returns after the device work is done,
 *     so device-side errors (barrier watchdog) are reported by that call.
 *     A handle is not thread-safe.
 *   - Return value: KIE_OK (0) or a negative kie_status.  All argument
 *     checks run before any launch, so a rejected call changes nothing.
 *     kie_last_error() gives a message for the calling thread.
 */
#ifndef KIE_H
#define KIE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kie_status {
  KIE_OK = 0,
  KIE_ERR_INVALID_ARG = -1,      /* NULL pointer, bad shape, bad size          */
  KIE_ERR_BAD_STATE = -2,        /* prefill on a used handle, decode w/o prompt,
                                    or a handle broken by an earlier device error */
  KIE_ERR_CONTEXT_OVERFLOW = -3, /* position would pass max_seq                */
  KIE_ERR_TOKEN_RANGE = -4,      /* prompt token id outside [0, vocab_in)      */
  KIE_ERR_OCCUPANCY = -5,        /* the grid cannot be co-resident             */
  KIE_ERR_HIP = -6,              /* a HIP runtime call failed                  */
  KIE_ERR_TIMEOUT = -7,          /* a device barrier wait passed timeout_ms    */
  KIE_ERR_UNSUPPORTED = -8       /* shape outside what the kernels implement   */
} kie_status;

/* flags */
#define KIE_MODE_GRAPH 0x1u   /* decode by replaying a hipGraph of per-stage
                                 kernels (one kernel per stage) instead of one
                                 persistent launch; same stage code, same
                                 results bit for bit */
#define KIE_TRACE 0x2u        /* persistent mode: record, for one decode step
                                 of every kie_decode call (step 1, or step 0
                                 of a one-step call), each workgroup's clock
                                 (100 MHz wall clock) at the step's start and
                                 three times per stage; read it back with
                                 kie_debug_read_trace.  Results are unchanged. */
#define KIE_PLAIN_LAUNCH 0x4u /* persistent mode: launch with an ordinary
                                 dispatch instead of the cooperative-launch API
                                 (for tools that do not follow cooperative
                                 launches).  Co-residency then rests on the
                                 occupancy check kie_create makes (one
                                 workgroup per compute unit fits) and on an
                                 otherwise idle device; if it is not met, the
                                 barrier watchdog ends the call with
                                 KIE_ERR_TIMEOUT instead of hanging. */
#define KIE_MOE_RENORM 0x10u  /* MoE models: the selected experts' softmax
                                 probabilities are rescaled to sum to 1
                                 before they weight the expert outputs
                                 (default: used as they are).  The pages name
                                 only "softmax top-k"; both readings are
                                 offered. */

typedef struct kie_config {
  int32_t n_layers;          /* 1..2048                                        */
  int32_t d_model, n_heads, n_kv_heads, head_dim, ffn_hidden;
  int32_t vocab_in;          /* embedding rows                                 */
  int32_t vocab_out;         /* lm_head rows; must be <= vocab_in              */
  int32_t max_seq;           /* KV capacity in positions                       */
  int32_t n_experts, top_k, n_shared_experts, expert_hidden; /* n_experts 0 = dense */
  float rms_eps, rope_base;
  uint32_t flags;            /* KIE_MODE_*                                     */
  int32_t n_workgroups;      /* persistent grid size; 0 = one per compute unit */
  int32_t timeout_ms;        /* barrier watchdog; 0 = 20000                    */
} kie_config;

typedef struct kie_layer_weights {   /* device pointers, fp16, row-major [out][in] */
  const void *attn_norm;             /* [d]                                        */
  const void *wq, *wk, *wv;          /* [H*hd][d], [n_kv*hd][d], [n_kv*hd][d]       */
  const void *wo;                    /* [d][H*hd]                                  */
  const void *ffn_norm;              /* [d]                                        */
  const void *w_gate, *w_up;         /* dense: [ffn_hidden][d]                     */
  const void *w_down;                /* dense: [d][ffn_hidden]                     */
  const void *router;                /* MoE: [n_experts][d]                        */
  const void *e_gate, *e_up;         /* MoE: [n_experts + n_shared][expert_hidden][d]
                                        (routed experts first, then shared)         */
  const void *e_down;                /* MoE: [n_experts + n_shared][d][expert_hidden] */
} kie_layer_weights;

typedef struct kie_weights {
  const void *tok_emb;               /* [vocab_in][d]                              */
  const void *final_norm;            /* [d]                                        */
  const void *lm_head;               /* [vocab_out][d]                             */
  const kie_layer_weights *layers;   /* host array of n_layers entries; copied     */
} kie_weights;

typedef struct kie_handle kie_handle;

/* Validates a configuration on the host only (no GPU needed).
 * KIE_OK, KIE_ERR_INVALID_ARG or KIE_ERR_UNSUPPORTED.  The pages describe
 * no API; the shapes are those of the model they benchmark, a 2B-class
 * decoder (page "Breaking the memory wall: 3,000 tokens/s inference on
 * standard GPUs", introduction). */
int kie_config_check(const kie_config *cfg);

/* Creates a decoder on the current HIP device.  Validates cfg and that every
 * weight pointer lies in device memory large enough for its shape; allocates
 * the fp16 KV cache ([L][n_kv][max_seq][hd] for K and for V), activation
 * scratch, barrier words and the RoPE cos/sin table (built in float64,
 * rounded to fp32).  `hip_stream` (a hipStream_t, NULL = default stream) is
 * the stream every later launch of this handle uses.  On success *out owns
 * all of that memory until kie_destroy.  KIE_ERR_OCCUPANCY if the
 * persistent grid cannot be co-resident: the monokernel stays resident for
 * the whole decode (same page, section "1. The Monokernel Runtime"). */
int kie_create(const kie_config *cfg, const kie_weights *w, void *hip_stream,
               kie_handle **out);

/* Copies `tokens` (host, int32 [n_tokens], n_tokens >= 1) to the device and
 * runs positions 0..n_tokens-2 through every layer (no lm_head) in one
 * persistent launch; tokens[n_tokens-1] becomes pending.  Needs a fresh or
 * reset handle (else KIE_ERR_BAD_STATE); KIE_ERR_TOKEN_RANGE for an id
 * outside [0, vocab_in); KIE_ERR_CONTEXT_OVERFLOW if n_tokens > max_seq.
 * The prompt runs in the same GPU-resident program as decoding, without
 * returning to the host between positions (same page, section "1. The
 * Monokernel Runtime"). */
int kie_prefill(kie_handle *h, const int32_t *tokens, int32_t n_tokens);

/* As kie_prefill (same arguments, state afterwards and errors), but the
 * prompt's positions go through each layer together, in chunks of 2048:
 * the weight products become dense matrix products on the matrix cores
 * (fp16 weights times activations split into fp16 hi + lo parts,
 * accumulated in fp32, so an fp32 product up to rounding order), followed
 * by causal attention over the cache.  The K/V rows written agree with
 * kie_prefill's up to fp32 rounding order.  MoE models route every
 * position (the routing record of kie_debug_expert_ids is filled), group
 * the positions by expert on the host and run each expert's products over
 * its rows.  Needs d_model, n_heads * head_dim and ffn_hidden (MoE:
 * expert_hidden) to be multiples of 32 and head_dim a multiple of 16;
 * otherwise KIE_ERR_UNSUPPORTED (use kie_prefill).  Its device workspace
 * belongs to the handle: allocated by the first call that needs more than
 * the handle holds, kept for later calls and freed by kie_destroy.  It
 * takes about 4 T (d + 2 qd + 2 kd + 2 F + max(d, qd, F)) bytes, with qd =
 * n_heads head_dim, kd = n_kv_heads head_dim, F = ffn_hidden (0 for MoE,
 * which adds its routing and per-expert buffers) and T = min(2048,
 * n_tokens - 1) positions per chunk.  A prompt's positions are all known
 * up front, so its products are dense matrix products; decode steps stay
 * on the GEMV path of the persistent kernel.  Cited: "Breaking the memory
 * wall: 3,000 tokens/s inference on standard GPUs", section "1. The
 * Monokernel Runtime" (the decode path; the prompt's own pass is not
 * described there). */
int kie_prefill_batched(kie_handle *h, const int32_t *tokens, int32_t n_tokens);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  As
 * kie_prefill_batched (same arguments, the same K/V rows and pending token
 * bit for bit, the same errors), but its workspace is a static device array
 * of KIE_PREFILL_SCRATCH_MIB MiB, which the library holds on every GPU it
 * runs on until the process ends, and it calls no hipMalloc or hipFree.
 * When the usual chunk's workspace (see kie_prefill_batched) exceeds the
 * array, the prompt goes through in smaller chunks; KIE_ERR_UNSUPPORTED if
 * one position's workspace exceeds it.  Every call on a GPU shares that
 * GPU's array, which keeps the last call's contents: calls that overlap on
 * one GPU (other threads, other handles' streams) race and must be
 * serialised by the caller.  The handle's device must be current
 * (KIE_ERR_BAD_STATE otherwise). */
#define KIE_PREFILL_SCRATCH_MIB 64
int kie_prefill_batched_noalloc(kie_handle *h, const int32_t *tokens, int32_t n_tokens);

/* Generates n_steps tokens in one launch.  out_tokens: device int32
 * [n_steps] (required when n_steps > 0).  out_logits: device fp32
 * [n_steps][vocab_out] or NULL.  n_steps == 0 is a no-op.
 * KIE_ERR_CONTEXT_OVERFLOW if position + n_steps > max_seq.  One kernel
 * launch for all the steps, with the greedy token fed back on the device:
 * the single-request decode the pages measure (same page, introduction
 * and section "1. The Monokernel Runtime"; launch overhead and CPU
 * sampling are among the losses listed in "Where the microseconds are
 * lost"). */
int kie_decode(kie_handle *h, int32_t n_steps, int32_t *out_tokens, float *out_logits);

/* As kie_decode, but each step draws its token from softmax(z / temperature)
 * instead of taking the argmax: sampling inside the monokernel (page
 * "Breaking the memory wall: 3,000 tokens/s inference on standard GPUs",
 * section "1. The Monokernel Runtime").  The draw is the Gumbel-max method:
 * the token is the first maximum over i of the float32 key
 * z_i / temperature - log(-log(u_i)), formed in float64, where u_i is the
 * top 53 bits (plus half a bin) of word i mod 4 of the Philox4x64-10 block
 * for counter (position, i div 4, 0, 0) and key (seed, 0); `position` is
 * the position of the step's input token.  So a (seed, position) pair
 * always gives the same draw, and decode(a); decode(b) equals decode(a+b).
 * temperature == 0 is greedy decoding (identical to kie_decode);
 * KIE_ERR_INVALID_ARG if it is negative, infinite or NaN.  out_logits, if
 * given, receives the logits z (not the keys).  Other arguments and errors
 * as kie_decode. */
int kie_decode_sampled(kie_handle *h, int32_t n_steps, uint64_t seed, float temperature,
                       int32_t *out_tokens, float *out_logits);

/* As kie_decode_sampled with temperature > 0, with the draw restricted to
 * top-k and top-p (nucleus) candidates; the pages name sampling in the
 * monokernel but no rule (same passage as kie_decode_sampled).  Candidates
 * are the vocabulary entries by logit, largest first, ties by the lower
 * index.  top_k in [1, KIE_MAX_TOP_K] keeps the first top_k of them;
 * top_k == 0 keeps the first KIE_MAX_TOP_K (so a nucleus wider than that is
 * cut there).  top_p in (0, 1) then keeps the shortest prefix whose mass
 * exp((z_j - z_0) / temperature), summed in float64 in that order (z_0 the
 * largest logit), reaches top_p of the kept pool's mass; top_p == 1 keeps
 * the pool.  The token is the Gumbel-max draw of kie_decode_sampled (same
 * keys) over what is kept, the lowest index winning on equal keys; so
 * top_k == 1 is the greedy token, and top_k == 0 with top_p == 1 is
 * exactly kie_decode_sampled.  Every workgroup selects the candidates from
 * the step's logits after the step's grid barrier.  KIE_ERR_INVALID_ARG for
 * temperature <= 0, infinite or NaN, top_k outside [0, KIE_MAX_TOP_K] or
 * top_p outside (0, 1]; KIE_ERR_UNSUPPORTED for a KIE_MODE_GRAPH handle
 * (unless nothing restricts the draw).  Other arguments and errors as
 * kie_decode. */
#define KIE_MAX_TOP_K 256
int kie_decode_sampled_topkp(kie_handle *h, int32_t n_steps, uint64_t seed, float temperature,
                             int32_t top_k, float top_p, int32_t *out_tokens, float *out_logits);

/* Drops the context: position 0, no pending token (KV contents are simply
 * overwritten by the next prefill).  Also clears a broken state. */
int kie_reset(kie_handle *h);

/* Next position to be written (P-1 after a prefill of P tokens). */
int kie_get_position(const kie_handle *h, int32_t *pos);

/* Frees everything the handle owns.  NULL is allowed. */
void kie_destroy(kie_handle *h);

/* Message for the last failed call on this thread ("" if none). */
const char *kie_last_error(void);

/* Device time of the last kie_prefill/kie_decode launch region of this
 * handle, in milliseconds (HIP events on the handle's stream). */
int kie_last_elapsed_ms(const kie_handle *h, float *ms);

/* ---- inspection entry points (used by the parity tests) ---------------- */

/* Copies K and V rows [pos0, pos1) of `layer`, all KV heads, to host
 * buffers laid out [n_kv][pos1-pos0][head_dim] fp16 (either may be NULL).
 * K rows are stored after RoPE. */
int kie_debug_read_kv(const kie_handle *h, int32_t layer, int32_t pos0, int32_t pos1,
                      void *k_host, void *v_host);

/* Test-only: one decode stage at a time, for checking each stage against a
 * float64 computation (the pages describe the stages only as the parts of
 * the monokernel: page "Breaking the memory wall: 3,000 tokens/s inference
 * on standard GPUs", section "1. The Monokernel Runtime").  On a handle with
 * a pending token (after a prefill), kie_debug_stage runs `stage` of layer
 * `layer` (0 for KIE_STAGE_LM_HEAD) of the next decode step, at the
 * handle's position, as the staged mode's kernels do (the attention stage
 * includes its split merge).  KIE_STAGE_QKV at layer 0 opens the step;
 * later stages read what the earlier ones of that step wrote, so they run
 * in model order.  The attention stage writes its K/V rows into the cache
 * (kie_debug_read_kv sees them); the position does not advance and the
 * next prefill, decode or reset closes the step.  KIE_ERR_BAD_STATE
 * without a pending token or an open step; KIE_ERR_INVALID_ARG for a stage
 * the model lacks or a layer out of range. */
#define KIE_STAGE_QKV 0          /* RMSNorm + Q/K/V products          */
#define KIE_STAGE_ATTENTION 1    /* RoPE, K/V append, split attention, merge */
#define KIE_STAGE_O 2            /* O product + residual              */
#define KIE_STAGE_GATEUP 3       /* RMSNorm + gate/up products + SwiGLU */
#define KIE_STAGE_DOWN 4         /* down product + residual           */
#define KIE_STAGE_ROUTER 5       /* MoE: RMSNorm + router product     */
#define KIE_STAGE_MOE_GATEUP 6   /* MoE: routing + experts' gate/up + SwiGLU */
#define KIE_STAGE_MOE_DOWN 7     /* MoE: experts' down + residual     */
#define KIE_STAGE_LM_HEAD 8      /* final RMSNorm + lm_head + argmax  */
int kie_debug_stage(kie_handle *h, int32_t stage, int32_t layer);

/* Test-only: copies what a stage of the open step (kie_debug_stage) wrote
 * to `out_host`, at least n elements, as fp32 (int32 for KIE_ACT_TOKEN):
 * the residual stream after the O product or after the FFN of `layer`
 * ([d_model]), its q|k|v ([n_heads + 2 n_kv_heads][head_dim]), the
 * attention output o ([n_heads][head_dim]), the FFN hidden u ([ffn_hidden],
 * MoE: [top_k + shared][expert_hidden]), the router logits ([n_experts]),
 * the logits ([vocab_out]) or the argmax token.  o and u cross between
 * workgroups as 24-bit values (a 16-bit significand) and are returned so.
 * KIE_ERR_BAD_STATE if a word was not written by that stage of the open
 * step (checked by its epoch). */
#define KIE_ACT_X_ATTN 0
#define KIE_ACT_X 1
#define KIE_ACT_QKV 2
#define KIE_ACT_O 3
#define KIE_ACT_U 4
#define KIE_ACT_ROUTER 5
#define KIE_ACT_LOGITS 6
#define KIE_ACT_TOKEN 7
int kie_debug_read_act(const kie_handle *h, int32_t what, int32_t layer, void *out_host, int32_t n);

/* MoE only: the routed expert ids chosen at positions [pos0, pos1) by
 * prefill or decode, host int32 [pos1-pos0][n_layers][top_k] in rank order
 * (largest probability first; ties to the lower id).  pos1 may not exceed
 * the current position (kie_get_position); INVALID_ARG otherwise. */
int kie_debug_expert_ids(const kie_handle *h, int32_t pos0, int32_t pos1, int32_t *ids_host);

/* y = W x with the decode kernel's GEMV stage code: W device fp16 [rows][cols]
 * row-major (cols a multiple of 8), x device fp32 [cols], y device fp32
 * [rows].  Synchronous on `hip_stream`.  Runs n_workgroups (0 = one per CU)
 * workgroups. */
int kie_debug_gemv(const void *w, const float *x, float *y, int32_t rows, int32_t cols,
                   int32_t n_workgroups, void *hip_stream);

/* c = a w^T (or c += a w^T with accumulate != 0) with the batched
 * prefill's matrix-core product: w device fp16 [n][k] row-major, a device
 * fp32 [m][k], c device fp32 [m][n]; k a positive multiple of 32; m, n, k at
 * most 65536, and n k and m k each under 2^30 elements (the kernel's byte
 * offsets are 32-bit), else KIE_ERR_INVALID_ARG.  Allocates and frees a
 * 4 m k byte workspace.  Synchronous on `hip_stream`. */
int kie_debug_gemm(const void *w, const float *a, float *c, int32_t m, int32_t n, int32_t k,
                   int32_t accumulate, void *hip_stream);

/* Grid-barrier stress test: n_rounds barriers over n_workgroups persistent
 * workgroups; each round every workgroup checks that all others reached the
 * previous round.  Returns KIE_OK, KIE_ERR_TIMEOUT, or KIE_ERR_INVALID_ARG
 * (*violations receives the number of failed checks).  spin_limit > 0 caps
 * each wait at that many polls (a host-forced watchdog test). */
int kie_debug_barrier(int32_t n_workgroups, int32_t n_rounds, int32_t spin_limit,
                      int32_t *violations, float *ms_per_barrier, void *hip_stream);

/* KIE_TRACE handles: copies the trace of the last kie_decode call to
 * `out` (host, uint64 [n_workgroups][max_events]) and sets *n_events to the
 * number of events each workgroup recorded: event 0 is the start of the
 * traced step, then three events for every stage of that step in execution
 * order (per layer Q/K/V, attention, O, then gate/up and down, or router,
 * expert gate/up and expert down; then lm_head): when the stage's inputs
 * were complete, when its main loop started (after the norm, or after RoPE
 * and the KV append) and when it ended.  KIE_ERR_BAD_STATE without
 * KIE_TRACE or before a decode call; KIE_ERR_INVALID_ARG if max_events is
 * smaller than the recorded count. */
int kie_debug_read_trace(const kie_handle *h, uint64_t *out, int32_t max_events,
                         int32_t *n_events, int32_t *n_workgroups);

/* HBM streaming probe: reads `bytes` (a multiple of 16) from device buffer
 * `src` with 128-bit non-temporal loads, grid-stride over n_workgroups
 * workgroups (0 = four per compute unit), and copies them to `dst` when it
 * is not NULL (same size, device memory, no overlap).  Launched `reps`
 * times back to back on `hip_stream`; *ms_per_launch receives the average
 * time of one launch.  Measures the device's achievable streaming
 * bandwidth, and gives a copy of known size against which memory counters
 * are calibrated. */
int kie_debug_stream(const void *src, void *dst, size_t bytes, int32_t n_workgroups,
                     int32_t reps, float *ms_per_launch, void *hip_stream);

/* The streaming probe with its shape chosen: `depth` (1, 2, 4, 8 or 16)
 * 128-bit loads in flight per lane, and `kind` the load: 0 non-temporal
 * global loads (what kie_debug_stream uses, with depth 8), 1 plain global
 * loads, 2 the raw buffer loads with the non-temporal policy that the
 * decode kernel streams its weights with (bytes below 4 GiB).  Other
 * arguments and errors as kie_debug_stream; KIE_ERR_INVALID_ARG for another
 * depth or kind.  A sweep over depth, kind and n_workgroups gives the
 * read rate this device reaches at all, the ceiling against which the
 * decode kernel's streaming is judged. */
int kie_debug_stream_ex(const void *src, void *dst, size_t bytes, int32_t n_workgroups,
                        int32_t depth, int32_t kind, int32_t reps, float *ms_per_launch,
                        void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* KIE_H */
