// Decode stages and the persistent monokernel for gfx950 (CDNA4, wave64).
//
// The pages' method: one GPU-resident program runs the whole per-token
// decode path (matrix multiplies, attention, normalisation, sampling) and
// never returns to the CPU between tokens (page "Breaking the memory wall:
// 3,000 tokens/s inference on standard GPUs", agentlenshq.com, section
// "1. The Monokernel Runtime"); normalisation, attention and matmul stages
// are fused so data stays near the compute units (page "Kog bets deeper GPU
// optimization can accelerate AI inference", remio.ai, co-design section).
// Batch-1 decode moves every active weight from HBM once per token and is
// bandwidth bound (agentlenshq.com page, section "The bottleneck: memory
// bandwidth, not compute"), so every stage is built around streaming fp16
// weight rows with 128-bit loads, not around matrix cores.
//
// Layout of one decode step (dense model), one workgroup per CU:
//   per layer:  [rmsnorm+QKV GEMV] | [RoPE + KV append + split-K attention,
//               last-arriving split merges] | [O GEMV + residual] |
//               [rmsnorm + gate/up GEMV + SwiGLU] | [down GEMV + residual] |
//   then        [final rmsnorm + lm_head GEMV + argmax] | token feedback
// '|' is a grid barrier in the persistent kernel and a kernel boundary in
// the staged (hipGraph) mode.  MoE layers replace the FFN with
//   [rmsnorm + router GEMV] | [routing + expert gate/up] | [expert down].
//
// Cross-XCD coherence without cache maintenance.  MI355X has one L2 per XCD
// and the L2s are not coherent with each other.  An agent-scope release or
// acquire fence writes back or invalidates a whole L2, and with 256
// workgroups doing that at every barrier the barrier costs tens of
// microseconds.  Instead, every value one workgroup writes and another
// reads (activations, KV rows, split partials, argmax slots) is stored and
// loaded with device-scope (sc1) accesses, which are coherent by
// themselves; a barrier then only has to wait for the issuing wave's stores
// to complete (s_waitcnt vmcnt(0)) before it signals.  Weights, the RoPE
// table and the prompt are read-only and use plain non-temporal loads.
//
// Prefetch across barriers.  Weights never depend on activations, so each
// workgroup issues the first loads of its next stage (weight rows, or the
// KV rows its attention split will read) right after it arrives at a
// barrier and before it waits; the HBM keeps streaming while the grid
// synchronises (the single-GPU counterpart of the pages' idea of
// overlapping weight movement with the dependency chain, agentlenshq.com
// page, section "3. Laneformer Architecture").
#include "kie_params.h"

namespace kie {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;         // finite "minus infinity" for softmax state
constexpr int kAuxSc1 = 16;                 // buffer-load cache policy: device scope (sc1)
constexpr int kAuxNt = 2;                   // buffer-load cache policy: non-temporal
constexpr unsigned kBufFlags = 0x00020000u; // raw 32-bit buffer resource word 3

// ---------------------------------------------------------------------------
// Memory access helpers
// ---------------------------------------------------------------------------
// Device-coherent scalar accesses for data shared between workgroups.
__device__ __forceinline__ float ld_c(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_c(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_cu(const unsigned* p) {
  return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_cu(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_c64(const unsigned long long* p) {
  return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_c64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Buffer resources.  A raw buffer load whose byte offset lies past the
// resource's size returns zero without touching memory, so loads are issued
// unconditionally (no divergent branch around them, which also keeps the
// compiler's wait counts exact) and unwanted lanes simply get kOffNone.
constexpr unsigned kOffNone = 0xFFFFFFF0u;  // out of range of every resource
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(unsigned)bytes,
                                           (int)kBufFlags);
}
// weights: read once per token, non-temporal
__device__ __forceinline__ u32x4 ld_w16(Rsrc r, unsigned byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kAuxNt));
}
// KV cache rows: written by other workgroups in earlier steps, device scope
__device__ __forceinline__ u32x4 ld_kv16(Rsrc r, unsigned byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kAuxSc1));
}

// Waits until every store this wave issued has completed (vmcnt(0)); the
// signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// fp16 x8 . fp32 x8 accumulated in fp32 (v_fma_mix_f32).  The 16-byte word
// is reinterpreted as a whole: bit-casting single elements of an ext_vector
// is miscompiled to element 0 by this toolchain.
__device__ __forceinline__ float dot8(u32x4 w, float4 a, float4 b, float acc) {
  const f16x8 v = __builtin_bit_cast(f16x8, w);
  acc = fmaf((float)v[0], a.x, acc);
  acc = fmaf((float)v[1], a.y, acc);
  acc = fmaf((float)v[2], a.z, acc);
  acc = fmaf((float)v[3], a.w, acc);
  acc = fmaf((float)v[4], b.x, acc);
  acc = fmaf((float)v[5], b.y, acc);
  acc = fmaf((float)v[6], b.z, acc);
  acc = fmaf((float)v[7], b.w, acc);
  return acc;
}

__device__ __forceinline__ void unpack8(u32x4 w, float* f) {
  const f16x8 v = __builtin_bit_cast(f16x8, w);
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (float)v[e];
}

// Cross-lane sums with DPP moves (VALU, no LDS round trip).  dpp_add(v, c,
// rows) adds the DPP-permuted v to v in the rows selected by `rows`; lanes
// in other rows add 0.
template <int kCtrl, int kRows>
__device__ __forceinline__ float dpp_add(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, kRows, 0xF,
                                                false);
  return v + __builtin_bit_cast(float, moved);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror
constexpr int kDppBcast15 = 0x142;    // row_bcast:15
constexpr int kDppBcast31 = 0x143;    // row_bcast:31

// Sum over each 16-lane row, left in every lane of the row.
__device__ __forceinline__ float group16_sum(float v) {
  v = dpp_add<kDppXor1, 0xF>(v);
  v = dpp_add<kDppXor2, 0xF>(v);
  v = dpp_add<kDppHalfMirror, 0xF>(v);
  v = dpp_add<kDppMirror, 0xF>(v);
  return v;
}

// Sum over the wave, returned uniformly (read from lane 63).
// The wave's index, known to the compiler as wave-uniform (kept in SGPRs).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ float wave_sum(float v) {
  v = group16_sum(v);
  v = dpp_add<kDppBcast15, 0xA>(v);   // rows 1, 3 += last lane of rows 0, 2
  v = dpp_add<kDppBcast31, 0xC>(v);   // rows 2, 3 += lane 31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

// Order-preserving map of a float to 32 bits, packed above the complemented
// index so that a 64-bit max picks the largest value and, on ties, the
// lowest index.
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
  unsigned u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)idx);
}
// Decodes a slot into a row index, clamped into [0, n) so that a slot no
// workgroup wrote can never address outside the embedding table.
__device__ __forceinline__ int argmax_index(unsigned long long key, int n) {
  const int i = (int)(0xFFFFFFFFu - (unsigned)(key & 0xFFFFFFFFull));
  return i < 0 ? 0 : (i >= n ? n - 1 : i);
}

__device__ __forceinline__ int split_begin(int s, int n, int S) {
  return (int)(((long long)s * n) / S);
}

// Even split of `total` items over `parts`: [begin, end) of part `i`.
__device__ __forceinline__ void even_range(int total, int parts, int i, int& b, int& e) {
  b = (int)(((long long)i * total) / parts);
  e = (int)(((long long)(i + 1) * total) / parts);
}

// ---------------------------------------------------------------------------
// Grid barrier: two-level arrival counters in HBM, no cache maintenance.
//
// Workgroup w belongs to group w mod 8 (the XCD the hardware dispatches it
// to).  Arrival: every wave waits for its own stores to complete, the
// workgroup meets at s_barrier, then one lane bumps its group's counter;
// the last arrival of a group bumps the global counter.  Waiting: one lane
// polls the global counter (device-scope loads) until all groups arrived
// for this epoch.  Counters only grow, so no reset is needed between
// barriers.  The wait is bounded: on timeout (or when another workgroup
// already failed) the error word is set and every workgroup leaves the
// kernel at its next barrier.
//
// arrive() and wait() are separate so that a workgroup can issue its next
// stage's weight loads in between.
// ---------------------------------------------------------------------------
struct GridSync {
  unsigned* ctr;      // [0] global counter, [kGroupStride * (1 + g)] group g counters
  int* err;
  unsigned epoch;
  unsigned ngrp;      // groups in use
  unsigned gsize;     // workgroups in this workgroup's group
  unsigned grp;
  long long ticks;
  int spin_limit;
};

__device__ __forceinline__ GridSync make_sync(unsigned* ctr, int* err, unsigned n, long long ticks,
                                              int spin_limit) {
  GridSync g;
  g.ctr = ctr;
  g.err = err;
  g.epoch = 0u;
  g.ngrp = n < (unsigned)kGroups ? n : (unsigned)kGroups;
  g.grp = blockIdx.x % g.ngrp;
  g.gsize = (n - g.grp + g.ngrp - 1) / g.ngrp;
  g.ticks = ticks;
  g.spin_limit = spin_limit;
  return g;
}

__device__ __forceinline__ void grid_arrive(GridSync& g) {
  wait_stores();
  __builtin_amdgcn_s_barrier();
  g.epoch += 1u;
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(g.ctr + kGroupStride * (1 + g.grp), 1u,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1u == g.epoch * g.gsize)
      __hip_atomic_fetch_add(g.ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void set_timeout(int* err) {
  int expected = 0;
  __hip_atomic_compare_exchange_strong(err, &expected, kErrTimeout, __ATOMIC_RELAXED,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool grid_wait(GridSync& g, int* flag) {
  if (threadIdx.x == 0) {
    const unsigned target = g.epoch * g.ngrp;
    int ok = 1;
    long long t0 = 0;
    int spins = 0;
    while ((int)(ld_cu(g.ctr) - target) < 0) {
      ++spins;
      if ((spins & 31) == 1) {
        if (spins == 1) t0 = wall_clock64();
        if (__hip_atomic_load(g.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
          ok = 0;
          break;
        }
        if (wall_clock64() - t0 > g.ticks) {
          set_timeout(g.err);
          ok = 0;
          break;
        }
      }
      if (g.spin_limit > 0 && spins >= g.spin_limit) {
        set_timeout(g.err);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!ok) *flag = 0;               // the flag is 1 until a failure (see wg_all)
  }
  __syncthreads();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return *flag != 0;
}

// ---------------------------------------------------------------------------
// GEMV engine.
//
// A workgroup owns rows [r0, r1) of a GEMV with `nch` 16-byte chunks per
// row.  Each row is cut into slices of 64 chunks (one 16-byte load per lane,
// 1 KiB contiguous per wave load); a (row, slice) pair is a task.  Rows are
// processed in blocks; a block's tasks are split evenly over the 8 waves,
// each wave streams its tasks in batches of kBatch loads per lane with the
// next batch always in flight, reduces each task across the wave and parks
// the partial in LDS; the block's row sums are then added in slice order
// (deterministic) and handed to the epilogue.
// ---------------------------------------------------------------------------
struct GemvWork {
  int r0, r1;    // rows of this workgroup
  int nch;       // 16-byte chunks per row
  int ks;        // slices per row
  int rb;        // rows per block
};

// Rows are dealt out in units of `unit` consecutive rows (rows % unit == 0),
// and row blocks hold whole units, so an epilogue can publish a unit's
// results together (gate and up rows of one output, or pair words).
__device__ __forceinline__ GemvWork gemv_work(int rows, int cols, int parts, int part, int unit) {
  GemvWork g;
  int b, e;
  even_range(rows / unit, parts, part, b, e);
  g.r0 = b * unit;
  g.r1 = e * unit;
  g.nch = cols >> 3;
  g.ks = (g.nch + 63) >> 6;
  const int rb = (kPartCap / g.ks / unit) * unit;
  g.rb = rb < unit ? unit : rb;
  return g;
}

struct WBatch {
  u32x4 w[kBatch];
};
struct WPre {                  // the first two batches of a wave's first block
  WBatch a, b;
};

__device__ __forceinline__ void wave_tasks(const GemvWork& g, int b0, int& t0, int& t1) {
  const int b1 = min(g.r1, b0 + g.rb);
  const int T = (b1 - b0) * g.ks;
  const int wave = wave_id();
  t0 = (wave * T) / kWaves;
  t1 = ((wave + 1) * T) / kWaves;
}

// Loads tasks [t, t + kBatch) ∩ [t, tend) of the block starting at row b0.
// A task's row is the same in every lane, so its resource is uniform; lanes
// past the row end and tasks past `tend` read zeros (kOffNone).
template <class Addr>
__device__ __forceinline__ WBatch wload(const Addr& addr, const GemvWork& g, int b0, int t, int tend) {
  const int lane = threadIdx.x & 63;
  int r = t / g.ks;
  int s = t - r * g.ks;
  WBatch B;
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    const int c = s * 64 + lane;
    const bool ok = (t + i < tend) && (c < g.nch);
    const int rr = min(b0 + r, g.r1 - 1);
    B.w[i] = ld_w16(addr.rsrc(rr), ok ? addr.off(rr, c) : kOffNone);
    if (++s == g.ks) {
      s = 0;
      ++r;
    }
  }
  // keep the issue order of batches: the wait counts assume it
  __builtin_amdgcn_sched_barrier(0);
  return B;
}

// The kBatch tasks of a batch are independent: their dot products and wave
// reductions are written as separate chains, with no branch between them,
// so the compiler interleaves them instead of running one latency-bound
// chain per task.  Tasks past `tend` and lanes past the row end hold zero
// weights (their loads used an out-of-range offset), so only the final
// partial store is conditional.
__device__ __forceinline__ void wconsume(const WBatch& B, const float* h, const GemvWork& g, int t,
                                         int tend, float* part) {
  const int lane = threadIdx.x & 63;
  const float4* h4 = reinterpret_cast<const float4*>(h);
  int s = t % g.ks;
  float a[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    const int c = min(s * 64 + lane, g.nch - 1);     // clamp the LDS index of lanes past the row end
    a[i] = dot8(B.w[i], h4[2 * c], h4[2 * c + 1], 0.f);
    if (++s == g.ks) s = 0;
  }
#pragma unroll
  for (int i = 0; i < kBatch; ++i) a[i] = wave_sum(a[i]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (t + i < tend) part[t + i] = a[i];
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <class Addr>
__device__ __forceinline__ WPre gemv_prefetch(const GemvWork& g, const Addr& addr) {
  int t0, t1;
  wave_tasks(g, g.r0, t0, t1);
  WPre P;
  P.a = wload(addr, g, g.r0, t0, t1);
  P.b = wload(addr, g, g.r0, t0 + kBatch, t1);
  return P;
}

// One row block [b0, b0 + nrows): A and B hold the wave's first two
// batches (already issued); the rest of the block streams through them.
template <class Addr, class Epi>
__device__ __forceinline__ void gemv_block(const GemvWork& g, const Addr& addr, const float* h,
                                           float* part, float* sums, int b0, WBatch A, WBatch B,
                                           Epi& epi) {
  const int nrows = min(g.r1 - b0, g.rb);
  int t0, t1;
  wave_tasks(g, b0, t0, t1);
  for (int t = t0; t < t1; t += 2 * kBatch) {
    wconsume(A, h, g, t, t1, part);
    if (t + 2 * kBatch < t1) A = wload(addr, g, b0, t + 2 * kBatch, t1);
    if (t + kBatch < t1) wconsume(B, h, g, t + kBatch, t1, part);
    if (t + 3 * kBatch < t1) B = wload(addr, g, b0, t + 3 * kBatch, t1);
  }
  __syncthreads();
  // row sums over the slices in order, four loads issued ahead of the adds
  for (int i = threadIdx.x; i < nrows; i += kThreads) {
    const float* pr = part + i * g.ks;
    float v = 0.f;
    int s = 0;
    for (; s + 4 <= g.ks; s += 4) {
      const float a0 = pr[s], a1 = pr[s + 1], a2 = pr[s + 2], a3 = pr[s + 3];
      v += a0;
      v += a1;
      v += a2;
      v += a3;
    }
    for (; s < g.ks; ++s) v += pr[s];
    sums[i] = v;
  }
  __syncthreads();
  epi(b0, nrows, sums);
  __syncthreads();
}

// Runs the workgroup's rows.  With kPre, `pre` is the first batch of the
// first block, already issued by gemv_prefetch with the same work and
// addresses.  epi(b0, n, sums) is called by every thread once per block
// with the block's n row sums in LDS.
template <bool kPre, class Addr, class Epi>
__device__ __forceinline__ void gemv_run(const GemvWork& g, const Addr& addr, const float* h,
                                         float* part, float* sums, WPre pre, Epi epi) {
  if (g.r0 >= g.r1) return;
  int b0 = g.r0;
  if (kPre) {
    gemv_block(g, addr, h, part, sums, b0, pre.a, pre.b, epi);
    b0 += g.rb;
  }
  for (; b0 < g.r1; b0 += g.rb) {
    int t0, t1;
    wave_tasks(g, b0, t0, t1);
    const WBatch A = wload(addr, g, b0, t0, t1);
    const WBatch B = wload(addr, g, b0, t0 + kBatch, t1);
    gemv_block(g, addr, h, part, sums, b0, A, B, epi);
  }
}

// ---------------------------------------------------------------------------
// Activation exchange: flag-in-data words.
//
// Every activation one workgroup hands to others (x, q/k/v, attention
// partials, o, the FFN hidden u, router logits) lives in one arena of 64-bit
// words holding a payload and the epoch of the stage that wrote it.  A
// plain word is (epoch << 32) | fp32 bits.  The vectors that every
// workgroup reads back in full as a GEMV input (x, o and u) travel as pair
// words instead: two values, each the top 24 bits of its fp32 pattern
// rounded to nearest even (sign, exponent and a 16-bit significand, relative
// error at most 2^-16), in bits [0, 24) and [24, 48), and a 16-bit tag of
// the epoch in bits [48, 64).  The cost of a gather follows the words each
// of the 256 workgroups reads, so pairs halve it.  All arithmetic stays
// fp32, and the residual stream also keeps plain words, which its owners,
// the router and lm_head read.  A producer writes each word with one device-scope
// 64-bit store (single-copy atomic), so a consumer that reads a word with
// the epoch it expects also has the value: one load both synchronises and
// delivers, and stages need no grid barrier and no store-completion wait.
// Epochs are unique per (call, step, layer, stage slot): flag(step, l, slot)
// = epoch0 + (step * L + l) * 8 + slot, with epoch0 advanced by the host
// for every launch, so stale words of earlier stages or calls never match.
//
// Reuse of a word by a later stage is safe without barriers because every
// stage that writes a buffer depends (through the data it consumes) on
// every workgroup having finished the stage that read the previous value:
// e.g. x written by the O projection of layer l+1 needs o of every head,
// hence every Q/K/V row of layer l+1, hence every workgroup's read of x in
// that layer's Q/K/V stage.  Consecutive decode steps are separated by the
// argmax grid barrier, consecutive prefill steps by an explicit barrier.
// ---------------------------------------------------------------------------
typedef unsigned long long u64;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

enum Slot : unsigned { kSlotQkv = 0, kSlotPart = 1, kSlotO = 2, kSlotXO = 3, kSlotRouter = 4,
                       kSlotU = 5, kSlotXDown = 6 };

__device__ __forceinline__ unsigned ll_flag(const Params& p, int step, int l, unsigned slot) {
  return p.epoch0 + ((unsigned)step * (unsigned)p.L + (unsigned)l) * 8u + slot;
}

__device__ __forceinline__ void ll_put(const Params& p, int word, float v, unsigned flag) {
  const u64 w = ((u64)flag << 32) | (u64)__float_as_uint(v);
  __hip_atomic_store(p.act + word, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The 16-bit tag of an epoch in a pair word: never 0, so a cleared word
// never matches.  Two epochs share a tag only when they are a multiple of
// 65535 apart.  A stale word is never that old when it is polled: within a
// launch every pair word is rewritten once per layer (8 epochs), and a
// launch's first wait on a word comes at most 16 * L + 16 epochs after that
// word's last write in the previous launch (the host hands each launch
// (steps + 1) * L * 8 + 8 epochs); n_layers <= 2048 keeps that below 65535.
__device__ __forceinline__ unsigned pair_tag(unsigned flag) { return flag % 65535u + 1u; }

// Top 24 bits of an fp32 pattern, rounded to nearest even.
__device__ __forceinline__ unsigned f32_to_24(float v) {
  const unsigned b = __float_as_uint(v);
  return (b + 0x7Fu + ((b >> 8) & 1u)) >> 8;
}

// Two values in one pair word: a is element 2j, b element 2j + 1.
__device__ __forceinline__ void ll_put2(const Params& p, int word, float a, float b, unsigned flag) {
  const unsigned ua = f32_to_24(a), ub = f32_to_24(b);
  const unsigned lo = ua | (ub << 24);
  const unsigned hi = (ub >> 8) | (pair_tag(flag) << 16);
  const u64 w = ((u64)hi << 32) | (u64)lo;
  __hip_atomic_store(p.act + word, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ Rsrc arena_rsrc(const Params& p) {
  return make_rsrc(p.act, (size_t)p.act_words * 8);
}

__device__ __forceinline__ u32x2 ld_ll(Rsrc r, unsigned byte_off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, kAuxSc1));
}

// A contiguous run of arena words to copy into LDS once they carry `want`.
typedef __attribute__((address_space(3))) float lds_float;
struct LLRange {
  int src;            // first arena word
  int n;              // words
  float* dst;         // LDS destination (2n floats for pair words)
  unsigned want;      // expected epoch
  int pk = 0;         // 1: pair words (2 values each)
};

// Control state shared by every bounded wait of a workgroup.
struct Ctl {
  int* err;
  long long ticks;
  int spin_limit;
  int* flag;          // LDS int used to make results workgroup-uniform
};

__device__ __forceinline__ Ctl make_ctl(const Params& p, int* flag) {
  return Ctl{p.err, p.timeout_ticks, p.spin_limit, flag};
}

// Workgroup-uniform AND of `ok` (every thread passes its own value).
// The flag is set to 1 when the kernel starts and only ever cleared on a
// failure, after which every thread leaves the kernel; one barrier suffices.
__device__ __forceinline__ bool wg_all(bool ok, int* flag) {
  if (!ok) *flag = 0;
  __syncthreads();
  return *flag != 0;
}

constexpr int kGatherPer = 8;    // words per thread per pass (the default width)

// One thread's share of a gather pass: up to NP arena words, their
// expected epochs and LDS destinations, and which of them are still pending.
template <int NP>
struct GatherSlots {
  unsigned pending;
  unsigned pk;                      // slots holding pair words
  unsigned off[NP];
  unsigned want[NP];
  lds_float* dst[NP];               // 32-bit LDS addresses
};

template <int NP, int NR>
__device__ __forceinline__ GatherSlots<NP> gather_slots(const LLRange (&rg)[NR], int total, int seg) {
  GatherSlots<NP> S;
  S.pending = 0;
  S.pk = 0;
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    int i = seg + (int)threadIdx.x + k * kThreads;
    S.off[k] = kOffNone;
    S.want[k] = 0u;
    S.dst[k] = nullptr;
    if (i < total) {
      S.pending |= 1u << k;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (i >= 0 && i < rg[r].n) {
          S.off[k] = (unsigned)(rg[r].src + i) * 8u;
          S.want[k] = rg[r].pk ? pair_tag(rg[r].want) : rg[r].want;
          S.dst[k] = (lds_float*)(rg[r].dst + (rg[r].pk ? 2 * i : i));
          S.pk |= (unsigned)(rg[r].pk != 0) << k;
        }
        i -= rg[r].n;
      }
    }
  }
  return S;
}

template <int NP>
__device__ __forceinline__ void gather_issue(Rsrc arena, const GatherSlots<NP>& S, u32x2 (&v)[NP]) {
#pragma unroll
  for (int k = 0; k < NP; ++k) v[k] = ld_ll(arena, ((S.pending >> k) & 1u) ? S.off[k] : kOffNone);
}

template <int NP>
__device__ __forceinline__ void gather_take(GatherSlots<NP>& S, const u32x2 (&v)[NP]) {
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const bool pk = (S.pk >> k) & 1u;
    if (((S.pending >> k) & 1u) && (pk ? v[k].y >> 16 : v[k].y) == S.want[k]) {
      if (pk) {
        S.dst[k][0] = __uint_as_float(v[k].x << 8);
        S.dst[k][1] = __uint_as_float(((v[k].y & 0xFFFFu) << 16) | ((v[k].x >> 24) << 8));
      } else {
        *S.dst[k] = __uint_as_float(v[k].x);
      }
      S.pending &= ~(1u << k);
    }
  }
}

// Bookkeeping of one poll round: false (with the timeout reported) once the
// wait has passed its time limit or spin limit, or another workgroup has
// reported an error.
__device__ __forceinline__ bool poll_check(const Ctl& c, int& spins, long long& t0) {
  ++spins;
  if ((spins & 15) == 1) {
    if (spins == 1) t0 = wall_clock64();
    if (__hip_atomic_load(c.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return false;
    if (wall_clock64() - t0 > c.ticks) {
      set_timeout(c.err);
      return false;
    }
  }
  if (c.spin_limit > 0 && spins >= c.spin_limit) {
    set_timeout(c.err);
    return false;
  }
  return true;
}

// Polls until every slot is valid; false on timeout or a reported error.
// One poll round per return: a second round in flight, or a longer pause
// between rounds, both measured slower (more poll traffic delays the data's
// own propagation; a pause delays its detection).
template <int NP>
__device__ __forceinline__ bool gather_wait(const Params& p, Rsrc arena, GatherSlots<NP>& S, const Ctl& c) {
  long long t0 = 0;
  int spins = 0;
  while (S.pending) {
    if (!poll_check(c, spins, t0)) return false;
    __builtin_amdgcn_s_sleep(1);
    u32x2 v[NP];
    gather_issue(arena, S, v);
    gather_take(S, v);
  }
  return true;
}

// Copies up to NR ranges of the arena into LDS, waiting until every word
// carries its range's epoch.  Thread t owns words t, t + kThreads, ... of
// the concatenated ranges and re-reads only the ones not yet valid; loads
// are issued for all of them at once.
//
// `issue()` is called once, right after the first poll loads are issued and
// before their results are used: loads it issues (the next weights) queue
// behind the first poll instead of in front of it, so that poll returns at
// the fabric's latency rather than after the prefetch has landed (a wave's
// loads return in issue order).  The first round is written out on its own
// so the compiler sees a single issue order there.  Returns false
// (uniformly) when a wait passes the timeout or another workgroup reported
// an error.
//
// Handing the polling and the prefetch to different waves of the workgroup
// measured slower: the exchange got no faster (the polls still meet the
// streaming traffic beyond the compute unit) and the polling waves started
// their share of the rows late.
template <int NP = kGatherPer, int NR, class Issue>
__device__ __forceinline__ bool ll_gather(const Params& p, const LLRange (&rg)[NR], const Ctl& c,
                                          Issue&& issue) {
  const Rsrc arena = arena_rsrc(p);
  int total = 0;
#pragma unroll
  for (int r = 0; r < NR; ++r) total += rg[r].n;
  GatherSlots<NP> S = gather_slots<NP>(rg, total, 0);
  {
    u32x2 v[NP];
    gather_issue(arena, S, v);
    issue();
    gather_take(S, v);
  }
  bool ok = gather_wait(p, arena, S, c);
  for (int seg = NP * kThreads; seg < total && ok; seg += NP * kThreads) {
    S = gather_slots<NP>(rg, total, seg);
    ok = gather_wait(p, arena, S, c);
  }
  return wg_all(ok, c.flag);
}

template <int NR>
__device__ __forceinline__ bool ll_gather(const Params& p, const LLRange (&rg)[NR], const Ctl& c) {
  return ll_gather(p, rg, c, [] {});
}

// A gather that prefetches the next stage's weights (issue) and the small
// loads needed right after it (early: the norm gains) behind its first poll.
template <int NP = kGatherPer, int NR, class Early, class Issue>
__device__ __forceinline__ bool ll_gather_pf(const Params& p, const LLRange (&rg)[NR], const Ctl& c,
                                             Early&& early, Issue&& issue) {
  return ll_gather<NP>(p, rg, c, [&]() {
    issue();
    early();
  });
}

// ---------------------------------------------------------------------------
// LDS carve-up (floats): [0, hcap) GEMV vector / attention area; part;
// sums; xown (this workgroup's rows of x); a small reduction / routing area.
// ---------------------------------------------------------------------------
struct Lds {
  float* h;
  float* part;
  float* sums;
  float* xown;
  float* red;
};

__device__ __forceinline__ Lds lds_carve(const Params& p, float* smem) {
  const LdsLayout L = lds_layout(p);
  Lds s;
  s.h = smem;
  s.part = smem + L.part_off;
  s.sums = smem + L.sums_off;
  s.xown = smem + L.xown_off;
  s.red = smem + L.red_off;
  return s;
}

// Norm gains are read-only: their loads are issued before the wait for the
// activations, for up to kGainPer * kThreads elements.
constexpr int kGainPer = 8;
struct GainPre {
  unsigned short g[kGainPer];      // raw fp16 bits
};
// Branch-free buffer loads: lanes past d use an out-of-range offset and read
// zero.  A guarded load (or a pointer the compiler cannot prove global)
// becomes a flat load followed by a wait for every outstanding load, which
// would drain the weight prefetch issued just before.
__device__ __forceinline__ GainPre gain_prefetch(const __half* gain, int d) {
  const Rsrc r = make_rsrc(gain, (size_t)d * 2);
  GainPre G;
#pragma unroll
  for (int k = 0; k < kGainPer; ++k) {
    const int i = threadIdx.x + k * kThreads;
    G.g[k] = __builtin_amdgcn_raw_buffer_load_b16(r, i < d ? (unsigned)i * 2u : kOffNone, 0, 0);
  }
  return G;
}

// RMSNorm folded into the GEMV that consumes it: rms(v) * gain = (v * gain)
// / sqrt(mean(v^2) + eps), and the divisor is one scalar, so it scales the
// GEMV's row sums instead of every input.  One pass over h (LDS, in place)
// multiplies by the gain and accumulates the sum of squares of the raw
// values in a fixed order; returns 1 / sqrt(mean(v^2) + eps), the same in
// every thread.
__device__ __forceinline__ float rmsnorm_lds(const Params& p, const __half* gain, const GainPre& G,
                                             float* h, float* red) {
  const int d = p.d;
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kGainPer; ++k) {
    const int i = threadIdx.x + k * kThreads;
    if (i < d) {
      const float v = h[i];
      ss = fmaf(v, v, ss);
      h[i] = v * __half2float(__ushort_as_half(G.g[k]));
    }
  }
  for (int i = threadIdx.x + kGainPer * kThreads; i < d; i += kThreads) {
    const float v = h[i];
    ss = fmaf(v, v, ss);
    h[i] = v * __half2float(gain[i]);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) tot += red[w];
  return 1.0f / sqrtf(tot / (float)d + p.eps);
}

// Appends one clock stamp to the workgroup's trace (traced steps only).
struct Tracer {
  unsigned long long* tr;
  int ev;
};
__device__ __forceinline__ void mark(Tracer& t) {
  if (t.tr != nullptr) {
    if (threadIdx.x == 0 && t.ev < kTraceEvents) t.tr[t.ev] = wall_clock64();
    ++t.ev;
  }
}

// ---------------------------------------------------------------------------
// Row address functors of each GEMV.
// ---------------------------------------------------------------------------
// Layer l's weight pointers, read through the constant address space so
// they are scalar loads into SGPRs (a vector load would leave them in VGPRs,
// and every later use would wait for all loads issued before it).
typedef const __attribute__((address_space(4))) unsigned long long* ConstU64Ptr;
__device__ __forceinline__ LayerPtrs layer(const Params& p, int l) {
  constexpr int kWords = (int)(sizeof(LayerPtrs) / sizeof(unsigned long long));
  const ConstU64Ptr q = (ConstU64Ptr)(p.layers + l);
  unsigned long long v[kWords];
#pragma unroll
  for (int i = 0; i < kWords; ++i) v[i] = q[i];
  return __builtin_bit_cast(LayerPtrs, v);
}

// A wave-uniform address as an opaque uniform value (readfirstlane of both
// halves): keeps it in SGPRs and keeps the optimiser from folding a choice
// between struct members into an indexed load of the struct.
__device__ __forceinline__ unsigned long long uniform_addr(const void* p) {
  const unsigned long long v = (unsigned long long)(uintptr_t)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

// Each GEMV's weights as buffer resources: rsrc(r) is the resource holding
// row r (uniform across the wave), off(r, c) the byte offset of 16-byte
// chunk c of that row.  Every resource spans its whole tensor (< 4 GiB).
struct QkvAddr {             // rows of Wq, then Wk, then Wv
  unsigned long long bq, bk, bv;   // uniform base addresses (SGPRs)
  int qd, kd, d;
  // The matrix is chosen by arithmetic on uniform values, not by branches or
  // selects over the members (either would cost waits or scratch memory).
  __device__ Rsrc rsrc(int r) const {
    const unsigned long long iq = r < qd, ik = (r >= qd) & (r < qd + kd), iv = r >= qd + kd;
    const unsigned long long b = iq * bq + ik * bk + iv * bv;
    return make_rsrc(reinterpret_cast<const void*>(b), (size_t)(iq ? qd : kd) * d * 2);
  }
  __device__ unsigned off(int r, int c) const {
    const int rr = r - (r >= qd) * qd - (r >= qd + kd) * kd;
    return (unsigned)rr * (unsigned)d * 2u + (unsigned)c * 16u;
  }
};
struct RowAddr {             // plain row-major [rows][cols]
  Rsrc w;
  int cols;
  __device__ Rsrc rsrc(int) const { return w; }
  __device__ unsigned off(int r, int c) const {
    return (unsigned)r * (unsigned)cols * 2u + (unsigned)c * 16u;
  }
};
struct PairAddr {            // virtual row 2f = gate row f, 2f+1 = up row f
  unsigned long long bg, bu;       // uniform base addresses
  int rows, cols;
  __device__ Rsrc rsrc(int vr) const {
    const unsigned long long iu = vr & 1;
    return make_rsrc(reinterpret_cast<const void*>((1ull - iu) * bg + iu * bu), (size_t)rows * cols * 2);
  }
  __device__ unsigned off(int vr, int c) const {
    return (unsigned)(vr >> 1) * (unsigned)cols * 2u + (unsigned)c * 16u;
  }
};
struct MoePairAddr {         // virtual row 2f (+1): pair f = (slot f / Fe, row f % Fe)
  unsigned long long bg, bu;       // whole stacked expert tensors [E + S][Fe][d]
  const int* ids;            // LDS: expert id per active slot
  int ne, Fe, d;
  __device__ Rsrc rsrc(int vr) const {
    const unsigned long long iu = vr & 1;
    return make_rsrc(reinterpret_cast<const void*>((1ull - iu) * bg + iu * bu), (size_t)ne * Fe * d * 2);
  }
  __device__ unsigned off(int vr, int c) const {
    const int f = vr >> 1;
    const int a = f / Fe, ff = f - a * Fe;
    return ((unsigned)ids[a] * (unsigned)Fe + (unsigned)ff) * (unsigned)d * 2u + (unsigned)c * 16u;
  }
};
struct MoeSharedPairAddr {   // as MoePairAddr over the shared experts only: pair f = (shared f / Fe, row f % Fe)
  unsigned long long bg, bu;
  int E, ne, Fe, d;
  __device__ Rsrc rsrc(int vr) const {
    const unsigned long long iu = vr & 1;
    return make_rsrc(reinterpret_cast<const void*>((1ull - iu) * bg + iu * bu), (size_t)ne * Fe * d * 2);
  }
  __device__ unsigned off(int vr, int c) const {
    const int f = vr >> 1;
    const int a = f / Fe, ff = f - a * Fe;
    return ((unsigned)(E + a) * (unsigned)Fe + (unsigned)ff) * (unsigned)d * 2u + (unsigned)c * 16u;
  }
};
struct MoeDownAddr {         // row r of the concatenated active experts' down rows
  Rsrc down;                 // whole stacked tensor [E + S][d][Fe]
  const int* ids;
  int Fe, d, cps;            // cps = chunks per expert segment (Fe / 8)
  __device__ Rsrc rsrc(int) const { return down; }
  __device__ unsigned off(int r, int c) const {
    const int a = c / cps, o = c - a * cps;
    return (((unsigned)ids[a] * (unsigned)d + (unsigned)r) * (unsigned)Fe) * 2u + (unsigned)o * 16u;
  }
};

__device__ __forceinline__ Rsrc mat_rsrc(const __half* w, int rows, int cols) {
  return make_rsrc(w, (size_t)rows * cols * 2);
}

// ---------------------------------------------------------------------------
// Stage: RMSNorm + fused Q/K/V GEMV (rows of Wq, Wk, Wv as one row space).
// Layer 0 normalises the embedding row; later layers wait for x of the
// previous layer's down projection.
// ---------------------------------------------------------------------------
__device__ __forceinline__ GemvWork qkv_work(const Params& p, int wg) {
  return gemv_work(p.H * p.hd + 2 * p.nkv * p.hd, p.d, p.n_wg, wg, 1);
}
__device__ __forceinline__ QkvAddr qkv_addr(const Params& p, int l) {
  const LayerPtrs w = layer(p, l);
  const int qd = p.H * p.hd, kd = p.nkv * p.hd;
  return QkvAddr{uniform_addr(w.wq), uniform_addr(w.wk), uniform_addr(w.wv), qd, kd, p.d};
}
// Every stage first issues the first loads of its own weight rows (or KV
// rows), then waits for its inputs: the loads stream while the workgroup
// waits.  The issued batches stay in registers local to the stage.
//
// At layer 0 the input is the embedding row of the step's token; `resolve`
// yields that token after the optional grid barrier `gs` (the previous
// step's argmax, or prefill ordering) and is called by every workgroup.
template <class Resolve>
__device__ __forceinline__ bool stage_qkv(const Params& p, int step, int l, int wg, Lds s,
                                          const Ctl& c, Tracer& tr, GridSync& gs, bool wait_first,
                                          int& tok, Resolve&& resolve) {
  const GemvWork g = qkv_work(p, wg);
  const QkvAddr addr = qkv_addr(p, l);
  const __half* gain = layer(p, l).attn_norm;
  WPre pre;
  GainPre G;
  auto gains = [&]() { G = gain_prefetch(gain, p.d); };
  auto weights = [&]() { pre = gemv_prefetch(g, addr); };
  // Layer 0 waits for the grid barrier or reads the embedding: prefetch
  // first.  Later layers prefetch behind the first poll of x.
  if (l == 0) {
    weights();
    gains();
  }
  if (wait_first) {
    if (!grid_wait(gs, c.flag)) return false;
    tok = resolve();
  }
  if (l == 0) {
    if (g.r0 < g.r1) {
      const __half* emb_row = p.tok_emb + (size_t)tok * p.d;
      for (int i = threadIdx.x; i < p.d; i += kThreads) s.h[i] = __half2float(emb_row[i]);
    }
  } else if (g.r0 < g.r1) {
    const LLRange rg[1] = {{p.off_xh, p.d / 2, s.h, ll_flag(p, step, l - 1, kSlotXDown), 1}};
    if (!ll_gather_pf(p, rg, c, gains, weights)) return false;
  }
  mark(tr);
  if (g.r0 >= g.r1) {
    mark(tr);
    return true;
  }
  const float inv = rmsnorm_lds(p, gain, G, s.h, s.red);
  mark(tr);
  const unsigned f = ll_flag(p, step, l, kSlotQkv);
  gemv_run<true>(g, addr, s.h, s.part, s.sums, pre,
                 [&](int b0, int n, const float* sums) {
                   for (int i = threadIdx.x; i < n; i += kThreads)
                     ll_put(p, p.off_qkv + b0 + i, sums[i] * inv, f);
                 });
  return true;
}

// ---------------------------------------------------------------------------
// Stage: RoPE + fp16 KV append + split-K flash-decode attention.
//
// Work unit = (KV head g, split s): the G query heads that share KV head g
// against positions [p0, p1) of the cache.  16 lanes own one position (8
// fp16 of the head dimension each), so a wave covers 4 positions per step
// and keeps an online-softmax state (max, sum, 8 accumulators per head) per
// 16-lane group; states are merged across groups, then waves, in a fixed
// order.  The split containing the current position rotates the new key,
// rounds K and V to fp16, appends them to the cache and uses the rounded
// values.  With one split per head the unit writes o directly; otherwise
// each split publishes its (acc, m, l) partial and split h of each head
// group merges query head h's partials in split order into o.  Scores carry log2(e)/sqrt(hd)
// so exp2 is the softmax exponential.
// ---------------------------------------------------------------------------
constexpr int kAttnStride = kWaves * 4;     // positions per workgroup per step
constexpr int kAU = 4;                      // steps in flight

struct KVPre {
  u32x4 k[kAU], v[kAU];
};

struct AttnUnit {
  int g, sidx, p0, pend;
  bool has_new, active;
};

// Splits per KV head at position pos: one per kSplitPositions cached
// positions (the depth of the cache prefetch, so a split's rows are all in
// flight before its inputs arrive), at most p.splits (the grid divided by
// the KV heads, which also sizes the partial buffers).  Fewer splits make
// the merge cheaper: its workgroup gathers every split's partial, and at
// short contexts a full grid of splits would hold a few positions each.
constexpr int kSplitPositions = kAU * kAttnStride;
__device__ __forceinline__ int attn_splits(const Params& p, int pos) {
  const int s = (pos + kSplitPositions) / kSplitPositions;     // ceil((pos + 1) / kSplitPositions)
  return s < p.splits ? s : p.splits;
}

__device__ __forceinline__ AttnUnit attn_unit_of(const Params& p, int pos, int unit) {
  AttnUnit u;
  const int S = attn_splits(p, pos);
  const int units = p.nkv * S;
  u.active = unit < units;
  u.g = u.active ? unit / S : 0;
  u.sidx = u.active ? unit % S : 0;
  const int n = pos + 1;
  u.p0 = split_begin(u.sidx, n, S);
  const int p1 = split_begin(u.sidx + 1, n, S);
  u.has_new = (p1 == n);
  u.pend = u.has_new ? pos : p1;               // cached positions [p0, pend)
  return u;
}

__device__ __forceinline__ void kv_load_step(const Params& p, Rsrc rk, Rsrc rv, int base, int pend,
                                             u32x4 (&k)[kAU], u32x4 (&v)[kAU]) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int grp = lane >> 4, sub = lane & 15;
  const bool lane_on = sub < (p.hd >> 3);
  const unsigned row_bytes = (unsigned)p.hd * 2u;
#pragma unroll
  for (int u = 0; u < kAU; ++u) {
    const int j = base + u * kAttnStride + wave * 4 + grp;
    const unsigned off = (lane_on && j < pend) ? (unsigned)j * row_bytes + (unsigned)sub * 16u : kOffNone;
    k[u] = ld_kv16(rk, off);
    v[u] = ld_kv16(rv, off);
  }
}

__device__ __forceinline__ size_t kv_head_base(const Params& p, int l, int g) {
  return ((size_t)l * p.nkv + g) * (size_t)p.cap * p.hd;
}

__device__ __forceinline__ KVPre prefetch_attn(const Params& p, int l, int pos, int wg) {
  const AttnUnit u = attn_unit_of(p, pos, wg);
  const unsigned bytes = (unsigned)((size_t)p.cap * p.hd * 2);
  const size_t hb = kv_head_base(p, l, u.g);
  const int pend = u.active ? u.pend : u.p0;
  KVPre P;
  kv_load_step(p, make_rsrc(p.kc + hb, bytes), make_rsrc(p.vc + hb, bytes), u.p0, pend, P.k, P.v);
  return P;
}

// LDS areas of an attention unit (floats, all inside [0, hcap)).
struct AttnLds {
  float *qs, *kn, *vn, *wst, *parts;
};
template <int G>
__device__ __forceinline__ AttnLds attn_lds(const Params& p, float* lds) {
  const int hd = p.hd;
  AttnLds a;
  a.qs = lds;                                  // [G][hd]
  a.kn = a.qs + G * hd;                        // [hd]
  a.vn = a.kn + hd;                            // [hd]
  a.wst = a.vn + hd;                           // [kWaves][G][hd + 2]
  a.parts = a.wst + kWaves * G * (hd + 2);     // [S][G][hd + 2] (merging split only)
  return a;
}

// Arena word of split s's partial for query head (g*G + h), element i.
// The partials of one query head are contiguous: [H][splits][hd + 2].
__device__ __forceinline__ int part_word(const Params& p, int g, int G, int s, int h, int i) {
  return p.off_part + (((g * G + h) * p.splits + s) * (p.hd + 2)) + i;
}

// Merges, in split order, the S partials of the query heads h0, h0 + hs, ...
// (< G) of head group g (in LDS, [head][S][hd+2]) and publishes their o.
template <int G>
__device__ __forceinline__ void attn_merge(const Params& p, int step, int l, int g, int S, int h0,
                                           int hs, const float* parts) {
  const int hd = p.hd, ws = hd + 2;
  const int nh = (G - h0 + hs - 1) / hs;
  const unsigned fo = ll_flag(p, step, l, kSlotO);
  for (int t = threadIdx.x; 2 * t < nh * hd; t += kThreads) {     // elements i, i + 1 of head j
    const int j = (2 * t) / hd, i = (2 * t) % hd;
    const float* hp = parts + j * S * ws;
    // split order throughout; loads are issued ahead of the dependent
    // max / multiply-add chains (four, then two splits at a time)
    float M = kNegBig;
    int s = 0;
    for (; s + 4 <= S; s += 4) {
      const float m0 = hp[s * ws + hd], m1 = hp[(s + 1) * ws + hd];
      const float m2 = hp[(s + 2) * ws + hd], m3 = hp[(s + 3) * ws + hd];
      M = fmaxf(M, m0);
      M = fmaxf(M, m1);
      M = fmaxf(M, m2);
      M = fmaxf(M, m3);
    }
    for (; s < S; ++s) M = fmaxf(M, hp[s * ws + hd]);
    float Ls = 0.f, A0 = 0.f, A1 = 0.f;
    for (s = 0; s + 2 <= S; s += 2) {
      const float* st = hp + s * ws;
      const float* su = st + ws;
      const float m0 = st[hd], l0 = st[hd + 1], x0 = st[i], y0 = st[i + 1];
      const float m1 = su[hd], l1 = su[hd + 1], x1 = su[i], y1 = su[i + 1];
      const float sc0 = exp2f(m0 - M), sc1 = exp2f(m1 - M);
      Ls = fmaf(l0, sc0, Ls);
      A0 = fmaf(x0, sc0, A0);
      A1 = fmaf(y0, sc0, A1);
      Ls = fmaf(l1, sc1, Ls);
      A0 = fmaf(x1, sc1, A0);
      A1 = fmaf(y1, sc1, A1);
    }
    for (; s < S; ++s) {
      const float* st = hp + s * ws;
      const float sc = exp2f(st[hd] - M);
      Ls = fmaf(st[hd + 1], sc, Ls);
      A0 = fmaf(st[i], sc, A0);
      A1 = fmaf(st[i + 1], sc, A1);
    }
    ll_put2(p, p.off_o + ((g * G + h0 + j * hs) * hd + i) / 2, A0 / Ls, A1 / Ls, fo);
  }
}

// Gathers the partials of query heads h0, h0 + hs, ... of head group g and
// merges them.  In the persistent kernel split s merges the heads h with
// h mod S == s, so a group's G heads are merged by up to G workgroups, each
// reading only its heads' partials; the staged mode's merge kernel gives
// every query head its own workgroup.
template <int G>
__device__ __forceinline__ bool attn_gather_merge(const Params& p, int step, int l, int g, int S,
                                                  int h0, int hs, float* lds, const Ctl& c) {
  const AttnLds a = attn_lds<G>(p, lds);
  const int ws = p.hd + 2;
  const unsigned want = ll_flag(p, step, l, kSlotPart);
  LLRange rg[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int h = h0 + j * hs;
    const bool on = h < G;
    rg[j] = LLRange{part_word(p, g, G, 0, on ? h : 0, 0), on ? S * ws : 0, a.parts + j * S * ws, want};
  }
  if (!ll_gather(p, rg, c)) return false;
  attn_merge<G>(p, step, l, g, S, h0, hs, a.parts);
  return true;
}

// The end of an attention unit, once every wave has written its online-
// softmax state (acc, m, l per query head) to a.wst: merges the waves in
// order and publishes this split's partial (or o itself when S == 1); the
// merging splits then gather and merge their heads.
template <int G, bool kMerge>
__device__ __forceinline__ bool attn_finish(const Params& p, int step, int l, int g, int S, int sidx,
                                            float* lds, const Ctl& c) {
  const int hd = p.hd, ws = hd + 2;
  const AttnLds a = attn_lds<G>(p, lds);
  __syncthreads();
  const unsigned fp = ll_flag(p, step, l, kSlotPart);
  const unsigned fo = ll_flag(p, step, l, kSlotO);
  for (int t = threadIdx.x; 2 * t < G * hd; t += kThreads) {      // elements i, i + 1 of head h
    const int h = (2 * t) / hd, i = (2 * t) % hd;
    float M = kNegBig;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, a.wst[(w * G + h) * ws + hd]);
    float Ls = 0.f, A0 = 0.f, A1 = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      const float* st = a.wst + (w * G + h) * ws;
      const float sc = exp2f(st[hd] - M);
      Ls = fmaf(st[hd + 1], sc, Ls);
      A0 = fmaf(st[i], sc, A0);
      A1 = fmaf(st[i + 1], sc, A1);
    }
    if (S == 1) {
      ll_put2(p, p.off_o + ((g * G + h) * hd + i) / 2, A0 / Ls, A1 / Ls, fo);
    } else {
      ll_put(p, part_word(p, g, G, sidx, h, i), A0, fp);
      ll_put(p, part_word(p, g, G, sidx, h, i + 1), A1, fp);
      if (i == 0) {
        ll_put(p, part_word(p, g, G, sidx, h, hd), M, fp);
        ll_put(p, part_word(p, g, G, sidx, h, hd + 1), Ls, fp);
      }
    }
  }
  if (kMerge && S > 1 && sidx < G) {
    __syncthreads();
    return attn_gather_merge<G>(p, step, l, g, S, sidx, S, lds, c);
  }
  return true;
}

// The start of an attention unit: gathers the raw q of the G heads (and
// the new k, v for the split holding pos), rotates q (scaled by
// log2(e)/sqrt(hd)) into a.qs, rounds the rotated new k and v to fp16 into
// a.kn / a.vn and appends them to the cache.  Marks the trace after the
// gather and at the end.
template <int G, class Issue>
__device__ __forceinline__ bool attn_prologue(const Params& p, int step, int l, int pos, int g, size_t hb,
                                              bool has_new, const AttnLds& a, const Ctl& c, Tracer& tr,
                                              Issue&& issue) {
  const int hd = p.hd, half = hd >> 1;
  const int qd = p.H * hd, kd = p.nkv * hd;
  // raw q of the G heads (and the new k, v for the split holding pos)
  {
    const unsigned fq = ll_flag(p, step, l, kSlotQkv);
    const LLRange rg[3] = {{p.off_qkv + g * G * hd, G * hd, a.qs, fq},
                           {p.off_qkv + qd + g * hd, has_new ? hd : 0, a.kn, fq},
                           {p.off_qkv + qd + kd + g * hd, has_new ? hd : 0, a.vn, fq}};
    if (!ll_gather(p, rg, c, issue)) return false;
  }
  mark(tr);

  const float* cs = p.rope_cos + (size_t)pos * half;
  const float* sn = p.rope_sin + (size_t)pos * half;
  const float qscale = kLog2e / sqrtf((float)hd);
  // rotate-half RoPE; every thread computes its elements from the raw values
  // before any is overwritten
  float qrot[(kMaxGroup * kMaxHeadDim + kThreads - 1) / kThreads];
#pragma unroll
  for (int k = 0; k < (kMaxGroup * kMaxHeadDim + kThreads - 1) / kThreads; ++k) {
    const int i = threadIdx.x + k * kThreads;
    qrot[k] = 0.f;
    if (i < G * hd) {
      const int h = i / hd, j = i % hd;
      const float* q = a.qs + h * hd;
      const int jj = j < half ? j : j - half;
      const float cc = cs[jj], sv = sn[jj];
      qrot[k] = (j < half ? q[j] * cc - q[j + half] * sv : q[j] * cc + q[j - half] * sv) * qscale;
    }
  }
  float krot = 0.f, vval = 0.f;
  if (has_new && threadIdx.x < hd) {
    const int j = threadIdx.x;
    const int jj = j < half ? j : j - half;
    const float cc = cs[jj], sv = sn[jj];
    krot = j < half ? a.kn[j] * cc - a.kn[j + half] * sv : a.kn[j] * cc + a.kn[j - half] * sv;
    vval = a.vn[j];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < (kMaxGroup * kMaxHeadDim + kThreads - 1) / kThreads; ++k) {
    const int i = threadIdx.x + k * kThreads;
    if (i < G * hd) a.qs[i] = qrot[k];
  }
  if (has_new && threadIdx.x < hd) {
    // round to fp16 (RNE), use the rounded values, append them to the cache
    const int j = threadIdx.x;
    const __half kh = __float2half_rn(krot);
    const __half vh = __float2half_rn(vval);
    a.kn[j] = __half2float(kh);
    a.vn[j] = __half2float(vh);
    // lanes j, j+1 pair up into one 32-bit device-scope store per row
    const unsigned kbits = (unsigned)__half_as_ushort(kh), vbits = (unsigned)__half_as_ushort(vh);
    const unsigned kpart = (unsigned)__shfl_xor((int)kbits, 1, 64);
    const unsigned vpart = (unsigned)__shfl_xor((int)vbits, 1, 64);
    if ((j & 1) == 0) {
      unsigned* kc32 = reinterpret_cast<unsigned*>(p.kc + hb + (size_t)pos * hd);
      unsigned* vc32 = reinterpret_cast<unsigned*>(p.vc + hb + (size_t)pos * hd);
      st_cu(kc32 + (j >> 1), kbits | (kpart << 16));
      st_cu(vc32 + (j >> 1), vbits | (vpart << 16));
    }
  }
  __syncthreads();
  mark(tr);
  return true;
}

template <int G, bool kPre, bool kMerge>
__device__ __forceinline__ bool attn_unit(const Params& p, int step, int l, int pos, const AttnUnit& U,
                                          float* lds, KVPre pre, const Ctl& c, Tracer& tr) {
  const int hd = p.hd, half = hd >> 1, S = attn_splits(p, pos);
  const int qd = p.H * hd, kd = p.nkv * hd;
  const int g = U.g, sidx = U.sidx, p0 = U.p0, pend = U.pend;
  const bool has_new = U.has_new;
  const AttnLds a = attn_lds<G>(p, lds);

  const size_t hb = kv_head_base(p, l, g);
  const unsigned bytes = (unsigned)((size_t)p.cap * hd * 2);
  const Rsrc rk = make_rsrc(p.kc + hb, bytes);
  const Rsrc rv = make_rsrc(p.vc + hb, bytes);

  // first step of cache rows: prefetched before the wait, or now
  u32x4 kr[kAU], vr[kAU];
  if (kPre) {
#pragma unroll
    for (int u = 0; u < kAU; ++u) {
      kr[u] = pre.k[u];
      vr[u] = pre.v[u];
    }
  } else {
    kv_load_step(p, rk, rv, p0, pend, kr, vr);
  }

  if (!attn_prologue<G>(p, step, l, pos, g, hb, has_new, a, c, tr, [] {})) return false;

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int grp = lane >> 4, sub = lane & 15;
  const int nsub = hd >> 3;
  const bool lane_on = sub < nsub;

  float qr[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[h][e] = lane_on ? a.qs[h * hd + sub * 8 + e] : 0.f;

  float m[G], lsum[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  auto consume = [&](const float (&kf)[8], const float (&vf)[8]) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float sc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sc = fmaf(qr[h][e], kf[e], sc);
      sc = group16_sum(sc);
      const float mn = fmaxf(m[h], sc);
      const float corr = exp2f(m[h] - mn);
      const float pw = exp2f(sc - mn);
      lsum[h] = lsum[h] * corr + pw;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(acc[h][e], corr, pw * vf[e]);
      m[h] = mn;
    }
  };

  // The kAU positions a 16-lane group holds per block are folded into the
  // online softmax together: their scores are independent chains, then one
  // new maximum and one rescale of the accumulators.  Positions past pend
  // (zero K/V rows) get weight exactly zero.  Same arithmetic as one position
  // at a time, in a different fixed order.
  auto consume_block = [&](const u32x4 (&kb)[kAU], const u32x4 (&vb)[kAU], const bool (&ok)[kAU]) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float sc[kAU];
#pragma unroll
      for (int u = 0; u < kAU; ++u) {
        float kf[8];
        unpack8(kb[u], kf);
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(qr[h][e], kf[e], d);
        sc[u] = d;
      }
#pragma unroll
      for (int u = 0; u < kAU; ++u) sc[u] = group16_sum(sc[u]);
      float mn = m[h];
#pragma unroll
      for (int u = 0; u < kAU; ++u) mn = ok[u] ? fmaxf(mn, sc[u]) : mn;
      const float corr = exp2f(m[h] - mn);
      float pw[kAU];
#pragma unroll
      for (int u = 0; u < kAU; ++u) pw[u] = ok[u] ? exp2f(sc[u] - mn) : 0.f;
      float ls = lsum[h] * corr;
#pragma unroll
      for (int u = 0; u < kAU; ++u) ls += pw[u];
      lsum[h] = ls;
      float av[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) av[e] = acc[h][e] * corr;
#pragma unroll
      for (int u = 0; u < kAU; ++u) {
        float vf[8];
        unpack8(vb[u], vf);
#pragma unroll
        for (int e = 0; e < 8; ++e) av[e] = fmaf(pw[u], vf[e], av[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = av[e];
      m[h] = mn;
    }
  };

  for (int base = p0; base < pend; base += kAttnStride * kAU) {
    if (base != p0) kv_load_step(p, rk, rv, base, pend, kr, vr);
    // a 16-lane group is wholly in or out, and its sums stay in the group
    bool ok[kAU];
#pragma unroll
    for (int u = 0; u < kAU; ++u) ok[u] = base + u * kAttnStride + wave * 4 + grp < pend;
    consume_block(kr, vr, ok);
  }
  if (has_new && wave == 0 && grp == 0) {
    float kf[8], vf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kf[e] = lane_on ? a.kn[sub * 8 + e] : 0.f;
      vf[e] = lane_on ? a.vn[sub * 8 + e] : 0.f;
    }
    // only lanes 0..15 take part: the 16-lane sum stays inside the group
    consume(kf, vf);
  }

  // merge the four 16-lane groups of the wave (xor 16, then xor 32)
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], o, 64);
      const float lo = __shfl_xor(lsum[h], o, 64);
      const float mn = fmaxf(m[h], mo);
      const float e0 = exp2f(m[h] - mn), e1 = exp2f(mo - mn);
      lsum[h] = lsum[h] * e0 + lo * e1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ao = __shfl_xor(acc[h][e], o, 64);
        acc[h][e] = acc[h][e] * e0 + ao * e1;
      }
      m[h] = mn;
    }
  }
  const int ws = hd + 2;
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* st = a.wst + (wave * G + h) * ws;
      if (lane_on)
#pragma unroll
        for (int e = 0; e < 8; ++e) st[sub * 8 + e] = acc[h][e];
      if (sub == 0) {
        st[hd] = m[h];
        st[hd + 1] = lsum[h];
      }
    }
  }
  return attn_finish<G, kMerge>(p, step, l, g, S, sidx, lds, c);
}

// ---- Matrix-core flash-decode unit (G >= 2 query heads per KV head, hd a
// multiple of 16 up to 80).  With G heads sharing every cached row the vector form
// spends most of its time on per-head dot products and lane reductions; here
// a wave takes 32 cached positions (a tile) at a time and both products run
// on v_mfma_f32_32x32x16_f16:
//   scores: rows = the G query heads (zero beyond G), columns = positions,
//           16 dimensions per step; q is split into fp16 high and low parts
//           (K is exact in fp16), so the product is fp32 up to rounding order;
//   output: rows = heads, columns = 32 dimensions per column tile, 16
//           positions per step, with P split high/low and V staged transposed
//           in the wave's own LDS tile.
// Lane l holds position l & 31 of the tile (dimensions 16 s + 8 (l >> 5) ..
// + 7 of step s) for the score product, and its lanes 0..31 hold the G
// scores of one position each, so the online softmax is a reduction across
// the wave.  Each wave keeps its own (acc, m, l) per head; attn_finish merges
// the waves as for the vector form.
typedef _Float16 mh8 __attribute__((ext_vector_type(8)));
typedef float mf16 __attribute__((ext_vector_type(16)));
constexpr int kMT = 32;                      // positions per tile
constexpr int kMTS = kMT + 8;                // LDS row stride (halves): transposed V, P
constexpr int kMaxNS = 5;                    // 16-wide steps of the score product: hd <= 80
constexpr int kMaxCT = (kMaxNS + 1) / 2;     // 32-wide column tiles of the output
// (a wider head keeps the vector form: its K/V fragments and accumulators
// would not fit the register budget)

__device__ __forceinline__ int mfma_cols(int hd) { return 32 * ((hd / 16 + 1) / 2); }

struct MfmaPre {
  u32x4 k[kMaxNS];
};

// Above the wave states (and over the merging split's partial buffer, which
// is used only once the tiles are done): q high/low [G][hd], each wave's
// transposed V tile [cols][kMTS] and P high/low [G][kMTS] (halves).
struct MfmaLds {
  _Float16 *qh, *ql, *vt, *ph, *pl;
};
template <int G>
__device__ __forceinline__ MfmaLds mfma_lds(const Params& p, const AttnLds& a) {
  const int hd = p.hd;
  const int base = (kWaves * G * (p.hd + 2) + 3) & ~3;        // floats past a.wst, 16-byte aligned
  MfmaLds m;
  m.qh = reinterpret_cast<_Float16*>(a.wst + base);
  m.ql = m.qh + G * hd;
  m.vt = m.ql + G * hd;
  m.ph = m.vt + kWaves * mfma_cols(hd) * kMTS;
  m.pl = m.ph + kWaves * G * kMTS;
  return m;
}

// The LDS writes of the calling wave are complete and visible to all its
// lanes (a wave-scope release/acquire around the wave barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int kCtrl, int kRows>
__device__ __forceinline__ float dpp_max(float v) {
  const int moved = __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, kNegBig), __builtin_bit_cast(int, v),
                                                kCtrl, kRows, 0xF, false);
  return fmaxf(v, __builtin_bit_cast(float, moved));
}
// Maximum over the wave, returned uniformly: DPP steps in the order of
// wave_sum (lanes outside a step's rows see kNegBig).  Cross-lane shuffles
// through the LDS crossbar measured 2% slower on the long-context decode.
__device__ __forceinline__ float wave_max(float v) {
  v = dpp_max<kDppXor1, 0xF>(v);
  v = dpp_max<kDppXor2, 0xF>(v);
  v = dpp_max<kDppHalfMirror, 0xF>(v);
  v = dpp_max<kDppMirror, 0xF>(v);
  v = dpp_max<kDppBcast15, 0xA>(v);
  v = dpp_max<kDppBcast31, 0xC>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// K (or V) rows of the tile starting at position kbase in the score
// product's layout; positions at or past pend read zeros.
__device__ __forceinline__ void mfma_rows_load(const Params& p, Rsrc r, int kbase, int pend,
                                               u32x4 (&k)[kMaxNS]) {
  const int lane = threadIdx.x & 63;
  const int j = kbase + (lane & 31), kin = 8 * (lane >> 5), NS = p.hd >> 4;
  const unsigned row = (unsigned)j * (unsigned)p.hd * 2u;
#pragma unroll
  for (int s = 0; s < kMaxNS; ++s)
    k[s] = ld_kv16(r, (s < NS && j < pend) ? row + (unsigned)(16 * s + kin) * 2u : kOffNone);
}

__device__ __forceinline__ u32x4 pack_h8(const float* f) {
  mh8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (_Float16)f[i];
  return __builtin_bit_cast(u32x4, h);
}

template <int G, bool kPre, bool kMerge>
__device__ __forceinline__ bool attn_unit_mfma(const Params& p, int step, int l, int pos, const AttnUnit& U,
                                               float* lds, const MfmaPre& pre, const Ctl& c, Tracer& tr) {
  const int hd = p.hd, S = attn_splits(p, pos), NS = hd >> 4, NCT = (NS + 1) >> 1, cols = mfma_cols(hd);
  const int g = U.g, sidx = U.sidx, p0 = U.p0, pend = U.pend;
  const bool has_new = U.has_new;
  const int kend = has_new ? pos + 1 : pend;          // this unit's positions: [p0, kend)
  const AttnLds a = attn_lds<G>(p, lds);
  const MfmaLds ml = mfma_lds<G>(p, a);
  const size_t hb = kv_head_base(p, l, g);
  const unsigned bytes = (unsigned)((size_t)p.cap * hd * 2);
  const Rsrc rk = make_rsrc(p.kc + hb, bytes);
  const Rsrc rv = make_rsrc(p.vc + hb, bytes);
  const int lane = threadIdx.x & 63, wave = wave_id(), l32 = lane & 31, kin = 8 * (lane >> 5);

  // K of the wave's first tile: prefetched before the wait, or now
  u32x4 kt[kMaxNS], vt[kMaxNS];
  if (kPre) {
#pragma unroll
    for (int s = 0; s < kMaxNS; ++s) kt[s] = pre.k[s];
  } else {
    mfma_rows_load(p, rk, p0 + kMT * wave, pend, kt);
  }
  // (V is loaded per tile once q has arrived: loads in flight during the
  // wait delay the polls behind them)
  if (!attn_prologue<G>(p, step, l, pos, g, hb, has_new, a, c, tr, [] {})) return false;

  // q as fp16 high and low parts; the padded columns of this wave's V tile
  for (int i = threadIdx.x; i < G * hd; i += kThreads) {
    const float v = a.qs[i];
    const _Float16 hi = (_Float16)v;
    ml.qh[i] = hi;
    ml.ql[i] = (_Float16)(v - (float)hi);
  }
  _Float16* vtw = ml.vt + wave * cols * kMTS;
  _Float16* phw = ml.ph + wave * G * kMTS;
  _Float16* plw = ml.pl + wave * G * kMTS;
  for (int e = lane; e < (cols - hd) * kMTS; e += 64) vtw[hd * kMTS + e] = (_Float16)0.f;
  __syncthreads();

  float m[G], ls[G];
  mf16 acc[kMaxCT];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    ls[h] = 0.f;
  }
#pragma unroll
  for (int ct = 0; ct < kMaxCT; ++ct) acc[ct] = (mf16){};
  const int ntiles = (kend - p0 + kMT - 1) / kMT;
  // per-lane LDS bases; every access below adds a constant offset
  const int qrow = l32 < G ? l32 : 0;                 // lanes past the heads read a valid row, then zero it
  const _Float16* qhr = ml.qh + qrow * hd + kin;      // q fragments
  const _Float16* qlr = ml.ql + qrow * hd + kin;
  _Float16* vw = vtw + kin * kMTS + l32;              // V transpose: this lane's position column
  const _Float16* vr = vtw + l32 * kMTS + kin;        // V fragments: dimension row l32 (+ 32 ct)
  _Float16* pwh = phw + l32;                          // P of this lane's position
  _Float16* pwl = plw + l32;
  const _Float16* prh = phw + qrow * kMTS + kin;      // P fragments: head row
  const _Float16* prl = plw + qrow * kMTS + kin;
  for (int t = wave; t < ntiles; t += kWaves) {
    const int kbase = p0 + kMT * t;
    if (t != wave) mfma_rows_load(p, rk, kbase, pend, kt);
    mfma_rows_load(p, rv, kbase, pend, vt);
    const int j = kbase + l32;
    const bool is_new = has_new && j == pos;            // the new position: its rounded rows from LDS
    if (is_new) {
#pragma unroll
      for (int s = 0; s < kMaxNS; ++s)
        if (s < NS) kt[s] = pack_h8(a.kn + 16 * s + kin);
    }
    // scores of the G heads against the tile's positions
    mf16 sa = (mf16){};
#pragma unroll
    for (int s = 0; s < kMaxNS; ++s) {
      if (s < NS) {
        mh8 ah = *reinterpret_cast<const mh8*>(qhr + 16 * s);
        mh8 al = *reinterpret_cast<const mh8*>(qlr + 16 * s);
        if (l32 >= G) {
          ah = (mh8){};
          al = (mh8){};
        }
        const mh8 b = __builtin_bit_cast(mh8, kt[s]);
        sa = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, b, sa, 0, 0, 0);
        sa = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, b, sa, 0, 0, 0);
      }
    }
    // online softmax: lanes 0..31 hold position j's score of head h in sa[h]
    const bool valid = lane < 32 && j < kend;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float sc = valid ? sa[h] : kNegBig;
      const float mn = fmaxf(m[h], wave_max(sc));
      const float corr = exp2f(m[h] - mn);
      const float pw = valid ? exp2f(sc - mn) : 0.f;
      ls[h] = ls[h] * corr + wave_sum(pw);
      m[h] = mn;
#pragma unroll
      for (int ct = 0; ct < kMaxCT; ++ct) acc[ct][h] *= corr;
      if (lane < 32) {
        const _Float16 hi = (_Float16)pw;
        pwh[h * kMTS] = hi;
        pwl[h * kMTS] = (_Float16)(pw - (float)hi);
      }
    }
    // V into the wave's LDS tile, transposed: [dimension][position]
    if (is_new) {
#pragma unroll
      for (int s = 0; s < kMaxNS; ++s)
        if (s < NS) vt[s] = pack_h8(a.vn + 16 * s + kin);
    }
#pragma unroll
    for (int s = 0; s < kMaxNS; ++s) {
      if (s < NS) {
        const mh8 vh = __builtin_bit_cast(mh8, vt[s]);
#pragma unroll
        for (int i = 0; i < 8; ++i) vw[(16 * s + i) * kMTS] = vh[i];
      }
    }
    wave_sync();                                       // the V tile and P are the wave's own
#pragma unroll
    for (int kk = 0; kk < kMT; kk += 16) {
      mh8 ah = *reinterpret_cast<const mh8*>(prh + kk);
      mh8 al = *reinterpret_cast<const mh8*>(prl + kk);
      if (l32 >= G) {
        ah = (mh8){};
        al = (mh8){};
      }
#pragma unroll
      for (int ct = 0; ct < kMaxCT; ++ct) {
        if (ct < NCT) {
          const mh8 b = *reinterpret_cast<const mh8*>(vr + 32 * ct * kMTS + kk);
          acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, b, acc[ct], 0, 0, 0);
          acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, b, acc[ct], 0, 0, 0);
        }
      }
    }
    wave_sync();                                       // reads done before the next tile's writes
  }
  // the wave's state: lanes 0..31 hold dimension 32 ct + l32 of head h in acc[ct][h]
  const int ws = hd + 2;
  if (lane < 32) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* st = a.wst + (wave * G + h) * ws;
#pragma unroll
      for (int ct = 0; ct < kMaxCT; ++ct) {
        const int d = 32 * ct + l32;
        if (ct < NCT && d < hd) st[d] = acc[ct][h];
      }
      if (lane == 0) {
        st[hd] = m[h];
        st[hd + 1] = ls[h];
      }
    }
  }
  return attn_finish<G, kMerge>(p, step, l, g, S, sidx, lds, c);
}

// Units wg, wg + n_wg, ... of this workgroup (one unit unless the grid is
// smaller than the number of KV heads, in which case there is one split per
// head and no merge); `pre` holds the first unit's first cache rows.
template <int G, bool kMerge>
__device__ __forceinline__ bool stage_attn(const Params& p, int step, int l, int pos, int wg, Lds s,
                                           const Ctl& c, Tracer& tr) {
  const int units = p.nkv * attn_splits(p, pos);
  if (wg >= units) {
    mark(tr);
    mark(tr);
    return true;
  }
  if constexpr (G >= 2) {
    if ((p.hd & 15) == 0 && p.hd <= 16 * kMaxNS) {
      const AttnUnit u0 = attn_unit_of(p, pos, wg);
      const size_t hb = kv_head_base(p, l, u0.g);
      const unsigned bytes = (unsigned)((size_t)p.cap * p.hd * 2);
      MfmaPre mp;
      mfma_rows_load(p, make_rsrc(p.kc + hb, bytes), u0.p0 + kMT * wave_id(), u0.pend, mp.k);
      if (!attn_unit_mfma<G, true, kMerge>(p, step, l, pos, u0, s.h, mp, c, tr)) return false;
      __syncthreads();
      for (int u = wg + p.n_wg; u < units; u += p.n_wg) {
        Tracer none{nullptr, 0};
        if (!attn_unit_mfma<G, false, kMerge>(p, step, l, pos, attn_unit_of(p, pos, u), s.h, MfmaPre{}, c,
                                              none))
          return false;
        __syncthreads();
      }
      return true;
    }
  }
  const KVPre pre = prefetch_attn(p, l, pos, wg);
  if (!attn_unit<G, true, kMerge>(p, step, l, pos, attn_unit_of(p, pos, wg), s.h, pre, c, tr))
    return false;
  __syncthreads();
  for (int u = wg + p.n_wg; u < units; u += p.n_wg) {
    Tracer none{nullptr, 0};
    if (!attn_unit<G, false, kMerge>(p, step, l, pos, attn_unit_of(p, pos, u), s.h, KVPre{}, c, none))
      return false;
    __syncthreads();
  }
  return true;
}

// Staged mode: merge kernel body (one workgroup per query head).
template <int G>
__device__ __forceinline__ bool stage_merge(const Params& p, int step, int l, int pos, int wg, Lds s,
                                            const Ctl& c) {
  const int S = attn_splits(p, pos);
  if (S <= 1) return true;
  for (int u = wg; u < p.H; u += p.n_wg) {
    if (!attn_gather_merge<G>(p, step, l, u / G, S, u % G, G, s.h, c)) return false;
    __syncthreads();
  }
  return true;
}

// ---------------------------------------------------------------------------
// Residual stages.  A workgroup owns the same rows [r0, r1) of x in the O
// and down projections; it reads its own previous x rows from the arena
// together with the stage input.
// ---------------------------------------------------------------------------
// Adds a block's row sums to the owned residual rows and publishes the new
// x twice: as plain fp32 words (read back by the owner, the router and
// lm_head) and as pair words (the GEMV input of the next stages).  Blocks
// start at even rows and hold an even number of them.
__device__ __forceinline__ void put_residual(const Params& p, int b0, int n, int r0, const float* xown,
                                             const float* sums, unsigned f) {
  for (int j = threadIdx.x; 2 * j < n; j += kThreads) {
    const int r = b0 + 2 * j;
    const float v0 = xown[r - r0] + sums[2 * j];
    const float v1 = xown[r + 1 - r0] + sums[2 * j + 1];
    ll_put(p, p.off_x + r, v0, f);
    ll_put(p, p.off_x + r + 1, v1, f);
    ll_put2(p, p.off_xh + (r >> 1), v0, v1, f);
  }
}

__device__ __forceinline__ GemvWork o_work(const Params& p, int wg) {
  return gemv_work(p.d, p.H * p.hd, p.n_wg, wg, 2);
}
__device__ __forceinline__ RowAddr o_addr(const Params& p, int l) {
  return RowAddr{mat_rsrc(layer(p, l).wo, p.d, p.H * p.hd), p.H * p.hd};
}
__device__ __forceinline__ bool stage_oproj(const Params& p, int step, int l, const __half* emb_row,
                                            int wg, Lds s, const Ctl& c, Tracer& tr) {
  const GemvWork g = o_work(p, wg);
  const RowAddr addr = o_addr(p, l);
  WPre pre;
  const int qd = p.H * p.hd;
  const int nown = g.r1 - g.r0;
  if (l == 0) {
    for (int i = threadIdx.x; i < nown; i += kThreads) s.xown[i] = __half2float(emb_row[g.r0 + i]);
  }
  const LLRange rg[2] = {{p.off_o, qd / 2, s.h, ll_flag(p, step, l, kSlotO), 1},
                         {p.off_x + g.r0, l == 0 ? 0 : nown, s.xown,
                          l == 0 ? 0u : ll_flag(p, step, l - 1, kSlotXDown)}};
  if (!ll_gather_pf(p, rg, c, [] {}, [&]() { pre = gemv_prefetch(g, addr); })) return false;
  mark(tr);
  mark(tr);
  const unsigned f = ll_flag(p, step, l, kSlotXO);
  gemv_run<true>(g, addr, s.h, s.part, s.sums, pre, [&](int b0, int n, const float* sums) {
    put_residual(p, b0, n, g.r0, s.xown, sums, f);
  });
  return true;
}

// Stage: RMSNorm + paired gate/up GEMV + SwiGLU (dense FFN).
__device__ __forceinline__ GemvWork gu_work(const Params& p, int wg) {
  return gemv_work(2 * p.F, p.d, p.n_wg, wg, 4);      // virtual rows: 2 outputs of u per unit
}
__device__ __forceinline__ PairAddr gu_addr(const Params& p, int l) {
  const LayerPtrs w = layer(p, l);
  return PairAddr{uniform_addr(w.w_gate), uniform_addr(w.w_up), p.F, p.d};
}
__device__ __forceinline__ bool stage_gateup(const Params& p, int step, int l, int wg, Lds s,
                                             const Ctl& c, Tracer& tr) {
  const GemvWork g = gu_work(p, wg);
  const PairAddr addr = gu_addr(p, l);
  if (g.r0 >= g.r1) {
    mark(tr);
    mark(tr);
    return true;
  }
  const __half* gain = layer(p, l).ffn_norm;
  WPre pre;
  GainPre G;
  const LLRange rg[1] = {{p.off_xh, p.d / 2, s.h, ll_flag(p, step, l, kSlotXO), 1}};
  if (!ll_gather_pf(p, rg, c, [&]() { G = gain_prefetch(gain, p.d); },
                    [&]() { pre = gemv_prefetch(g, addr); }))
    return false;
  mark(tr);
  const float inv = rmsnorm_lds(p, gain, G, s.h, s.red);
  mark(tr);
  const unsigned f = ll_flag(p, step, l, kSlotU);
  gemv_run<true>(g, addr, s.h, s.part, s.sums, pre, [&](int b0, int n, const float* sums) {
    // virtual rows 4j .. 4j + 3 = (gate, up) of u[2j] and of u[2j + 1]
    for (int j = threadIdx.x; 4 * j < n; j += kThreads)
      ll_put2(p, p.off_u + (b0 >> 2) + j, silu(sums[4 * j] * inv) * (sums[4 * j + 1] * inv),
              silu(sums[4 * j + 2] * inv) * (sums[4 * j + 3] * inv), f);
  });
  return true;
}

// Stage: down GEMV + residual (dense FFN).
__device__ __forceinline__ GemvWork down_work(const Params& p, int wg) {
  return gemv_work(p.d, p.F, p.n_wg, wg, 2);
}
__device__ __forceinline__ RowAddr down_addr(const Params& p, int l) {
  return RowAddr{mat_rsrc(layer(p, l).w_down, p.d, p.F), p.F};
}
__device__ __forceinline__ bool stage_down(const Params& p, int step, int l, int wg, Lds s,
                                           const Ctl& c, Tracer& tr) {
  const GemvWork g = down_work(p, wg);
  const RowAddr addr = down_addr(p, l);
  WPre pre;
  const int nown = g.r1 - g.r0;
  const LLRange rg[2] = {{p.off_u, p.F / 2, s.h, ll_flag(p, step, l, kSlotU), 1},
                         {p.off_x + g.r0, nown, s.xown, ll_flag(p, step, l, kSlotXO)}};
  if (!ll_gather_pf(p, rg, c, [] {}, [&]() { pre = gemv_prefetch(g, addr); })) return false;
  mark(tr);
  mark(tr);
  const unsigned f = ll_flag(p, step, l, kSlotXDown);
  gemv_run<true>(g, addr, s.h, s.part, s.sums, pre, [&](int b0, int n, const float* sums) {
    put_residual(p, b0, n, g.r0, s.xown, sums, f);
  });
  return true;
}

// ---------------------------------------------------------------------------
// MoE stages.  A few workgroups compute the router logits; every workgroup
// then derives the same routing (softmax, top-k with the lower id on ties)
// from them.
// ---------------------------------------------------------------------------
__device__ __forceinline__ GemvWork router_work(const Params& p, int wg) {
  return gemv_work(p.E, p.d, p.n_wg, wg, 1);
}
__device__ __forceinline__ RowAddr router_addr(const Params& p, int l) {
  return RowAddr{mat_rsrc(layer(p, l).router, p.E, p.d), p.d};
}
__device__ __forceinline__ bool stage_router(const Params& p, int step, int l, int wg, Lds s,
                                             const Ctl& c, Tracer& tr) {
  const GemvWork g = router_work(p, wg);
  const RowAddr addr = router_addr(p, l);
  if (g.r0 >= g.r1) {
    mark(tr);
    mark(tr);
    return true;
  }
  const __half* gain = layer(p, l).ffn_norm;
  WPre pre;
  GainPre G;
  const LLRange rg[1] = {{p.off_x, p.d, s.h, ll_flag(p, step, l, kSlotXO)}};
  if (!ll_gather_pf(p, rg, c, [&]() { G = gain_prefetch(gain, p.d); },
                    [&]() { pre = gemv_prefetch(g, addr); }))
    return false;
  mark(tr);
  const float inv = rmsnorm_lds(p, gain, G, s.h, s.red);
  mark(tr);
  const unsigned f = ll_flag(p, step, l, kSlotRouter);
  gemv_run<true>(g, addr, s.h, s.part, s.sums, pre, [&](int b0, int n, const float* sums) {
    for (int i = threadIdx.x; i < n; i += kThreads) ll_put(p, p.off_router + b0 + i, sums[i] * inv, f);
  });
  return true;
}

// Routing in LDS from the router logits in `rl` (LDS): ids[a], wts[a] for
// the active slots a < topk + nshared (routed experts in rank order, then
// the shared experts with weight 1).
// The maximum and the softmax denominator are wave reductions (lane i takes
// logits i, i + 64, ...), the same in every wave of every workgroup, so all
// workgroups agree on the routing bit for bit.  The rank of logit e (how many
// logits are larger, or equal with a lower index) is counted by all the
// workgroup's threads, each comparing e with a slice of the others, and the
// partial counts are added with LDS integer atomics into `cnt` (int[E]
// scratch), so the ranks are exact whatever the order.  One wave comparing
// every pair took ~2 us per layer with 64 experts.
__device__ __forceinline__ void moe_routing(const Params& p, int* ids, float* wts, const float* rl,
                                            int* cnt) {
  const int E = p.E, K = p.topk;
  const int lane = threadIdx.x & 63;
  for (int e = threadIdx.x; e < E; e += kThreads) cnt[e] = 0;
  float mx = kNegBig;
  for (int e = lane; e < E; e += 64) mx = fmaxf(mx, rl[e]);
  mx = wave_max(mx);
  float den = 0.f;
  for (int e = lane; e < E; e += 64) den += __expf(rl[e] - mx);
  den = wave_sum(den);
  __syncthreads();
  const int nch = E >= kThreads ? 1 : kThreads / E;      // slices of the compared logits
  const int jlen = (E + nch - 1) / nch;
  for (int t = threadIdx.x; t < E * nch; t += kThreads) {
    const int e = t % E, j0 = (t / E) * jlen, j1 = min(E, j0 + jlen);
    const float re = rl[e];
    int r = 0;
    for (int j = j0; j < j1; ++j) {
      const float rj = rl[j];
      r += (rj > re) || (rj == re && j < e);
    }
    if (r) atomicAdd(&cnt[e], r);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) {
    const int rank = cnt[e];
    if (rank < K) {
      ids[rank] = e;
      wts[rank] = __expf(rl[e] - mx) / den;
    }
  }
  for (int a = threadIdx.x; a < p.nshared; a += kThreads) {
    ids[K + a] = E + a;
    wts[K + a] = 1.0f;
  }
  __syncthreads();
  if (p.moe_renorm) {
    // the selected probabilities rescaled to sum to 1 (summed in rank order,
    // the same in every workgroup)
    float sel = 0.f;
    for (int a = 0; a < K; ++a) sel += wts[a];
    __syncthreads();
    if ((int)threadIdx.x < K) wts[threadIdx.x] = wts[threadIdx.x] / sel;
    __syncthreads();
  }
}

__device__ __forceinline__ int* moe_ids(Lds s) { return reinterpret_cast<int*>(s.red + kRedIdsOff); }
__device__ __forceinline__ float* moe_wts(Lds s) { return s.red + kRedWtsOff; }

// The gate/up rows of the active experts are dealt out in two parts: the
// shared experts' rows, which do not depend on the routing, and the routed
// experts' rows.  Every workgroup streams its share of the shared rows first
// (their first batches issued behind the poll for x), so the router logits'
// hand-off and the routing overlap weight streaming instead of stalling it.
// The routed part is dealt in reverse workgroup order so that the workgroups
// holding an extra unit of one part do not also hold one of the other.
__device__ __forceinline__ GemvWork moe_gu_shared_work(const Params& p, int wg) {
  return gemv_work(2 * p.nshared * p.Fe, p.d, p.n_wg, wg, 4);
}
__device__ __forceinline__ GemvWork moe_gu_routed_work(const Params& p, int wg) {
  return gemv_work(2 * p.topk * p.Fe, p.d, p.n_wg, p.n_wg - 1 - wg, 4);
}
__device__ __forceinline__ bool stage_moe_gateup(const Params& p, int step, int l, int wg, Lds s,
                                                 const Ctl& c, Tracer& tr) {
  const LayerPtrs w = layer(p, l);
  int* ids = moe_ids(s);
  float* wts = moe_wts(s);
  const GemvWork gs = moe_gu_shared_work(p, wg);
  const GemvWork gr = moe_gu_routed_work(p, wg);
  const int Fe = p.Fe, K = p.topk, ne = p.E + p.nshared;
  const MoeSharedPairAddr saddr{uniform_addr(w.e_gate), uniform_addr(w.e_up), p.E, ne, Fe, p.d};
  const __half* gain = w.ffn_norm;
  const GainPre G = gain_prefetch(gain, p.d);
  const bool srows = gs.r0 < gs.r1;
  const bool rows = srows || gr.r0 < gr.r1;
  WPre pre = {};
  const LLRange rx[1] = {{p.off_x, rows ? p.d : 0, s.h, ll_flag(p, step, l, kSlotXO)}};
  if (!ll_gather_pf(p, rx, c, [] {}, [&]() {
        if (srows) pre = gemv_prefetch(gs, saddr);
      }))
    return false;
  mark(tr);
  const float inv = rows ? rmsnorm_lds(p, gain, G, s.h, s.red) : 0.f;
  mark(tr);
  const unsigned f = ll_flag(p, step, l, kSlotU);
  // u of the shared experts (routing weight 1): slots K, K + 1, ...
  gemv_run<true>(gs, saddr, s.h, s.part, s.sums, pre, [&](int b0, int n, const float* sums) {
    for (int j = threadIdx.x; 4 * j < n; j += kThreads) {
      const int ff = K * Fe + (b0 >> 1) + 2 * j;
      ll_put2(p, p.off_u + (ff >> 1), silu(sums[4 * j] * inv) * (sums[4 * j + 1] * inv),
              silu(sums[4 * j + 2] * inv) * (sums[4 * j + 3] * inv), f);
    }
  });
  __syncthreads();
  const LLRange rl[1] = {{p.off_router, p.E, s.sums, ll_flag(p, step, l, kSlotRouter)}};
  if (!ll_gather(p, rl, c)) return false;
  moe_routing(p, ids, wts, s.sums, reinterpret_cast<int*>(s.part));
  if (wg == 0 && threadIdx.x < K)
    p.expert_log[((size_t)(p.pos0 + step) * p.L + l) * K + threadIdx.x] = ids[threadIdx.x];
  const MoePairAddr addr{uniform_addr(w.e_gate), uniform_addr(w.e_up), ids, ne, Fe, p.d};
  gemv_run<false>(gr, addr, s.h, s.part, s.sums, WPre{}, [&](int b0, int n, const float* sums) {
    for (int j = threadIdx.x; 4 * j < n; j += kThreads) {     // u[ff], u[ff + 1]
      const int ff = (b0 >> 1) + 2 * j;
      ll_put2(p, p.off_u + (ff >> 1),
              wts[ff / Fe] * silu(sums[4 * j] * inv) * (sums[4 * j + 1] * inv),
              wts[(ff + 1) / Fe] * silu(sums[4 * j + 2] * inv) * (sums[4 * j + 3] * inv), f);
    }
  });
  return true;
}

// Down projection of all active experts as one GEMV whose row r is the
// concatenation of each active expert's down row r (segments of Fe).
__device__ __forceinline__ GemvWork moe_down_work(const Params& p, int wg) {
  return gemv_work(p.d, (p.topk + p.nshared) * p.Fe, p.n_wg, wg, 2);
}
__device__ __forceinline__ MoeDownAddr moe_down_addr(const Params& p, int l, Lds s) {
  return MoeDownAddr{mat_rsrc(layer(p, l).e_down, (p.E + p.nshared) * p.d, p.Fe), moe_ids(s), p.Fe,
                     p.d, p.Fe >> 3};
}
// With have_routing the expert ids are already in LDS (from this layer's
// gate/up stage), so the first expert rows can be issued before the wait.
__device__ __forceinline__ bool stage_moe_down(const Params& p, int step, int l, int wg, Lds s,
                                               bool have_routing, const Ctl& c, Tracer& tr) {
  const GemvWork g = moe_down_work(p, wg);
  WPre pre = {};
  const int nown = g.r1 - g.r0;
  const int A = p.topk + p.nshared;
  const LLRange rg[3] = {{p.off_u, A * p.Fe / 2, s.h, ll_flag(p, step, l, kSlotU), 1},
                         {p.off_x + g.r0, nown, s.xown, ll_flag(p, step, l, kSlotXO)},
                         {p.off_router, have_routing ? 0 : p.E, s.sums, ll_flag(p, step, l, kSlotRouter)}};
  // 12 words per thread: the active experts' u (5,632 pair words for 8
  // experts of 1,408) arrives in one pass instead of two, each pass costing a
  // poll round trip; the extra slot registers only count in the MoE kernel
  const bool ok = have_routing
                      ? ll_gather_pf<12>(p, rg, c, [] {}, [&]() { pre = gemv_prefetch(g, moe_down_addr(p, l, s)); })
                      : ll_gather<12>(p, rg, c, [] {});
  if (!ok) return false;
  mark(tr);
  if (!have_routing) {
    moe_routing(p, moe_ids(s), moe_wts(s), s.sums, reinterpret_cast<int*>(s.part));
    int t0, t1;
    wave_tasks(g, g.r0, t0, t1);
    pre.a = wload(moe_down_addr(p, l, s), g, g.r0, t0, t1);
    pre.b = wload(moe_down_addr(p, l, s), g, g.r0, t0 + kBatch, t1);
  }
  mark(tr);
  const unsigned f = ll_flag(p, step, l, kSlotXDown);
  gemv_run<true>(g, moe_down_addr(p, l, s), s.h, s.part, s.sums, pre,
                 [&](int b0, int n, const float* sums) {
                   put_residual(p, b0, n, g.r0, s.xown, sums, f);
                 });
  return true;
}

// ---------------------------------------------------------------------------
// Stage: final RMSNorm + lm_head GEMV + greedy argmax.  Each workgroup
// reduces its rows to one packed key and folds it into the step's slot with
// a 64-bit atomic max (order independent, so deterministic).
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Temperature sampling.  The pages put sampling inside the monokernel ("1. The
// Monokernel Runtime"); a step draws its token from softmax(z / T) by the
// Gumbel-max method: token = first argmax of z_i / T + g_i with Gumbel noise
// g_i = -log(-log u_i), so the draw folds into the same packed 64-bit argmax
// as greedy decoding.  u_i comes from Philox4x64-10 (Salmon et al., "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011): word i mod 4 of the block
// for counter (pos, i div 4, 0, 0) and key (seed, 0), top 53 bits, centred
// in their bin so u is never 0 or 1.  The key is formed in float64 and
// rounded once to float32.
// ---------------------------------------------------------------------------
constexpr unsigned long long kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr unsigned long long kPhiloxM1 = 0xCA5A826395121157ull;
constexpr unsigned long long kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr unsigned long long kPhiloxW1 = 0xBB67AE8584CAA73Bull;

// Word `w` (0..3) of the Philox4x64-10 block for counter (c0, c1, 0, 0) and
// key (k0, 0).
__device__ __forceinline__ unsigned long long philox4x64_word(unsigned long long c0, unsigned long long c1,
                                                              unsigned long long k0, int w) {
  unsigned long long x0 = c0, x1 = c1, x2 = 0ull, x3 = 0ull, k1 = 0ull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const unsigned long long hi0 = __umul64hi(kPhiloxM0, x0), lo0 = kPhiloxM0 * x0;
    const unsigned long long hi1 = __umul64hi(kPhiloxM1, x2), lo1 = kPhiloxM1 * x2;
    const unsigned long long n0 = hi1 ^ x1 ^ k0, n2 = hi0 ^ x3 ^ k1;
    x0 = n0;
    x1 = lo1;
    x2 = n2;
    x3 = lo0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return w == 0 ? x0 : w == 1 ? x1 : w == 2 ? x2 : x3;
}

// float32 sampling key of logit v at vocabulary index i, decode position pos.
__device__ __forceinline__ float sample_key(float v, float temperature, unsigned long long seed, int pos, int i) {
  const unsigned long long w = philox4x64_word((unsigned long long)pos, (unsigned long long)(i >> 2), seed, i & 3);
  const double u = ((double)(w >> 11) + 0.5) * 0x1p-53;
  const double g = -log(-log(u));
  return (float)((double)v / (double)temperature + g);
}

// ---------------------------------------------------------------------------
// Top-k / top-p draw (sample == 2).  Candidates are the logits in order,
// largest first, ties by the lower index (the greedy argmax's order); top-k
// keeps the first K of them (K = top_k, or kMaxTopK without one), top-p the
// shortest prefix whose mass exp((z_j - z_0) / T), summed in float64 in
// that order, reaches top_p of the kept pool's; the token is the Gumbel-max
// draw of temperature sampling over what is kept, the lowest index winning
// on equal keys.  Runs once the step's logits in p.zbuf are complete (after
// the step's grid barrier); every workgroup computes the same token from
// the same logits, so no exchange follows.  Called by every thread of the
// workgroup; `lds`: kSelWords floats of scratch.
// ---------------------------------------------------------------------------
constexpr int kSelWords = 256 + kThreads + 8 + 4 * kMaxTopK;
static_assert(kSelWords <= 2 * kPartCap, "selection scratch exceeds the GEMV scratch it reuses");

__device__ __forceinline__ unsigned ord_key(float v) {
  const unsigned u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(unsigned long long key) {
  const unsigned u = (unsigned)(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
__device__ __forceinline__ int key_index(unsigned long long key) {
  return (int)(0xFFFFFFFFu - (unsigned)(key & 0xFFFFFFFFull));
}

__device__ int select_topkp(const Params& p, int step, float* lds) {
  const int V = p.Vout, tid = threadIdx.x;
  const int K = min(p.top_k > 0 ? p.top_k : kMaxTopK, V);
  unsigned* hist = reinterpret_cast<unsigned*>(lds);               // [256]
  unsigned* tcnt = hist + 256;                                      // [kThreads]
  unsigned* misc = tcnt + kThreads;                                 // [8]
  unsigned long long* cand = reinterpret_cast<unsigned long long*>(misc + 8);   // [kMaxTopK]
  double* q = reinterpret_cast<double*>(cand + kMaxTopK);          // [kMaxTopK]
  const float* zb = p.zbuf;
  // 1. the K-th largest key, a byte at a time from the top: the count of
  //    keys above the prefix's bucket decides the next byte
  unsigned prefix = 0u, mask = 0u, r = (unsigned)K;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kThreads) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < V; i += kThreads) {
      const unsigned u = ord_key(ld_c(zb + i));
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 0xFFu], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      unsigned above = 0u;
      int d = 255;
      for (; d > 0 && above + hist[d] < r; --d) above += hist[d];
      misc[0] = (unsigned)d;
      misc[1] = above;
    }
    __syncthreads();
    prefix |= misc[0] << shift;
    mask |= 0xFFu << shift;
    r -= misc[1];
    __syncthreads();
  }
  // 2. the keys above the K-th, and the first r equal to it in index order
  //    (each thread takes a contiguous run of indices)
  const int per = (V + kThreads - 1) / kThreads;
  const int i0 = min(V, tid * per), i1 = min(V, i0 + per);
  unsigned ties = 0u;
  for (int i = i0; i < i1; ++i) ties += ord_key(ld_c(zb + i)) == prefix ? 1u : 0u;
  tcnt[tid] = ties;
  if (tid == 0) misc[2] = 0u;
  __syncthreads();
  if (tid == 0) {
    unsigned acc = 0u;
    for (int t = 0; t < kThreads; ++t) {
      const unsigned v = tcnt[t];
      tcnt[t] = acc;
      acc += v;
    }
  }
  __syncthreads();
  unsigned before = tcnt[tid];
  for (int i = i0; i < i1; ++i) {
    const unsigned u = ord_key(ld_c(zb + i));
    const bool keep = u > prefix || (u == prefix && before < r);
    before += u == prefix ? 1u : 0u;
    if (keep) {
      const unsigned slot = atomicAdd(&misc[2], 1u);     // exactly K keys are kept
      if (slot < (unsigned)kMaxTopK) cand[slot] = ((unsigned long long)u << 32) | (0xFFFFFFFFu - (unsigned)i);
    }
  }
  __syncthreads();
  // 3. the K candidates in candidate order (their packed keys, descending):
  //    a bitonic sort, padded with zero keys that sort last
  int n2 = 1;
  while (n2 < K) n2 <<= 1;
  for (int j = K + tid; j < n2; j += kThreads) cand[j] = 0ull;
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int j = tid; j < n2; j += kThreads) {
        const int o = j ^ stride;
        if (o > j) {
          const unsigned long long a = cand[j], b = cand[o];
          if ((j & size) == 0 ? a < b : a > b) {
            cand[j] = b;
            cand[o] = a;
          }
        }
      }
      __syncthreads();
    }
  // 4. top-p: the shortest prefix reaching top_p of the pool's mass
  int m = K;
  if (p.top_p < 1.0f) {
    const double z0 = (double)key_value(cand[0]), t = (double)p.temperature;
    for (int j = tid; j < K; j += kThreads) q[j] = exp(((double)key_value(cand[j]) - z0) / t);
    __syncthreads();
    if (tid == 0) {
      double tot = 0.0;
      for (int j = 0; j < K; ++j) tot += q[j];
      const double goal = (double)p.top_p * tot;
      double run = 0.0;
      int j = 0;
      for (; j < K - 1; ++j) {
        run += q[j];
        if (run >= goal) break;
      }
      misc[3] = (unsigned)(j + 1);
    }
    __syncthreads();
    m = (int)misc[3];
  }
  // 5. Gumbel-max over the kept candidates
  const int pos = p.pos0 + step;
  unsigned long long best = 0ull;
  for (int j = tid; j < m; j += kThreads) {
    const int idx = key_index(cand[j]);
    const unsigned long long k = argmax_key(sample_key(key_value(cand[j]), p.temperature, p.seed, pos, idx), idx);
    best = k > best ? k : best;
  }
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long other = __shfl_xor(best, o, 64);
    best = other > best ? other : best;
  }
  unsigned long long* red = reinterpret_cast<unsigned long long*>(tcnt);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = best;
  __syncthreads();
  unsigned long long b = 0ull;
  for (int w = 0; w < kWaves; ++w) b = red[w] > b ? red[w] : b;
  __syncthreads();                                   // the scratch is free again
  return argmax_index(b, V);
}

__device__ __forceinline__ GemvWork lm_work(const Params& p, int wg) {
  return gemv_work(p.Vout, p.d, p.n_wg, wg, 1);
}
__device__ __forceinline__ bool stage_lmhead(const Params& p, int step, int wg, Lds s, const Ctl& c,
                                             Tracer& tr) {
  const GemvWork g = lm_work(p, wg);
  const RowAddr addr{mat_rsrc(p.lm_head, p.Vout, p.d), p.d};
  if (g.r0 >= g.r1) {
    mark(tr);
    mark(tr);
    return true;
  }
  WPre pre;
  GainPre G;
  const LLRange rg[1] = {{p.off_x, p.d, s.h, ll_flag(p, step, p.L - 1, kSlotXDown)}};
  if (!ll_gather_pf(p, rg, c, [&]() { G = gain_prefetch(p.final_norm, p.d); },
                    [&]() { pre = gemv_prefetch(g, addr); }))
    return false;
  mark(tr);
  const float inv = rmsnorm_lds(p, p.final_norm, G, s.h, s.red);
  mark(tr);
  float* logits = p.out_logits ? p.out_logits + (size_t)step * p.Vout : nullptr;
  const bool sample = p.sample == 1;
  const bool select = p.sample == 2;       // the logits go to zbuf; the draw follows the barrier
  const int pos = p.pos0 + step;           // position of this step's input token
  unsigned long long best = 0ull;
  gemv_run<true>(g, addr, s.h, s.part, s.sums, pre,
                 [&](int b0, int n, const float* sums) {
                   for (int i = threadIdx.x; i < n; i += kThreads) {
                     const float v = sums[i] * inv;
                     if (logits) logits[b0 + i] = v;
                     if (select) {
                       st_c(p.zbuf + b0 + i, v);
                       continue;
                     }
                     const float key = sample ? sample_key(v, p.temperature, p.seed, pos, b0 + i) : v;
                     const unsigned long long k = argmax_key(key, b0 + i);
                     best = k > best ? k : best;
                   }
                 });
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long other = __shfl_xor(best, o, 64);
    best = other > best ? other : best;
  }
  unsigned long long* red64 = reinterpret_cast<unsigned long long*>(s.red);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red64[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long b = 0ull;
    for (int i = 0; i < kWaves; ++i) b = red64[i] > b ? red64[i] : b;
    if (b != 0ull)
      __hip_atomic_fetch_max(p.amax + (step & 1), b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return true;
}

// ---------------------------------------------------------------------------
// The persistent kernel.  Each stage issues the next stage's first weight
// (or KV) loads as soon as it has stored its own outputs, then waits only
// for the activations it consumes.  One grid barrier per step publishes the
// argmax (decode) or orders prefill steps.
// ---------------------------------------------------------------------------
// The parameter block lives in device memory and is re-read (scalar loads,
// scalar-cache hits) at every stage: `fresh` hides the pointer from the
// optimiser, so parameter loads are not hoisted out of the step and layer
// loops and kept live in SGPRs for the whole kernel.
typedef const __attribute__((address_space(4))) Params* ConstParamsPtr;
__device__ __forceinline__ const Params& fresh(const Params* pp) {
  ConstParamsPtr c = (ConstParamsPtr)pp;
  asm volatile("" : "+s"(c));
  return *(const Params*)c;
}

// The persistent kernel, one build per query-head group G and FFN kind: a
// dense build carries no expert code and the MoE build no dense FFN, so
// each is allocated the registers of its own path (the dense G = 1 build
// uses 212 VGPRs, the MoE one 240).
template <int G, bool kMoe>
__global__ __launch_bounds__(kThreads, 1) void mono_kernel(const Params* __restrict__ pp) {
  // 16-byte aligned: the GEMV reads the input vector with 16-byte LDS loads
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int flag;
  if (threadIdx.x == 0) flag = 1;
  __syncthreads();
  const int wg = blockIdx.x;
  GridSync gs;
  Lds s;
  Ctl c;
  Tracer tr{nullptr, 0};
  int tok, n_steps, L, pos0, trace_step;
  bool decode;
  unsigned long long* trace;
  {
    const Params& p = fresh(pp);
    s = lds_carve(p, smem);
    gs = make_sync(p.bar, p.err, (unsigned)p.n_wg, p.timeout_ticks, p.spin_limit);
    c = make_ctl(p, &flag);
    decode = p.mode == kDecode;
    n_steps = p.n_steps;
    L = p.L;
    pos0 = p.pos0;
    tok = decode ? p.state[0] : (n_steps > 0 ? p.prompt[0] : 0);
    trace = (decode && p.trace != nullptr) ? p.trace + (size_t)wg * kTraceEvents : nullptr;
    trace_step = p.trace_step;
  }
  // Input token of step `prev + 1`, once the grid barrier that closed step
  // `prev` has been passed: the argmax of its logits (decode) or the next
  // prompt token (prefill).
  auto resolve = [&](int prev) -> int {
    const Params& p = fresh(pp);
    if (!decode) return p.prompt[prev + 1];
    const int t = p.sample == 2 ? select_topkp(p, prev, s.part) : argmax_index(ld_c64(p.amax + (prev & 1)), p.Vout);
    if (wg == 0 && threadIdx.x == 0) {
      p.out_tokens[prev] = t;
      st_c64(p.amax + ((prev + 1) & 1), 0ull);
    }
    return t;
  };
  for (int step = 0; step < n_steps; ++step) {
    const int pos = pos0 + step;
    tr.tr = (step == trace_step) ? trace : nullptr;
    tr.ev = 0;
    mark(tr);
    for (int l = 0; l < L; ++l) {
      if (!stage_qkv(fresh(pp), step, l, wg, s, c, tr, gs, l == 0 && step > 0, tok,
                     [&]() { return resolve(step - 1); }))
        return;
      mark(tr);
      if (!stage_attn<G, true>(fresh(pp), step, l, pos, wg, s, c, tr)) return;
      mark(tr);
      {
        const Params& p = fresh(pp);
        if (!stage_oproj(p, step, l, p.tok_emb + (size_t)tok * p.d, wg, s, c, tr)) return;
      }
      mark(tr);
      if constexpr (!kMoe) {
        if (!stage_gateup(fresh(pp), step, l, wg, s, c, tr)) return;
        mark(tr);
        if (!stage_down(fresh(pp), step, l, wg, s, c, tr)) return;
      } else {
        if (!stage_router(fresh(pp), step, l, wg, s, c, tr)) return;
        mark(tr);
        if (!stage_moe_gateup(fresh(pp), step, l, wg, s, c, tr)) return;
        mark(tr);
        if (!stage_moe_down(fresh(pp), step, l, wg, s, true, c, tr)) return;
      }
      mark(tr);
    }
    if (decode) {
      if (!stage_lmhead(fresh(pp), step, wg, s, c, tr)) return;
      mark(tr);
    }
    // closes the step: the argmax is complete (decode); this step's KV rows,
    // read by the next step's attention, are written (prefill)
    grid_arrive(gs);
  }
  if (n_steps > 0) {
    if (!grid_wait(gs, &flag)) return;
    tok = resolve(n_steps - 1);
  }
  if (wg == 0 && threadIdx.x == 0) {
    const Params& p = fresh(pp);
    p.state[0] = decode ? tok : p.prompt[n_steps];
  }
}

// ---- staged mode: one kernel per stage, the step counter lives on device.
// Kernel boundaries order the stages, so every wait for activations is
// satisfied at its first read.
enum StageId : int { kSQkv, kSAttn, kSMerge, kSO, kSGateUp, kSDown, kSRouter, kSMoeGateUp, kSMoeDown, kSLm };

__global__ __launch_bounds__(kThreads, 1) void stage_kernel(Params p, int stage, int l) {
  // 16-byte aligned: the GEMV reads the input vector with 16-byte LDS loads
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int flag;
  if (threadIdx.x == 0) flag = 1;
  __syncthreads();
  const Lds s = lds_carve(p, smem);
  const Ctl c = make_ctl(p, &flag);
  const int wg = blockIdx.x;
  const int step = p.state[1];
  const int pos = p.pos0 + step;
  const int tok = (p.mode == kPrefill) ? p.prompt[step] : p.state[0];
  const __half* emb = p.tok_emb + (size_t)tok * p.d;
  Tracer none{nullptr, 0};
  GridSync no_sync = make_sync(p.bar, p.err, (unsigned)p.n_wg, p.timeout_ticks, p.spin_limit);
  int t = tok;
  switch (stage) {
    case kSQkv: (void)stage_qkv(p, step, l, wg, s, c, none, no_sync, false, t, [&]() { return tok; }); break;
    case kSAttn:
      switch (p.H / p.nkv) {
        case 1: (void)stage_attn<1, false>(p, step, l, pos, wg, s, c, none); break;
        case 2: (void)stage_attn<2, false>(p, step, l, pos, wg, s, c, none); break;
        default: (void)stage_attn<4, false>(p, step, l, pos, wg, s, c, none); break;
      }
      break;
    case kSMerge:
      switch (p.H / p.nkv) {
        case 1: (void)stage_merge<1>(p, step, l, pos, wg, s, c); break;
        case 2: (void)stage_merge<2>(p, step, l, pos, wg, s, c); break;
        default: (void)stage_merge<4>(p, step, l, pos, wg, s, c); break;
      }
      break;
    case kSO: (void)stage_oproj(p, step, l, emb, wg, s, c, none); break;
    case kSGateUp: (void)stage_gateup(p, step, l, wg, s, c, none); break;
    case kSDown: (void)stage_down(p, step, l, wg, s, c, none); break;
    case kSRouter: (void)stage_router(p, step, l, wg, s, c, none); break;
    case kSMoeGateUp: (void)stage_moe_gateup(p, step, l, wg, s, c, none); break;
    case kSMoeDown: (void)stage_moe_down(p, step, l, wg, s, false, c, none); break;
    case kSLm: (void)stage_lmhead(p, step, wg, s, c, none); break;
  }
}

// End of a step in staged mode (one workgroup of one thread's work).
__global__ void step_end_kernel(Params p) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const int step = p.state[1];
  if (p.mode == kDecode) {
    const int tok = argmax_index(p.amax[step & 1], p.Vout);
    p.out_tokens[step] = tok;
    p.state[0] = tok;
    p.amax[(step + 1) & 1] = 0ull;
  } else if (step + 1 == p.n_steps) {
    p.state[0] = p.prompt[p.n_steps];
  }
  p.state[1] = step + 1;
}

// ---- inspection kernels
__global__ __launch_bounds__(kThreads, 1) void gemv_kernel(const __half* w, const float* x, float* y,
                                                           int rows, int cols, int n_wg) {
  // 16-byte aligned: the GEMV reads the input vector with 16-byte LDS loads
  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* h = smem;
  float* part = smem + ((cols + 63) & ~63);
  float* sums = part + kPartCap;
  for (int i = threadIdx.x; i < cols; i += kThreads) h[i] = x[i];
  __syncthreads();
  gemv_run<false>(gemv_work(rows, cols, n_wg, blockIdx.x, 1), RowAddr{mat_rsrc(w, rows, cols), cols},
                  h, part, sums, WPre{}, [&](int b0, int n, const float* sm) {
                    for (int i = threadIdx.x; i < n; i += kThreads) y[b0 + i] = sm[i];
                  });
}

__global__ __launch_bounds__(kThreads, 1) void barrier_test_kernel(unsigned* bar, unsigned* slots,
                                                                   int* violations, int* err,
                                                                   int rounds, long long ticks,
                                                                   int spin_limit) {
  __shared__ int flag;
  __shared__ int bad;
  const unsigned nwg = gridDim.x;
  GridSync gs = make_sync(bar, err, nwg, ticks, spin_limit);
  if (threadIdx.x == 0) {
    bad = 0;
    flag = 1;
  }
  __syncthreads();
  for (int r = 1; r <= rounds; ++r) {
    if (threadIdx.x == 0) st_cu(slots + blockIdx.x, (unsigned)r);
    grid_arrive(gs);
    if (!grid_wait(gs, &flag)) return;
    int local = 0;
    for (unsigned j = threadIdx.x; j < nwg; j += kThreads) local += (ld_cu(slots + j) < (unsigned)r);
    if (local) atomicAdd(&bad, local);
    __syncthreads();
    // nobody may run ahead and overwrite a slot before everyone checked it
    grid_arrive(gs);
    if (!grid_wait(gs, &flag)) return;
  }
  if (threadIdx.x == 0 && bad) atomicAdd(violations, bad);
}

// Plain HBM streaming probe: reads n16 16-byte words grid-stride with kU
// loads in flight per lane and either copies them to dst or folds them into
// a value that is stored only if it equals an arbitrary constant (so the
// reads cannot be dropped).  kKind picks the load: 0 a non-temporal global
// load, 1 a plain global load, 2 the raw buffer load with the non-temporal
// policy that the decode kernel streams its weights with.  Gives the
// achievable read bandwidth of the device and a copy of known size for
// calibrating the memory counters.
template <int kKind>
__device__ __forceinline__ u32x4 stream_ld(const u32x4* src, Rsrc r, size_t i) {
  if constexpr (kKind == 0) return __builtin_nontemporal_load(src + i);
  else if constexpr (kKind == 1) return src[i];
  else return ld_w16(r, (unsigned)(i * 16u));
}

template <int kU, int kKind>
__global__ __launch_bounds__(kThreads) void stream_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, size_t n16,
                                                          unsigned* sink) {
  const Rsrc r = make_rsrc(src, kKind == 2 ? n16 * 16u : 16u);
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kU - 1) * stride < n16; i += kU * stride) {
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = stream_ld<kKind>(src, r, i + u * stride);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (dst) dst[i + u * stride] = v[u];
      else acc ^= v[u];
    }
  }
  for (; i < n16; i += stride) {
    const u32x4 v = stream_ld<kKind>(src, r, i);
    if (dst) dst[i] = v;
    else acc ^= v;
  }
  if (!dst && (acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[0] = 1u;
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
static const void* mono_for(int group, bool moe) {
  switch (group) {
    case 1: return moe ? reinterpret_cast<const void*>(mono_kernel<1, true>)
                       : reinterpret_cast<const void*>(mono_kernel<1, false>);
    case 2: return moe ? reinterpret_cast<const void*>(mono_kernel<2, true>)
                       : reinterpret_cast<const void*>(mono_kernel<2, false>);
    default: return moe ? reinterpret_cast<const void*>(mono_kernel<4, true>)
                        : reinterpret_cast<const void*>(mono_kernel<4, false>);
  }
}

int max_blocks_per_cu(int group, bool moe, size_t lds_bytes) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, mono_for(group, moe), kThreads, lds_bytes) !=
      hipSuccess)
    return 0;
  return nb;
}

hipError_t launch_mono(const Params& p, const Params* p_dev, size_t lds_bytes, bool plain,
                       hipStream_t s) {
  void* args[] = {const_cast<Params**>(&p_dev)};
  if (plain)
    return hipLaunchKernel(mono_for(p.H / p.nkv, p.E != 0), dim3(p.n_wg), dim3(kThreads), args,
                           (unsigned)lds_bytes, s);
  return hipLaunchCooperativeKernel(mono_for(p.H / p.nkv, p.E != 0), dim3(p.n_wg), dim3(kThreads), args,
                                    (unsigned)lds_bytes, s);
}

hipError_t launch_staged_step(const Params& p, size_t lds_bytes, hipStream_t s) {
  const dim3 grid(p.n_wg), block(kThreads);
  const unsigned lds = (unsigned)lds_bytes;
  for (int l = 0; l < p.L; ++l) {
    hipLaunchKernelGGL(stage_kernel, grid, block, lds, s, p, (int)kSQkv, l);
    hipLaunchKernelGGL(stage_kernel, grid, block, lds, s, p, (int)kSAttn, l);
    if (p.splits > 1) hipLaunchKernelGGL(stage_kernel, grid, block, lds, s, p, (int)kSMerge, l);
    hipLaunchKernelGGL(stage_kernel, grid, block, lds, s, p, (int)kSO, l);
    if (p.E == 0) {
      hipLaunchKernelGGL(stage_kernel, grid, block, lds, s, p, (int)kSGateUp, l);
      hipLaunchKernelGGL(stage_kernel, grid, block, lds, s, p, (int)kSDown, l);
    } else {
      hipLaunchKernelGGL(stage_kernel, grid, block, lds, s, p, (int)kSRouter, l);
      hipLaunchKernelGGL(stage_kernel, grid, block, lds, s, p, (int)kSMoeGateUp, l);
      hipLaunchKernelGGL(stage_kernel, grid, block, lds, s, p, (int)kSMoeDown, l);
    }
  }
  if (p.mode == kDecode) hipLaunchKernelGGL(stage_kernel, grid, block, lds, s, p, (int)kSLm, 0);
  hipLaunchKernelGGL(step_end_kernel, dim3(1), dim3(64), 0, s, p);
  return hipGetLastError();
}

// One stage of the staged mode (the attention stage with its merge).
hipError_t launch_stage(const Params& p, size_t lds_bytes, int stage, int l, hipStream_t s) {
  const dim3 grid(p.n_wg), block(kThreads);
  const unsigned lds = (unsigned)lds_bytes;
  hipLaunchKernelGGL(stage_kernel, grid, block, lds, s, p, stage, l);
  if (stage == kSAttn && p.splits > 1) hipLaunchKernelGGL(stage_kernel, grid, block, lds, s, p, (int)kSMerge, l);
  return hipGetLastError();
}

size_t gemv_lds_bytes(int cols) {
  return ((size_t)((cols + 63) & ~63) + 2 * kPartCap) * sizeof(float);
}

hipError_t launch_gemv(const __half* w, const float* x, float* y, int rows, int cols, int n_wg,
                       hipStream_t s) {
  hipLaunchKernelGGL(gemv_kernel, dim3(n_wg), dim3(kThreads), (unsigned)gemv_lds_bytes(cols), s, w,
                     x, y, rows, cols, n_wg);
  return hipGetLastError();
}

hipError_t launch_barrier_test(unsigned* bar, unsigned* slots, int* violations, int* err, int n_wg,
                               int rounds, long long timeout_ticks, int spin_limit,
                               hipStream_t s) {
  void* args[] = {&bar, &slots, &violations, &err, &rounds, &timeout_ticks, &spin_limit};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(barrier_test_kernel),
                                    dim3(n_wg), dim3(kThreads), args, 0u, s);
}

template <int kKind>
static const void* stream_for(int depth) {
  switch (depth) {
    case 1: return reinterpret_cast<const void*>(stream_kernel<1, kKind>);
    case 2: return reinterpret_cast<const void*>(stream_kernel<2, kKind>);
    case 4: return reinterpret_cast<const void*>(stream_kernel<4, kKind>);
    case 16: return reinterpret_cast<const void*>(stream_kernel<16, kKind>);
    default: return reinterpret_cast<const void*>(stream_kernel<8, kKind>);
  }
}

hipError_t launch_stream(const void* src, void* dst, size_t bytes, int n_wg, int depth, int kind,
                         unsigned* sink, hipStream_t s) {
  const void* k = kind == 1 ? stream_for<1>(depth) : kind == 2 ? stream_for<2>(depth)
                                                               : stream_for<0>(depth);
  size_t n16 = bytes / 16;
  void* args[] = {&src, &dst, &n16, &sink};
  return hipLaunchKernel(k, dim3(n_wg), dim3(kThreads), args, 0u, s);
}

}  // namespace kie
