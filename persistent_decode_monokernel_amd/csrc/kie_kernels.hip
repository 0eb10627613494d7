// Decode stages and the persistent monokernel for gfx950 (CDNA4, wave64).
//
// The pages' method: one GPU-resident program runs the whole per-token
// decode path (matrix multiplies, attention, normalisation, sampling) and
// never returns to the CPU between tokens (page "Breaking the memory wall:
// 3,000 tokens/s on standard GPUs", agentlenshq.com, section "1. The
// Monokernel Runtime"); normalisation, attention and matmul stages are fused
// so data stays near the compute units (page "Kog bets deeper GPU
// optimization can accelerate AI inference", remio.ai, section on co-design).
// Batch-1 decode moves every active weight from HBM once per token and is
// bandwidth bound (first page, section "The bottleneck: memory bandwidth,
// not compute"), so every stage here is built around streaming fp16 weight
// rows with 128-bit loads, not around matrix cores.
//
// Layout of one decode step (dense model), one workgroup per CU:
//   per layer:  [rmsnorm+QKV GEMV] | [RoPE + KV append + split-K attention,
//               last-arriving split merges] | [O GEMV + residual] |
//               [rmsnorm + gate/up GEMV + SwiGLU] | [down GEMV + residual] |
//   then        [final rmsnorm + lm_head GEMV + argmax] | token feedback
// '|' is a grid barrier in the persistent kernel and a kernel boundary in
// the staged (hipGraph) mode.  MoE layers replace the FFN with
//   [rmsnorm + router GEMV] | [routing + expert gate/up] | [expert down].
#include "kie_params.h"

namespace kie {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kUnroll = 4;                  // 16-byte chunks per lane per batch
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;         // finite "minus infinity" for softmax state

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 ld_stream16(const __half* p) {
  // weights are read once per token: non-temporal
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16(const __half* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// fp16 x8 . fp32 x8 accumulated in fp32 (v_fma_mix_f32).  The 16-byte word
// is reinterpreted as a whole: bit-casting single elements of an ext_vector
// (w.y, ...) is miscompiled to element 0 by this toolchain.
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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over a 16-lane group (lanes differing in bits 0..3).
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Workgroup sum in a fixed order: every workgroup computes bit-identical
// results from identical inputs.  `red` holds kWaves floats of LDS.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) s += red[i];
  return s;
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
// Grid barrier on an HBM counter (agent-scope atomics).
//
// Every wave publishes its own stores (agent release: L2 write-back + wait),
// one lane per workgroup bumps the monotonically increasing counter and
// polls it with agent-coherent loads until all workgroups of this round
// arrived, then every wave acquires (L2/L1 invalidate) before reading data
// written elsewhere on the chip.  The wait is bounded: on timeout (or when
// another workgroup already failed) the error word is set and every
// workgroup leaves the kernel at its next barrier.
// ---------------------------------------------------------------------------
struct GridSync {
  unsigned* bar;
  int* err;
  unsigned target;
  unsigned nwg;
  long long ticks;
  int spin_limit;
};

__device__ __forceinline__ bool grid_sync(GridSync& g, int* flag) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __builtin_amdgcn_s_barrier();
  g.target += g.nwg;
  if (threadIdx.x == 0) {
    int ok = 1;
    __hip_atomic_fetch_add(g.bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const long long t0 = wall_clock64();
    int spins = 0;
    while ((int)(__hip_atomic_load(g.bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - g.target) < 0) {
      if (__hip_atomic_load(g.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) { ok = 0; break; }
      ++spins;
      if ((g.spin_limit > 0 && spins >= g.spin_limit) || wall_clock64() - t0 > g.ticks) {
        int expected = 0;
        __hip_atomic_compare_exchange_strong(g.err, &expected, kErrTimeout, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    *flag = ok;
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return *flag != 0;
}

// ---------------------------------------------------------------------------
// GEMV core.  One wave computes NR dot products of fp16 rows with the fp32
// vector h in LDS.  Lane l reads 16-byte chunks l, l+64, ... of each row
// (fully coalesced 1 KiB per wave per load), up to NR*kUnroll loads in
// flight per lane; the fp32 sums are reduced across the wave at the end.
// ---------------------------------------------------------------------------
template <int NR>
__device__ __forceinline__ void wave_dot(const __half* const (&rowp)[NR], int nvalid, int nch,
                                         const float* __restrict__ h, float (&out)[NR]) {
  const int lane = threadIdx.x & 63;
  const float4* h4 = reinterpret_cast<const float4*>(h);
  float acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.f;
  for (int c0 = 0; c0 < nch; c0 += 64 * kUnroll) {
    u32x4 w[NR][kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int idx = c0 + u * 64 + lane;
#pragma unroll
      for (int r = 0; r < NR; ++r)
        w[r][u] = (idx < nch && r < nvalid) ? ld_stream16(rowp[r] + (size_t)idx * 8)
                                            : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int idx = c0 + u * 64 + lane;
      if (idx < nch) {
        const float4 a = h4[2 * idx];
        const float4 b = h4[2 * idx + 1];
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r] = dot8(w[r][u], a, b, acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) out[r] = wave_sum(acc[r]);
}

// Rows [r0, r1) of a GEMV for this workgroup: groups of NR consecutive rows
// go to the waves round-robin.  row(r) gives the fp16 row pointer,
// epi(r, value) consumes one result (called by lane (r - group start)).
template <int NR, class RowFn, class EpiFn>
__device__ __forceinline__ void gemv_rows(int r0, int r1, int ncols, const float* h, RowFn row,
                                          EpiFn epi) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nch = ncols >> 3;
  for (int g0 = r0 + wave * NR; g0 < r1; g0 += kWaves * NR) {
    const int nvalid = min(NR, r1 - g0);
    const __half* rp[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) rp[r] = row(min(g0 + r, r1 - 1));
    float res[NR];
    wave_dot<NR>(rp, nvalid, nch, h, res);
#pragma unroll
    for (int r = 0; r < NR; ++r)
      if (r < nvalid && lane == r) epi(g0 + r, res[r]);
  }
}

template <class RowFn, class EpiFn>
__device__ __forceinline__ void gemv_dispatch(int r0, int r1, int ncols, const float* h, RowFn row,
                                              EpiFn epi) {
  const int per_wave = (r1 - r0 + kWaves - 1) / kWaves;
  if (per_wave <= 1)
    gemv_rows<1>(r0, r1, ncols, h, row, epi);
  else if (per_wave <= 2)
    gemv_rows<2>(r0, r1, ncols, h, row, epi);
  else
    gemv_rows<4>(r0, r1, ncols, h, row, epi);
}

// Paired rows (gate f, up f) -> one SwiGLU output; NP pairs per wave group.
template <int NP, class RowFn, class EpiFn>
__device__ __forceinline__ void gemv_pairs(int f0, int f1, int ncols, const float* h, RowFn row,
                                           EpiFn epi) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nch = ncols >> 3;
  for (int g0 = f0 + wave * NP; g0 < f1; g0 += kWaves * NP) {
    const int nvalid = min(NP, f1 - g0);
    const __half* rp[2 * NP];
#pragma unroll
    for (int r = 0; r < NP; ++r) {
      const int f = min(g0 + r, f1 - 1);
      rp[2 * r] = row(f, 0);
      rp[2 * r + 1] = row(f, 1);
    }
    float res[2 * NP];
    wave_dot<2 * NP>(rp, 2 * nvalid, nch, h, res);
#pragma unroll
    for (int r = 0; r < NP; ++r)
      if (r < nvalid && lane == r) epi(g0 + r, silu(res[2 * r]) * res[2 * r + 1]);
  }
}

template <class RowFn, class EpiFn>
__device__ __forceinline__ void gemv_pairs_dispatch(int f0, int f1, int ncols, const float* h,
                                                    RowFn row, EpiFn epi) {
  const int per_wave = (f1 - f0 + kWaves - 1) / kWaves;
  if (per_wave <= 1)
    gemv_pairs<1>(f0, f1, ncols, h, row, epi);
  else
    gemv_pairs<2>(f0, f1, ncols, h, row, epi);
}

// ---------------------------------------------------------------------------
// RMSNorm into LDS, recomputed by every workgroup (deterministic, no extra
// barrier): h = v / sqrt(mean(v^2) + eps) * gain with v = x (fp32, global)
// or, at layer 0, the fp16 embedding row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rmsnorm_to_lds(const Params& p, const float* xg, const __half* xe,
                                               const __half* gain, float* h, float* red) {
  const int d = p.d;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += kThreads) {
    const float v = xg ? xg[i] : __half2float(xe[i]);
    h[i] = v;
    ss = fmaf(v, v, ss);
  }
  ss = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)d + p.eps);
  for (int i = threadIdx.x; i < d; i += kThreads) h[i] = h[i] * inv * __half2float(gain[i]);
  __syncthreads();
}

__device__ __forceinline__ void copy_to_lds(const float* src, int n, float* h) {
  for (int i = threadIdx.x; i < n; i += kThreads) h[i] = src[i];
  __syncthreads();
}

// LDS carve-up (floats): [0, hcap) GEMV vector; then a small reduction area.
struct Lds {
  float* h;
  float* red;
};

// ---------------------------------------------------------------------------
// Stage: RMSNorm + fused Q/K/V GEMV (rows of Wq, Wk, Wv as one row space).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void stage_qkv(const Params& p, int l, const __half* emb_row, int wg, Lds s) {
  const LayerPtrs& w = p.layers[l];
  rmsnorm_to_lds(p, l == 0 ? nullptr : p.x, emb_row, w.attn_norm, s.h, s.red);
  const int qd = p.H * p.hd, kd = p.nkv * p.hd;
  int r0, r1;
  even_range(qd + 2 * kd, p.n_wg, wg, r0, r1);
  const int d = p.d;
  float* out = p.qkv;
  gemv_dispatch(
      r0, r1, d, s.h,
      [&](int r) -> const __half* {
        if (r < qd) return w.wq + (size_t)r * d;
        if (r < qd + kd) return w.wk + (size_t)(r - qd) * d;
        return w.wv + (size_t)(r - qd - kd) * d;
      },
      [&](int r, float v) { out[r] = v; });
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
// values.  Each split writes (acc, m, l) to HBM; the last split to arrive
// at the per-head counter merges all splits in split order into o.
// Scores carry log2(e)/sqrt(hd) so exp2 is the softmax exponential.
// ---------------------------------------------------------------------------
template <int G>
__device__ __forceinline__ void attn_unit(const Params& p, int l, int pos, int g, int sidx, float* lds, int* flag) {
  const int hd = p.hd, half = hd >> 1, S = p.splits;
  const int qd = p.H * hd, kd = p.nkv * hd;
  const int n = pos + 1;
  const int p0 = split_begin(sidx, n, S), p1 = split_begin(sidx + 1, n, S);
  const bool has_new = (p1 == n);
  const int pend = has_new ? pos : p1;           // cached positions [p0, pend)

  float* qs = lds;                               // [G][hd]
  float* kn = qs + G * hd;                       // [hd]
  float* vn = kn + hd;                           // [hd]
  float* wst = vn + hd;                          // [kWaves][G][hd + 2]

  const float* qkv = p.qkv;
  const float* cs = p.rope_cos + (size_t)pos * half;
  const float* sn = p.rope_sin + (size_t)pos * half;
  const float qscale = kLog2e / sqrtf((float)hd);

  for (int i = threadIdx.x; i < G * hd; i += kThreads) {
    const int hq = g * G + i / hd, j = i % hd;
    const float* q = qkv + (size_t)hq * hd;
    const int jj = j < half ? j : j - half;
    const float c = cs[jj], sv = sn[jj];
    const float rot = j < half ? q[j] * c - q[j + half] * sv : q[j] * c + q[j - half] * sv;
    qs[i] = rot * qscale;
  }
  const size_t head_base = ((size_t)l * p.nkv + g) * (size_t)p.cap * hd;
  __half* kcache = p.kc + head_base;
  __half* vcache = p.vc + head_base;
  if (has_new) {
    const float* k = qkv + qd + (size_t)g * hd;
    const float* v = qkv + qd + kd + (size_t)g * hd;
    for (int j = threadIdx.x; j < hd; j += kThreads) {
      const int jj = j < half ? j : j - half;
      const float c = cs[jj], sv = sn[jj];
      const float rot = j < half ? k[j] * c - k[j + half] * sv : k[j] * c + k[j - half] * sv;
      const __half kh = __float2half_rn(rot);
      const __half vh = __float2half_rn(v[j]);
      kcache[(size_t)pos * hd + j] = kh;
      vcache[(size_t)pos * hd + j] = vh;
      kn[j] = __half2float(kh);
      vn[j] = __half2float(vh);
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, sub = lane & 15;
  const int nsub = hd >> 3;
  const bool lane_on = sub < nsub;

  float qr[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[h][e] = lane_on ? qs[h * hd + sub * 8 + e] : 0.f;

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

  constexpr int kStride = kWaves * 4;             // positions per workgroup per step
  constexpr int kAU = 4;                          // steps in flight
  for (int base = p0; base < pend; base += kStride * kAU) {
    u32x4 kr[kAU], vr[kAU];
#pragma unroll
    for (int u = 0; u < kAU; ++u) {
      const int j = base + u * kStride + wave * 4 + grp;
      const bool ok = lane_on && j < pend;
      kr[u] = ok ? ld16(kcache + (size_t)j * hd + sub * 8) : u32x4{0u, 0u, 0u, 0u};
      vr[u] = ok ? ld16(vcache + (size_t)j * hd + sub * 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kAU; ++u) {
      const int j0 = base + u * kStride + wave * 4;   // first position of this wave's step
      if (j0 < pend) {                                // wave-uniform
        const int j = j0 + grp;
        float kf[8], vf[8];
        unpack8(kr[u], kf);
        unpack8(vr[u], vf);
        // a 16-lane group is wholly in or out, and its sums stay in the group
        if (j < pend) consume(kf, vf);
      }
    }
  }
  if (has_new && wave == 0 && grp == 0) {
    float kf[8], vf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kf[e] = lane_on ? kn[sub * 8 + e] : 0.f;
      vf[e] = lane_on ? vn[sub * 8 + e] : 0.f;
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
      const float a = exp2f(m[h] - mn), b = exp2f(mo - mn);
      lsum[h] = lsum[h] * a + lo * b;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ao = __shfl_xor(acc[h][e], o, 64);
        acc[h][e] = acc[h][e] * a + ao * b;
      }
      m[h] = mn;
    }
  }
  const int wstride = hd + 2;
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* st = wst + ((size_t)wave * G + h) * wstride;
      if (lane_on)
#pragma unroll
        for (int e = 0; e < 8; ++e) st[sub * 8 + e] = acc[h][e];
      if (sub == 0) {
        st[hd] = m[h];
        st[hd + 1] = lsum[h];
      }
    }
  }
  __syncthreads();
  // merge the waves in order and write this split's partial
  for (int t = threadIdx.x; t < G * hd; t += kThreads) {
    const int h = t / hd, i = t % hd;
    float M = kNegBig;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wst[((size_t)w * G + h) * wstride + hd]);
    float Ls = 0.f, A = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      const float* st = wst + ((size_t)w * G + h) * wstride;
      const float sc = exp2f(st[hd] - M);
      Ls = fmaf(st[hd + 1], sc, Ls);
      A = fmaf(st[i], sc, A);
    }
    float* out = p.part + ((size_t)(g * G + h) * S + sidx) * wstride;
    out[i] = A;
    if (i == 0) {
      out[hd] = M;
      out[hd + 1] = Ls;
    }
  }
  // publish the partial, count the arrival; the last split merges
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __builtin_amdgcn_s_barrier();
  if (threadIdx.x == 0) {
    const unsigned old =
        __hip_atomic_fetch_add(p.head_ctr + g, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const int last = (old == (unsigned)(S - 1));
    if (last) __hip_atomic_store(p.head_ctr + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  if (!*flag) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int t = threadIdx.x; t < G * hd; t += kThreads) {
    const int h = t / hd, i = t % hd;
    const float* pp = p.part + (size_t)(g * G + h) * S * wstride;
    float M = kNegBig;
    for (int s = 0; s < S; ++s) M = fmaxf(M, pp[(size_t)s * wstride + hd]);
    float Ls = 0.f, A = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* st = pp + (size_t)s * wstride;
      const float sc = exp2f(st[hd] - M);
      Ls = fmaf(st[hd + 1], sc, Ls);
      A = fmaf(st[i], sc, A);
    }
    p.o[(size_t)(g * G + h) * hd + i] = A / Ls;
  }
}

__device__ __forceinline__ void stage_attn(const Params& p, int l, int pos, int wg, Lds s, int* flag) {
  const int G = p.H / p.nkv;
  const int units = p.nkv * p.splits;
  for (int u = wg; u < units; u += p.n_wg) {
    const int g = u / p.splits, sidx = u % p.splits;
    switch (G) {
      case 1: attn_unit<1>(p, l, pos, g, sidx, s.h, flag); break;
      case 2: attn_unit<2>(p, l, pos, g, sidx, s.h, flag); break;
      default: attn_unit<4>(p, l, pos, g, sidx, s.h, flag); break;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Stage: O GEMV + residual.  Rows of x are owned by the same workgroup in
// this stage and in the down stage, so the residual update needs no atomics.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void stage_oproj(const Params& p, int l, const __half* emb_row, int wg, Lds s) {
  const LayerPtrs& w = p.layers[l];
  const int qd = p.H * p.hd;
  copy_to_lds(p.o, qd, s.h);
  int r0, r1;
  even_range(p.d, p.n_wg, wg, r0, r1);
  float* x = p.x;
  const bool first = (l == 0);
  gemv_dispatch(
      r0, r1, qd, s.h, [&](int r) { return w.wo + (size_t)r * qd; },
      [&](int r, float v) { x[r] = (first ? __half2float(emb_row[r]) : x[r]) + v; });
}

// Stage: RMSNorm + paired gate/up GEMV + SwiGLU (dense FFN).
__device__ __forceinline__ void stage_gateup(const Params& p, int l, int wg, Lds s) {
  const LayerPtrs& w = p.layers[l];
  rmsnorm_to_lds(p, p.x, nullptr, w.ffn_norm, s.h, s.red);
  int f0, f1;
  even_range(p.F, p.n_wg, wg, f0, f1);
  const int d = p.d;
  float* u = p.u;
  gemv_pairs_dispatch(
      f0, f1, d, s.h,
      [&](int f, int which) { return (which ? w.w_up : w.w_gate) + (size_t)f * d; },
      [&](int f, float v) { u[f] = v; });
}

// Stage: down GEMV + residual (dense FFN).
__device__ __forceinline__ void stage_down(const Params& p, int l, int wg, Lds s) {
  const LayerPtrs& w = p.layers[l];
  copy_to_lds(p.u, p.F, s.h);
  int r0, r1;
  even_range(p.d, p.n_wg, wg, r0, r1);
  const int F = p.F;
  float* x = p.x;
  gemv_dispatch(
      r0, r1, F, s.h, [&](int r) { return w.w_down + (size_t)r * F; },
      [&](int r, float v) { x[r] = x[r] + v; });
}

// ---------------------------------------------------------------------------
// MoE stages.  Router logits are computed by a few workgroups; after the
// barrier every workgroup derives the same routing (softmax, top-k with the
// lower id on ties) from them, so routing costs one barrier, not two.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void stage_router(const Params& p, int l, int wg, Lds s) {
  const LayerPtrs& w = p.layers[l];
  int r0, r1;
  even_range(p.E, p.n_wg, wg, r0, r1);
  if (r0 >= r1) return;
  rmsnorm_to_lds(p, p.x, nullptr, w.ffn_norm, s.h, s.red);
  const int d = p.d;
  float* out = p.router_logits;
  gemv_dispatch(
      r0, r1, d, s.h, [&](int r) { return w.router + (size_t)r * d; },
      [&](int r, float v) { out[r] = v; });
}

// Routing in LDS: ids[a], wts[a] for the active slots a < topk + nshared
// (routed experts in rank order, then the shared experts with weight 1).
__device__ __forceinline__ void moe_routing(const Params& p, int* ids, float* wts, float* red) {
  const int E = p.E, K = p.topk;
  const float* r = p.router_logits;
  float mx = kNegBig;
  for (int e = 0; e < E; ++e) mx = fmaxf(mx, r[e]);   // same order in every thread
  float den = 0.f;
  for (int e = 0; e < E; ++e) den += __expf(r[e] - mx);
  for (int e = threadIdx.x; e < E; e += kThreads) {
    const float re = r[e];
    int rank = 0;
    for (int j = 0; j < E; ++j) {
      const float rj = r[j];
      rank += (rj > re) || (rj == re && j < e);
    }
    if (rank < K) {
      ids[rank] = e;
      wts[rank] = __expf(re - mx) / den;
    }
  }
  for (int a = threadIdx.x; a < p.nshared; a += kThreads) {
    ids[K + a] = E + a;
    wts[K + a] = 1.0f;
  }
  __syncthreads();
  (void)red;
}

__device__ __forceinline__ void stage_moe_gateup(const Params& p, int l, int step, int wg, Lds s) {
  const LayerPtrs& w = p.layers[l];
  int* ids = reinterpret_cast<int*>(s.red + 2 * kWaves);
  float* wts = s.red + 2 * kWaves + kMaxActiveExperts;
  moe_routing(p, ids, wts, s.red);
  if (p.mode == kDecode && wg == 0 && threadIdx.x < p.topk)
    p.expert_log[((size_t)step * p.L + l) * p.topk + threadIdx.x] = ids[threadIdx.x];
  const int A = p.topk + p.nshared, Fe = p.Fe, d = p.d;
  int f0, f1;
  even_range(A * Fe, p.n_wg, wg, f0, f1);
  if (f0 >= f1) return;
  rmsnorm_to_lds(p, p.x, nullptr, w.ffn_norm, s.h, s.red);
  float* u = p.u;
  gemv_pairs_dispatch(
      f0, f1, d, s.h,
      [&](int f, int which) {
        const int a = f / Fe, ff = f - a * Fe;
        const __half* base = which ? w.e_up : w.e_gate;
        return base + ((size_t)ids[a] * Fe + ff) * d;
      },
      [&](int f, float v) { u[f] = wts[f / Fe] * v; });
}

// Down projection of all active experts as one GEMV whose row r is the
// concatenation of each active expert's down row r (segments of Fe).
template <int NR>
__device__ __forceinline__ void moe_down_rows(const Params& p, const LayerPtrs& w, const int* ids, int r0, int r1,
                              const float* h) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int Fe = p.Fe, d = p.d, A = p.topk + p.nshared;
  const int cps = Fe >> 3;                 // chunks per segment
  const int nch = A * cps;
  const float4* h4 = reinterpret_cast<const float4*>(h);
  for (int g0 = r0 + wave * NR; g0 < r1; g0 += kWaves * NR) {
    const int nvalid = min(NR, r1 - g0);
    float acc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = 0.f;
    for (int c0 = 0; c0 < nch; c0 += 64 * kUnroll) {
      u32x4 wv[NR][kUnroll];
#pragma unroll
      for (int uu = 0; uu < kUnroll; ++uu) {
        const int idx = c0 + uu * 64 + lane;
        const int a = idx / cps, off = idx - a * cps;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int row = min(g0 + r, r1 - 1);
          wv[r][uu] = (idx < nch && r < nvalid)
                          ? ld_stream16(w.e_down + ((size_t)ids[a] * d + row) * Fe + (size_t)off * 8)
                          : u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int uu = 0; uu < kUnroll; ++uu) {
        const int idx = c0 + uu * 64 + lane;
        if (idx < nch) {
          const float4 a = h4[2 * idx], b = h4[2 * idx + 1];
#pragma unroll
          for (int r = 0; r < NR; ++r) acc[r] = dot8(wv[r][uu], a, b, acc[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float v = wave_sum(acc[r]);
      if (r < nvalid && lane == r) p.x[g0 + r] += v;
    }
  }
}

__device__ __forceinline__ void stage_moe_down(const Params& p, int l, int wg, Lds s) {
  const LayerPtrs& w = p.layers[l];
  int* ids = reinterpret_cast<int*>(s.red + 2 * kWaves);
  float* wts = s.red + 2 * kWaves + kMaxActiveExperts;
  moe_routing(p, ids, wts, s.red);
  const int A = p.topk + p.nshared;
  copy_to_lds(p.u, A * p.Fe, s.h);
  int r0, r1;
  even_range(p.d, p.n_wg, wg, r0, r1);
  const int per_wave = (r1 - r0 + kWaves - 1) / kWaves;
  if (per_wave <= 1) moe_down_rows<1>(p, w, ids, r0, r1, s.h);
  else if (per_wave <= 2) moe_down_rows<2>(p, w, ids, r0, r1, s.h);
  else moe_down_rows<4>(p, w, ids, r0, r1, s.h);
}

// ---------------------------------------------------------------------------
// Stage: final RMSNorm + lm_head GEMV + greedy argmax.  Each workgroup
// reduces its rows to one packed key and folds it into the step's slot with
// a 64-bit atomic max (order independent, so deterministic).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void stage_lmhead(const Params& p, int step, int wg, Lds s) {
  rmsnorm_to_lds(p, p.x, nullptr, p.final_norm, s.h, s.red);
  int r0, r1;
  even_range(p.Vout, p.n_wg, wg, r0, r1);
  const int d = p.d;
  float* logits = p.out_logits ? p.out_logits + (size_t)step * p.Vout : nullptr;
  unsigned long long best = 0ull;
  gemv_dispatch(
      r0, r1, d, s.h, [&](int r) { return p.lm_head + (size_t)r * d; },
      [&](int r, float v) {
        if (logits) logits[r] = v;
        const unsigned long long k = argmax_key(v, r);
        best = k > best ? k : best;
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
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------
__device__ __forceinline__ Lds lds_carve(const Params& p, float* smem) {
  const LdsLayout L = lds_layout(p);
  Lds s;
  s.h = smem;
  s.red = smem + L.red_off;
  return s;
}

// The layer loop shared by the persistent kernel (barriers) and nothing
// else; the staged mode launches each stage as its own kernel instead.
__global__ __launch_bounds__(kThreads, 1) void mono_kernel(Params p) {
  extern __shared__ float smem[];
  __shared__ int flag;
  const Lds s = lds_carve(p, smem);
  const int wg = blockIdx.x;
  GridSync gs{p.bar, p.err, 0u, (unsigned)p.n_wg, p.timeout_ticks, p.spin_limit};
  int tok = (p.mode == kDecode) ? p.state[0] : 0;
  for (int step = 0; step < p.n_steps; ++step) {
    const int pos = p.pos0 + step;
    if (p.mode == kPrefill) tok = p.prompt[step];
    const __half* emb = p.tok_emb + (size_t)tok * p.d;
    for (int l = 0; l < p.L; ++l) {
      stage_qkv(p, l, emb, wg, s);
      if (!grid_sync(gs, &flag)) return;
      stage_attn(p, l, pos, wg, s, &flag);
      if (!grid_sync(gs, &flag)) return;
      stage_oproj(p, l, emb, wg, s);
      if (!grid_sync(gs, &flag)) return;
      if (p.E == 0) {
        stage_gateup(p, l, wg, s);
        if (!grid_sync(gs, &flag)) return;
        stage_down(p, l, wg, s);
        if (!grid_sync(gs, &flag)) return;
      } else {
        stage_router(p, l, wg, s);
        if (!grid_sync(gs, &flag)) return;
        stage_moe_gateup(p, l, step, wg, s);
        if (!grid_sync(gs, &flag)) return;
        stage_moe_down(p, l, wg, s);
        if (!grid_sync(gs, &flag)) return;
      }
    }
    if (p.mode == kDecode) {
      stage_lmhead(p, step, wg, s);
      if (!grid_sync(gs, &flag)) return;
      tok = argmax_index(p.amax[step & 1], p.Vout);
      if (wg == 0 && threadIdx.x == 0) {
        p.out_tokens[step] = tok;
        p.amax[(step + 1) & 1] = 0ull;
      }
    }
  }
  if (wg == 0 && threadIdx.x == 0) p.state[0] = (p.mode == kPrefill) ? p.prompt[p.n_steps] : tok;
}

// ---- staged mode: one kernel per stage, the step counter lives on device
enum StageId : int { kSQkv, kSAttn, kSO, kSGateUp, kSDown, kSRouter, kSMoeGateUp, kSMoeDown, kSLm };

__global__ __launch_bounds__(kThreads, 1) void stage_kernel(Params p, int stage, int l) {
  extern __shared__ float smem[];
  __shared__ int flag;
  const Lds s = lds_carve(p, smem);
  const int wg = blockIdx.x;
  const int step = p.state[1];
  const int pos = p.pos0 + step;
  const int tok = (p.mode == kPrefill) ? p.prompt[step] : p.state[0];
  const __half* emb = p.tok_emb + (size_t)tok * p.d;
  switch (stage) {
    case kSQkv: stage_qkv(p, l, emb, wg, s); break;
    case kSAttn: stage_attn(p, l, pos, wg, s, &flag); break;
    case kSO: stage_oproj(p, l, emb, wg, s); break;
    case kSGateUp: stage_gateup(p, l, wg, s); break;
    case kSDown: stage_down(p, l, wg, s); break;
    case kSRouter: stage_router(p, l, wg, s); break;
    case kSMoeGateUp: stage_moe_gateup(p, l, step, wg, s); break;
    case kSMoeDown: stage_moe_down(p, l, wg, s); break;
    case kSLm: stage_lmhead(p, step, wg, s); break;
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
  extern __shared__ float smem[];
  copy_to_lds(x, cols, smem);
  int r0, r1;
  even_range(rows, n_wg, blockIdx.x, r0, r1);
  gemv_dispatch(
      r0, r1, cols, smem, [&](int r) { return w + (size_t)r * cols; },
      [&](int r, float v) { y[r] = v; });
}

__global__ __launch_bounds__(kThreads, 1) void barrier_test_kernel(unsigned* bar, int* slots,
                                                                   int* violations, int* err,
                                                                   int rounds, long long ticks,
                                                                   int spin_limit) {
  __shared__ int flag;
  __shared__ int bad;
  const int nwg = gridDim.x;
  GridSync gs{bar, err, 0u, (unsigned)nwg, ticks, spin_limit};
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  for (int r = 1; r <= rounds; ++r) {
    if (threadIdx.x == 0) slots[blockIdx.x] = r;
    if (!grid_sync(gs, &flag)) return;
    int local = 0;
    for (int j = threadIdx.x; j < nwg; j += kThreads) local += (slots[j] < r);
    if (local) atomicAdd(&bad, local);
    __syncthreads();
    // nobody may run ahead and overwrite a slot before everyone checked it
    if (!grid_sync(gs, &flag)) return;
  }
  if (threadIdx.x == 0 && bad) atomicAdd(violations, bad);
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
int max_blocks_per_cu(size_t lds_bytes) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(mono_kernel),
                                                   kThreads, lds_bytes) != hipSuccess)
    return 0;
  return nb;
}

hipError_t launch_mono(const Params& p, size_t lds_bytes, hipStream_t s) {
  void* args[] = {const_cast<Params*>(&p)};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(mono_kernel), dim3(p.n_wg),
                                    dim3(kThreads), args, (unsigned)lds_bytes, s);
}

hipError_t launch_staged_step(const Params& p, size_t lds_bytes, hipStream_t s) {
  const dim3 grid(p.n_wg), block(kThreads);
  const unsigned lds = (unsigned)lds_bytes;
  for (int l = 0; l < p.L; ++l) {
    hipLaunchKernelGGL(stage_kernel, grid, block, lds, s, p, (int)kSQkv, l);
    hipLaunchKernelGGL(stage_kernel, grid, block, lds, s, p, (int)kSAttn, l);
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

hipError_t launch_gemv(const __half* w, const float* x, float* y, int rows, int cols, int n_wg,
                       hipStream_t s) {
  const size_t lds = (size_t)((cols + 63) & ~63) * sizeof(float);
  hipLaunchKernelGGL(gemv_kernel, dim3(n_wg), dim3(kThreads), (unsigned)lds, s, w, x, y, rows,
                     cols, n_wg);
  return hipGetLastError();
}

hipError_t launch_barrier_test(unsigned* bar, int* slots, int* violations, int* err, int n_wg,
                               int rounds, long long timeout_ticks, int spin_limit,
                               hipStream_t s) {
  void* args[] = {&bar, &slots, &violations, &err, &rounds, &timeout_ticks, &spin_limit};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(barrier_test_kernel),
                                    dim3(n_wg), dim3(kThreads), args, 0u, s);
}

}  // namespace kie
