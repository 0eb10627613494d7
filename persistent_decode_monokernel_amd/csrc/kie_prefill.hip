// Batched prefill for gfx950: the prompt's positions go through each layer
// together, so the weight products are dense matrix products (M = tokens)
// and run on the matrix cores (MFMA), while the persistent decode kernel
// keeps the one-token-per-step path.
//
// The pages put the model's matrix multiplies inside one GPU-resident
// program for decode (page "Breaking the memory wall: 3,000 tokens/s
// inference on standard GPUs", agentlenshq.com, section "1. The Monokernel
// Runtime"); a prompt, unlike a decode step, has every position's input up
// front, so its products have M > 1 and are a dense contraction.
//
// Precision.  Weights are fp16.  The fp32 activations are split into two
// fp16 parts, hi = fp16(v) and lo = fp16(v - hi), and each product is
// W * hi + W * lo accumulated in fp32: fp16 x fp16 products are exact in
// fp32, and hi + lo carries ~22 significant bits of v, so the result is an
// fp32 product up to accumulation order.  The arithmetic of every other step
// (RMSNorm, RoPE, attention, SwiGLU, residual) is fp32, and the K/V rows are
// rounded to fp16 (RNE) when stored, as in the decode kernel.
#include "kie_params.h"

namespace kie {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16acc __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// hi/lo split of an fp32 matrix [M][K] (row stride ldx) into fp16 [M][K].
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split_store(float v, __half* hi, __half* lo, size_t i) {
  const __half h = __float2half_rn(v);
  hi[i] = h;
  lo[i] = __float2half_rn(v - __half2float(h));
}

__global__ void split_kernel(const float* __restrict__ x, int ldx, __half* __restrict__ hi,
                             __half* __restrict__ lo, int M, int K) {
  const size_t n = (size_t)M * K;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const size_t m = i / K, k = i - m * K;
    split_store(x[m * ldx + k], hi, lo, i);
  }
}

// ---------------------------------------------------------------------------
// C[M][N] (+)= (Ahi + Alo)[M][K] * W[N][K]^T with v_mfma_f32_32x32x16_f16,
// CDNA4's double-rate fp16 MFMA (16 products of the inner index per
// instruction and output element).
//
// Block: 4 waves, a 64 x 64 WN tile of C (64 rows of A, 64 WN rows of W,
// WN = 1 or 2); wave (wm, wn) owns 32 x 32 WN of it, WN MFMA tiles that
// share the A operands.  WN = 2 serves 128 outputs per A byte (A is sent
// twice, as hi and lo) and is launched where it still gives two blocks per
// CU.
// K advances kGK = 64 at a time through LDS (rows padded by 8 halves); the
// next step's tiles are loaded into registers while the current step's
// MFMAs run.  Operand layout: lane l holds A[l % 32][8 (l / 32) + i] and
// B[8 (l / 32) + i][l % 32], i < 8, and accumulator j of lane l is
// D[8 (j / 4) + 4 (l / 32) + j % 4][l % 32].  A and B are read with the same
// inner-index map, so the contraction is the same whichever of the 16
// inner positions the unit pairs with each register element.  B[k][n] is
// W[n][k], so both operands are read as 8 consecutive halves of a row.
// Requires K % 32 == 0 and 16-byte aligned rows (lda, ldw multiples of 8);
// a last step of 32 is zero-padded.
// ---------------------------------------------------------------------------
constexpr int kGT = 64;                  // rows (positions) per block
constexpr int kGK = 64;
constexpr int kGPad = kGK + 8;
static_assert(kGPad % 8 == 0, "LDS rows must stay 16-byte aligned for the 8-half operand reads");

// Raw buffer loads: an offset past the resource's size reads zeros, so the
// ragged rows and the zero-padded last K step need no branches.
constexpr unsigned kGOff = 0xFFFFFFF0u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void* p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(unsigned)bytes, (int)0x00020000u);
}
__device__ __forceinline__ uint4 gemm_ld(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

//
// Grouped form (tiles != nullptr): row block y takes the rows [tiles[3y],
// tiles[3y + 1]) of A and C (at most 64) and the weight matrix
// w + tiles[3y + 2] * wstride, so the products of several experts over
// their own rows of one compact A run as one launch.
template <int WN>
__global__ __launch_bounds__(256) void gemm_kernel(const __half* __restrict__ ahi,
                                                   const __half* __restrict__ alo, int lda,
                                                   const __half* __restrict__ w, int ldw,
                                                   float* __restrict__ c, int ldc, int M, int N, int K,
                                                   int accumulate, const int* __restrict__ tiles,
                                                   size_t wstride) {
  __shared__ __attribute__((aligned(16))) _Float16 sAh[kGT * kGPad];
  __shared__ __attribute__((aligned(16))) _Float16 sAl[kGT * kGPad];
  constexpr int kGN = kGT * WN;           // output columns per block
  __shared__ __attribute__((aligned(16))) _Float16 sW[kGN * kGPad];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int m0 = blockIdx.y * kGT;
  const int n0 = blockIdx.x * kGN;
  if (tiles) {
    m0 = tiles[3 * blockIdx.y];
    M = tiles[3 * blockIdx.y + 1];
    if (m0 >= M) return;                  // an unused tile slot (the grid covers the most there can be)
    w += (size_t)tiles[3 * blockIdx.y + 2] * wstride;
  }
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32 * WN;
  // loader: row lr, 8 halves at columns lc and lc + 32 of each 64-wide step
  const int lr = tid >> 2, lc = (tid & 3) * 8;
  const __amdgpu_buffer_rsrc_t rh = gemm_rsrc(ahi, (size_t)M * lda * 2);
  const __amdgpu_buffer_rsrc_t rl = gemm_rsrc(alo, (size_t)M * lda * 2);
  const __amdgpu_buffer_rsrc_t rw = gemm_rsrc(w, (size_t)N * ldw * 2);
  const bool am = m0 + lr < M, wnok = n0 + lr < N, wnok2 = WN == 2 && n0 + 64 + lr < N;
  const unsigned abase = (unsigned)((m0 + lr) * lda + lc) * 2u;
  const unsigned wbase = (unsigned)((n0 + lr) * ldw + lc) * 2u;
  const unsigned wbase2 = (unsigned)((n0 + 64 + lr) * ldw + lc) * 2u;
  f16acc acc = {}, acc2 = {};
  const int ar = (wm + (lane & 31)) * kGPad, br = (wn + (lane & 31)) * kGPad, br2 = br + 32 * kGPad;
  const int kin = 8 * (lane >> 5);                 // the lane's inner-index offset
  uint4 h0, h1, l0, l1, w0, w1, v0, v1;
  auto load = [&](int k0) {
    const bool k1in = k0 + 32 < K;
    const unsigned a0 = am ? abase + (unsigned)k0 * 2u : kGOff;
    const unsigned a1 = (am && k1in) ? abase + (unsigned)(k0 + 32) * 2u : kGOff;
    const unsigned b0 = wnok ? wbase + (unsigned)k0 * 2u : kGOff;
    const unsigned b1 = (wnok && k1in) ? wbase + (unsigned)(k0 + 32) * 2u : kGOff;
    h0 = gemm_ld(rh, a0);
    h1 = gemm_ld(rh, a1);
    l0 = gemm_ld(rl, a0);
    l1 = gemm_ld(rl, a1);
    w0 = gemm_ld(rw, b0);
    w1 = gemm_ld(rw, b1);
    if constexpr (WN == 2) {
      v0 = gemm_ld(rw, wnok2 ? wbase2 + (unsigned)k0 * 2u : kGOff);
      v1 = gemm_ld(rw, (wnok2 && k1in) ? wbase2 + (unsigned)(k0 + 32) * 2u : kGOff);
    }
  };
  load(0);
  for (int k0 = 0; k0 < K; k0 += kGK) {
    __syncthreads();                                 // the previous step's reads are done
    const int o = lr * kGPad + lc;
    *reinterpret_cast<uint4*>(&sAh[o]) = h0;
    *reinterpret_cast<uint4*>(&sAh[o + 32]) = h1;
    *reinterpret_cast<uint4*>(&sAl[o]) = l0;
    *reinterpret_cast<uint4*>(&sAl[o + 32]) = l1;
    *reinterpret_cast<uint4*>(&sW[o]) = w0;
    *reinterpret_cast<uint4*>(&sW[o + 32]) = w1;
    if constexpr (WN == 2) {
      *reinterpret_cast<uint4*>(&sW[o + 64 * kGPad]) = v0;
      *reinterpret_cast<uint4*>(&sW[o + 64 * kGPad + 32]) = v1;
    }
    __syncthreads();
    if (k0 + kGK < K) load(k0 + kGK);                // in flight during the MFMAs
#pragma unroll
    for (int kk = 0; kk < kGK; kk += 16) {
      const h8 a_h = *reinterpret_cast<const h8*>(&sAh[ar + kk + kin]);
      const h8 a_l = *reinterpret_cast<const h8*>(&sAl[ar + kk + kin]);
      const h8 b = *reinterpret_cast<const h8*>(&sW[br + kk + kin]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_h, b, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_l, b, acc, 0, 0, 0);
      if constexpr (WN == 2) {
        const h8 b2 = *reinterpret_cast<const h8*>(&sW[br2 + kk + kin]);
        acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_h, b2, acc2, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_l, b2, acc2, 0, 0, 0);
      }
    }
  }
  const int n = n0 + wn + (lane & 31);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int m = m0 + wm + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
    if (m < M && n < N) {
      float* p = c + (size_t)m * ldc + n;
      *p = accumulate ? *p + acc[j] : acc[j];
    }
    if (WN == 2 && m < M && n + 32 < N) {
      float* p = c + (size_t)m * ldc + n + 32;
      *p = accumulate ? *p + acc2[j] : acc2[j];
    }
  }
}

// ---------------------------------------------------------------------------
// The other steps of a layer, over the T positions of a chunk.
// ---------------------------------------------------------------------------
constexpr int kPT = 256;          // threads of the per-position kernels

// Fixed-order block sum over kPT threads (every thread gets the total).
__device__ __forceinline__ float block_sum(float v, float* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int s = kPT / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const float t = red[0];
  __syncthreads();
  return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int s = kPT / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  const float t = red[0];
  __syncthreads();
  return t;
}

// X[t] = fp32(E[tok[t]])
__global__ __launch_bounds__(kPT) void embed_kernel(const __half* __restrict__ emb, const int* __restrict__ tok,
                                                   int d, float* __restrict__ X) {
  const int t = blockIdx.x;
  const __half* row = emb + (size_t)tok[t] * d;
  for (int i = threadIdx.x; i < d; i += kPT) X[(size_t)t * d + i] = __half2float(row[i]);
}

// H[t] = X[t] / sqrt(mean(X[t]^2) + eps) * gain, split into hi/lo fp16.
__global__ __launch_bounds__(kPT) void rmsnorm_split_kernel(const float* __restrict__ X, const __half* __restrict__ gain,
                                                           int d, float eps, __half* __restrict__ hi,
                                                           __half* __restrict__ lo) {
  __shared__ float red[kPT];
  const int t = blockIdx.x;
  const float* x = X + (size_t)t * d;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += kPT) ss = fmaf(x[i], x[i], ss);
  const float inv = 1.0f / sqrtf(block_sum(ss, red) / (float)d + eps);
  for (int i = threadIdx.x; i < d; i += kPT)
    split_store(x[i] * inv * __half2float(gain[i]), hi, lo, (size_t)t * d + i);
}

// Rotate-half RoPE of q (in place) and k at position pos0 + t from the
// host-built angle tables; k and v are rounded to fp16 (RNE) and stored
// into the layer's cache rows kc/vc [nkv][cap][hd].
__global__ __launch_bounds__(kPT) void rope_kv_kernel(float* __restrict__ QKV, int ldq, int H, int nkv, int hd,
                                                     int pos0, const float* __restrict__ cosT,
                                                     const float* __restrict__ sinT, __half* __restrict__ kc,
                                                     __half* __restrict__ vc, int cap) {
  const int t = blockIdx.x, pos = pos0 + t, half = hd >> 1;
  float* q = QKV + (size_t)t * ldq;
  const float* k = q + H * hd;
  const float* v = k + nkv * hd;
  const float* cs = cosT + (size_t)pos * half;
  const float* sn = sinT + (size_t)pos * half;
  for (int e = threadIdx.x; e < H * half; e += kPT) {
    const int h = e / half, j = e - h * half;
    const float a = q[h * hd + j], b = q[h * hd + j + half];
    q[h * hd + j] = a * cs[j] - b * sn[j];
    q[h * hd + j + half] = b * cs[j] + a * sn[j];
  }
  for (int e = threadIdx.x; e < nkv * half; e += kPT) {
    const int g = e / half, j = e - g * half;
    const float a = k[g * hd + j], b = k[g * hd + j + half];
    __half* row = kc + ((size_t)g * cap + pos) * hd;
    row[j] = __float2half_rn(a * cs[j] - b * sn[j]);
    row[j + half] = __float2half_rn(b * cs[j] + a * sn[j]);
  }
  for (int e = threadIdx.x; e < nkv * hd; e += kPT) {
    const int g = e / hd, j = e - g * hd;
    vc[((size_t)g * cap + pos) * hd + j] = __float2half_rn(v[g * hd + j]);
  }
}

// Causal attention over the cache for a chunk's positions, on the matrix
// cores.  A block of 4 waves takes 128 rows: 128 / G consecutive positions
// of the chunk times the G query heads that share KV head g (blockIdx.y);
// row r is position r / G, query head g * G + r % G, and wave w owns rows
// [32 w, 32 w + 32).  The block walks the cached positions 0 .. (its last
// position) in tiles of 32, staged once in LDS for all four waves:
//   S = Q K^T       per wave one 32x32 MFMA tile over hd / 16 steps, Q held
//                   in registers as fp16 hi + lo;
//   online softmax  2 lanes per row: causal mask, running maximum and sum;
//   O = O f + P V   per wave hd / 32 (rounded up) column tiles, P split into
//                   fp16 hi + lo, V staged transposed.
// Scores, P and the rescale factors are per wave, so only the K/V staging
// takes block barriers (two per tile); the rest is ordered within the wave.
// Both products use v_mfma_f32_32x32x16_f16 with the operand and
// accumulator layout of the weight product above; LDS rows are padded by 8
// halves so every 8-half operand read is 16-byte aligned.  K and V are the
// fp16 cache rows, so every product is fp32 up to rounding order.
constexpr int kMK = 32;                       // cached positions per tile
constexpr int kAW = 4;                        // waves per block

// The LDS writes of the calling wave are complete and visible to all its
// lanes (a wave-scope release/acquire around the wave barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
constexpr int kAR = 32 * kAW;                 // query rows per block
constexpr int kQS = kMaxHeadDim + 8;          // K tile row stride (halves)
constexpr int kPS = kMK + 8;                  // P and transposed V row stride (halves)
static_assert(kQS % 8 == 0 && kPS % 8 == 0, "LDS rows must stay 16-byte aligned");

template <int NS>   // NS = hd / 16 inner steps of the score product
__global__ __launch_bounds__(kPT, 2) void attn_prefill_kernel(const float* __restrict__ QKV, int ldq,
                                                          const __half* __restrict__ kc,
                                                          const __half* __restrict__ vc, int cap, int H,
                                                          int nkv, int pos0, int T, float* __restrict__ O) {
  constexpr int hd = 16 * NS, NCT = (NS + 1) / 2, hdp = 32 * NCT;
  __shared__ __attribute__((aligned(16))) _Float16 Ks[kMK * kQS];       // [key][dim]
  __shared__ __attribute__((aligned(16))) _Float16 Vt[kMaxHeadDim * kPS];   // [dim][key]
  __shared__ __attribute__((aligned(16))) _Float16 Ph[kAW][32 * kPS];
  __shared__ __attribute__((aligned(16))) _Float16 Pl[kAW][32 * kPS];
  __shared__ float Sw[kAW][32 * (kMK + 1)];
  __shared__ float rfw[kAW][32];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int G = H / nkv, QP = kAR / G;
  const int t0 = blockIdx.x * QP, g = blockIdx.y;
  const int tn = min(QP, T - t0);
  const float scale = 1.0f / sqrtf((float)hd);
  // kq0: accumulator row offset of the lane; kin: its inner-index offset
  const int kq0 = 4 * (lane >> 5), kin = 8 * (lane >> 5), l32 = lane & 31;
  // this lane's query row as an MFMA A operand, split hi/lo, per 16-wide step
  h8 qh[NS], ql[NS];
  {
    const int r = wave * 32 + l32, tq = r / G, h = g * G + r % G;
    const float* q = QKV + (size_t)(t0 + tq) * ldq + h * hd + kin;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = tq < tn ? q[16 * s + i] * scale : 0.f;
        const _Float16 hi = (_Float16)v;
        qh[s][i] = hi;
        ql[s][i] = (_Float16)(v - (float)hi);
      }
    }
  }
  for (int e = tid; e < (hdp - hd) * kPS; e += kPT) Vt[hd * kPS + e] = (_Float16)0.f;   // padded columns
  // softmax lanes: row sr of the wave, keys si, si + 2, ... of the tile
  const int sr = lane >> 1, si = lane & 1;
  const int stq = (wave * 32 + sr) / G, spos = pos0 + t0 + stq;
  const bool svalid = stq < tn;
  float rm = -3.0e38f, rl = 0.f;
  // the wave's last position, and the block's
  const int wlast = pos0 + t0 + min(tn - 1, (wave * 32 + 31) / G);
  const bool wactive = wave * 32 / G < tn;
  const int last = pos0 + t0 + tn - 1;
  f16acc acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = (f16acc){};
  const __half* K = kc + (size_t)g * cap * hd;
  const __half* V = vc + (size_t)g * cap * hd;
  // K/V tile staging: 16-byte chunks e = tid, tid + 256 of the tile's 32 rows;
  // K puts a row's chunks on neighbouring lanes, V the rows.  Two register
  // stages alternate by tile, so each tile's K/V is loaded two tiles ahead.
  constexpr int kC = hd / 8;                         // 16-byte chunks per row
  constexpr int kIt = (kMK * kC + kPT - 1) / kPT;    // 1 or 2
  uint4 kpre[2][kIt];
  h8 vpre[2][kIt];
  auto kv_load = [&](int r, int k0) {
    const int nk = min(kMK, last + 1 - k0);
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int e = tid + it * kPT;
      if (e < kMK * kC) {
        const int jk = e / kC, ck = e - jk * kC, jv = e & (kMK - 1), cv = e / kMK;
        kpre[r][it] = *reinterpret_cast<const uint4*>(K + (size_t)(k0 + (jk < nk ? jk : 0)) * hd + 8 * ck);
        if (jk >= nk) kpre[r][it] = make_uint4(0u, 0u, 0u, 0u);
        vpre[r][it] = *reinterpret_cast<const h8*>(V + (size_t)(k0 + (jv < nk ? jv : 0)) * hd + 8 * cv);
        if (jv >= nk) vpre[r][it] = (h8){};
      }
    }
  };
  auto tile = [&](int r, int k0) {
    const int nk = min(kMK, last + 1 - k0);
    const bool run = wactive && k0 <= wlast;        // the tile holds keys some row of the wave sees
    __syncthreads();                                 // the previous tile's reads are done
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int e = tid + it * kPT;
      if (e < kMK * kC) {
        const int jk = e / kC, ck = e - jk * kC, jv = e & (kMK - 1), cv = e / kMK;
        *reinterpret_cast<uint4*>(&Ks[jk * kQS + 8 * ck]) = kpre[r][it];
#pragma unroll
        for (int i = 0; i < 8; ++i) Vt[(8 * cv + i) * kPS + jv] = vpre[r][it][i];
      }
    }
    __syncthreads();
    if (k0 + 2 * kMK <= last) kv_load(r, k0 + 2 * kMK);   // two tiles ahead
    if (run) {
      f16acc sa = {};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const h8 b = *reinterpret_cast<const h8*>(&Ks[l32 * kQS + 16 * s + kin]);
        sa = __builtin_amdgcn_mfma_f32_32x32x16_f16(qh[s], b, sa, 0, 0, 0);
        sa = __builtin_amdgcn_mfma_f32_32x32x16_f16(ql[s], b, sa, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) Sw[wave][(8 * (j >> 2) + kq0 + (j & 3)) * (kMK + 1) + l32] = sa[j];
      wave_sync();                                   // Sw[wave] is the wave's own
      float sc[16];
      float mx = rm;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int j = si + 2 * k;
        float v = Sw[wave][sr * (kMK + 1) + j];
        if (!svalid || j >= nk || k0 + j > spos) v = -3.0e38f;
        sc[k] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float pk = sc[k] > -1.0e38f ? __expf(sc[k] - mx) : 0.f;
        const _Float16 hi = (_Float16)pk;
        Ph[wave][sr * kPS + si + 2 * k] = hi;
        Pl[wave][sr * kPS + si + 2 * k] = (_Float16)(pk - (float)hi);
        sum += pk;
      }
      sum += __shfl_xor(sum, 1, 64);
      const float f = __expf(rm - mx);
      rl = rl * f + sum;
      rm = mx;
      if (si == 0) rfw[wave][sr] = f;
      wave_sync();                                   // so are Ph, Pl and rfw[wave]
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[c][j] *= rfw[wave][8 * (j >> 2) + kq0 + (j & 3)];
      }
#pragma unroll
      for (int kk = 0; kk < kMK; kk += 16) {
        const h8 a_h = *reinterpret_cast<const h8*>(&Ph[wave][l32 * kPS + kk + kin]);
        const h8 a_l = *reinterpret_cast<const h8*>(&Pl[wave][l32 * kPS + kk + kin]);
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          const h8 b = *reinterpret_cast<const h8*>(&Vt[(32 * c + l32) * kPS + kk + kin]);
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_h, b, acc[c], 0, 0, 0);
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_l, b, acc[c], 0, 0, 0);
        }
      }
    }
  };
  kv_load(0, 0);
  if (kMK <= last) kv_load(1, kMK);
  for (int k0 = 0; k0 <= last; k0 += 2 * kMK) {
    tile(0, k0);
    if (k0 + kMK <= last) tile(1, k0 + kMK);
  }
  // the row sums, from the softmax lanes to the accumulator lanes
  __syncthreads();
  if (si == 0) rfw[wave][sr] = rl;
  __syncthreads();
  if (!wactive) return;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int rw = 8 * (j >> 2) + kq0 + (j & 3), r = wave * 32 + rw;
    const int tq = r / G;
    if (tq >= tn) continue;
    const float l = rfw[wave][rw];
    float* out = O + (size_t)(t0 + tq) * H * hd + (g * G + r % G) * hd;
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int d = 32 * c + l32;
      if (d < hd) out[d] = acc[c][j] / l;
    }
  }
}

// S = silu(G) * U, split into hi/lo fp16.
__global__ void swiglu_split_kernel(const float* __restrict__ G, const float* __restrict__ U, size_t n,
                                    __half* __restrict__ hi, __half* __restrict__ lo) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const float a = G[i];
    split_store(a / (1.0f + __expf(-a)) * U[i], hi, lo, i);
  }
}

// ---------------------------------------------------------------------------
// Mixture-of-experts FFN over a chunk: routing per position, then the
// positions grouped by expert (the host builds the grouping from the
// routing) so each expert's products are dense products over its rows.
// ---------------------------------------------------------------------------
// Routing of position t from its router logits R[t][E]: softmax in fp32, the
// top_k probabilities (lower id on ties) as ids[t][a] and weights wts[t][a]
// in rank order (rescaled to sum to 1 with renorm); the ids also go to the
// routing record by position.  One block per position.
__global__ __launch_bounds__(kPT) void route_kernel(const float* __restrict__ R, int E, int topk, int renorm,
                                                   int* __restrict__ ids, float* __restrict__ wts,
                                                   int* __restrict__ log, int L, int l, int pos0) {
  __shared__ float red[kPT];
  __shared__ float sw[kMaxActiveExperts];
  const int t = blockIdx.x;
  const float* r = R + (size_t)t * E;
  float mx = -3.0e38f;
  for (int e = threadIdx.x; e < E; e += kPT) mx = fmaxf(mx, r[e]);
  mx = block_max(mx, red);
  float den = 0.f;
  for (int e = threadIdx.x; e < E; e += kPT) den += __expf(r[e] - mx);
  den = block_sum(den, red);
  for (int e = threadIdx.x; e < E; e += kPT) {
    const float re = r[e];
    int rank = 0;
    for (int j = 0; j < E; ++j) {
      const float rj = r[j];
      rank += (rj > re) || (rj == re && j < e);
    }
    if (rank < topk) {
      ids[t * topk + rank] = e;
      sw[rank] = __expf(re - mx) / den;
      log[((size_t)(pos0 + t) * L + l) * topk + rank] = e;
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < topk) {
    float sel = 1.f;
    if (renorm) {
      sel = 0.f;
      for (int a = 0; a < topk; ++a) sel += sw[a];
    }
    wts[t * topk + threadIdx.x] = sw[threadIdx.x] / sel;
  }
}

// Compact row q takes position perm[q] / topk: its hi/lo input row.
__global__ __launch_bounds__(kPT) void gather_rows_kernel(const __half* __restrict__ hi, const __half* __restrict__ lo,
                                                         int d, const int* __restrict__ perm, int topk,
                                                         __half* __restrict__ ch, __half* __restrict__ cl) {
  const int q = blockIdx.x, t = perm[q] / topk;
  for (int i = threadIdx.x; i < d; i += kPT) {
    ch[(size_t)q * d + i] = hi[(size_t)t * d + i];
    cl[(size_t)q * d + i] = lo[(size_t)t * d + i];
  }
}

// S[q] = w[q] * silu(G[q]) * U[q] over rows q < rows, split into hi/lo; the
// weight of compact row q is wts[perm[q]] (or 1 without perm).
__global__ void swiglu_w_split_kernel(const float* __restrict__ G, const float* __restrict__ U, int F, int rows,
                                      const int* __restrict__ perm, const float* __restrict__ wts,
                                      __half* __restrict__ hi, __half* __restrict__ lo) {
  const size_t n = (size_t)rows * F;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int q = (int)(i / F);
    const float w = perm ? wts[perm[q]] : 1.f;
    const float a = G[i];
    split_store(w * (a / (1.0f + __expf(-a)) * U[i]), hi, lo, i);
  }
}

// X[t] += sum over a < topk (rank order) of Y[inv[t * topk + a]].
__global__ __launch_bounds__(kPT) void combine_kernel(float* __restrict__ X, int d, const float* __restrict__ Y,
                                                     const int* __restrict__ inv, int topk) {
  const int t = blockIdx.x;
  for (int i = threadIdx.x; i < d; i += kPT) {
    float v = 0.f;
    for (int a = 0; a < topk; ++a) v += Y[(size_t)inv[t * topk + a] * d + i];
    X[(size_t)t * d + i] += v;
  }
}

// Groups the compact rows by expert on the device.  moe_group_kernel (one
// block) counts the rows of each expert, places each expert's rows at the
// exclusive prefix sum of the counts (fill[e] = first row of expert e) and
// writes the row tiles: expert e's rows in tiles of at most 64, in expert
// order, and every tile slot past the last one empty.  moe_scatter_kernel
// then gives each row i its compact row q by an atomic increment of its
// expert's fill.  The order of rows within an expert is not fixed, but no
// result depends on it: each compact row's products are computed on their
// own, and the combine sums a position's experts in rank order.
constexpr int kGroupThreads = 1024;
__global__ __launch_bounds__(kGroupThreads) void moe_group_kernel(const int* __restrict__ ids, int rows, int E,
                                                                 int* __restrict__ fill, int* __restrict__ tiles,
                                                                 int max_tiles) {
  __shared__ int cnt[kGroupThreads], off[kGroupThreads], toff[kGroupThreads];
  const int t = threadIdx.x;
  cnt[t] = 0;
  __syncthreads();
  for (int i = t; i < rows; i += kGroupThreads) atomicAdd(&cnt[ids[i]], 1);
  __syncthreads();
  const int c = t < E ? cnt[t] : 0;
  const int tc = (c + 63) / 64;
  off[t] = c;
  toff[t] = tc;
  __syncthreads();
  for (int o = 1; o < kGroupThreads; o <<= 1) {       // inclusive scans of counts and tile counts
    const int a = t >= o ? off[t - o] : 0;
    const int b = t >= o ? toff[t - o] : 0;
    __syncthreads();
    off[t] += a;
    toff[t] += b;
    __syncthreads();
  }
  const int r0 = off[t] - c, y0 = toff[t] - tc;
  if (t < E) {
    fill[t] = r0;
    for (int j = 0; j < tc; ++j) {
      const int y = y0 + j;
      tiles[3 * y] = r0 + 64 * j;
      tiles[3 * y + 1] = min(r0 + 64 * (j + 1), r0 + c);
      tiles[3 * y + 2] = t;
    }
  }
  for (int y = toff[kGroupThreads - 1] + t; y < max_tiles; y += kGroupThreads) {
    tiles[3 * y] = 0;
    tiles[3 * y + 1] = 0;
    tiles[3 * y + 2] = 0;
  }
}

__global__ __launch_bounds__(kPT) void moe_scatter_kernel(const int* __restrict__ ids, int rows,
                                                          int* __restrict__ fill, int* __restrict__ perm,
                                                          int* __restrict__ inv) {
  const int i = blockIdx.x * kPT + threadIdx.x;
  if (i < rows) {
    const int q = atomicAdd(&fill[ids[i]], 1);
    perm[q] = i;
    inv[i] = q;
  }
}

hipError_t launch_moe_group(const int* ids, int rows, int E, int* fill, int* tiles, int max_tiles, int* perm,
                            int* inv, hipStream_t s) {
  if (E > kGroupThreads) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(kGroupThreads), 0, s, ids, rows, E, fill, tiles, max_tiles);
  if (rows > 0)
    hipLaunchKernelGGL(moe_scatter_kernel, dim3((rows + kPT - 1) / kPT), dim3(kPT), 0, s, ids, rows, fill, perm,
                       inv);
  return hipGetLastError();
}

hipError_t launch_route(const float* R, int E, int topk, int renorm, int* ids, float* wts, int* log, int L, int l,
                        int pos0, int T, hipStream_t s) {
  hipLaunchKernelGGL(route_kernel, dim3(T), dim3(kPT), 0, s, R, E, topk, renorm, ids, wts, log, L, l, pos0);
  return hipGetLastError();
}
hipError_t launch_gather_rows(const __half* hi, const __half* lo, int d, const int* perm, int topk, __half* ch,
                              __half* cl, int rows, hipStream_t s) {
  hipLaunchKernelGGL(gather_rows_kernel, dim3(rows), dim3(kPT), 0, s, hi, lo, d, perm, topk, ch, cl);
  return hipGetLastError();
}
hipError_t launch_swiglu_w_split(const float* G, const float* U, int F, int rows, const int* perm, const float* wts,
                                 __half* hi, __half* lo, hipStream_t s) {
  const size_t blocks = ((size_t)rows * F + 255) / 256;
  const int grid = (int)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(swiglu_w_split_kernel, dim3(grid), dim3(256), 0, s, G, U, F, rows, perm, wts, hi, lo);
  return hipGetLastError();
}
hipError_t launch_combine(float* X, int d, const float* Y, const int* inv, int topk, int T, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(kPT), 0, s, X, d, Y, inv, topk);
  return hipGetLastError();
}

hipError_t launch_embed(const __half* emb, const int* tok, int d, float* X, int T, hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3(T), dim3(kPT), 0, s, emb, tok, d, X);
  return hipGetLastError();
}
hipError_t launch_rmsnorm_split(const float* X, const __half* gain, int d, float eps, __half* hi, __half* lo,
                                int T, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_split_kernel, dim3(T), dim3(kPT), 0, s, X, gain, d, eps, hi, lo);
  return hipGetLastError();
}
hipError_t launch_rope_kv(float* QKV, int ldq, int H, int nkv, int hd, int pos0, const float* cosT,
                          const float* sinT, __half* kc, __half* vc, int cap, int T, hipStream_t s) {
  hipLaunchKernelGGL(rope_kv_kernel, dim3(T), dim3(kPT), 0, s, QKV, ldq, H, nkv, hd, pos0, cosT, sinT, kc,
                     vc, cap);
  return hipGetLastError();
}
hipError_t launch_attn_prefill(const float* QKV, int ldq, const __half* kc, const __half* vc, int cap, int H,
                               int nkv, int hd, int pos0, float* O, int T, hipStream_t s) {
  const int qp = kAR / (H / nkv);                   // positions per block (H / nkv is 1, 2 or 4)
  const dim3 grid((T + qp - 1) / qp, nkv);
  switch (hd / 16) {
#define KIE_ATTN_CASE(ns)                                                                                     \
  case ns:                                                                                                    \
    hipLaunchKernelGGL(attn_prefill_kernel<ns>, grid, dim3(kPT), 0, s, QKV, ldq, kc, vc, cap, H, nkv, pos0, T, O); \
    break;
    KIE_ATTN_CASE(1) KIE_ATTN_CASE(2) KIE_ATTN_CASE(3) KIE_ATTN_CASE(4)
    KIE_ATTN_CASE(5) KIE_ATTN_CASE(6) KIE_ATTN_CASE(7) KIE_ATTN_CASE(8)
#undef KIE_ATTN_CASE
    default:
      return hipErrorInvalidValue;                  // head_dim must be 16, 32, ..., 128
  }
  return hipGetLastError();
}
hipError_t launch_swiglu_split(const float* G, const float* U, size_t n, __half* hi, __half* lo,
                               hipStream_t s) {
  const size_t blocks = (n + 255) / 256;
  const int grid = (int)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(swiglu_split_kernel, dim3(grid), dim3(256), 0, s, G, U, n, hi, lo);
  return hipGetLastError();
}

hipError_t launch_split(const float* x, int ldx, __half* hi, __half* lo, int M, int K, hipStream_t s) {
  const size_t n = (size_t)M * K;
  const size_t blocks = (n + 255) / 256;
  const int grid = (int)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(split_kernel, dim3(grid), dim3(256), 0, s, x, ldx, hi, lo, M, K);
  return hipGetLastError();
}

hipError_t launch_gemm(const __half* ahi, const __half* alo, int lda, const __half* w, int ldw, float* c,
                       int ldc, int M, int N, int K, bool accumulate, hipStream_t s) {
  const int rows = (M + kGT - 1) / kGT, wide = (N + 2 * kGT - 1) / (2 * kGT);
  if (wide * rows >= 512) {                         // two 64 x 128 blocks per CU or more
    hipLaunchKernelGGL(gemm_kernel<2>, dim3(wide, rows), dim3(256), 0, s, ahi, alo, lda, w, ldw, c, ldc, M,
                       N, K, accumulate ? 1 : 0, (const int*)nullptr, (size_t)0);
  } else {
    hipLaunchKernelGGL(gemm_kernel<1>, dim3((N + kGT - 1) / kGT, rows), dim3(256), 0, s, ahi, alo, lda, w,
                       ldw, c, ldc, M, N, K, accumulate ? 1 : 0, (const int*)nullptr, (size_t)0);
  }
  return hipGetLastError();
}
hipError_t launch_gemm_grouped(const __half* ahi, const __half* alo, int lda, const __half* w, size_t wstride,
                               int ldw, float* c, int ldc, const int* tiles, int ntiles, int N, int K,
                               hipStream_t s) {
  if (ntiles == 0) return hipSuccess;
  const int wide = (N + 2 * kGT - 1) / (2 * kGT);
  if (wide * ntiles >= 512) {                       // two 64 x 128 blocks per CU or more
    hipLaunchKernelGGL(gemm_kernel<2>, dim3(wide, ntiles), dim3(256), 0, s, ahi, alo, lda, w, ldw, c, ldc, 0, N,
                       K, 0, tiles, wstride);
  } else {
    hipLaunchKernelGGL(gemm_kernel<1>, dim3((N + kGT - 1) / kGT, ntiles), dim3(256), 0, s, ahi, alo, lda, w,
                       ldw, c, ldc, 0, N, K, 0, tiles, wstride);
  }
  return hipGetLastError();
}

}  // namespace kie
