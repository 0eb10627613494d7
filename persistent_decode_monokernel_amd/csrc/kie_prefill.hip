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
// C[M][N] (+)= (Ahi + Alo)[M][K] * W[N][K]^T with v_mfma_f32_32x32x8_f16.
//
// Block: 4 waves, a 64 x 64 tile of C; wave (wm, wn) owns a 32 x 32 quarter.
// K advances 32 at a time through LDS (rows padded by 8 halves).  Operand
// layout of the 32x32x8 MFMA: lane l holds A[l % 32][4 (l / 32) + i] and
// B[4 (l / 32) + i][l % 32], i < 4, and accumulator j of lane l is
// D[8 (j / 4) + 4 (l / 32) + j % 4][l % 32].  B[k][n] is W[n][k], so both
// operands are read as 4 consecutive halves of a row.
// Requires K % 32 == 0 and 16-byte aligned rows (lda, ldw multiples of 8).
// ---------------------------------------------------------------------------
constexpr int kGT = 64;
constexpr int kGK = 32;
constexpr int kGPad = kGK + 8;

__global__ __launch_bounds__(256) void gemm_kernel(const __half* __restrict__ ahi,
                                                   const __half* __restrict__ alo, int lda,
                                                   const __half* __restrict__ w, int ldw,
                                                   float* __restrict__ c, int ldc, int M, int N, int K,
                                                   int accumulate) {
  __shared__ __attribute__((aligned(16))) _Float16 sAh[kGT * kGPad];
  __shared__ __attribute__((aligned(16))) _Float16 sAl[kGT * kGPad];
  __shared__ __attribute__((aligned(16))) _Float16 sW[kGT * kGPad];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m0 = blockIdx.y * kGT, n0 = blockIdx.x * kGT;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const int lr = tid >> 2, lc = (tid & 3) * 8;      // loader: row lr, 8 halves at column lc
  const bool am = m0 + lr < M, wnok = n0 + lr < N;
  const __half* pa_h = ahi + (size_t)(am ? m0 + lr : 0) * lda + lc;
  const __half* pa_l = alo + (size_t)(am ? m0 + lr : 0) * lda + lc;
  const __half* pw = w + (size_t)(wnok ? n0 + lr : 0) * ldw + lc;
  f16acc acc = {};
  const int ar = (wm + (lane & 31)) * kGPad, br = (wn + (lane & 31)) * kGPad;
  const int kq0 = 4 * (lane >> 5);
  for (int k0 = 0; k0 < K; k0 += kGK) {
    uint4 vh = {0u, 0u, 0u, 0u}, vl = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
    if (am) {
      vh = *reinterpret_cast<const uint4*>(pa_h + k0);
      vl = *reinterpret_cast<const uint4*>(pa_l + k0);
    }
    if (wnok) vw = *reinterpret_cast<const uint4*>(pw + k0);
    __syncthreads();                                 // the previous step's reads are done
    *reinterpret_cast<uint4*>(&sAh[lr * kGPad + lc]) = vh;
    *reinterpret_cast<uint4*>(&sAl[lr * kGPad + lc]) = vl;
    *reinterpret_cast<uint4*>(&sW[lr * kGPad + lc]) = vw;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kGK; kk += 8) {
      const h4 a_h = *reinterpret_cast<const h4*>(&sAh[ar + kk + kq0]);
      const h4 a_l = *reinterpret_cast<const h4*>(&sAl[ar + kk + kq0]);
      const h4 b = *reinterpret_cast<const h4*>(&sW[br + kk + kq0]);
      acc = __builtin_amdgcn_mfma_f32_32x32x8f16(a_h, b, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x8f16(a_l, b, acc, 0, 0, 0);
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

// Causal attention over the cache for a chunk's positions, tiled so that
// the K/V rows staged in LDS serve many query rows: a block takes R / G
// consecutive positions of the chunk and the G query heads that share KV
// head g (blockIdx.y), i.e. R rows (row r = position r / G, query head
// g * G + r % G; R = 64, or 32 for head sizes above 64 so that the block's
// LDS stays under 64 KiB), and walks the cached positions 0 .. (its last
// position) in tiles of kAK.  Each row belongs to TPR = 256 / R adjacent
// threads of one wave: thread i of a row scores keys i, i + TPR, ... of the
// tile in registers, the row's maximum and sum are reduced across the TPR
// lanes (online softmax), and the thread accumulates output dimensions
// [i * hd / TPR, (i + 1) * hd / TPR) of P V.  fp32 throughout; K/V are the
// fp16 cache rows.  Needs hd % 16 == 0.
constexpr int kAK = 64;                       // cached positions per tile
constexpr int kAReg = 16;                     // per-thread registers: keys (kAK / TPR) and dims (hd / TPR)

__host__ __device__ inline int attn_prefill_rows(int hd) { return hd > 64 ? 32 : 64; }

size_t attn_prefill_lds(int hd) {
  const size_t R = (size_t)attn_prefill_rows(hd);
  return sizeof(float) * (R * (hd + 2) + R * (kAK + 1)) +
         sizeof(__half) * ((size_t)kAK * (hd + 2) + (size_t)kAK * hd);
}

template <int TPR>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
template <int TPR>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int TPR>
__device__ __forceinline__ void attn_prefill_body(const float* __restrict__ QKV, int ldq,
                                                  const __half* __restrict__ kc, const __half* __restrict__ vc,
                                                  int cap, int H, int nkv, int hd, int pos0, int T,
                                                  float* __restrict__ O, float* lds) {
  constexpr int R = kPT / TPR, KPT = kAK / TPR;
  const int G = H / nkv, QP = R / G, DPT = hd / TPR;
  const int qs = hd + 2;                     // Q row stride (floats), keeps 2-word reads conflict-free
  const int ks = hd + 2;                     // K row stride (halves), odd in 32-bit words
  float* Qs = lds;                           // [R][hd + 2], pre-scaled
  float* Pm = Qs + (size_t)R * qs;           // [R][kAK + 1] probabilities of the tile
  __half* Ks = reinterpret_cast<__half*>(Pm + (size_t)R * (kAK + 1));   // [kAK][hd + 2]
  __half* Vs = Ks + (size_t)kAK * ks;                                     // [kAK][hd]
  const int t0 = blockIdx.x * QP, g = blockIdx.y;
  const int tn = min(QP, T - t0);
  const float scale = 1.0f / sqrtf((float)hd);
  for (int e = threadIdx.x; e < R * hd; e += kPT) {
    const int r = e / hd, d = e - r * hd;
    const int tq = r / G, h = g * G + r % G;
    Qs[r * qs + d] = tq < tn ? QKV[(size_t)(t0 + tq) * ldq + h * hd + d] * scale : 0.f;
  }
  const int r = threadIdx.x / TPR, i = threadIdx.x - r * TPR;
  const int tq = r / G, pos = pos0 + t0 + tq;
  const bool valid = tq < tn;
  float m = -3.0e38f, l = 0.f, acc[kAReg];
#pragma unroll
  for (int k = 0; k < kAReg; ++k) acc[k] = 0.f;
  const __half* K = kc + (size_t)g * cap * hd;
  const __half* V = vc + (size_t)g * cap * hd;
  const int last = pos0 + t0 + tn - 1;
  const float* qr = Qs + r * qs;
  float* pr = Pm + r * (kAK + 1);
  __syncthreads();
  for (int k0 = 0; k0 <= last; k0 += kAK) {
    const int nk = min(kAK, last + 1 - k0);
    for (int e = threadIdx.x; e < nk * (hd >> 1); e += kPT) {          // 2 halves at a time
      const int j = e / (hd >> 1), d = 2 * (e - j * (hd >> 1));
      *reinterpret_cast<__half2*>(&Ks[j * ks + d]) = *reinterpret_cast<const __half2*>(&K[(size_t)(k0 + j) * hd + d]);
      *reinterpret_cast<__half2*>(&Vs[j * hd + d]) = *reinterpret_cast<const __half2*>(&V[(size_t)(k0 + j) * hd + d]);
    }
    __syncthreads();
    float sc[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) sc[k] = 0.f;
    for (int d = 0; d < hd; d += 2) {
      const float2 q2 = *reinterpret_cast<const float2*>(qr + d);
#pragma unroll
      for (int k = 0; k < KPT; ++k) {
        const float2 k2 = __half22float2(*reinterpret_cast<const __half2*>(&Ks[(i + TPR * k) * ks + d]));
        sc[k] = fmaf(q2.x, k2.x, fmaf(q2.y, k2.y, sc[k]));
      }
    }
    float mx = m;
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int j = i + TPR * k;
      if (!valid || j >= nk || k0 + j > pos) sc[k] = -3.0e38f;
      mx = fmaxf(mx, sc[k]);
    }
    mx = group_max<TPR>(mx);
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const float pk = sc[k] > -1.0e38f ? __expf(sc[k] - mx) : 0.f;
      pr[i + TPR * k] = pk;
      sum += pk;
    }
    sum = group_sum<TPR>(sum);
    const float f = __expf(m - mx);
    l = l * f + sum;
    m = mx;
    __syncthreads();                         // the row's probabilities are in LDS
    const int d0 = i * DPT;
#pragma unroll
    for (int k = 0; k < kAReg; ++k) acc[k] *= f;
    for (int j = 0; j < nk; ++j) {
      const float pj = pr[j];
      const __half* vr = Vs + j * hd + d0;
#pragma unroll
      for (int k = 0; k < kAReg; k += 2) {
        if (k < DPT) {
          const float2 v2 = __half22float2(*reinterpret_cast<const __half2*>(vr + k));
          acc[k] = fmaf(pj, v2.x, acc[k]);
          acc[k + 1] = fmaf(pj, v2.y, acc[k + 1]);
        }
      }
    }
    __syncthreads();                         // before the next tile overwrites K, V and P
  }
  if (valid) {
    const int h = g * G + r % G;
    float* out = O + (size_t)(t0 + tq) * H * hd + h * hd + i * DPT;
    for (int k = 0; k < DPT; ++k) out[k] = acc[k] / l;
  }
}

__global__ __launch_bounds__(kPT) void attn_prefill_kernel(const float* __restrict__ QKV, int ldq,
                                                          const __half* __restrict__ kc,
                                                          const __half* __restrict__ vc, int cap, int H,
                                                          int nkv, int hd, int pos0, int T, float* __restrict__ O) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  if (attn_prefill_rows(hd) == 32)
    attn_prefill_body<8>(QKV, ldq, kc, vc, cap, H, nkv, hd, pos0, T, O, lds);
  else
    attn_prefill_body<4>(QKV, ldq, kc, vc, cap, H, nkv, hd, pos0, T, O, lds);
}

// S = silu(G) * U, split into hi/lo fp16.
__global__ void swiglu_split_kernel(const float* __restrict__ G, const float* __restrict__ U, size_t n,
                                    __half* __restrict__ hi, __half* __restrict__ lo) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const float a = G[i];
    split_store(a / (1.0f + __expf(-a)) * U[i], hi, lo, i);
  }
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
  const size_t lds = attn_prefill_lds(hd);          // < 64 KiB for every head size <= 128
  const int qp = attn_prefill_rows(hd) / (H / nkv);
  hipLaunchKernelGGL(attn_prefill_kernel, dim3((T + qp - 1) / qp, nkv), dim3(kPT), lds, s, QKV, ldq, kc, vc,
                     cap, H, nkv, hd, pos0, T, O);
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
  const dim3 grid((N + kGT - 1) / kGT, (M + kGT - 1) / kGT);
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, s, ahi, alo, lda, w, ldw, c, ldc, M, N, K,
                     accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace kie
