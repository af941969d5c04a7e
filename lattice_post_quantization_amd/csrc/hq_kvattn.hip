// Decode attention over a compressed (E8, tile 128, optionally dithered)
// K/V cache, in the rotated domain.
//
// Passages: [ICLR abstract] "HyperQuant: A Near-Entropy-Optimal Lattice
// Quantization Pipeline ..." (subtractive dither keeps each cached inner
// product unbiased; algebraic decoding); [arXiv abstract] "HyperQuant: A
// Rate-Distortion-Optimal Quantization Pipeline ..." ideas (i)-(iv).
//
// A cached vector decodes to s (.) H yhat / sqrt(n), yhat = Delta (p - d).
// For query j, tau q_j . khat_k = <H (s_K (.) q_j) tau / sqrt(n), yhatK_k>,
// and sum_k a_jk vhat_k = s_V (.) H (sum_k a_jk yhatV_k) / sqrt(n): keys and
// values stay in the lattice domain, each query is rotated once before and
// its weighted value sum once after.
//
// rotate_kernel: qr = H (s_K (.) q) tau log2(e) / sqrt(n) (fp64 butterflies,
// one fp32 rounding), so scores come out in base-2 exponent units.
// attn_kernel: a block owns a range of keys of one head and up to 4 of its
// queries (8 from LDS when a head has more), each wave a quarter of the
// range; lane
// (r, b) = (lane / 16, lane % 16) decodes E8 block b of keys k0 + 4 i + r for
// K and V (the dither regenerated from the encoder's counter hash and E8
// decision), the block's partial score is summed over the 16 lanes of its
// key, and an online softmax keeps a wave-uniform running maximum per query
// (m), each lane's share of the exponent sum (l) and of the weighted yhatV
// (8 coordinates per query).  The four key residues are summed at the end,
// the four waves merged through LDS in wave order, and the range's
// (m, l, acc) written out.
// combine_kernel: per head and query, the ranges in order: M = max m,
// L = sum l 2^(m - M), acc likewise; out = s_V (.) H (acc / L) / sqrt(n) in
// fp64.
#include "hq.h"
#include "hq_device.h"
#include "hq_kvattn.h"
#include "hq_dither.h"

namespace hq {
namespace {

constexpr int kHd = 128;

__global__ __launch_bounds__(kHd) void rotate_kernel(AttnLaunch a) {
  __shared__ double v[kHd];
  const int j = threadIdx.x;
  const int64_t c = (int64_t)blockIdx.x * kHd + j;
  const bool neg = (a.k_signs[j >> 5] >> (j & 31)) & 1u;
  const double x = (double)a.q[c];
  v[j] = neg ? -x : x;
  __syncthreads();
#pragma unroll
  for (int h = 1; h < kHd; h <<= 1) {
    const double mine = v[j], other = v[j ^ h];
    __syncthreads();
    v[j] = (j & h) ? other - mine : mine + other;
    __syncthreads();
  }
  a.qr[c] = (float)(v[j] * a.q_scale);
}

// yhat of E8 block b of a cached vector: stored bytes d0, d1 (z0..z6, t7),
// coset bit c, scale delta; with the dither, d = w - Q_E8(w) for the
// vector's counter-hash box sample w (global vector index vec).
__device__ inline void block_yhat(uint32_t d0, uint32_t d1, int c, float delta, bool dither,
                                  uint32_t seed, uint64_t vec, int b, float* y) {
  int32_t s[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[i] = __builtin_amdgcn_sbfe((int32_t)d0, 8 * i, 8);
    s[4 + i] = __builtin_amdgcn_sbfe((int32_t)d1, 8 * i, 8);
  }
  const int32_t par = s[0] + s[1] + s[2] + s[3] + s[4] + s[5] + s[6];
  int32_t P[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int32_t z = (i == 7) ? 2 * s[7] + (par & 1) : s[i];
    P[i] = 2 * z + c;
  }
  if (dither) {
    int32_t W[8], d24[8];                          // w and d in 2^-24 units
    const DitherVec dk = dither_vec(seed, vec);
#pragma unroll
    for (int i = 0; i < 8; ++i) W[i] = dither_w(dk, (uint32_t)(8 * b + i));
    e8_dither_block(W, d24);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      y[i] = delta * ((float)P[i] * 0.5f - (float)d24[i] * 5.9604644775390625e-08f);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = delta * ((float)P[i] * 0.5f);
  }
}

__device__ inline float sum16(float x) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <int QG>
__global__ __launch_bounds__(256) void attn_kernel(AttnLaunch a) {
  constexpr bool kLdsQ = QG > 4;     // queries read from LDS at each step
  __shared__ float wm[4][QG], wl[4][QG];
  __shared__ float wacc[4][QG][kHd];
  __shared__ float4 qs[kLdsQ ? QG : 1][kHd / 4];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t range = blockIdx.x, head = blockIdx.z;
  const int r = lane >> 4, b = lane & 15;
  const int64_t q0 = (int64_t)blockIdx.y * QG;
  const int nq = (int)(a.n_q - q0 < QG ? a.n_q - q0 : QG);
  // this wave's keys (possibly none at the end of the head)
  const int64_t k_begin0 = (range * 4 + w) * a.keys_per_wave;
  const int64_t k_begin = k_begin0 < a.n_keys ? k_begin0 : a.n_keys;
  const int64_t k_end = k_begin + a.keys_per_wave < a.n_keys ? k_begin + a.keys_per_wave
                                                             : a.n_keys;
  const int64_t kv0 = head * a.n_keys;             // the head's first vector
  const float* qr = a.qr + (head * a.n_q + q0) * kHd;

  // the queries' coordinates of block b: registers, or LDS for 8 queries
  float qv[kLdsQ ? 1 : QG][8];
  if constexpr (kLdsQ) {
    for (int e = threadIdx.x; e < QG * (kHd / 4); e += 256) {
      const int jj = e / (kHd / 4) < nq ? e / (kHd / 4) : 0;
      qs[e / (kHd / 4)][e % (kHd / 4)] =
          reinterpret_cast<const float4*>(qr + jj * kHd)[e % (kHd / 4)];
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int j = 0; j < QG; ++j) {
      const int jj = j < nq ? j : 0;
      const float4 lo = *reinterpret_cast<const float4*>(qr + jj * kHd + 8 * b);
      const float4 hi = *reinterpret_cast<const float4*>(qr + jj * kHd + 8 * b + 4);
      qv[j][0] = lo.x; qv[j][1] = lo.y; qv[j][2] = lo.z; qv[j][3] = lo.w;
      qv[j][4] = hi.x; qv[j][5] = hi.y; qv[j][6] = hi.z; qv[j][7] = hi.w;
    }
  }
  float m[QG], l[QG], acc[QG][8];
#pragma unroll
  for (int j = 0; j < QG; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = 0.0f;
  }

  const int64_t steps = (k_end - k_begin + 3) / 4;
  for (int64_t st = 0; st < steps; ++st) {
    const int64_t key_raw = k_begin + 4 * st + r;
    const bool live = key_raw < k_end;
    const int64_t key = kv0 + (live ? key_raw : k_end - 1);   // loads stay inside the cache
    const uint2 kb = *reinterpret_cast<const uint2*>(a.k_idx + key * kHd + 8 * b);
    const uint2 vb = *reinterpret_cast<const uint2*>(a.v_idx + key * kHd + 8 * b);
    float yk[8], yv[8];
    block_yhat(kb.x, kb.y, (int)((a.k_coset[key] >> b) & 1u), a.k_scale[key], a.k_dither,
               a.k_seed, (uint64_t)(a.k_base + key), b, yk);
    block_yhat(vb.x, vb.y, (int)((a.v_coset[key] >> b) & 1u), a.v_scale[key], a.v_dither,
               a.v_seed, (uint64_t)(a.v_base + key), b, yv);
#pragma unroll
    for (int j = 0; j < QG; ++j) {
      float q8[8];
      if constexpr (kLdsQ) {
        const float4 lo = qs[j][2 * b], hi = qs[j][2 * b + 1];
        q8[0] = lo.x; q8[1] = lo.y; q8[2] = lo.z; q8[3] = lo.w;
        q8[4] = hi.x; q8[5] = hi.y; q8[6] = hi.z; q8[7] = hi.w;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) q8[i] = qv[j][i];
      }
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) part = fmaf(q8[i], yk[i], part);
      float s = sum16(part);                       // this key's score (log2 units)
      if (!live) s = -INFINITY;
      float smax = fmaxf(s, __shfl_xor(s, 16, 64));
      smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
      const float m_new = fmaxf(m[j], smax);       // finite: every step has a live key
      const float sc = exp2f(m[j] - m_new);
      const float p = exp2f(s - m_new);
      l[j] = fmaf(l[j], sc, p);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[j][i] = fmaf(acc[j][i], sc, p * yv[i]);
      m[j] = m_new;
    }
  }
  // sum the four key residues (a wave without keys has m = -inf, l = 0)
#pragma unroll
  for (int j = 0; j < QG; ++j) {
    l[j] += __shfl_xor(l[j], 16, 64);
    l[j] += __shfl_xor(l[j], 32, 64);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[j][i] += __shfl_xor(acc[j][i], 16, 64);
      acc[j][i] += __shfl_xor(acc[j][i], 32, 64);
    }
  }
  if (r == 0) {
#pragma unroll
    for (int j = 0; j < QG; ++j) {
      if (b == 0) {
        wm[w][j] = m[j];
        wl[w][j] = l[j];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) wacc[w][j][8 * b + i] = acc[j][i];
    }
  }
  __syncthreads();
  // merge the four waves in order: thread (j, d) for j < nq
  const int jt = threadIdx.x >> 7, d = threadIdx.x & 127;
#pragma unroll
  for (int jb = 0; jb < QG; jb += 2) {
    const int j = jb + jt;
    if (j >= nq) continue;
    float M = wm[0][j];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, wm[ww][j]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = wm[ww][j] == -INFINITY ? 0.0f : exp2f(wm[ww][j] - M);
      L = fmaf(wl[ww][j], f, L);
      O = fmaf(wacc[ww][j][d], f, O);
    }
    float* dst = a.part + ((head * a.n_ranges + range) * a.n_q + q0 + j) * (2 + kHd);
    if (d == 0) {
      dst[0] = M;
      dst[1] = L;
    }
    dst[2 + d] = O;
  }
}

__global__ __launch_bounds__(kHd) void combine_kernel(AttnLaunch a) {
  __shared__ double v[kHd];
  const int d = threadIdx.x;
  const int64_t qj = blockIdx.x, head = blockIdx.y;
  const int64_t stride = a.n_q * (2 + kHd);
  const float* p0 = a.part + (head * a.n_ranges * a.n_q + qj) * (2 + kHd);
  float M = -INFINITY;
#pragma unroll 8
  for (int64_t s = 0; s < a.n_ranges; ++s) M = fmaxf(M, p0[s * stride]);
  float L = 0.0f, O = 0.0f;
#pragma unroll 8
  for (int64_t s = 0; s < a.n_ranges; ++s) {
    const float* p = p0 + s * stride;
    const float f = exp2f(p[0] - M);
    L = fmaf(p[1], f, L);
    O = fmaf(p[2 + d], f, O);
  }
  v[d] = (double)O / (double)L;
  __syncthreads();
#pragma unroll
  for (int h = 1; h < kHd; h <<= 1) {
    const double mine = v[d], other = v[d ^ h];
    __syncthreads();
    v[d] = (d & h) ? other - mine : mine + other;
    __syncthreads();
  }
  const bool neg = (a.v_signs[d >> 5] >> (d & 31)) & 1u;
  const double o = v[d] * 0.08838834764831845;   // 1 / sqrt(128)
  a.out[(head * a.n_q + qj) * kHd + d] = (float)(neg ? -o : o);
}

}  // namespace

// Keys per wave: about 2048 waves in all, at least 64 keys each (fewer
// ranges keep the merge short), a multiple of 4.
void attn_plan(int64_t n_heads, int64_t n_q, int64_t n_keys, int64_t& keys_per_wave,
               int64_t& n_ranges) {
  const int64_t groups = (n_q + attn_group(n_q) - 1) / attn_group(n_q);
  const int64_t per_head = (2048 + n_heads * groups - 1) / (n_heads * groups);   // waves
  int64_t kpw = (n_keys + per_head - 1) / per_head;
  kpw = kpw < 64 ? 64 : kpw;
  keys_per_wave = (kpw + 3) / 4 * 4;
  n_ranges = (n_keys + 4 * keys_per_wave - 1) / (4 * keys_per_wave);
}

int64_t attn_blocks(int64_t n_heads, int64_t n_q, int64_t n_keys) {
  int64_t kpw, nr;
  attn_plan(n_heads, n_q, n_keys, kpw, nr);
  return nr * ((n_q + attn_group(n_q) - 1) / attn_group(n_q)) * n_heads;
}

size_t attn_workspace(int64_t n_heads, int64_t n_q, int64_t n_keys) {
  int64_t kpw, nr;
  attn_plan(n_heads, n_q, n_keys, kpw, nr);
  return (size_t)4 * (size_t)(n_heads * n_q) * kHd +
         (size_t)4 * (size_t)(n_heads * nr * n_q) * (2 + kHd);
}

hipError_t launch_attention(const AttnLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL(rotate_kernel, dim3((unsigned)(a.n_heads * a.n_q)), dim3(kHd), 0, s, a);
  const int qg = attn_group(a.n_q);
  const dim3 grid((unsigned)a.n_ranges, (unsigned)((a.n_q + qg - 1) / qg), (unsigned)a.n_heads);
  if (qg == 4)
    hipLaunchKernelGGL((attn_kernel<4>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<8>), grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)a.n_q, (unsigned)a.n_heads), dim3(kHd), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace hq
