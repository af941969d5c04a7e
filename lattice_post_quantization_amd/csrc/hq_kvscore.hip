// Attention scores against compressed keys, in the rotated domain.
//
// Passages: [ICLR abstract] "HyperQuant: A Near-Entropy-Optimal Lattice
// Quantization Pipeline ..." (subtractive dither keeps each cached inner
// product unbiased; algebraic decoding); [arXiv abstract] "HyperQuant: A
// Rate-Distortion-Optimal Quantization Pipeline ..." ideas (i)-(iii).
//
// A key decodes to khat = s (.) H yhat / sqrt(n) with yhat = Delta (p - d)
// (p the lattice point, d the dither, 0 without dither).  H is symmetric, so
// q . khat = <H (s (.) q), yhat> / sqrt(n): queries are rotated once
// (rotate_q_kernel, fp64 butterflies, stored fp32) and the keys never leave
// the lattice domain.  score_kernel: one lane per key holds yhat in 128
// registers (the dither regenerated from the same counter hash and E8
// decision as the encoder), the block's four waves share chunks of 32
// rotated queries in LDS (read as broadcasts), and each lane writes one
// score per query: 64 consecutive keys per store.
#include "hq.h"
#include "hq_device.h"
#include "hq_internal.h"
#include "hq_dither.h"

namespace hq {
namespace {

constexpr int kHd = 128;        // head dimension (tile)
constexpr int kQChunk = 32;     // queries per LDS chunk

__global__ __launch_bounds__(kHd) void rotate_q_kernel(ScoreLaunch a) {
  __shared__ double v[kHd];
  const int j = threadIdx.x;
  const int64_t c = (int64_t)blockIdx.x * kHd + j;
  const bool neg = (a.signs[j >> 5] >> (j & 31)) & 1u;
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
  a.qr[c] = (float)v[j];
}

__global__ __launch_bounds__(256) void score_kernel(ScoreLaunch a) {
  __shared__ float4 qs[kQChunk][kHd / 4];
  const int64_t key_raw = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = key_raw < a.n_keys;
  const int64_t key = live ? key_raw : a.n_keys - 1;   // whole block stays for the syncs

  // ---- yhat of this lane's key, in the lattice domain
  float y[kHd];
  {
    const uint4* src = reinterpret_cast<const uint4*>(a.idx + key * kHd);
    const uint32_t cw = a.coset[key];
    const float delta = a.scale[key];
#pragma unroll
    for (int blk = 0; blk < kHd / 8; ++blk) {
      const uint4 q = src[blk >> 1];
      const uint32_t d0 = (blk & 1) ? q.z : q.x, d1 = (blk & 1) ? q.w : q.y;
      int32_t s[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = __builtin_amdgcn_sbfe((int32_t)d0, 8 * i, 8);
        s[4 + i] = __builtin_amdgcn_sbfe((int32_t)d1, 8 * i, 8);
      }
      const int c = (cw >> blk) & 1;
      const int32_t par = s[0] + s[1] + s[2] + s[3] + s[4] + s[5] + s[6];
      int32_t P[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int32_t z = (i == 7) ? 2 * s[7] + (par & 1) : s[i];
        P[i] = 2 * z + c;
      }
      if (a.dither) {
        // d = w - Q_E8(w), w = 2^-23 h - 1, h the top 24 bits of the hash
        int32_t W[8], d24[8];                      // w and d in 2^-24 units
        const DitherVec dk = dither_vec(a.dither_seed, (uint64_t)(a.dither_base + key));
#pragma unroll
        for (int i = 0; i < 8; ++i) W[i] = dither_w(dk, (uint32_t)(8 * blk + i));
        e8_dither_block(W, d24);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          y[8 * blk + i] = delta * ((float)P[i] * 0.5f - (float)d24[i] * 5.9604644775390625e-08f);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) y[8 * blk + i] = delta * ((float)P[i] * 0.5f);
      }
    }
  }

  // ---- scores against chunks of rotated queries
  for (int64_t j0 = 0; j0 < a.n_q; j0 += kQChunk) {
    const int nq = (int)(a.n_q - j0 < kQChunk ? a.n_q - j0 : kQChunk);
    __syncthreads();   // the previous chunk is no longer read
    for (int e = threadIdx.x; e < nq * (kHd / 4); e += 256)
      qs[e / (kHd / 4)][e % (kHd / 4)] =
          reinterpret_cast<const float4*>(a.qr + (j0 + e / (kHd / 4)) * kHd)[e % (kHd / 4)];
    __syncthreads();
    for (int jj = 0; jj < nq; ++jj) {
      float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
      for (int i = 0; i < kHd / 4; i += 2) {
        const float4 q0 = qs[jj][i], q1 = qs[jj][i + 1];
        acc0 = fmaf(y[4 * i], q0.x, acc0);
        acc0 = fmaf(y[4 * i + 1], q0.y, acc0);
        acc0 = fmaf(y[4 * i + 2], q0.z, acc0);
        acc0 = fmaf(y[4 * i + 3], q0.w, acc0);
        acc1 = fmaf(y[4 * i + 4], q1.x, acc1);
        acc1 = fmaf(y[4 * i + 5], q1.y, acc1);
        acc1 = fmaf(y[4 * i + 6], q1.z, acc1);
        acc1 = fmaf(y[4 * i + 7], q1.w, acc1);
      }
      if (live) a.scores[(j0 + jj) * a.n_keys + key] = (acc0 + acc1) * (float)a.inv_sqrt_n;
    }
  }
}

}  // namespace

hipError_t launch_scores(const ScoreLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL(rotate_q_kernel, dim3((unsigned)a.n_q), dim3(kHd), 0, s, a);
  const int64_t blocks = (a.n_keys + 255) / 256;
  hipLaunchKernelGGL(score_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hq
