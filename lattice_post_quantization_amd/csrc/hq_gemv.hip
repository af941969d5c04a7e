// y = W x straight from E8 indices (tile 256): the consumer of the format.
//
// Passages: GitHub issue "HyperQuant ... #9", "Is your feature request
// related to a problem?" (the compressed weights must serve inference);
// [ICLR abstract] "HyperQuant: A Near-Entropy-Optimal Lattice Quantization
// Pipeline ..." (algebraic decoding of the lattice indices).
//
// Tile t of row r decodes to w = s (.) H P Delta / (2 sqrt(n)) with P = 2p
// the lattice point (2 z + c per coordinate, z7 restored from the parity of
// z0..z6).  H is symmetric, so w . x_t = Delta / (2 sqrt(n)) <P, H (s (.) x_t)>:
// rotate_kernel forms xr = H (s (.) x) once per 256-column slice (fp64
// butterflies, stored as fp32), and gemv_kernel reads only the stored bytes
// of W: per weight a byte, an unstrip and one fused multiply-add per vector.
//
// gemv_kernel: a wave owns kGemvRows rows and a range of column slices (the
// columns are split so that small matrices still fill the chip; the splits'
// partial sums are added in a fixed order); lane l holds columns 4l .. 4l + 3 of
// the current slice (half of 8-block l / 2), so the wave's idx loads are
// 256 contiguous bytes per row and the slice of xr is loaded once for all
// kGemvRows rows.  The odd lane of a block gets the even lane's bytes by a DPP
// move for the parity of z0..z6.
#include "hq.h"
#include "hq_device.h"
#include "hq_internal.h"

namespace hq {
namespace {

constexpr int kGemvRows = 4;    // rows per wave

// xr[v][c] = (H (s (.) x_t))_j for c = 256 t + j, one 256-thread block per
// (vector, slice); fp64 butterflies through LDS, one rounding to fp32.
__global__ __launch_bounds__(256) void rotate_kernel(GemvLaunch a) {
  __shared__ double v[256];
  const int j = threadIdx.x;
  const int64_t slices = a.cols / 256;
  const int64_t vec = blockIdx.x / slices, t = blockIdx.x % slices;
  const int64_t c = vec * a.cols + t * 256 + j;
  const bool neg = (a.signs[j >> 5] >> (j & 31)) & 1u;
  double x = (double)a.x[c];
  v[j] = neg ? -x : x;
  __syncthreads();
#pragma unroll
  for (int h = 1; h < 256; h <<= 1) {
    const double mine = v[j], other = v[j ^ h];
    __syncthreads();
    v[j] = (j & h) ? other - mine : mine + other;
    __syncthreads();
  }
  a.xr[c] = (float)v[j];
}

__device__ inline uint32_t dpp_row_shr1(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// Work item (row block, column split): a wave sums kGemvRows rows over the
// slices [split * a.span, ...) and writes its partial sums to the workspace
// (part[split][v][row]); reduce_kernel adds the splits in a fixed order
// (a single split writes y directly).
// The next slice's bytes and rotated input are loaded while the current
// slice is computed.
template <int M>
__global__ __launch_bounds__(256) void gemv_kernel(GemvLaunch a) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row_blocks = (a.rows + kGemvRows - 1) / kGemvRows;
  if (wave >= row_blocks * a.splits) return;   // whole waves only
  const int64_t rb = wave % row_blocks, split = wave / row_blocks;
  const int64_t r0 = rb * kGemvRows;
  const int64_t slices = a.cols / 256;
  const int64_t t0 = split * a.span;
  const int64_t t1 = t0 + a.span < slices ? t0 + a.span : slices;
  const int b = lane >> 1;          // 8-block of the slice
  const bool odd = lane & 1;        // holds coordinates 4..7 of the block
  float acc[kGemvRows][M];
#pragma unroll
  for (int i = 0; i < kGemvRows; ++i)
#pragma unroll
    for (int v = 0; v < M; ++v) acc[i][v] = 0.0f;

  int64_t rr[kGemvRows];
#pragma unroll
  for (int i = 0; i < kGemvRows; ++i) rr[i] = r0 + i < a.rows ? r0 + i : a.rows - 1;  // past the end: discarded

  uint32_t dq[kGemvRows];
  float4 xq[M];
  auto fetch = [&](int64_t t) {
#pragma unroll
    for (int i = 0; i < kGemvRows; ++i)
      dq[i] = *reinterpret_cast<const uint32_t*>(a.idx + rr[i] * a.cols + t * 256 + 4 * lane);
#pragma unroll
    for (int v = 0; v < M; ++v)
      xq[v] = *reinterpret_cast<const float4*>(a.xr + v * a.cols + t * 256 + 4 * lane);
  };
  if (t0 < t1) fetch(t0);
  for (int64_t t = t0; t < t1; ++t) {
    uint32_t dc[kGemvRows];
    float xr[M][4], xs[M];
#pragma unroll
    for (int i = 0; i < kGemvRows; ++i) dc[i] = dq[i];
#pragma unroll
    for (int v = 0; v < M; ++v) {
      xr[v][0] = xq[v].x; xr[v][1] = xq[v].y; xr[v][2] = xq[v].z; xr[v][3] = xq[v].w;
      xs[v] = (xr[v][0] + xr[v][1]) + (xr[v][2] + xr[v][3]);
    }
    if (t + 1 < t1) fetch(t + 1);
#pragma unroll
    for (int i = 0; i < kGemvRows; ++i) {
      const int64_t tile = rr[i] * slices + t;
      const uint32_t d = dc[i];
      const uint32_t dn = dpp_row_shr1(d);   // the even lane's bytes (z0..z3)
      const uint32_t cw = a.coset[tile];
      const float delta = a.scale[tile];
      const float c = (float)((cw >> b) & 1u);
      // parity of z0..z6: XOR of the bytes of dn and of d's first three
      uint32_t px = dn ^ (d & 0x00FFFFFFu);
      px ^= px >> 16;
      px ^= px >> 8;
      int32_t z[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = __builtin_amdgcn_sbfe((int32_t)d, 8 * e, 8);
      if (odd) z[3] = 2 * z[3] + (int32_t)(px & 1u);   // z7 = 2 floor(z7 / 2) + parity
#pragma unroll
      for (int v = 0; v < M; ++v) {
        float dot = (float)z[0] * xr[v][0];
        dot = fmaf((float)z[1], xr[v][1], dot);
        dot = fmaf((float)z[2], xr[v][2], dot);
        dot = fmaf((float)z[3], xr[v][3], dot);
        // <P, xr> over this lane's coordinates, P = 2 z + c
        acc[i][v] = fmaf(delta, fmaf(2.0f, dot, c * xs[v]), acc[i][v]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kGemvRows; ++i) {
#pragma unroll
    for (int v = 0; v < M; ++v) {
      const float s = wave_sum(acc[i][v]);
      if (lane == 0 && r0 + i < a.rows) {
        if (a.splits == 1)
          a.y[v * a.rows + r0 + i] = s * 0.03125f;   // y = (sum) / (2 sqrt(256))
        else
          a.part[(split * a.m + v) * a.rows + r0 + i] = s;
      }
    }
  }
}

// y[v][r] = (sum over the splits, in order) / (2 sqrt(256))
__global__ __launch_bounds__(256) void reduce_kernel(GemvLaunch a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // v * rows + r
  if (i >= (int64_t)a.m * a.rows) return;
  float s = 0.0f;
  for (int64_t k = 0; k < a.splits; ++k) s += a.part[k * a.m * a.rows + i];
  a.y[i] = s * 0.03125f;
}

template <int M>
hipError_t launch_m(const GemvLaunch& a, hipStream_t s) {
  const int64_t waves = (a.rows + kGemvRows - 1) / kGemvRows * a.splits;
  hipLaunchKernelGGL(gemv_kernel<M>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
  if (a.splits > 1) {
    const int64_t n = (int64_t)a.m * a.rows;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

// Column splits so that a launch has at least kTargetWaves waves.
constexpr int64_t kTargetWaves = 2048;

void gemv_split(int64_t rows, int64_t cols, int64_t& splits, int64_t& span) {
  const int64_t row_blocks = (rows + kGemvRows - 1) / kGemvRows;
  const int64_t slices = cols / 256;
  int64_t want = (kTargetWaves + row_blocks - 1) / row_blocks;
  want = want < 1 ? 1 : (want > slices ? slices : want);
  span = (slices + want - 1) / want;
  splits = (slices + span - 1) / span;
}

hipError_t launch_gemv(const GemvLaunch& a, hipStream_t s) {
  const int64_t rot_blocks = (int64_t)a.m * (a.cols / 256);
  hipLaunchKernelGGL(rotate_kernel, dim3((unsigned)rot_blocks), dim3(256), 0, s, a);
  switch (a.m) {
    case 1: return launch_m<1>(a, s);
    case 2: return launch_m<2>(a, s);
    case 3: return launch_m<3>(a, s);
    case 4: return launch_m<4>(a, s);
    case 5: return launch_m<5>(a, s);
    case 6: return launch_m<6>(a, s);
    case 7: return launch_m<7>(a, s);
    default: return launch_m<8>(a, s);
  }
}

}  // namespace hq
