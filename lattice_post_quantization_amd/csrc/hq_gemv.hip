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
// butterflies, stored as fp32, with the fp32 sum of every 8-block), and
// gemv_kernel reads only the stored bytes of W.  Per block,
// <P, xr> = 2 <z, xr> + c sum(xr), and <z, xr> = sum_i t_i xr'_i + par xr_7
// with t the stored integers and xr'_7 = 2 xr_7: a byte conversion and one
// fused multiply-add per weight and vector.
//
// gemv_kernel: a wave owns a chunk of J pieces of 1024 columns (lane l holds
// columns 16 l .. 16 l + 15 of each piece: two blocks of one tile) and a
// group of rows.  The rotated input of the chunk stays in registers for the
// whole group (J = 4 for one vector, so a 4096-column row is one chunk); the
// rows stream through with several rows of index bytes, coset words and
// scales in flight.  Each row's 64 lane sums are added by DPP (a fixed
// tree), the totals collect in LDS and leave as one coalesced store per
// vector.  With several chunks per row the chunk totals go to the workspace
// and reduce_kernel adds them in chunk order.
#include "hq.h"
#include "hq_device.h"
#include "hq_internal.h"

namespace hq {
namespace {

constexpr int kPieceCols = 1024;   // columns of one piece: 64 lanes x 16
constexpr int kMaxRowsPerWave = 64;

// pieces per chunk for m vectors (registers for the rotated input: 16 J m)
__host__ __device__ constexpr int pieces_for(int m) { return m == 1 ? 4 : (m == 2 ? 2 : 1); }

// LDS exchange among the lanes of one wave: its LDS operations run in
// order, so the fences only keep the compiler from moving them
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// xr[v][c] = (H (s (.) x_v))_j for c = 256 t + j and xs[v][c / 8] the sum of
// its 8-block: one wave per (vector, slice), lane l holding elements
// 4 l .. 4 l + 3.  Butterflies in fp64 (stages 1 and 2 in registers, the
// others through the wave's LDS), one rounding to fp32 each.
// Matrix of the batch that holds index g of a numbering (wave-uniform; the
// batch is small).
template <typename F>
__device__ inline int item_at(const GemvBatch& b, int64_t g, F first) {
  int i = 0;
#pragma unroll
  for (int k = 1; k < kGemvMaxItems; ++k)
    if (k < b.n && g >= first(b.it[k])) i = k;
  return i;
}

__global__ __launch_bounds__(256) void rotate_kernel(GemvBatch b) {
  __shared__ double v[4][256];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t g = (int64_t)blockIdx.x * 4 + w;
  if (g >= b.n_rot) return;
  const GemvItem& a = b.it[item_at(b, g, [](const GemvItem& t) { return t.rot0; })];
  const int64_t slices = a.cols / 256;
  const int64_t item = g - a.rot0;
  const int64_t vec = item / slices, t = item % slices;
  const int64_t c0 = vec * a.cols + t * 256 + 4 * lane;
  const float4 xv = *reinterpret_cast<const float4*>(a.x + c0);
  const uint32_t sg = b.signs[lane >> 3] >> (4 * (lane & 7));
  double e[4] = {(double)xv.x, (double)xv.y, (double)xv.z, (double)xv.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if ((sg >> i) & 1u) e[i] = -e[i];
  // element bits 0 and 1
  double p = e[0], q = e[1];
  e[0] = p + q; e[1] = p - q;
  p = e[2]; q = e[3];
  e[2] = p + q; e[3] = p - q;
  p = e[0]; q = e[2];
  e[0] = p + q; e[2] = p - q;
  p = e[1]; q = e[3];
  e[1] = p + q; e[3] = p - q;
  // element bits 2 .. 7 = lane bits 0 .. 5
  double* vw = v[w];
#pragma unroll
  for (int hb = 1; hb < 64; hb <<= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) vw[4 * lane + i] = e[i];
    wave_sync();
    double o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = vw[4 * (lane ^ hb) + i];
    wave_sync();
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = (lane & hb) ? o[i] - e[i] : e[i] + o[i];
  }
  *reinterpret_cast<float4*>(a.xr + c0) = make_float4((float)e[0], (float)e[1], (float)e[2], (float)e[3]);
#pragma unroll
  for (int i = 0; i < 4; ++i) vw[4 * lane + i] = e[i];
  wave_sync();
  if (!(lane & 1)) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += vw[4 * lane + i];
    a.xs[c0 >> 3] = (float)s;
  }
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// x plus the value DPP control CTRL brings from another lane (0 where the
// row mask excludes the lane or the source is outside its row)
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_add(float x) {
  return x + __int_as_float(
                 __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, true));
}

// Sum over the wave's 64 lanes in a fixed tree (row inclusive scans, then
// the row totals); the total lands in lane 63.
__device__ inline float wave_total(float x) {
  x = dpp_add<0x111, 0xF>(x);   // row_shr:1
  x = dpp_add<0x112, 0xF>(x);   // row_shr:2
  x = dpp_add<0x114, 0xF>(x);   // row_shr:4
  x = dpp_add<0x118, 0xF>(x);   // row_shr:8
  x = dpp_add<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
  x = dpp_add<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}

template <int J>
struct RowIn {
  uint4 q[J];       // 16 index bytes of each piece
  uint32_t cw[J];   // coset word of each piece's tile
  float sc[J];      // its scale
};

template <int M, int J>
__global__ __launch_bounds__(256) void gemv_kernel(GemvBatch b) {
  constexpr int kDepth = J >= 4 ? 2 : 4;   // rows in flight per register set
  __shared__ float sums[4][M][kMaxRowsPerWave];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t g = (int64_t)blockIdx.x * 4 + wave;
  if (g >= b.n_waves) return;   // whole waves only
  const GemvItem& a = b.it[item_at(b, g, [](const GemvItem& t) { return t.wave0; })];
  const int64_t item = g - a.wave0;
  const int64_t R = a.rows_per_wave;
  const int64_t ch = item % a.n_chunks, rg = item / a.n_chunks;
  const int64_t r0 = rg * R;
  const int n = (int)(a.rows - r0 < R ? a.rows - r0 : R);   // rows of this group
  const int64_t slices = a.cols / 256;
  const int bb = 2 * (lane & 15);   // tile block index of the lane's first block
  int64_t col[J];
  bool live[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    col[j] = (ch * J + j) * kPieceCols + 16 * lane;
    live[j] = col[j] < a.cols;
  }

  // rotated input of the lane's columns (zero past the last column)
  float xr[M][J][16], xs[M][J][2];
#pragma unroll
  for (int v = 0; v < M; ++v) {
    const auto rx = rsrc(a.xr + v * a.cols, (uint32_t)(a.cols * 4));
    const auto rs = rsrc(a.xs + v * (a.cols / 8), (uint32_t)(a.cols / 2));
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t off = live[j] ? (uint32_t)(col[j] * 4) : 0x80000000u;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(off + 16 * k), 0, 0);
        xr[v][j][4 * k] = __uint_as_float(q.x);
        xr[v][j][4 * k + 1] = __uint_as_float(q.y);
        xr[v][j][4 * k + 2] = __uint_as_float(q.z);
        xr[v][j][4 * k + 3] = __uint_as_float(q.w);
      }
      const uint32_t offs = live[j] ? (uint32_t)(col[j] / 2) : 0x80000000u;
      xs[v][j][0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)offs, 0, 0));
      xs[v][j][1] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)(offs + 4), 0, 0));
    }
  }

  // rows r0 .. r0 + n - 1; loads past the group read zeros
  const auto ri = rsrc(a.idx + r0 * a.cols, (uint32_t)(n * a.cols));
  const auto rc = rsrc(a.coset + r0 * slices, (uint32_t)(n * slices * 4));
  const auto rsc = rsrc(a.scale + r0 * slices, (uint32_t)(n * slices * 4));
  uint32_t ioff[J], toff[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    ioff[j] = live[j] ? (uint32_t)col[j] : 0x80000000u;
    toff[j] = live[j] ? (uint32_t)((col[j] >> 8) * 4) : 0x80000000u;
  }
  const uint32_t irow = (uint32_t)a.cols, trow = (uint32_t)(slices * 4);
  auto fetch = [&](int row, RowIn<J>& in) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(
          ri, (int)(ioff[j] + (uint32_t)row * irow), 0, 0);
      in.q[j] = make_uint4(q.x, q.y, q.z, q.w);
      in.cw[j] = __builtin_amdgcn_raw_buffer_load_b32(rc, (int)(toff[j] + (uint32_t)row * trow),
                                                      0, 0);
      in.sc[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rsc, (int)(toff[j] + (uint32_t)row * trow), 0, 0));
    }
  };

  // row r of the group (wave-uniform r < n): its lane partials, wave totals
  // into LDS
  auto row = [&](const RowIn<J>& in, int r) {
    float part[M];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t dw[4] = {in.q[j].x, in.q[j].y, in.q[j].z, in.q[j].w};
      const uint32_t cb = in.cw[j] >> bb;
      const float c0 = (float)(cb & 1u), c1 = (float)((cb >> 1) & 1u);
      float dz[2][M];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const uint32_t d0 = dw[2 * b], d1 = dw[2 * b + 1];
        // parity of z0..z6: XOR of the seven bytes' low bits
        uint32_t px = d0 ^ (d1 & 0x00FFFFFFu);
        px ^= px >> 16;
        px ^= px >> 8;
        const float par = (float)(px & 1u);
        float s[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // the builtin's result is unsigned: convert it as a signed value
          s[e] = (float)(int32_t)__builtin_amdgcn_sbfe((int32_t)d0, 8 * e, 8);
          s[4 + e] = (float)(int32_t)__builtin_amdgcn_sbfe((int32_t)d1, 8 * e, 8);
        }
#pragma unroll
        for (int v = 0; v < M; ++v) {
          const float* x = &xr[v][j][8 * b];
          float acc = s[0] * x[0];
#pragma unroll
          for (int e = 1; e < 7; ++e) acc = fmaf(s[e], x[e], acc);
          acc = fmaf(s[7], 2.0f * x[7], acc);   // z7 = 2 t7 + par
          dz[b][v] = fmaf(par, x[7], acc);
        }
      }
#pragma unroll
      for (int v = 0; v < M; ++v) {
        // <P, xr> over the piece's two blocks, P = 2 z + c, times Delta
        float u = fmaf(c1, xs[v][j][1], c0 * xs[v][j][0]);
        u = fmaf(2.0f, dz[0][v], u);
        u = fmaf(2.0f, dz[1][v], u);
        part[v] = j == 0 ? in.sc[j] * u : fmaf(in.sc[j], u, part[v]);
      }
    }
#pragma unroll
    for (int v = 0; v < M; ++v) {
      const float tot = wave_total(part[v]);
      if (lane == 63) sums[wave][v][r] = tot;
    }
  };

  // two register sets of kDepth rows: one is consumed while the other fills
  // (issued in row order, so a slot's loads are never younger than the
  // next slot's: each row then waits only for its own loads)
  RowIn<J> A[kDepth], B[kDepth];
#pragma unroll
  for (int k = 0; k < kDepth; ++k) {
    fetch(k, A[k]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int rb = 0; rb < n; rb += 2 * kDepth) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      fetch(rb + kDepth + k, B[k]);
      if (rb + k < n) row(A[k], rb + k);
    }
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      fetch(rb + 2 * kDepth + k, A[k]);
      if (rb + kDepth + k < n) row(B[k], rb + kDepth + k);
    }
  }

  // one coalesced store per vector: lane i holds row r0 + i
  wave_sync();
  if (lane < n) {
#pragma unroll
    for (int v = 0; v < M; ++v) {
      const float s = sums[wave][v][lane];
      if (a.n_chunks == 1)
        a.y[v * a.rows + r0 + lane] = s * 0.03125f;   // y = (sum) / (2 sqrt(256))
      else
        a.part[(ch * M + v) * a.rows + r0 + lane] = s;
    }
  }
}

// y[v][r] = (sum over the chunks, in order) / (2 sqrt(256)), for the
// matrices with more than one chunk per row
__global__ __launch_bounds__(256) void reduce_kernel(GemvBatch b) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= b.n_red) return;
  // the element's matrix (lanes may differ: a plain scan)
  int k = 0;
  for (int j = 1; j < b.n; ++j)
    if (b.it[j].n_chunks > 1 && g >= b.it[j].red0) k = j;
  const GemvItem& a = b.it[k];
  const int64_t i = g - a.red0;   // v * rows + r
  float s = 0.0f;
  for (int64_t c = 0; c < a.n_chunks; ++c) s += a.part[c * b.m * a.rows + i];
  a.y[i] = s * 0.03125f;
}

template <int M>
hipError_t launch_m(const GemvBatch& b, hipStream_t s) {
  hipLaunchKernelGGL((gemv_kernel<M, pieces_for(M)>), dim3((unsigned)((b.n_waves + 3) / 4)),
                     dim3(256), 0, s, b);
  if (b.n_red > 0)
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((b.n_red + 255) / 256)), dim3(256), 0, s, b);
  return hipGetLastError();
}

}  // namespace

// Chunks of pieces_for(m) pieces per row, and rows per wave so that a
// launch has about kTargetWaves waves (at least 4 rows, so the rotated input
// a wave loads is at most as large as the index bytes it streams).  The
// buffer offsets of a wave stay below 2^31 for cols <= kGemvMaxCols.
constexpr int64_t kTargetWaves = 2048;

void gemv_plan(int64_t rows, int64_t cols, int m, int64_t& n_chunks, int64_t& rows_per_wave) {
  const int64_t chunk = (int64_t)kPieceCols * pieces_for(m);
  n_chunks = (cols + chunk - 1) / chunk;
  int64_t r = (rows * n_chunks + kTargetWaves - 1) / kTargetWaves;
  r = r < 4 ? 4 : (r > kMaxRowsPerWave ? kMaxRowsPerWave : r);
  rows_per_wave = r;
}

size_t gemv_workspace(int64_t rows, int64_t cols, int m) {
  int64_t n_chunks, rows_per_wave;
  gemv_plan(rows, cols, m, n_chunks, rows_per_wave);
  // the rotated vectors, their 8-block sums, then the chunk totals (each
  // 16-byte aligned)
  const size_t xr = ((size_t)cols * (size_t)m * sizeof(float) + 15) / 16 * 16;
  const size_t xs = ((size_t)cols / 8 * (size_t)m * sizeof(float) + 15) / 16 * 16;
  const size_t part =
      n_chunks > 1 ? ((size_t)n_chunks * (size_t)m * (size_t)rows * sizeof(float) + 15) / 16 * 16 : 0;
  return xr + xs + part;
}

void gemv_layout(GemvBatch& b, char* workspace) {
  b.n_waves = b.n_rot = b.n_red = 0;
  for (int i = 0; i < b.n; ++i) {
    GemvItem& it = b.it[i];
    gemv_plan(it.rows, it.cols, b.m, it.n_chunks, it.rows_per_wave);
    const size_t xr = ((size_t)it.cols * (size_t)b.m * sizeof(float) + 15) / 16 * 16;
    const size_t xs = ((size_t)it.cols / 8 * (size_t)b.m * sizeof(float) + 15) / 16 * 16;
    it.xr = reinterpret_cast<float*>(workspace);
    it.xs = reinterpret_cast<float*>(workspace + xr);
    it.part = reinterpret_cast<float*>(workspace + xr + xs);
    workspace += gemv_workspace(it.rows, it.cols, b.m);
    it.wave0 = b.n_waves;
    it.rot0 = b.n_rot;
    it.red0 = b.n_red;
    b.n_waves += (it.rows + it.rows_per_wave - 1) / it.rows_per_wave * it.n_chunks;
    b.n_rot += (int64_t)b.m * (it.cols / 256);
    if (it.n_chunks > 1) b.n_red += (int64_t)b.m * it.rows;
  }
  for (int i = b.n; i < kGemvMaxItems; ++i) b.it[i] = b.it[0];
}

hipError_t launch_gemv(const GemvBatch& b, hipStream_t s) {
  hipLaunchKernelGGL(rotate_kernel, dim3((unsigned)((b.n_rot + 3) / 4)), dim3(256), 0, s, b);
  switch (b.m) {
    case 1: return launch_m<1>(b, s);
    case 2: return launch_m<2>(b, s);
    case 3: return launch_m<3>(b, s);
    case 4: return launch_m<4>(b, s);
    case 5: return launch_m<5>(b, s);
    case 6: return launch_m<6>(b, s);
    case 7: return launch_m<7>(b, s);
    default: return launch_m<8>(b, s);
  }
}

}  // namespace hq
