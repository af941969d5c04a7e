// Launch descriptors shared by the C ABI (hq_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

constexpr int kBlock = 256;         // threads per block, every kernel
constexpr int kElemsPerLane = 16;   // tile elements held by one lane

constexpr int kMaxTile = 512;       // largest tile (elements)

struct EncodeLaunch {
  const void* x;
  int in_bf16;
  int64_t n_tiles;
  int lattice;          // 8, 4, 2, 1
  int tile;             // 128 or 256
  float* scale;
  int auto_scale;
  int8_t* idx;
  uint32_t* coset;
  uint8_t* rice_k;
  uint32_t* tile_bits;
  int16_t* coords;      // nullptr unless requested
  uint32_t* status;     // may be nullptr
  uint32_t signs[kMaxTile / 32];   // bit j set: sign of element j is -1
  double c;             // auto-scale constant c(L, R)
  double sqrt_n;        // fp64 sqrt(tile)
  int dither;
  uint32_t dither_seed;
  int64_t dither_base;
  int rate_control;     // per-tile scales by bisection (generic kernel)
  uint32_t rc_budget;   // bits one tile may take: floor(bps * tile)
  int wide;             // int16 index mode: idx holds int16 values (generic kernel)
};

// bf16 bit patterns the rate control searches on each side of the
// automatic scale (eight binades)
constexpr int32_t kRcSpan = 1024;

struct DecodeLaunch {
  const int8_t* idx;
  const uint32_t* coset;
  const float* scale;
  int64_t n_tiles;
  int lattice;
  int tile;
  void* y;
  int out_bf16;
  uint32_t* status;
  uint32_t signs[kMaxTile / 32];
  double inv_sqrt_n;    // fp64 1/sqrt(tile)
  int dither;
  uint32_t dither_seed;
  int64_t dither_base;
  int wide;             // int16 index mode: idx holds int16 values (generic kernel)
};

struct RateLaunch {
  const int8_t* idx;
  const uint32_t* coset;
  int64_t n_tiles;
  int tile;
  int coset_bits;       // per tile
  int coset_words;      // per tile
  uint8_t* rice_k;
  uint32_t* tile_bits;
  uint64_t* total_bits;
  uint32_t* stream;     // nullptr: rate only
  uint64_t capacity;
  uint64_t* tile_word_offset;
  uint64_t* block_words;   // workspace: words per rate block (nullptr: no workspace)
  uint64_t* block_bits;    // workspace: bits per rate block
  uint64_t* wave_words;    // workspace: words per rate wave
  uint32_t* status;
  int given;               // rice_k and tile_bits are inputs (the encoder's)
  int wide;                // int16 index mode: idx holds int16 values
};

// One packed matrix of an unpack launch; wave0 numbers its first wave (64
// tiles per wave) among the launch's waves.
struct UnpackItem {
  const uint32_t* stream;
  const uint64_t* tile_word_offset;
  int64_t n_tiles;
  int8_t* idx;
  uint32_t* coset;      // nullptr iff coset_words == 0
  uint8_t* rice_k;      // may be nullptr
  int64_t wave0;
};

constexpr int kUnpackMaxItems = 8;

// One matrix of an hq_gemm batch.  The workspace pointers and the plan are
// filled in by gemm_layout; blk0 / split0 / sum0 number the matrix's GEMM
// blocks, split waves and summed elements across the batch.
struct GemmItem {
  const int8_t* idx;
  const uint32_t* coset;
  const float* scale;
  int64_t rows;
  int64_t cols;         // multiple of 256 (E8, tile 256), at most kGemmMaxCols
  const float* x;       // [m][cols]
  float* y;             // [m][rows]
  uint16_t* xh;         // workspace: the rotated inputs' bf16 terms, [m][cols]
  uint16_t* xl;
  float* part;          // workspace: [kchunks][m][rows] partial sums (kchunks > 1)
  int64_t kchunks;      // slice ranges summed by separate blocks
  int64_t spc;          // slices per range
  int64_t blk0;
  int64_t split0;
  int64_t sum0;
};

constexpr int kGemmMaxItems = 8;   // matrices per launch

struct GemmBatch {
  int32_t n;            // matrices, 1..kGemmMaxItems
  int32_t m;            // vectors
  int64_t n_blocks;     // GEMM blocks of the batch
  int64_t n_split;      // split waves
  int64_t n_sum;        // summed elements
  uint32_t signs[8];
  GemmItem it[kGemmMaxItems];
};

// limits that keep the kernels' 32-bit buffer offsets in range
constexpr int64_t kGemmMaxCols = (int64_t)1 << 22;
constexpr int64_t kGemmMaxRows = (int64_t)1 << 23;
// limits that keep the launch grids within 2^32 work-items
constexpr int64_t kGemmMaxVecs = 65536;
constexpr int64_t kGemmMaxProduct = (int64_t)1 << 31;   // m cols and m rows
// The slice ranges of every matrix of b (kchunks, spc), a function of the
// group's sizes and m alone, so a call repeats its bits on any device.
void gemm_plan(GemmBatch& b);
constexpr int64_t kGemmMaxRanges = 64;
// Whether a planned group's three launches stay within 2^32 work-items.
bool gemm_fits_launch(const GemmBatch& b);
// Workspace of one planned matrix: the inputs' bf16 terms, then the partial
// sums when its slices are split.
size_t gemm_item_workspace(const GemmItem& it, int32_t m);
// Plans b, then fills the workspace pointers and the numbering of
// b.it[0 .. b.n).
void gemm_layout(GemmBatch& b, char* workspace);
hipError_t launch_gemm(const GemmBatch& b, hipStream_t s);

struct UnpackLaunch {
  int n;                // items in use
  int tile;
  int coset_bits;       // per tile
  int coset_words;      // per tile
  uint32_t* status;     // may be nullptr
  int64_t n_waves;      // waves of all items
  int wide;             // int16 index mode: idx receives int16 values
  UnpackItem it[kUnpackMaxItems];
};

// One matrix of an hq_gemv batch.  The workspace pointers and the plan are
// filled in by the API; wave0 / rot0 / red0 number the matrix's waves,
// rotate waves and reduce elements across the batch.
struct GemvItem {
  const int8_t* idx;
  const uint32_t* coset;
  const float* scale;
  int64_t rows;
  int64_t cols;         // multiple of 256 (E8, tile 256), at most kGemvMaxCols
  const float* x;       // [m][cols]
  float* y;             // [m][rows]
  float* xr;            // workspace: H (s (.) x) per 256-column slice, [m][cols]
  float* xs;            // workspace: sums of xr over each 8-block, [m][cols / 8]
  float* part;          // workspace: chunk totals [n_chunks][m][rows] (n_chunks > 1)
  int64_t n_chunks;     // column chunks per row
  int64_t rows_per_wave;
  int64_t wave0;        // first gemv wave of this matrix
  int64_t rot0;         // first rotate wave
  int64_t red0;         // first reduce element
};

constexpr int kGemvMaxItems = 8;   // matrices per launch

struct GemvBatch {
  int32_t n;            // matrices, 1..kGemvMaxItems
  int32_t m;            // vectors, 1..8
  int64_t n_waves;      // gemv waves of the batch
  int64_t n_rot;        // rotate waves
  int64_t n_red;        // reduce elements
  uint32_t signs[8];
  GemvItem it[kGemvMaxItems];
};

// Largest cols hq_gemv accepts, its work split (column chunks per row, rows
// per wave) and the workspace one matrix needs.
constexpr int64_t kGemvMaxCols = (int64_t)1 << 24;
void gemv_plan(int64_t rows, int64_t cols, int m, int64_t& n_chunks, int64_t& rows_per_wave);
size_t gemv_workspace(int64_t rows, int64_t cols, int m);
// Fills the workspace pointers, the plan and the numbering of b.it[0 .. b.n).
void gemv_layout(GemvBatch& b, char* workspace);

struct ScoreLaunch {
  const float* q;       // [n_q][128]
  int64_t n_q;
  const int8_t* idx;    // [n_keys][128]
  const uint32_t* coset;
  const float* scale;
  int64_t n_keys;
  float* scores;        // [n_q][n_keys]
  float* qr;            // workspace: H (s (.) q), [n_q][128]
  uint32_t signs[8];
  double inv_sqrt_n;
  int dither;
  uint32_t dither_seed;
  int64_t dither_base;
};

hipError_t launch_encode(const EncodeLaunch& a, hipStream_t s);
hipError_t launch_decode(const DecodeLaunch& a, hipStream_t s);
hipError_t launch_rate(const RateLaunch& a, hipStream_t s);
hipError_t launch_unpack(const UnpackLaunch& a, hipStream_t s);
hipError_t launch_gemv(const GemvBatch& b, hipStream_t s);
hipError_t launch_scores(const ScoreLaunch& a, hipStream_t s);

// Fast path for E8 / tile 256 / bf16 input (encode) and E8 / tile 256
// (decode).  One launch covers up to kMaxItems matrices that share the
// parameters; groups of 16 tiles are numbered across the items.
constexpr int kMaxItems = 8;

struct EncItem {
  const void* x;
  int8_t* idx;
  float* scale;
  uint32_t* coset;
  uint8_t* rice_k;
  uint32_t* tile_bits;
  int64_t n_tiles;
  int64_t group0;       // first global group of this item
};

struct EncBatch {
  int32_t n;
  int32_t pad;
  int64_t n_groups;
  EncItem it[kMaxItems];
};

struct DecItem {
  const int8_t* idx;
  const uint32_t* coset;
  const float* scale;
  void* y;
  int64_t n_tiles;
  int64_t group0;
};

struct DecBatch {
  int32_t n;
  int32_t pad;
  int64_t n_groups;
  DecItem it[kMaxItems];
};

bool e8_fast_encode_ok(const EncodeLaunch& a);
bool e8_fast_decode_ok(const DecodeLaunch& a);
// a: shared parameters (its per-matrix fields are ignored); b: the matrices
hipError_t launch_encode_e8_fast(const EncodeLaunch& a, const EncBatch& b, hipStream_t s);
hipError_t launch_decode_e8_fast(const DecodeLaunch& a, const DecBatch& b, hipStream_t s);
// One launch that runs an encode batch and an independent decode batch
// together (every wave alternates a group of each); same results as the two
// launches above.
hipError_t launch_codec_e8_fast(const EncodeLaunch& a, const EncBatch& b, const DecodeLaunch& ad,
                               const DecBatch& bd, hipStream_t s);

// Fast path for tile 128, every lattice (E8 with or without the KV dither):
// bf16 input (encode), either output type (decode); groups of 32 tiles.
bool fast128_encode_ok(const EncodeLaunch& a);
bool fast128_decode_ok(const DecodeLaunch& a);
hipError_t launch_encode_fast128(const EncodeLaunch& a, hipStream_t s);
hipError_t launch_decode_fast128(const DecodeLaunch& a, hipStream_t s);

// Rate blocks the hq_rate workspace provides for: per block a word sum and a
// bit sum, per wave (4 per block) a word sum.
int64_t rate_workspace_blocks(int64_t n_tiles);

}  // namespace hq
