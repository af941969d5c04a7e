/*
 * hq.h - C ABI of the HyperQuant hot path on MI355X (gfx950).
 *
 * The method (sources are web pages, cited by title):
 *   [arXiv abstract]  "HyperQuant: A Rate-Distortion-Optimal Quantization
 *       Pipeline for Large Language and Diffusion Models", arXiv abstract as
 *       shown on mlsanity.com (paper 2606.23406), enumerated ideas (i)-(iv).
 *   [ICLR abstract]   "HyperQuant: A Near-Entropy-Optimal Lattice Quantization
 *       Pipeline for Large Language and Diffusion Models", abstract on
 *       acceptodds.com (iclr2027-3515).
 *   [issue]           GitHub issue "HyperQuant: A Rate-Distortion-Optimal
 *       Quantization Pipeline ... #9", section "Additional context".
 *
 * Pipeline per tile of n consecutive elements: random signs, Walsh-Hadamard
 * rotation, per-tile scale, nearest point of the E8 / D4 / A2 / Z lattice,
 * lossless strip of the membership-fixed bits, Rice rate; decode inverts it
 * algebraically; the KV path adds a subtractive dither.
 *
 * Conventions for every entry point
 *   - All array arguments are caller-allocated DEVICE pointers (hipMalloc or
 *     equivalent) on the current HIP device; `p` is host memory read during
 *     the call only.  The library allocates nothing on any path.  The
 *     exceptions are the host helpers and the checkpoint-file calls
 *     (hq_ckpt_*), whose arrays are host memory and which make no device
 *     call (their status codes add HQ_EIO, HQ_EFORMAT and HQ_ENOTFOUND).
 *   - Calls enqueue kernels on `stream` and return without synchronising.
 *     The return code reports argument validation (HQ_EINVAL,
 *     HQ_EUNSUPPORTED), the auto-scale index range bound (HQ_ERANGE) and
 *     launch failure (HQ_EDEVICE).  Validation happens before any device
 *     call; on a nonzero return nothing was enqueued.
 *   - Data-dependent faults (non-finite input, a quantizer value |u| > 124
 *     with an explicit scale, a packed stream larger than its capacity) are
 *     OR-ed into the optional device word `*status` (HQ_ST_* bits); the caller
 *     reads it after synchronising.  Outputs of an affected tile are
 *     unspecified.  `status` may be NULL.
 *   - A call with zero tiles is a no-op returning HQ_OK.
 *   - Stateless and reentrant.  Results are bitwise deterministic and, on
 *     inputs whose Hadamard partial sums are exact in fp64 (every bf16 tile
 *     whose magnitudes span less than 2^37), bit-identical to the fp64
 *     definition below, ties included.
 *
 * Data layout
 *   A matrix is row-major and contiguous; tile t is flat elements
 *   [n t, n t + n), so cols must be a multiple of n.  idx holds one int8 per
 *   element in the same order; coset holds hq_coset_words(p) uint32 words per
 *   tile; scale, rice_k and tile_bits hold one entry per tile.
 */
#ifndef HQ_H
#define HQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t hq_status;
enum {
  HQ_OK = 0,
  HQ_EINVAL = -1,       /* bad argument (null pointer, size, tile, dtype)  */
  HQ_ERANGE = -2,       /* auto scale cannot keep indices inside int8
                           (int16 with HQ_IDX16)                           */
  HQ_EDEVICE = -3,      /* a HIP call or kernel launch failed              */
  HQ_EUNSUPPORTED = -4, /* a valid combination the library does not offer */
  HQ_EIO = -5,          /* checkpoint file: cannot open, write or read     */
  HQ_EFORMAT = -6,      /* checkpoint file: not one, truncated, or a record
                           whose checksum or offsets do not hold          */
  HQ_ENOTFOUND = -7     /* checkpoint file: no record of that name        */
};

/* Lattice; the value is the lattice dimension. [arXiv abstract] item (ii). */
typedef enum { HQ_Z = 1, HQ_A2 = 2, HQ_D4 = 4, HQ_E8 = 8 } hq_lattice;

/* Element type of weight / KV / decoded arrays. */
typedef enum { HQ_F32 = 0, HQ_BF16 = 1 } hq_dtype;

/* hq_params.flags */
enum {
  HQ_SCALE_AUTO = 1u,   /* encode computes the scales (else reads them)    */
  HQ_DITHER = 2u,       /* subtractive dither (E8 only; KV encode/decode)  */
  HQ_WANT_COORDS = 4u,  /* encode also writes full lattice coordinates     */
  HQ_RATE_CONTROL = 8u, /* encode: per-tile scales by bisection so that each
                           tile fits floor(bps * tile) bits (see below);
                           requires HQ_SCALE_AUTO; not with HQ_DITHER       */
  HQ_RATE_GIVEN = 16u,  /* hq_rate: rice_k and tile_bits are inputs (the
                           values hq_encode_tiles wrote for these indices);
                           other calls ignore it                           */
  HQ_IDX16 = 32u        /* int16 index mode, for bit rates whose indices
                           leave int8 (R >= 6 at tile 256: the stripped
                           integers reach |u| + 2 with |u| <= sqrt(n)/c).
                           Every `int8_t* idx` argument of the call then
                           points to int16 values (2 bytes per index, the
                           same count and order); grid values are held in
                           64 bits and clamped at |u| = 32000; Rice k runs
                           over [0, 15].  Taken by hq_encode_tiles,
                           hq_decode_tiles, hq_rate, hq_rate_noalloc,
                           hq_rate_batch, hq_unpack and hq_unpack_batch
                           (all on the generic kernels); the other calls,
                           HQ_DITHER and HQ_RATE_CONTROL refuse it with
                           HQ_EUNSUPPORTED                                 */
};

/* Device status bits (OR-ed into *status by kernels). */
enum {
  HQ_ST_NONFINITE = 1u,   /* NaN or Inf in the input of a tile            */
  HQ_ST_OVERFLOW = 2u,    /* a grid value |u| passed 124 (32000 with
                             HQ_IDX16), where encode clamps it (explicit
                             scale; covers every index that would leave
                             int8, or int16)                              */
  HQ_ST_STREAM_FULL = 4u, /* hq_rate: packed stream exceeded capacity     */
  HQ_ST_CORRUPT = 8u      /* hq_unpack: a tile's codes overran its words,
                             or decoded to a value outside int8; hq_rate
                             with HQ_RATE_GIVEN: given values that cannot
                             hold a tile's codes                          */
};

typedef struct {
  uint32_t struct_size;   /* must equal sizeof(hq_params)                   */
  int32_t lattice;        /* hq_lattice                                     */
  int32_t tile;           /* n: 64, 128, 256 or 512, any lattice (at most  
                             256 with HQ_DITHER, else HQ_EUNSUPPORTED)     */
  float bps;              /* target rate R in bits per scalar, 0 < R <= 8   */
  uint32_t rht_seed;      /* seed of the RHT sign vector                    */
  uint32_t dither_seed;   /* HQ_DITHER only; must be < 2^24                 */
  int64_t dither_base;    /* HQ_DITHER only: global index of vector 0       */
  uint32_t flags;         /* HQ_SCALE_AUTO | HQ_DITHER | HQ_WANT_COORDS     */
  uint32_t reserved;      /* must be 0                                      */
} hq_params;

/*
 * hq_encode_tiles - forward pipeline on a row-major matrix.
 *
 * Passages: [arXiv abstract] items (i)-(iii); [ICLR abstract] (rotation,
 * lattice, lossless strip, Rice).  Per tile t:
 *   s      = sign vector: s_j = -1 iff bit 63 of SplitMix64(((seed) << 32) ^ j)
 *   S      = H_n (s * x_t)                      (Sylvester Hadamard, exact)
 *   Delta  = scale[t], or with HQ_SCALE_AUTO
 *            bf16_rne(sqrt(sum x^2 / n) * sqrt(2 pi e) 2^-R / vol^(1/d)),
 *            1 when that rounds to 0
 *   u      = rne(S * (2^24 / (sqrt(n) * Delta))) * 2^-24    (quantizer input)
 *   p      = nearest lattice point per block (ties: see the oracle's rules)
 *   idx    = stripped integers: E8 (z0..z6, floor(z7/2)) with z = p - c/2,
 *            D4 (z0, z1, z2, floor(z3/2)), A2 (a, b), Z (z)
 *   coset  = one bit per E8 block / A2 pair, block j at bit j (LSB first)
 *   rice_k = argmin_k sum(floor(zeta/2^k) + 1 + k), zeta = zigzag(idx)
 *   tile_bits = 4 + coset bits + that minimum
 * With HQ_RATE_CONTROL (per-tile rate control, a variant the pages name as
 * a direction only): Delta is searched over bf16 bit patterns within eight
 * binades of the automatic one (patterns a -/+ 1024, kept among normal
 * values) for the finest scale whose indices fit int8 and whose tile_bits
 * <= floor(bps * n): the top of the window is probed first (if it does not
 * fit, the tile takes it), then bisection with mid = floor((lo + hi) / 2)
 * keeping the top feasible.  All-zero and non-finite tiles keep the
 * automatic scale.  Generic kernels only (about a dozen candidate encodes per
 * tile); no HQ_ERANGE check, since the search keeps the indices in range.
 *
 * x       [rows*cols] of x_dtype (bf16 or fp32)
 * scale   [n_tiles] fp32: output with HQ_SCALE_AUTO, input otherwise
 * idx     [rows*cols] int8
 * coset   [n_tiles * hq_coset_words(p)] uint32; may be NULL iff that is 0
 * rice_k  [n_tiles] uint8,  tile_bits [n_tiles] uint32
 * coords  [rows*cols] int16 iff HQ_WANT_COORDS (E8: 2p; A2: 2 * (a + c/2,
 *         b + c/2); D4, Z: p), else ignored and may be NULL
 * Errors: HQ_EINVAL (null pointer, rows or cols <= 0, cols % tile != 0,
 * bad tile/lattice/dtype/bps/flags), HQ_ERANGE (auto scale with
 * sqrt(n)/c(L,R) + 2 > 127), HQ_EUNSUPPORTED (HQ_DITHER here: use
 * hq_kv_encode), HQ_EDEVICE.
 */
hq_status hq_encode_tiles(const hq_params* p, const void* x, int32_t x_dtype,
                          int64_t rows, int64_t cols, float* scale, int8_t* idx,
                          uint32_t* coset, uint8_t* rice_k, uint32_t* tile_bits,
                          int16_t* coords, uint32_t* status, hipStream_t stream);

/*
 * hq_decode_tiles - inverse pipeline ([ICLR abstract]: decoding is
 * algebraic, no codebook).  Per tile: unstrip (E8: z7 = 2 t7 + (z0+..+z6 mod
 * 2)), point p, yhat = Delta p (HQ_DITHER: Delta (p - d) with the same
 * dither_seed and dither_base as the encode), x = s * ((H_n yhat) / sqrt(n)),
 * rounded to y_dtype (fp32: nearest; bf16: nearest even).
 *
 * idx [rows*cols] int8, coset as for encode, scale [n_tiles] fp32,
 * y [rows*cols] of y_dtype.  Errors as for encode; HQ_DITHER requires E8.
 */
hq_status hq_decode_tiles(const hq_params* p, const int8_t* idx,
                          const uint32_t* coset, const float* scale,
                          int64_t rows, int64_t cols, void* y, int32_t y_dtype,
                          uint32_t* status, hipStream_t stream);

/*
 * hq_rate - Rice rate and optional packing of stripped indices.
 *
 * Passages: [arXiv abstract] item (iii), [ICLR abstract] (Rice code; one
 * itemized rate accounting), [issue] (packed Rice-coded index format).
 * Per tile: rice_k and tile_bits as in hq_encode_tiles; *total_bits = sum of
 * tile_bits (written, not accumulated).  If stream_words is not NULL the
 * tiles are also packed: per tile, k (4 bits), the coset bits, then each code
 * (floor(zeta/2^k) one-bits, a zero bit, the k low bits of zeta, LSB first);
 * stream bit j is bit (j mod 32) of word j/32; each tile starts on a word
 * boundary, zero padded; tile_word_offset[t] = sum over earlier tiles of
 * ceil(tile_bits/32), tile_word_offset[n_tiles] = total words.  A tile that
 * does not fit in capacity_words is not written and sets HQ_ST_STREAM_FULL.
 *
 * With HQ_RATE_GIVEN, rice_k and tile_bits are read instead of computed:
 * the rate pass then reads 4 bytes per tile instead of the tile's indices,
 * and the indices are read once, by the packing.  They must be the values
 * the encoder wrote for these indices; otherwise the stream contents are
 * unspecified, nothing is accessed outside the buffers, a tile whose given
 * k exceeds 8 or whose codes do not fit its given tile_bits sets
 * HQ_ST_CORRUPT (its codes are not written), and a tile past
 * capacity_words still sets HQ_ST_STREAM_FULL.
 *
 * idx [n_tiles * tile] int8 (may be NULL with HQ_RATE_GIVEN when not
 * packing); coset as for encode (used only when packing);
 * rice_k [n_tiles] uint8, tile_bits [n_tiles] uint32 (outputs, or inputs
 * with HQ_RATE_GIVEN), total_bits: 1 uint64;
 * tile_word_offset [n_tiles + 1] uint64 (required when packing);
 * workspace: device scratch of at least hq_rate_workspace_bytes(n_tiles)
 * bytes, 8-byte aligned (required when packing; optional otherwise, where it
 * replaces one 64-bit atomic per block on *total_bits by a per-block sum).
 */
hq_status hq_rate(const hq_params* p, const int8_t* idx, const uint32_t* coset,
                  int64_t n_tiles, uint8_t* rice_k, uint32_t* tile_bits,
                  uint64_t* total_bits, uint32_t* stream_words,
                  uint64_t capacity_words, uint64_t* tile_word_offset,
                  void* workspace, size_t workspace_bytes, uint32_t* status,
                  hipStream_t stream);

/*
 * hq_rate_noalloc - hq_rate for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The arguments, checks and results (bit for bit) are those of
 * hq_rate with a workspace, and it likewise packs when stream_words is
 * given; there is no workspace argument.  The per-block sums live in a
 * static device array of the library, 96 KiB per GPU, allocated with the
 * code object and held until the process ends; it holds the workspace of
 * any tile count (a size that would need more is refused with HQ_ERANGE).
 * The first call on a device looks up that array's address there.  The
 * call allocates nothing.  Every call on one GPU shares the array (each
 * call writes every word it reads, so nothing needs clearing): calls that
 * overlap on one GPU, on different streams or from different host threads,
 * race and leave unspecified results.
 */
hq_status hq_rate_noalloc(const hq_params* p, const int8_t* idx, const uint32_t* coset,
                          int64_t n_tiles, uint8_t* rice_k, uint32_t* tile_bits,
                          uint64_t* total_bits, uint32_t* stream_words,
                          uint64_t capacity_words, uint64_t* tile_word_offset,
                          uint32_t* status, hipStream_t stream);

/*
 * hq_rate_batch - hq_rate for `count` matrices that share p (a layer's
 * projections), enqueued as at most four kernel launches per group of up to
 * eight matrices instead of up to four per matrix.  Same passages,
 * arguments per item and results (bit for bit) as one hq_rate call per item
 * with a workspace.  The workspace (device, 8-byte aligned, at least
 * hq_rate_batch_workspace_bytes(count, items) bytes: each item's
 * hq_rate_workspace_bytes, in item order) is required; an item with
 * n_tiles 0 is skipped.
 */
typedef struct {
  const int8_t* idx;            /* [n_tiles * tile] (NULL: HQ_RATE_GIVEN, no packing) */
  const uint32_t* coset;        /* [n_tiles * words] (packing, E8 / A2)           */
  int64_t n_tiles;
  uint8_t* rice_k;              /* [n_tiles]                                      */
  uint32_t* tile_bits;          /* [n_tiles]                                      */
  uint64_t* total_bits;         /* one value                                      */
  uint32_t* stream_words;       /* NULL: rate only                                */
  uint64_t capacity_words;
  uint64_t* tile_word_offset;   /* [n_tiles + 1] (packing)                        */
} hq_rate_item;

hq_status hq_rate_batch(const hq_params* p, int32_t count, const hq_rate_item* items,
                        void* workspace, size_t workspace_bytes, uint32_t* status,
                        hipStream_t stream);

/* Device workspace bytes hq_rate_batch needs; 0 for invalid arguments. */
size_t hq_rate_batch_workspace_bytes(int32_t count, const hq_rate_item* items);

/*
 * hq_unpack - decode a packed stream back to stripped indices, coset words
 * and Rice parameters: the inverse of the packing done by hq_rate.
 *
 * Passages: [issue] "Additional context" (a packed, Rice-coded lattice-index
 * checkpoint format, to be read back), [arXiv abstract] item (iii) and
 * [ICLR abstract] (the Rice code itself).  The layout is the one written by
 * hq_rate: per tile k (4 bits), the coset bits, then per index a run of
 * floor(zeta/2^k) one-bits, a zero bit and the k low bits of zeta (LSB
 * first), with zeta the zigzag map of the index; stream bit j is bit
 * (j mod 32) of word j/32; tile t occupies words [tile_word_offset[t],
 * tile_word_offset[t + 1]).  Any k in 0..15 is accepted.
 *
 * stream_words: the words (device, read only within the tiles' ranges);
 * tile_word_offset [n_tiles + 1] uint64 (device); idx [n_tiles * tile] int8
 * out; coset [n_tiles * hq_coset_words(p)] uint32 out (NULL iff that is 0);
 * rice_k [n_tiles] uint8 out, or NULL.  Only lattice, tile and HQ_IDX16 of
 * p are used (with HQ_IDX16 idx receives int16 values).
 * A tile whose codes run past its words, whose word range is reversed, or
 * that decodes an index outside int8 (int16) sets HQ_ST_CORRUPT; its outputs are
 * unspecified and no word outside its range is read.  idx must be 16-byte
 * aligned.
 */
hq_status hq_unpack(const hq_params* p, const uint32_t* stream_words,
                    const uint64_t* tile_word_offset, int64_t n_tiles,
                    int8_t* idx, uint32_t* coset, uint8_t* rice_k,
                    uint32_t* status, hipStream_t stream);

/*
 * hq_unpack_batch - hq_unpack for `count` packed matrices that share p (a
 * layer's projections), enqueued as one launch per group of up to eight.
 * The decoder runs one lane per tile, so a single small matrix occupies a
 * fraction of the GPU; a layer's matrices decoded together fill it.  Same
 * passages, arguments per item and results (bit for bit) as one hq_unpack
 * call per item.  `items` is a host array read during the call; every item
 * is validated and nothing is enqueued unless all pass; an item with
 * n_tiles 0 is skipped.
 */
typedef struct {
  const uint32_t* stream_words;        /* device, read only in the ranges  */
  const uint64_t* tile_word_offset;    /* [n_tiles + 1]                    */
  int64_t n_tiles;
  int8_t* idx;                         /* [n_tiles * tile], 16-byte aligned */
  uint32_t* coset;                     /* [n_tiles * hq_coset_words(p)]    */
  uint8_t* rice_k;                     /* [n_tiles] or NULL                */
} hq_unpack_item;

hq_status hq_unpack_batch(const hq_params* p, int32_t count, const hq_unpack_item* items,
                          uint32_t* status, hipStream_t stream);

/*
 * hq_gemv - y = W x for E8-coded weights, without forming W: the consumer
 * of the format ([issue] "Is your feature request related to a problem?":
 * decode must be usable at inference; [ICLR abstract]: algebraic decoding).
 *
 * W is the matrix hq_decode_tiles reconstructs (before its output rounding):
 * tile t of row r is w = s (.) H P Delta / (2 sqrt(n)), P = 2p the stored
 * lattice point.  Since H is symmetric, w . x_t = Delta / (2 sqrt(n)) *
 * <P, H (s (.) x_t)>, so the kernel rotates each n-column slice of x once
 * (into the workspace) and then needs only the stored indices of W.
 *
 * p: lattice E8, tile 256, rht_seed of the encode; no dither.
 * idx [rows*cols] int8 (cols a multiple of 256, at most 2^24), coset
 * [n_tiles] words, scale [n_tiles] fp32 (tile t = row t / (cols/256),
 * column slice t mod (cols/256)); x [m][cols] fp32 (m vectors, each
 * contiguous), 1 <= m <= 8; y [m][rows] fp32 out; workspace: device
 * scratch of at least hq_gemv_workspace_bytes(rows, cols, m) bytes,
 * 16-byte aligned.  Results are fp32 sums of the products in a fixed order
 * (deterministic).  Errors as for decode; HQ_EUNSUPPORTED for another
 * lattice or tile, or HQ_DITHER.
 */
hq_status hq_gemv(const hq_params* p, const int8_t* idx, const uint32_t* coset,
                  const float* scale, int64_t rows, int64_t cols, const float* x,
                  int32_t m, float* y, void* workspace, size_t workspace_bytes,
                  uint32_t* status, hipStream_t stream);

/* Device workspace bytes hq_gemv needs for a rows x cols matrix and m
   vectors (the rotated vectors, their 8-block sums, and the totals of the
   column chunks when a row has more than one); 0 for invalid sizes. */
size_t hq_gemv_workspace_bytes(int64_t rows, int64_t cols, int32_t m);

/*
 * hq_gemv_batch - hq_gemv for `count` matrices with the same m and the same
 * p (a layer's projections), enqueued as three kernel launches per group of
 * up to eight matrices instead of up to three per matrix.  Same passages,
 * arguments per item and results (bit for bit) as one hq_gemv call per item.
 * `items` is a host array read during the call; every item is validated and
 * nothing is enqueued unless all pass.  The workspace (16-byte aligned, at
 * least hq_gemv_batch_workspace_bytes(count, items, m) bytes) is divided
 * among the items in order; an item with rows or cols 0 is skipped.
 */
typedef struct {
  const int8_t* idx;      /* [rows*cols]                                */
  const uint32_t* coset;  /* [n_tiles]                                  */
  const float* scale;     /* [n_tiles]                                  */
  int64_t rows, cols;
  const float* x;         /* [m][cols]                                  */
  float* y;               /* [m][rows]                                  */
} hq_gemv_item;

hq_status hq_gemv_batch(const hq_params* p, int32_t count, const hq_gemv_item* items,
                        int32_t m, void* workspace, size_t workspace_bytes,
                        uint32_t* status, hipStream_t stream);

/* Device workspace bytes hq_gemv_batch needs (the sum over the items of
   hq_gemv_workspace_bytes); 0 for invalid arguments. */
size_t hq_gemv_batch_workspace_bytes(int32_t count, const hq_gemv_item* items, int32_t m);

/*
 * hq_gemm - Y = W X^T for many vectors on the bf16 matrix cores, from the
 * stored indices of W: the GEMM counterpart of hq_gemv (same passages,
 * same W).  Per 256-column slice, (Delta / 32) <P, H (s (.) x)>: the lattice
 * points |P| <= 255 are exact in bf16, the rotated inputs H (s (.) x) are
 * formed in fp64 and held as two bf16 terms (their rounding and the
 * rounding of the rest, |error| <= 2^-17 of each value), the products are
 * exact and accumulate in fp32 inside the MFMA; each slice's sum is scaled
 * by its tile's Delta / 32 and added in fp32.  Deterministic.
 *
 * p: lattice E8, tile 256, rht_seed of the encode; no dither.
 * idx [rows*cols] int8 (16-byte aligned), coset [n_tiles] words, scale
 * [n_tiles] fp32 as for hq_gemv; cols a multiple of 256 and at most 2^22,
 * rows at most 2^23; x [m][cols] fp32 (16-byte aligned), 1 <= m <= 65536
 * with m cols and m rows at most 2^31 (and each launch's grid below 2^32
 * work-items, which only the largest of these sizes reach); y [m][rows]
 * fp32 out; workspace:
 * device scratch of at least hq_gemm_workspace_bytes(rows, cols, m) bytes,
 * 16-byte aligned.  Errors as for hq_gemv (HQ_EINVAL for sizes out of
 * range).
 */
hq_status hq_gemm(const hq_params* p, const int8_t* idx, const uint32_t* coset,
                  const float* scale, int64_t rows, int64_t cols, const float* x,
                  int32_t m, float* y, void* workspace, size_t workspace_bytes,
                  uint32_t* status, hipStream_t stream);

/* Device workspace bytes hq_gemm needs: the rotated inputs as two bf16
   terms (4 m cols bytes) and, when the slices are split over several blocks
   to occupy the device, their partial sums (4 m rows bytes per range, added
   in range order; the split is a function of the sizes alone, so results
   repeat bit for bit); 0 for invalid sizes. */
size_t hq_gemm_workspace_bytes(int64_t rows, int64_t cols, int32_t m);

/*
 * hq_gemm_batch - hq_gemm for `count` matrices with the same m and the same
 * p (a layer's projections), enqueued as three kernel launches per group of
 * up to eight matrices instead of up to three per matrix.  Same passages,
 * arguments per item (hq_gemv_item) and error bound as hq_gemm.  The slice
 * ranges summed by separate blocks are chosen for each group of eight as a
 * whole, so an item may round differently than in a call of its own; the
 * same call repeats its bits.  The workspace (device, 16-byte aligned, at
 * least hq_gemm_batch_workspace_bytes(count, items, m) bytes) is divided
 * among the groups in order; an item with rows or cols 0 is skipped.
 */
hq_status hq_gemm_batch(const hq_params* p, int32_t count, const hq_gemv_item* items,
                        int32_t m, void* workspace, size_t workspace_bytes,
                        uint32_t* status, hipStream_t stream);

/* Device workspace bytes hq_gemm_batch needs (each item's input terms and,
   where its group's plan splits its slices, its partial sums); 0 for
   invalid arguments. */
size_t hq_gemm_batch_workspace_bytes(int32_t count, const hq_gemv_item* items, int32_t m);

/*
 * hq_kv_scores - attention scores of queries against one head's compressed
 * keys: scores[j][k] = q_j . khat_k, khat_k the key hq_decode_tiles would
 * reconstruct (dither subtracted), without forming khat.
 *
 * Passages: [ICLR abstract] (subtractive dither keeps each cached inner
 * product unbiased; algebraic decoding), [arXiv abstract] ideas (i)-(iii).
 * khat = s (.) H yhat / sqrt(n) with yhat = Delta (p - d), and H is
 * symmetric, so q . khat = <H (s (.) q), yhat> / sqrt(n): the queries are
 * rotated once (into the workspace) and each key's yhat is formed from its
 * stored indices and regenerated dither.
 *
 * p: lattice E8, tile 128 (the head dimension), rht_seed of the encode;
 * HQ_DITHER with the encode's dither_seed, and dither_base = global index of
 * key 0 (as for hq_kv_encode), or no dither (rotation-only keys).
 * q [n_q][128] fp32; idx [n_keys][128] int8, coset [n_keys] uint32 (16 coset
 * bits), scale [n_keys] fp32 as written by hq_kv_encode; scores [n_q][n_keys]
 * fp32 out (n_q < 2^25, n_keys <= 2^32 - 256); workspace: device scratch of
 * at least hq_kv_scores_workspace_bytes(n_q) bytes.  fp32 arithmetic in a
 * fixed order.
 */
hq_status hq_kv_scores(const hq_params* p, const float* q, int64_t n_q,
                       const int8_t* idx, const uint32_t* coset, const float* scale,
                       int64_t n_keys, float* scores, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* Device workspace bytes hq_kv_scores needs for n_q queries. */
size_t hq_kv_scores_workspace_bytes(int64_t n_q);

/*
 * hq_kv_attention - decode attention over compressed K and V, per head:
 * out_hj = sum_k a_hjk vhat_hk, a_hjk = softmax over k of tau q_hj . khat_hk,
 * with khat and vhat the vectors hq_decode_tiles would reconstruct (dither
 * subtracted), without forming either.
 *
 * Passages: as hq_kv_scores.  The pages give no attention procedure; this
 * is softmax attention of one head over the decoded cache.  Both caches
 * stay in the lattice domain: scores as in hq_kv_scores (queries rotated
 * once, scaled by tau log2(e) / sqrt(n), so the softmax runs in base 2), the
 * weighted sum of the values' yhat = Delta (p - d) is formed per query and
 * rotated back once: sum_k a_jk vhat_k = s_V (.) H (sum_k a_jk yhatV_k) /
 * sqrt(n).  Keys are split into ranges; each keeps a running maximum, its
 * exponent sum and weighted sum (fp32), and the ranges are merged in order
 * (deterministic).
 *
 * pk, pv: the K and V encodes' parameters (lattice E8, tile 128; rht_seed;
 * HQ_DITHER with dither_seed and dither_base = global index of vector 0, or
 * no dither).  k_* and v_*: [n_heads][n_keys] vectors as hq_kv_encode writes
 * them for the whole cache (key k of head h is vector h n_keys + k; idx
 * 16-byte aligned); n_keys >= 1 when n_q > 0.  q [n_heads][n_q][128] fp32
 * (16-byte aligned), 1 <= n_heads <= 65535, n_q <= 65536 queries per head
 * (grouped queries share a head), n_heads n_q < 2^25, n_heads n_keys <= 2^32
 * (and the launch grid below 2^32 work-items, which only extreme sizes
 * reach); tau the score scale (finite; 1/sqrt(128)
 * for standard attention); out [n_heads][n_q][128] fp32; workspace: device
 * scratch of at least hq_kv_attention_workspace_bytes(n_heads, n_q, n_keys)
 * bytes, 16-byte aligned.  Errors as hq_kv_scores.
 */
hq_status hq_kv_attention(const hq_params* pk, const int8_t* k_idx, const uint32_t* k_coset,
                          const float* k_scale, const hq_params* pv, const int8_t* v_idx,
                          const uint32_t* v_coset, const float* v_scale, int64_t n_heads,
                          int64_t n_keys, const float* q, int64_t n_q, float tau, float* out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Device workspace bytes hq_kv_attention needs; 0 for invalid sizes. */
size_t hq_kv_attention_workspace_bytes(int64_t n_heads, int64_t n_q, int64_t n_keys);

/*
 * hq_kv_encode - encode KV-cache vectors ([ICLR abstract]: subtractive
 * dither keeps each cached inner product unbiased per vector; [arXiv
 * abstract] item (iv)).  The vectors are tiles of n = p->tile = head_dim
 * (128 or 256), lattice E8.  With HQ_DITHER, vector v (global index
 * dither_base + v) gets the dither d = w - Q_E8(w), w_i = 2^-23 *
 * (SplitMix64((seed << 40) ^ ((v << 8) | i)) >> 40) - 1, and is encoded as
 * Q_E8(u + d).  Without HQ_DITHER this is hq_encode_tiles on the vectors
 * (the rotation-only control).  Outputs as for hq_encode_tiles; decode with
 * hq_decode_tiles and the same flags, seed and base.
 */
hq_status hq_kv_encode(const hq_params* p, const void* kv, int32_t kv_dtype,
                       int64_t n_vectors, float* scale, int8_t* idx,
                       uint32_t* coset, uint8_t* rice_k, uint32_t* tile_bits,
                       uint32_t* status, hipStream_t stream);

/*
 * Batched calls.  A transformer layer's projections share one parameter
 * block (lattice, tile, rate, RHT seed, flags); encoding or decoding them in
 * one call lets the library cover several matrices with one persistent
 * launch (up to 8 matrices per launch on the E8 / tile 256 path), which
 * keeps the GPU full on small matrices and removes per-matrix launch gaps.
 * Results are bit-identical to one hq_encode_tiles / hq_decode_tiles call per
 * item.  `items` is a host array of `count` descriptors read during the call;
 * every item is validated as the single call would be, and nothing is
 * enqueued unless all of them pass.  HQ_WANT_COORDS and HQ_DITHER are not
 * accepted here (HQ_EUNSUPPORTED).  Same passages as the single calls.
 */
typedef struct {
  const void* x;          /* [rows*cols] of x_dtype                     */
  int64_t rows, cols;
  float* scale;           /* [n_tiles]: out with HQ_SCALE_AUTO, else in */
  int8_t* idx;            /* [rows*cols]                                */
  uint32_t* coset;        /* [n_tiles * hq_coset_words(p)]              */
  uint8_t* rice_k;        /* [n_tiles]                                  */
  uint32_t* tile_bits;    /* [n_tiles]                                  */
} hq_encode_item;

typedef struct {
  const int8_t* idx;      /* [rows*cols]                                */
  const uint32_t* coset;  /* [n_tiles * hq_coset_words(p)]              */
  const float* scale;     /* [n_tiles]                                  */
  int64_t rows, cols;
  void* y;                /* [rows*cols] of y_dtype                     */
} hq_decode_item;

hq_status hq_encode_batch(const hq_params* p, int32_t x_dtype, int32_t count,
                          const hq_encode_item* items, uint32_t* status,
                          hipStream_t stream);

hq_status hq_decode_batch(const hq_params* p, int32_t y_dtype, int32_t count,
                          const hq_decode_item* items, uint32_t* status,
                          hipStream_t stream);

/*
 * Encode one batch and decode another, independent batch in one call: the
 * results are exactly those of hq_encode_batch(enc_p, x_dtype, enc_count,
 * enc_items) followed by hq_decode_batch(dec_p, y_dtype, dec_count,
 * dec_items), with the same validation of every item.  For a model streamed
 * through the codec ([arXiv abstract] "HyperQuant: A Rate-Distortion-Optimal
 * Quantization Pipeline ..." ideas (i)-(iii), [ICLR abstract] "HyperQuant: A
 * Near-Entropy-Optimal Lattice Quantization Pipeline ...": rotation, lattice
 * point, strip and Rice rate, then the algebraic decode) the caller encodes
 * layer l + 1 while it decodes layer l.  On the E8 / tile 256 / bf16-input
 * path, with at most 8 non-empty matrices on each side, one launch runs both
 * (each wave alternates an encode group and a decode group, so the encoder's
 * arithmetic overlaps the decoder's memory traffic); otherwise the two
 * batches are enqueued one after the other.  The batches must be
 * independent: HQ_EINVAL when an encode output (idx, scale, coset, rice_k,
 * tile_bits) overlaps a decode input or output, or a decode output overlaps
 * an encode input.  `status` (optional device word) collects both sides'
 * status bits.
 */
hq_status hq_encode_decode_batch(const hq_params* enc_p, int32_t x_dtype,
                                 int32_t enc_count, const hq_encode_item* enc_items,
                                 const hq_params* dec_p, int32_t y_dtype,
                                 int32_t dec_count, const hq_decode_item* dec_items,
                                 uint32_t* status, hipStream_t stream);

/* Coset words per tile: E8 ceil(n/256), A2 ceil(n/64), D4 and Z 0;
 * -1 on an invalid p. */
int32_t hq_coset_words(const hq_params* p);

/* Device workspace bytes hq_rate needs to pack n_tiles tiles. */
size_t hq_rate_workspace_bytes(int64_t n_tiles);

/* Static description of a status code (never NULL). */
const char* hq_status_string(hq_status s);

/* Host-side helpers (no device work; usable without a GPU). */

/* SplitMix64 output for state `key` (Steele, Lea & Flood, OOPSLA 2014). */
uint64_t hq_splitmix64(uint64_t key);

/* Writes the n RHT signs (+1 / -1) for `seed` into host memory `out`. */
hq_status hq_rht_signs(uint32_t seed, int32_t n, int8_t* out);

/* The auto-scale constant c(L, R) = sqrt(2 pi e) 2^-R / vol^(1/d) for p. */
hq_status hq_scale_constant(const hq_params* p, double* out);

/* Library version as 10000*major + 100*minor + patch. */
int32_t hq_version(void);

/*
 * Checkpoint files - the packed, Rice-coded lattice-index format on disk
 * ([issue] "Additional context": a packed, Rice-coded lattice-index
 * checkpoint format, to be read back; [arXiv abstract] item (iii)).  Host
 * code only: every array below is host memory, and no device call is made.
 *
 * A file holds records, one per packed matrix, each named.  Layout (host
 * byte order; little-endian on every supported host): the file magic
 * "HQCKPT" 0 1, then per record a 136-byte header (magic "HQRE", header
 * size, the hq_ckpt_entry below, payload bytes, FNV-1a 64 checksum of the
 * payload) and the payload: scale[n_tiles] fp32, padded to 8 bytes;
 * tile_word_offset[n_tiles + 1] uint64; words[n_words] uint32, padded to 8
 * bytes.  The stream is the one hq_rate packs and hq_unpack decodes (each
 * tile's k and coset bits inline), so loading a matrix is: read the record,
 * copy the three arrays to the device, hq_unpack (or hq_unpack_batch).
 */
typedef struct {
  char name[64];          /* NUL-terminated, 1..63 bytes, unique per file   */
  int32_t lattice;        /* hq_lattice of the encode                       */
  int32_t tile;           /* 64, 128, 256 or 512                            */
  float bps;              /* rate R of the encode, 0 < R <= 8               */
  uint32_t rht_seed;      /* RHT seed of the encode                         */
  int64_t rows, cols;     /* the matrix; rows * cols = n_tiles * tile       */
  int64_t n_tiles;
  uint64_t n_words;       /* stream words, tile_word_offset[n_tiles]        */
} hq_ckpt_entry;

/* Appends one record to `path` (created with the file magic if missing).
 * scale [n_tiles], tile_word_offset [n_tiles + 1] (starting at 0, never
 * decreasing, ending at n_words) and words [n_words] are host arrays.
 * HQ_EINVAL: an invalid entry or offsets, a NULL array, or a name the file
 * already holds; HQ_EFORMAT: the file exists but is not a checkpoint;
 * HQ_EIO: the file cannot be opened or written. */
hq_status hq_ckpt_append(const char* path, const hq_ckpt_entry* e, const float* scale,
                         const uint64_t* tile_word_offset, const uint32_t* words);

/* Number of records in `path` (HQ_EIO / HQ_EFORMAT as above). */
hq_status hq_ckpt_count(const char* path, int32_t* count);

/* The entry of record i (0-based, file order); HQ_ENOTFOUND past the end. */
hq_status hq_ckpt_entry_at(const char* path, int32_t i, hq_ckpt_entry* e);

/* Reads the record named `name` into e and the host arrays: scale holds
 * capacity_tiles values, tile_word_offset capacity_tiles + 1, words
 * capacity_words (HQ_EINVAL if the record needs more; at most 2^48 weights
 * per record).  HQ_ENOTFOUND: no such record;
 * HQ_EFORMAT: a truncated record, a checksum mismatch or offsets that do
 * not hold (the arrays' contents are then unspecified). */
hq_status hq_ckpt_read(const char* path, const char* name, hq_ckpt_entry* e, float* scale,
                       uint64_t* tile_word_offset, uint32_t* words, int64_t capacity_tiles,
                       uint64_t capacity_words);

#ifdef __cplusplus
}
#endif

#endif /* HQ_H */
