// C ABI of the HyperQuant hot path: argument validation, sign vectors,
// kernel launches.  Every check that needs no device call runs first, so a
// rejected call touches nothing on the GPU.
//
// Passages: [arXiv abstract] "HyperQuant: A Rate-Distortion-Optimal
// Quantization Pipeline ..." ideas (i)-(iv); [ICLR abstract] "HyperQuant: A
// Near-Entropy-Optimal Lattice Quantization Pipeline ..."; the statement of
// the problem there (tile, lattice, target rate, per-tile scale and seed in;
// lattice indices, coset bits, Rice parameters and bit lengths out) is the
// shape of this interface.
#include <math.h>
#include <string.h>

#include <mutex>

#include "hq.h"
#include "hq_device.h"
#include "hq_internal.h"
#include "hq_kvattn.h"
#include "hq_ratebatch.h"

namespace hq {
}

// Scratch of hq_rate_noalloc: the per-block word and bit sums and per-wave
// word sums that hq_rate keeps in its caller's workspace.  The rate pass
// runs at most 8192 waves (2048 blocks), so 6 * 2048 uint64 hold the
// workspace of any tile count.  Each GPU the library runs on holds its own
// copy until the process ends.
constexpr size_t kRateScratchWords = 6 * 2048;
static __device__ __align__(256) uint64_t scratch[kRateScratchWords];

namespace {

using namespace hq;

// Device address of `scratch` on the current device, looked up once per
// device (the host-side name is not a device address).
constexpr int kScratchDevices = 64;
void* g_scratch_ptr[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];
std::once_flag g_scratch_once[kScratchDevices];

hq_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) {
    (void)hipGetLastError();
    return HQ_EDEVICE;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* q = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = q;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return HQ_EDEVICE;
  *out = g_scratch_ptr[dev];
  return HQ_OK;
}

constexpr uint32_t kKnownFlags =
    HQ_SCALE_AUTO | HQ_DITHER | HQ_WANT_COORDS | HQ_RATE_CONTROL | HQ_RATE_GIVEN | HQ_IDX16;

bool lattice_ok(int32_t l) { return l == HQ_E8 || l == HQ_D4 || l == HQ_A2 || l == HQ_Z; }

// Validates the parameter block; `need_range` adds the auto-scale bound.
hq_status check_params(const hq_params* p) {
  if (p == nullptr || p->struct_size != sizeof(hq_params)) return HQ_EINVAL;
  if (!lattice_ok(p->lattice)) return HQ_EINVAL;
  if (p->tile != 64 && p->tile != 128 && p->tile != 256 && p->tile != kMaxTile) return HQ_EINVAL;
  if (!(p->bps > 0.0f) || !(p->bps <= 8.0f)) return HQ_EINVAL;
  if ((p->flags & ~kKnownFlags) != 0 || p->reserved != 0) return HQ_EINVAL;
  if (p->flags & HQ_RATE_CONTROL) {
    if (!(p->flags & HQ_SCALE_AUTO)) return HQ_EINVAL;     // the scales are outputs
    if (p->flags & HQ_DITHER) return HQ_EUNSUPPORTED;
  }
  // the int16 index mode runs on the generic kernels, without dither or
  // rate control
  if ((p->flags & HQ_IDX16) && (p->flags & (HQ_DITHER | HQ_RATE_CONTROL))) return HQ_EUNSUPPORTED;
  if (p->flags & HQ_DITHER) {
    if (p->lattice != HQ_E8) return HQ_EUNSUPPORTED;
    if (p->tile > 256) return HQ_EUNSUPPORTED;   // the dither key holds coordinates < 256
    if (p->dither_seed >= (1u << 24)) return HQ_EINVAL;
    if (p->dither_base < 0) return HQ_EINVAL;
  }
  return HQ_OK;
}

double vol_root(int32_t lattice) {
  switch (lattice) {
    case HQ_D4: return sqrt(sqrt(2.0));
    case HQ_A2: return sqrt(sqrt(3.0) / 2.0);
    default: return 1.0;
  }
}

// c(L, R) = sqrt(2 pi e) 2^-R / vol^(1/d)   (high-resolution scale constant)
double scale_constant(const hq_params* p) {
  return sqrt(2.0 * M_PI * M_E) * pow(2.0, -(double)p->bps) / vol_root(p->lattice);
}

// Auto scale keeps |index| <= sqrt(n)/c + 2 inside int8, or in the int16
// index mode within the 64-bit grid's clamp (|u| <= 32000, inside int16).
bool range_ok(const hq_params* p) {
  const double bound = (p->flags & HQ_IDX16) ? 32000.0 : 127.0;
  return sqrt((double)p->tile) / scale_constant(p) + 2.0 <= bound;
}

// Calls that take int8 indices only.
bool idx16(const hq_params* p) { return (p->flags & HQ_IDX16) != 0; }

int32_t coset_words(const hq_params* p) {
  if (p->lattice == HQ_E8) return (p->tile / 8 + 31) / 32;
  if (p->lattice == HQ_A2) return (p->tile / 2 + 31) / 32;
  return 0;
}

int32_t coset_bits(const hq_params* p) {
  if (p->lattice == HQ_E8) return p->tile / 8;
  if (p->lattice == HQ_A2) return p->tile / 2;
  return 0;
}

bool aligned16(const void* q) { return ((uintptr_t)q & 15u) == 0; }

// out: (n + 31) / 32 words
void make_signs(uint32_t seed, int n, uint32_t* out) {
  for (int w = 0; w < (n + 31) / 32; ++w) out[w] = 0;
  for (int j = 0; j < n; ++j) {
    const uint64_t h = splitmix64(((uint64_t)seed << 32) ^ (uint64_t)j);
    if (h >> 63) out[j >> 5] |= 1u << (j & 31);
  }
}

// Device-pointer check (one HIP query per pointer); clears the error a
// failed query leaves behind.
bool on_device(const void* q) {
  if (q == nullptr) return false;
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof(attr));
  if (hipPointerGetAttributes(&attr, q) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged ||
         attr.type == hipMemoryTypeUnified;
}

hq_status launched(hipError_t e) { return e == hipSuccess ? HQ_OK : HQ_EDEVICE; }

void set_rate_control(const hq_params* p, EncodeLaunch& a) {
  a.rate_control = (p->flags & HQ_RATE_CONTROL) != 0;
  a.rc_budget = (uint32_t)floor((double)p->bps * (double)p->tile);
}

// Shared validation of an encode-shaped call.
hq_status check_encode(const hq_params* p, const void* x, int32_t x_dtype, int64_t rows,
                       int64_t cols, const float* scale, const int8_t* idx,
                       const uint32_t* coset, const uint8_t* rice_k,
                       const uint32_t* tile_bits, const int16_t* coords) {
  hq_status st = check_params(p);
  if (st != HQ_OK) return st;
  if (x_dtype != HQ_F32 && x_dtype != HQ_BF16) return HQ_EINVAL;
  if (rows < 0 || cols < 0) return HQ_EINVAL;
  if (cols % p->tile != 0) return HQ_EINVAL;
  if (rows == 0 || cols == 0) return HQ_OK;   // zero tiles: a no-op, buffers unused
  if (x == nullptr || scale == nullptr || idx == nullptr || rice_k == nullptr ||
      tile_bits == nullptr)
    return HQ_EINVAL;
  if (coset_words(p) > 0 && coset == nullptr) return HQ_EINVAL;
  if ((p->flags & HQ_WANT_COORDS) && coords == nullptr) return HQ_EINVAL;
  if (!aligned16(x) || !aligned16(idx) || ((p->flags & HQ_WANT_COORDS) && !aligned16(coords)))
    return HQ_EINVAL;
  if (rows > 0 && cols > 0 && rows > INT64_MAX / cols) return HQ_EINVAL;
  // (rate control keeps the indices in range by itself)
  if ((p->flags & HQ_SCALE_AUTO) && !(p->flags & HQ_RATE_CONTROL) && !range_ok(p))
    return HQ_ERANGE;
  return HQ_OK;
}

}  // namespace

extern "C" {

hq_status hq_encode_tiles(const hq_params* p, const void* x, int32_t x_dtype, int64_t rows,
                          int64_t cols, float* scale, int8_t* idx, uint32_t* coset,
                          uint8_t* rice_k, uint32_t* tile_bits, int16_t* coords,
                          uint32_t* status, hipStream_t stream) {
  hq_status st = check_encode(p, x, x_dtype, rows, cols, scale, idx, coset, rice_k, tile_bits,
                              coords);
  if (st != HQ_OK) return st;
  if (p->flags & HQ_DITHER) return HQ_EUNSUPPORTED;
  const int64_t n_tiles = rows * cols / p->tile;
  if (n_tiles == 0) return HQ_OK;
  if (!on_device(x) || !on_device(scale) || !on_device(idx) || !on_device(rice_k) ||
      !on_device(tile_bits) || (coset_words(p) > 0 && !on_device(coset)) ||
      ((p->flags & HQ_WANT_COORDS) && !on_device(coords)) ||
      (status != nullptr && !on_device(status)))
    return HQ_EINVAL;
  EncodeLaunch a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.in_bf16 = x_dtype == HQ_BF16;
  a.n_tiles = n_tiles;
  a.lattice = p->lattice;
  a.tile = p->tile;
  a.scale = scale;
  a.auto_scale = (p->flags & HQ_SCALE_AUTO) != 0;
  a.idx = idx;
  a.coset = coset;
  a.rice_k = rice_k;
  a.tile_bits = tile_bits;
  a.coords = (p->flags & HQ_WANT_COORDS) ? coords : nullptr;
  a.status = status;
  make_signs(p->rht_seed, p->tile, a.signs);
  a.c = scale_constant(p);
  a.sqrt_n = sqrt((double)p->tile);
  set_rate_control(p, a);
  a.wide = idx16(p) ? 1 : 0;
  return launched(launch_encode(a, stream));
}

hq_status hq_kv_encode(const hq_params* p, const void* kv, int32_t kv_dtype, int64_t n_vectors,
                       float* scale, int8_t* idx, uint32_t* coset, uint8_t* rice_k,
                       uint32_t* tile_bits, uint32_t* status, hipStream_t stream) {
  hq_status st = check_params(p);
  if (st != HQ_OK) return st;
  if (p->lattice != HQ_E8) return HQ_EUNSUPPORTED;
  if (p->flags & (HQ_WANT_COORDS | HQ_IDX16)) return HQ_EUNSUPPORTED;
  if (n_vectors < 0) return HQ_EINVAL;
  st = check_encode(p, kv, kv_dtype, n_vectors, p->tile, scale, idx, coset, rice_k, tile_bits,
                    nullptr);
  if (st != HQ_OK) return st;
  if ((p->flags & HQ_DITHER) && p->dither_base + n_vectors > ((int64_t)1 << 32))
    return HQ_EINVAL;
  if (n_vectors == 0) return HQ_OK;
  if (!on_device(kv) || !on_device(scale) || !on_device(idx) || !on_device(rice_k) ||
      !on_device(tile_bits) || !on_device(coset) || (status != nullptr && !on_device(status)))
    return HQ_EINVAL;
  EncodeLaunch a;
  memset(&a, 0, sizeof(a));
  a.x = kv;
  a.in_bf16 = kv_dtype == HQ_BF16;
  a.n_tiles = n_vectors;
  a.lattice = HQ_E8;
  a.tile = p->tile;
  a.scale = scale;
  a.auto_scale = (p->flags & HQ_SCALE_AUTO) != 0;
  a.idx = idx;
  a.coset = coset;
  a.rice_k = rice_k;
  a.tile_bits = tile_bits;
  a.coords = nullptr;
  a.status = status;
  make_signs(p->rht_seed, p->tile, a.signs);
  a.c = scale_constant(p);
  a.sqrt_n = sqrt((double)p->tile);
  set_rate_control(p, a);
  a.dither = (p->flags & HQ_DITHER) != 0;
  a.dither_seed = p->dither_seed;
  a.dither_base = p->dither_base;
  return launched(launch_encode(a, stream));
}

hq_status hq_decode_tiles(const hq_params* p, const int8_t* idx, const uint32_t* coset,
                          const float* scale, int64_t rows, int64_t cols, void* y,
                          int32_t y_dtype, uint32_t* status, hipStream_t stream) {
  hq_status st = check_params(p);
  if (st != HQ_OK) return st;
  if (y_dtype != HQ_F32 && y_dtype != HQ_BF16) return HQ_EINVAL;
  if (rows < 0 || cols < 0 || cols % p->tile != 0) return HQ_EINVAL;
  if (rows == 0 || cols == 0) return HQ_OK;   // zero tiles: a no-op
  if (idx == nullptr || scale == nullptr || y == nullptr) return HQ_EINVAL;
  if (coset_words(p) > 0 && coset == nullptr) return HQ_EINVAL;
  if (!aligned16(idx) || !aligned16(y)) return HQ_EINVAL;
  if (rows > 0 && cols > 0 && rows > INT64_MAX / cols) return HQ_EINVAL;
  const int64_t n_tiles = rows * cols / p->tile;
  if ((p->flags & HQ_DITHER) && p->dither_base + n_tiles > ((int64_t)1 << 32))
    return HQ_EINVAL;
  if (n_tiles == 0) return HQ_OK;
  if (!on_device(idx) || !on_device(scale) || !on_device(y) ||
      (coset_words(p) > 0 && !on_device(coset)) || (status != nullptr && !on_device(status)))
    return HQ_EINVAL;
  DecodeLaunch a;
  memset(&a, 0, sizeof(a));
  a.idx = idx;
  a.coset = coset;
  a.scale = scale;
  a.n_tiles = n_tiles;
  a.lattice = p->lattice;
  a.tile = p->tile;
  a.y = y;
  a.out_bf16 = y_dtype == HQ_BF16;
  a.status = status;
  make_signs(p->rht_seed, p->tile, a.signs);
  a.inv_sqrt_n = 1.0 / sqrt((double)p->tile);
  a.dither = (p->flags & HQ_DITHER) != 0;
  a.dither_seed = p->dither_seed;
  a.dither_base = p->dither_base;
  a.wide = idx16(p) ? 1 : 0;
  return launched(launch_decode(a, stream));
}

extern "C++" {
namespace {

// Validation of an encode batch: every item as hq_encode_tiles would check
// it, and device residence of every pointer.
hq_status check_encode_batch(const hq_params* p, int32_t x_dtype, int32_t count,
                             const hq_encode_item* items, uint32_t* status) {
  hq_status st = check_params(p);
  if (st != HQ_OK) return st;
  if (p->flags & (HQ_WANT_COORDS | HQ_DITHER | HQ_IDX16)) return HQ_EUNSUPPORTED;
  if (count < 0 || (count > 0 && items == nullptr)) return HQ_EINVAL;
  for (int32_t i = 0; i < count; ++i) {
    const hq_encode_item& it = items[i];
    st = check_encode(p, it.x, x_dtype, it.rows, it.cols, it.scale, it.idx, it.coset, it.rice_k,
                      it.tile_bits, nullptr);
    if (st != HQ_OK) return st;
  }
  for (int32_t i = 0; i < count; ++i) {
    const hq_encode_item& it = items[i];
    if (it.rows == 0 || it.cols == 0) continue;
    if (!on_device(it.x) || !on_device(it.scale) || !on_device(it.idx) || !on_device(it.rice_k) ||
        !on_device(it.tile_bits) || (coset_words(p) > 0 && !on_device(it.coset)))
      return HQ_EINVAL;
  }
  if (status != nullptr && !on_device(status)) return HQ_EINVAL;
  return HQ_OK;
}

EncodeLaunch encode_launch(const hq_params* p, int32_t x_dtype, uint32_t* status) {
  EncodeLaunch a;
  memset(&a, 0, sizeof(a));
  a.in_bf16 = x_dtype == HQ_BF16;
  a.lattice = p->lattice;
  a.tile = p->tile;
  a.auto_scale = (p->flags & HQ_SCALE_AUTO) != 0;
  a.status = status;
  make_signs(p->rht_seed, p->tile, a.signs);
  a.c = scale_constant(p);
  a.sqrt_n = sqrt((double)p->tile);
  set_rate_control(p, a);
  return a;
}

// the fast E8 encoder (with or without the per-tile rate control)
bool encode_batch_fast(const EncodeLaunch& a) { return e8_fast_encode_ok(a); }

// Launch groups of the fast encoder: up to kMaxItems non-empty matrices each.
// Calls emit(batch) per group; returns false when a launch fails.
template <typename F>
bool encode_groups(const hq_params* p, int32_t count, const hq_encode_item* items, F emit) {
  EncBatch b;
  memset(&b, 0, sizeof(b));
  for (int32_t i = 0; i <= count; ++i) {
    const bool flush = (i == count) || b.n == kMaxItems;
    if (flush && b.n > 0) {
      for (int k = b.n; k < kMaxItems; ++k) b.it[k] = b.it[0];
      if (!emit(b)) return false;
      memset(&b, 0, sizeof(b));
    }
    if (i == count) break;
    const hq_encode_item& it = items[i];
    const int64_t nt = it.rows * it.cols / p->tile;
    if (nt == 0) continue;
    b.it[b.n] = EncItem{it.x, it.idx, it.scale, it.coset, it.rice_k, it.tile_bits, nt, b.n_groups};
    b.n_groups += (nt + 15) / 16;
    b.n += 1;
  }
  return true;
}

hq_status enqueue_encode_batch(const hq_params* p, EncodeLaunch a, int32_t count,
                               const hq_encode_item* items, hipStream_t stream) {
  if (encode_batch_fast(a)) {
    const bool ok = encode_groups(p, count, items, [&](const EncBatch& b) {
      return launch_encode_e8_fast(a, b, stream) == hipSuccess;
    });
    return ok ? HQ_OK : HQ_EDEVICE;
  }
  for (int32_t i = 0; i < count; ++i) {
    const hq_encode_item& it = items[i];
    const int64_t nt = it.rows * it.cols / p->tile;
    if (nt == 0) continue;
    a.x = it.x;
    a.n_tiles = nt;
    a.scale = it.scale;
    a.idx = it.idx;
    a.coset = it.coset;
    a.rice_k = it.rice_k;
    a.tile_bits = it.tile_bits;
    a.coords = nullptr;
    if (launch_encode(a, stream) != hipSuccess) return HQ_EDEVICE;
  }
  return HQ_OK;
}

hq_status check_decode_batch(const hq_params* p, int32_t y_dtype, int32_t count,
                             const hq_decode_item* items, uint32_t* status) {
  hq_status st = check_params(p);
  if (st != HQ_OK) return st;
  if (p->flags & (HQ_WANT_COORDS | HQ_DITHER | HQ_IDX16)) return HQ_EUNSUPPORTED;
  if (y_dtype != HQ_F32 && y_dtype != HQ_BF16) return HQ_EINVAL;
  if (count < 0 || (count > 0 && items == nullptr)) return HQ_EINVAL;
  for (int32_t i = 0; i < count; ++i) {
    const hq_decode_item& it = items[i];
    if (it.rows < 0 || it.cols < 0 || it.cols % p->tile != 0) return HQ_EINVAL;
    if (it.rows == 0 || it.cols == 0) continue;
    if (it.idx == nullptr || it.scale == nullptr || it.y == nullptr) return HQ_EINVAL;
    if (coset_words(p) > 0 && it.coset == nullptr) return HQ_EINVAL;
    if (!aligned16(it.idx) || !aligned16(it.y)) return HQ_EINVAL;
    if (it.rows > INT64_MAX / it.cols) return HQ_EINVAL;
  }
  for (int32_t i = 0; i < count; ++i) {
    const hq_decode_item& it = items[i];
    if (it.rows == 0 || it.cols == 0) continue;
    if (!on_device(it.idx) || !on_device(it.scale) || !on_device(it.y) ||
        (coset_words(p) > 0 && !on_device(it.coset)))
      return HQ_EINVAL;
  }
  if (status != nullptr && !on_device(status)) return HQ_EINVAL;
  return HQ_OK;
}

DecodeLaunch decode_launch(const hq_params* p, int32_t y_dtype, uint32_t* status) {
  DecodeLaunch a;
  memset(&a, 0, sizeof(a));
  a.lattice = p->lattice;
  a.tile = p->tile;
  a.out_bf16 = y_dtype == HQ_BF16;
  a.status = status;
  make_signs(p->rht_seed, p->tile, a.signs);
  a.inv_sqrt_n = 1.0 / sqrt((double)p->tile);
  return a;
}

template <typename F>
bool decode_groups(const hq_params* p, int32_t count, const hq_decode_item* items, F emit) {
  DecBatch b;
  memset(&b, 0, sizeof(b));
  for (int32_t i = 0; i <= count; ++i) {
    const bool flush = (i == count) || b.n == kMaxItems;
    if (flush && b.n > 0) {
      for (int k = b.n; k < kMaxItems; ++k) b.it[k] = b.it[0];
      if (!emit(b)) return false;
      memset(&b, 0, sizeof(b));
    }
    if (i == count) break;
    const hq_decode_item& it = items[i];
    const int64_t nt = it.rows * it.cols / p->tile;
    if (nt == 0) continue;
    b.it[b.n] = DecItem{it.idx, it.coset, it.scale, it.y, nt, b.n_groups};
    b.n_groups += (nt + 15) / 16;
    b.n += 1;
  }
  return true;
}

hq_status enqueue_decode_batch(const hq_params* p, DecodeLaunch a, int32_t count,
                               const hq_decode_item* items, hipStream_t stream) {
  if (e8_fast_decode_ok(a)) {
    const bool ok = decode_groups(p, count, items, [&](const DecBatch& b) {
      return launch_decode_e8_fast(a, b, stream) == hipSuccess;
    });
    return ok ? HQ_OK : HQ_EDEVICE;
  }
  for (int32_t i = 0; i < count; ++i) {
    const hq_decode_item& it = items[i];
    const int64_t nt = it.rows * it.cols / p->tile;
    if (nt == 0) continue;
    a.idx = it.idx;
    a.coset = it.coset;
    a.scale = it.scale;
    a.n_tiles = nt;
    a.y = it.y;
    if (launch_decode(a, stream) != hipSuccess) return HQ_EDEVICE;
  }
  return HQ_OK;
}

// Non-empty items of a batch (launch groups hold up to kMaxItems).
template <typename I>
int32_t live_items(const hq_params* p, int32_t count, const I* items) {
  int32_t n = 0;
  for (int32_t i = 0; i < count; ++i)
    if (items[i].rows * items[i].cols / p->tile > 0) ++n;
  return n;
}

struct Span {
  uintptr_t lo, hi;   // [lo, hi)
};

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

Span span(const void* ptr, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
  return Span{lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

}  // namespace
}  // extern "C++"

hq_status hq_encode_batch(const hq_params* p, int32_t x_dtype, int32_t count,
                          const hq_encode_item* items, uint32_t* status, hipStream_t stream) {
  hq_status st = check_encode_batch(p, x_dtype, count, items, status);
  if (st != HQ_OK) return st;
  return enqueue_encode_batch(p, encode_launch(p, x_dtype, status), count, items, stream);
}

hq_status hq_decode_batch(const hq_params* p, int32_t y_dtype, int32_t count,
                          const hq_decode_item* items, uint32_t* status, hipStream_t stream) {
  hq_status st = check_decode_batch(p, y_dtype, count, items, status);
  if (st != HQ_OK) return st;
  return enqueue_decode_batch(p, decode_launch(p, y_dtype, status), count, items, stream);
}

hq_status hq_encode_decode_batch(const hq_params* enc_p, int32_t x_dtype, int32_t enc_count,
                                 const hq_encode_item* enc_items, const hq_params* dec_p,
                                 int32_t y_dtype, int32_t dec_count,
                                 const hq_decode_item* dec_items, uint32_t* status,
                                 hipStream_t stream) {
  hq_status st = check_encode_batch(enc_p, x_dtype, enc_count, enc_items, status);
  if (st != HQ_OK) return st;
  st = check_decode_batch(dec_p, y_dtype, dec_count, dec_items, status);
  if (st != HQ_OK) return st;
  // the two batches must be independent: no buffer the encode writes may be
  // read or written by the decode, and the decode's outputs may not overlap
  // the encode's inputs
  for (int32_t i = 0; i < enc_count; ++i) {
    const hq_encode_item& e = enc_items[i];
    const int64_t ne = e.rows * e.cols;
    if (ne == 0) continue;
    const int64_t te = ne / enc_p->tile;
    const int xb = x_dtype == HQ_BF16 ? 2 : 4;
    const Span ew[5] = {span(e.idx, ne), span(e.scale, 4 * te),
                        span(e.coset, 4 * te * coset_words(enc_p)), span(e.rice_k, te),
                        span(e.tile_bits, 4 * te)};
    const Span ex = span(e.x, ne * xb);
    for (int32_t j = 0; j < dec_count; ++j) {
      const hq_decode_item& d = dec_items[j];
      const int64_t nd = d.rows * d.cols;
      if (nd == 0) continue;
      const int64_t td = nd / dec_p->tile;
      const Span dr[4] = {span(d.idx, nd), span(d.scale, 4 * td),
                          span(d.coset, 4 * td * coset_words(dec_p)),
                          span(d.y, nd * (y_dtype == HQ_BF16 ? 2 : 4))};
      for (const Span& w : ew)
        for (const Span& r : dr)
          if (overlap(w, r)) return HQ_EINVAL;
      if (overlap(ex, dr[3])) return HQ_EINVAL;
    }
  }
  const EncodeLaunch a = encode_launch(enc_p, x_dtype, status);
  const DecodeLaunch ad = decode_launch(dec_p, y_dtype, status);
  const int32_t le = live_items(enc_p, enc_count, enc_items);
  const int32_t ld = live_items(dec_p, dec_count, dec_items);
  // (the fused kernel encodes without rate control)
  if (!a.rate_control && a.tile == 256 && ad.tile == 256 && encode_batch_fast(a) &&
      e8_fast_decode_ok(ad) && le <= kMaxItems &&
      ld <= kMaxItems && le + ld > 0) {
    EncBatch b;
    DecBatch bd;
    memset(&b, 0, sizeof(b));
    memset(&bd, 0, sizeof(bd));
    encode_groups(enc_p, enc_count, enc_items, [&](const EncBatch& g) { b = g; return true; });
    decode_groups(dec_p, dec_count, dec_items, [&](const DecBatch& g) { bd = g; return true; });
    return launch_codec_e8_fast(a, b, ad, bd, stream) == hipSuccess ? HQ_OK : HQ_EDEVICE;
  }
  st = enqueue_encode_batch(enc_p, a, enc_count, enc_items, stream);
  if (st != HQ_OK) return st;
  return enqueue_decode_batch(dec_p, ad, dec_count, dec_items, stream);
}

size_t hq_rate_workspace_bytes(int64_t n_tiles) {
  if (n_tiles <= 0) return 0;
  // word and bit sums of each rate block, word sums of each rate wave
  return 6 * (size_t)rate_workspace_blocks(n_tiles) * sizeof(uint64_t);
}

// hq_rate's checks and launch; scratch_ws: the workspace is the library's
// static scratch (known device memory, not checked by pointer attributes);
// check_only: return after the checks, launching nothing.
static hq_status rate_impl(const hq_params* p, const int8_t* idx, const uint32_t* coset,
                           int64_t n_tiles, uint8_t* rice_k, uint32_t* tile_bits,
                           uint64_t* total_bits, uint32_t* stream_words, uint64_t capacity_words,
                           uint64_t* tile_word_offset, void* workspace, size_t workspace_bytes,
                           uint32_t* status, hipStream_t stream, bool scratch_ws,
                           bool check_only = false) {
  hq_status st = check_params(p);
  if (st != HQ_OK) return st;
  if (n_tiles < 0) return HQ_EINVAL;
  if (n_tiles == 0) return HQ_OK;   // zero tiles: a no-op (nothing is written)
  const bool given = (p->flags & HQ_RATE_GIVEN) != 0;
  const bool pack = stream_words != nullptr;
  if ((idx == nullptr && (pack || !given)) || rice_k == nullptr || tile_bits == nullptr ||
      total_bits == nullptr)
    return HQ_EINVAL;
  if (!aligned16(idx) || ((uintptr_t)total_bits & 7u) || ((uintptr_t)tile_bits & 3u))
    return HQ_EINVAL;
  if (pack) {
    if (tile_word_offset == nullptr || workspace == nullptr) return HQ_EINVAL;
    if (coset_words(p) > 0 && coset == nullptr) return HQ_EINVAL;
    if (workspace_bytes < hq_rate_workspace_bytes(n_tiles)) return HQ_EINVAL;
    if (((uintptr_t)workspace & 7u) || ((uintptr_t)tile_word_offset & 7u)) return HQ_EINVAL;
  }
  if (n_tiles > INT64_MAX / p->tile) return HQ_EINVAL;
  if (n_tiles == 0) return HQ_OK;
  if ((idx != nullptr && !on_device(idx)) || !on_device(rice_k) || !on_device(tile_bits) ||
      !on_device(total_bits) || (status != nullptr && !on_device(status)))
    return HQ_EINVAL;
  if (pack && (!on_device(stream_words) || !on_device(tile_word_offset) ||
               (!scratch_ws && !on_device(workspace)) ||
               (coset_words(p) > 0 && !on_device(coset))))
    return HQ_EINVAL;
  if (!pack && workspace != nullptr && !scratch_ws && !on_device(workspace)) return HQ_EINVAL;
  if (check_only) return HQ_OK;
  RateLaunch a;
  memset(&a, 0, sizeof(a));
  a.idx = idx;
  a.coset = coset;
  a.n_tiles = n_tiles;
  a.tile = p->tile;
  a.coset_bits = coset_bits(p);
  a.coset_words = coset_words(p);
  a.rice_k = rice_k;
  a.tile_bits = tile_bits;
  a.total_bits = total_bits;
  a.stream = pack ? stream_words : nullptr;
  a.capacity = capacity_words;
  a.tile_word_offset = tile_word_offset;
  // with a workspace the block sums go there (no atomics); packing needs one
  const bool ws = workspace != nullptr && workspace_bytes >= hq_rate_workspace_bytes(n_tiles) &&
                  ((uintptr_t)workspace & 7u) == 0;
  a.block_words = ws ? static_cast<uint64_t*>(workspace) : nullptr;
  const int64_t nb = rate_workspace_blocks(n_tiles);
  a.block_bits = ws ? static_cast<uint64_t*>(workspace) + nb : nullptr;
  a.wave_words = ws ? static_cast<uint64_t*>(workspace) + 2 * nb : nullptr;
  a.status = status;
  a.given = given ? 1 : 0;
  a.wide = idx16(p) ? 1 : 0;
  return launched(launch_rate(a, stream));
}

hq_status hq_rate(const hq_params* p, const int8_t* idx, const uint32_t* coset, int64_t n_tiles,
                  uint8_t* rice_k, uint32_t* tile_bits, uint64_t* total_bits,
                  uint32_t* stream_words, uint64_t capacity_words, uint64_t* tile_word_offset,
                  void* workspace, size_t workspace_bytes, uint32_t* status,
                  hipStream_t stream) {
  return rate_impl(p, idx, coset, n_tiles, rice_k, tile_bits, total_bits, stream_words,
                   capacity_words, tile_word_offset, workspace, workspace_bytes, status, stream,
                   false);
}

hq_status hq_rate_noalloc(const hq_params* p, const int8_t* idx, const uint32_t* coset,
                          int64_t n_tiles, uint8_t* rice_k, uint32_t* tile_bits,
                          uint64_t* total_bits, uint32_t* stream_words, uint64_t capacity_words,
                          uint64_t* tile_word_offset, uint32_t* status, hipStream_t stream) {
  // the workspace of any tile count fits the scratch; a size past it (none
  // exists while the rate pass is capped at 8192 waves) is refused
  if (n_tiles > 0 && hq_rate_workspace_bytes(n_tiles) > sizeof(scratch)) return HQ_ERANGE;
  // hq_rate's argument checks first, with the scratch standing in for the
  // workspace (a placeholder address: nothing is read in the checks)
  hq_status st = rate_impl(p, idx, coset, n_tiles, rice_k, tile_bits, total_bits, stream_words,
                           capacity_words, tile_word_offset, reinterpret_cast<void*>(256),
                           sizeof(scratch), status, stream, true, true);
  if (st != HQ_OK || n_tiles == 0) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != HQ_OK) return st;
  return rate_impl(p, idx, coset, n_tiles, rice_k, tile_bits, total_bits, stream_words,
                   capacity_words, tile_word_offset, ws, sizeof(scratch), status, stream, true);
}

// Validation of one hq_rate_batch item with n_tiles > 0 (a workspace is
// given to the call).
static hq_status check_rate_item(const hq_params* p, const hq_rate_item& it) {
  const bool given = (p->flags & HQ_RATE_GIVEN) != 0;
  const bool pack = it.stream_words != nullptr;
  if ((it.idx == nullptr && (pack || !given)) || it.rice_k == nullptr ||
      it.tile_bits == nullptr || it.total_bits == nullptr)
    return HQ_EINVAL;
  if (!aligned16(it.idx) || ((uintptr_t)it.total_bits & 7u) || ((uintptr_t)it.tile_bits & 3u))
    return HQ_EINVAL;
  if (pack) {
    if (it.tile_word_offset == nullptr || ((uintptr_t)it.tile_word_offset & 7u)) return HQ_EINVAL;
    if (coset_words(p) > 0 && it.coset == nullptr) return HQ_EINVAL;
  }
  if (it.n_tiles > INT64_MAX / p->tile) return HQ_EINVAL;
  if ((it.idx != nullptr && !on_device(it.idx)) || !on_device(it.rice_k) ||
      !on_device(it.tile_bits) || !on_device(it.total_bits))
    return HQ_EINVAL;
  if (pack && (!on_device(it.stream_words) || !on_device(it.tile_word_offset) ||
               (coset_words(p) > 0 && !on_device(it.coset))))
    return HQ_EINVAL;
  return HQ_OK;
}

size_t hq_rate_batch_workspace_bytes(int32_t count, const hq_rate_item* items) {
  if (count < 0 || (count > 0 && items == nullptr)) return 0;
  size_t total = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (items[i].n_tiles < 0) return 0;
    total += hq_rate_workspace_bytes(items[i].n_tiles);
  }
  return total;
}

hq_status hq_rate_batch(const hq_params* p, int32_t count, const hq_rate_item* items,
                        void* workspace, size_t workspace_bytes, uint32_t* status,
                        hipStream_t stream) {
  hq_status st = check_params(p);
  if (st != HQ_OK) return st;
  if (count < 0 || (count > 0 && items == nullptr)) return HQ_EINVAL;
  bool any = false;
  for (int32_t i = 0; i < count; ++i) {
    if (items[i].n_tiles < 0) return HQ_EINVAL;
    if (items[i].n_tiles == 0) continue;
    st = check_rate_item(p, items[i]);
    if (st != HQ_OK) return st;
    any = true;
  }
  if (!any) return HQ_OK;
  if (workspace == nullptr || ((uintptr_t)workspace & 7u) ||
      workspace_bytes < hq_rate_batch_workspace_bytes(count, items) || !on_device(workspace) ||
      (status != nullptr && !on_device(status)))
    return HQ_EINVAL;
  // groups of up to kRateMaxItems matrices, each with its own workspace slice
  RateBatch b;
  memset(&b, 0, sizeof(b));
  char* ws = static_cast<char*>(workspace);
  for (int32_t i = 0; i <= count; ++i) {
    if ((i == count || b.n == kRateMaxItems) && b.n > 0) {
      for (int k = b.n; k < kRateMaxItems; ++k) b.it[k] = b.it[0];
      for (int k = b.n + 1; k <= kRateMaxItems; ++k) b.block0[k] = b.block0[b.n];
      if (launch_rate_batch(b, stream) != hipSuccess) return HQ_EDEVICE;
      memset(&b, 0, sizeof(b));
    }
    if (i == count) break;
    const hq_rate_item& it = items[i];
    if (it.n_tiles == 0) {
      ws += hq_rate_workspace_bytes(0);
      continue;
    }
    RateLaunch& a = b.it[b.n];
    a.idx = it.idx;
    a.coset = it.coset;
    a.n_tiles = it.n_tiles;
    a.tile = p->tile;
    a.coset_bits = coset_bits(p);
    a.coset_words = coset_words(p);
    a.rice_k = it.rice_k;
    a.tile_bits = it.tile_bits;
    a.total_bits = it.total_bits;
    a.stream = it.stream_words;
    a.capacity = it.capacity_words;
    a.tile_word_offset = it.tile_word_offset;
    const int64_t nb = rate_workspace_blocks(it.n_tiles);
    a.block_words = reinterpret_cast<uint64_t*>(ws);
    a.block_bits = a.block_words + nb;
    a.wave_words = a.block_words + 2 * nb;
    ws += hq_rate_workspace_bytes(it.n_tiles);
    a.status = status;
    a.given = (p->flags & HQ_RATE_GIVEN) ? 1 : 0;
    a.wide = idx16(p) ? 1 : 0;
    b.block0[b.n + 1] = b.block0[b.n] + rate_blocks(p->tile, it.n_tiles);
    ++b.n;
  }
  return HQ_OK;
}

namespace {

// Validation of one packed matrix (n_tiles > 0).
hq_status check_unpack(const hq_params* p, const hq_unpack_item& it) {
  if (it.stream_words == nullptr || it.tile_word_offset == nullptr || it.idx == nullptr)
    return HQ_EINVAL;
  if (coset_words(p) > 0 && it.coset == nullptr) return HQ_EINVAL;
  if (!aligned16(it.idx) || ((uintptr_t)it.tile_word_offset & 7u) ||
      ((uintptr_t)it.stream_words & 3u) || ((uintptr_t)it.coset & 3u))
    return HQ_EINVAL;
  if (it.n_tiles > INT64_MAX / p->tile) return HQ_EINVAL;
  if (!on_device(it.stream_words) || !on_device(it.tile_word_offset) || !on_device(it.idx) ||
      (coset_words(p) > 0 && !on_device(it.coset)) ||
      (it.rice_k != nullptr && !on_device(it.rice_k)))
    return HQ_EINVAL;
  return HQ_OK;
}

}  // namespace

hq_status hq_unpack_batch(const hq_params* p, int32_t count, const hq_unpack_item* items,
                          uint32_t* status, hipStream_t stream) {
  hq_status st = check_params(p);
  if (st != HQ_OK) return st;
  if (count < 0 || (count > 0 && items == nullptr)) return HQ_EINVAL;
  for (int32_t i = 0; i < count; ++i) {
    if (items[i].n_tiles < 0) return HQ_EINVAL;
    if (items[i].n_tiles == 0) continue;   // skipped: nothing is read or written
    st = check_unpack(p, items[i]);
    if (st != HQ_OK) return st;
  }
  if (status != nullptr && !on_device(status)) return HQ_EINVAL;
  // launches of up to kUnpackMaxItems matrices, waves numbered across them
  UnpackLaunch a;
  memset(&a, 0, sizeof(a));
  a.tile = p->tile;
  a.coset_bits = coset_bits(p);
  a.coset_words = coset_words(p);
  a.status = status;
  a.wide = idx16(p) ? 1 : 0;
  for (int32_t i = 0; i <= count; ++i) {
    if ((i == count || a.n == kUnpackMaxItems) && a.n > 0) {
      if (launch_unpack(a, stream) != hipSuccess) return HQ_EDEVICE;
      a.n = 0;
      a.n_waves = 0;
    }
    if (i == count) break;
    const hq_unpack_item& it = items[i];
    if (it.n_tiles == 0) continue;
    UnpackItem& u = a.it[a.n++];
    u.stream = it.stream_words;
    u.tile_word_offset = it.tile_word_offset;
    u.n_tiles = it.n_tiles;
    u.idx = it.idx;
    u.coset = a.coset_words > 0 ? it.coset : nullptr;
    u.rice_k = it.rice_k;
    u.wave0 = a.n_waves;
    a.n_waves += (it.n_tiles + 63) / 64;
  }
  return HQ_OK;
}

hq_status hq_unpack(const hq_params* p, const uint32_t* stream_words,
                    const uint64_t* tile_word_offset, int64_t n_tiles, int8_t* idx,
                    uint32_t* coset, uint8_t* rice_k, uint32_t* status, hipStream_t stream) {
  hq_status st = check_params(p);
  if (st != HQ_OK) return st;
  if (n_tiles < 0) return HQ_EINVAL;
  if (n_tiles == 0) return HQ_OK;   // zero tiles: a no-op (nothing is read or written)
  const hq_unpack_item it{stream_words, tile_word_offset, n_tiles, idx, coset, rice_k};
  return hq_unpack_batch(p, 1, &it, status, stream);
}

size_t hq_gemv_workspace_bytes(int64_t rows, int64_t cols, int32_t m) {
  if (rows <= 0 || cols <= 0 || m <= 0 || m > 8 || cols % 256 != 0 || cols > kGemvMaxCols)
    return 0;
  return gemv_workspace(rows, cols, m);
}

namespace {

// Argument checks of one hq_gemv matrix (device residency checked apart).
hq_status check_gemv(const int8_t* idx, const uint32_t* coset, const float* scale, int64_t rows,
                     int64_t cols, const float* x, const float* y) {
  if (rows < 0 || cols < 0 || cols % 256 != 0 || cols > kGemvMaxCols) return HQ_EINVAL;
  if (rows == 0 || cols == 0) return HQ_OK;   // nothing to compute
  if (idx == nullptr || coset == nullptr || scale == nullptr || x == nullptr || y == nullptr)
    return HQ_EINVAL;
  if (rows > INT64_MAX / cols) return HQ_EINVAL;
  if (!aligned16(idx) || !aligned16(x) || ((uintptr_t)y & 3u) || ((uintptr_t)coset & 3u) ||
      ((uintptr_t)scale & 3u))
    return HQ_EINVAL;
  return HQ_OK;
}

bool gemv_on_device(const hq_gemv_item& it) {
  return on_device(it.idx) && on_device(it.coset) && on_device(it.scale) && on_device(it.x) &&
         on_device(it.y);
}

}  // namespace

// Sizes hq_gemm accepts (m checked separately).
static bool gemm_sizes_ok(int64_t rows, int64_t cols, int32_t m) {
  return rows >= 0 && cols >= 0 && cols % 256 == 0 && rows <= kGemmMaxRows &&
         cols <= kGemmMaxCols && m * cols <= kGemmMaxProduct && m * rows <= kGemmMaxProduct;
}

extern "C++" {
// The launch groups of a batch (up to kGemmMaxItems non-empty matrices
// each, in item order): fn(group) for each, planned.
template <typename F>
static void gemm_groups(int32_t count, const hq_gemv_item* items, int32_t m, F fn) {
  GemmBatch b;
  memset(&b, 0, sizeof(b));
  b.m = m;
  for (int32_t i = 0; i <= count; ++i) {
    if ((i == count || b.n == kGemmMaxItems) && b.n > 0) {
      gemm_plan(b);
      fn(b);
      b.n = 0;
    }
    if (i == count) break;
    const hq_gemv_item& it = items[i];
    if (it.rows == 0 || it.cols == 0) continue;
    GemmItem& g = b.it[b.n++];
    memset(&g, 0, sizeof(g));
    g.idx = it.idx;
    g.coset = it.coset;
    g.scale = it.scale;
    g.rows = it.rows;
    g.cols = it.cols;
    g.x = it.x;
    g.y = it.y;
  }
}

static size_t gemm_group_workspace(const GemmBatch& b) {
  size_t total = 0;
  for (int k = 0; k < b.n; ++k) total += gemm_item_workspace(b.it[k], b.m);
  return total;
}
}  // extern "C++"

size_t hq_gemm_batch_workspace_bytes(int32_t count, const hq_gemv_item* items, int32_t m) {
  if (count < 0 || (count > 0 && items == nullptr) || m < 1 || m > kGemmMaxVecs) return 0;
  for (int32_t i = 0; i < count; ++i)
    if (!gemm_sizes_ok(items[i].rows, items[i].cols, m)) return 0;
  size_t total = 0;
  bool fits = true;
  gemm_groups(count, items, m, [&](const GemmBatch& b) {
    total += gemm_group_workspace(b);
    fits = fits && gemm_fits_launch(b);
  });
  return fits ? total : 0;
}

size_t hq_gemm_workspace_bytes(int64_t rows, int64_t cols, int32_t m) {
  if (rows <= 0 || cols <= 0) return 0;
  hq_gemv_item it;
  memset(&it, 0, sizeof(it));
  it.rows = rows;
  it.cols = cols;
  return hq_gemm_batch_workspace_bytes(1, &it, m);
}

hq_status hq_gemm_batch(const hq_params* p, int32_t count, const hq_gemv_item* items, int32_t m,
                        void* workspace, size_t workspace_bytes, uint32_t* status,
                        hipStream_t stream) {
  (void)status;
  hq_status st = check_params(p);
  if (st != HQ_OK) return st;
  if (p->lattice != HQ_E8 || p->tile != 256 || (p->flags & (HQ_DITHER | HQ_IDX16)))
    return HQ_EUNSUPPORTED;
  if (count < 0 || (count > 0 && items == nullptr) || m < 1 || m > kGemmMaxVecs)
    return HQ_EINVAL;
  bool any = false;
  for (int32_t i = 0; i < count; ++i) {
    const hq_gemv_item& it = items[i];
    if (!gemm_sizes_ok(it.rows, it.cols, m)) return HQ_EINVAL;
    if (it.rows == 0 || it.cols == 0) continue;
    if (it.idx == nullptr || it.coset == nullptr || it.scale == nullptr || it.x == nullptr ||
        it.y == nullptr)
      return HQ_EINVAL;
    if (!aligned16(it.idx) || !aligned16(it.x) || ((uintptr_t)it.y & 3u) ||
        ((uintptr_t)it.coset & 3u) || ((uintptr_t)it.scale & 3u))
      return HQ_EINVAL;
    any = true;
  }
  if (!any) return HQ_OK;
  const size_t need = hq_gemm_batch_workspace_bytes(count, items, m);   // 0: too large a launch
  if (need == 0 || workspace == nullptr || !aligned16(workspace) || workspace_bytes < need)
    return HQ_EINVAL;
  for (int32_t i = 0; i < count; ++i) {
    const hq_gemv_item& it = items[i];
    if (it.rows == 0 || it.cols == 0) continue;
    if (!on_device(it.idx) || !on_device(it.coset) || !on_device(it.scale) || !on_device(it.x) ||
        !on_device(it.y))
      return HQ_EINVAL;
  }
  if (!on_device(workspace)) return HQ_EINVAL;
  // launches of up to kGemmMaxItems matrices, each group with its own
  // workspace slice in item order
  uint32_t signs[8];
  make_signs(p->rht_seed, p->tile, signs);
  char* ws = static_cast<char*>(workspace);
  bool ok = true;
  gemm_groups(count, items, m, [&](const GemmBatch& planned) {
    if (!ok) return;
    GemmBatch b = planned;
    memcpy(b.signs, signs, sizeof(signs));
    const size_t bytes = gemm_group_workspace(b);
    gemm_layout(b, ws);
    ws += bytes;
    ok = launch_gemm(b, stream) == hipSuccess;
  });
  return ok ? HQ_OK : HQ_EDEVICE;
}

hq_status hq_gemm(const hq_params* p, const int8_t* idx, const uint32_t* coset, const float* scale,
                  int64_t rows, int64_t cols, const float* x, int32_t m, float* y,
                  void* workspace, size_t workspace_bytes, uint32_t* status, hipStream_t stream) {
  hq_gemv_item it;
  it.idx = idx;
  it.coset = coset;
  it.scale = scale;
  it.rows = rows;
  it.cols = cols;
  it.x = x;
  it.y = y;
  return hq_gemm_batch(p, 1, &it, m, workspace, workspace_bytes, status, stream);
}

size_t hq_gemv_batch_workspace_bytes(int32_t count, const hq_gemv_item* items, int32_t m) {
  if (count < 0 || (count > 0 && items == nullptr) || m < 1 || m > 8) return 0;
  size_t total = 0;
  for (int32_t i = 0; i < count; ++i) {
    const hq_gemv_item& it = items[i];
    if (it.rows < 0 || it.cols < 0 || it.cols % 256 != 0 || it.cols > kGemvMaxCols) return 0;
    if (it.rows > 0 && it.cols > 0) total += gemv_workspace(it.rows, it.cols, m);
  }
  return total;
}

hq_status hq_gemv_batch(const hq_params* p, int32_t count, const hq_gemv_item* items, int32_t m,
                        void* workspace, size_t workspace_bytes, uint32_t* status,
                        hipStream_t stream) {
  (void)status;
  hq_status st = check_params(p);
  if (st != HQ_OK) return st;
  if (p->lattice != HQ_E8 || p->tile != 256 || (p->flags & (HQ_DITHER | HQ_IDX16)))
    return HQ_EUNSUPPORTED;
  if (count < 0 || (count > 0 && items == nullptr) || m < 1 || m > 8) return HQ_EINVAL;
  bool any = false;
  for (int32_t i = 0; i < count; ++i) {
    const hq_gemv_item& it = items[i];
    st = check_gemv(it.idx, it.coset, it.scale, it.rows, it.cols, it.x, it.y);
    if (st != HQ_OK) return st;
    any = any || (it.rows > 0 && it.cols > 0);
  }
  if (!any) return HQ_OK;
  if (workspace == nullptr || !aligned16(workspace) ||
      workspace_bytes < hq_gemv_batch_workspace_bytes(count, items, m))
    return HQ_EINVAL;
  for (int32_t i = 0; i < count; ++i)
    if (items[i].rows > 0 && items[i].cols > 0 && !gemv_on_device(items[i])) return HQ_EINVAL;
  if (!on_device(workspace)) return HQ_EINVAL;
  // launches of up to kGemvMaxItems matrices, each with its own workspace
  // slice in item order
  GemvBatch b;
  memset(&b, 0, sizeof(b));
  b.m = m;
  make_signs(p->rht_seed, p->tile, b.signs);
  char* ws = static_cast<char*>(workspace);
  for (int32_t i = 0; i <= count; ++i) {
    if ((i == count || b.n == kGemvMaxItems) && b.n > 0) {
      char* base = ws;
      for (int k = 0; k < b.n; ++k) ws += gemv_workspace(b.it[k].rows, b.it[k].cols, m);
      gemv_layout(b, base);
      if (launch_gemv(b, stream) != hipSuccess) return HQ_EDEVICE;
      b.n = 0;
    }
    if (i == count) break;
    const hq_gemv_item& it = items[i];
    if (it.rows == 0 || it.cols == 0) continue;
    GemvItem& g = b.it[b.n++];
    memset(&g, 0, sizeof(g));
    g.idx = it.idx;
    g.coset = it.coset;
    g.scale = it.scale;
    g.rows = it.rows;
    g.cols = it.cols;
    g.x = it.x;
    g.y = it.y;
  }
  return HQ_OK;
}

hq_status hq_gemv(const hq_params* p, const int8_t* idx, const uint32_t* coset,
                  const float* scale, int64_t rows, int64_t cols, const float* x, int32_t m,
                  float* y, void* workspace, size_t workspace_bytes, uint32_t* status,
                  hipStream_t stream) {
  const hq_gemv_item it{idx, coset, scale, rows, cols, x, y};
  return hq_gemv_batch(p, 1, &it, m, workspace, workspace_bytes, status, stream);
}

size_t hq_kv_scores_workspace_bytes(int64_t n_q) {
  if (n_q <= 0) return 0;
  return (size_t)n_q * 128u * sizeof(float);
}

hq_status hq_kv_scores(const hq_params* p, const float* q, int64_t n_q, const int8_t* idx,
                       const uint32_t* coset, const float* scale, int64_t n_keys, float* scores,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  hq_status st = check_params(p);
  if (st != HQ_OK) return st;
  if (p->lattice != HQ_E8 || p->tile != 128 || idx16(p)) return HQ_EUNSUPPORTED;
  if (n_q < 0 || n_keys < 0) return HQ_EINVAL;
  if (n_q == 0 || n_keys == 0) return HQ_OK;   // nothing to compute
  if (q == nullptr || idx == nullptr || coset == nullptr || scale == nullptr ||
      scores == nullptr || workspace == nullptr)
    return HQ_EINVAL;
  // grids below 2^32 work-items: n_q blocks of 128, n_keys / 256 blocks of 256
  if (n_q >= ((int64_t)1 << 25) || n_keys > ((int64_t)1 << 32) - 256 ||
      n_keys > INT64_MAX / n_q || workspace_bytes < hq_kv_scores_workspace_bytes(n_q))
    return HQ_EINVAL;
  if ((p->flags & HQ_DITHER) && p->dither_base + n_keys > ((int64_t)1 << 32)) return HQ_EINVAL;
  if (!aligned16(q) || !aligned16(idx) || !aligned16(workspace) || ((uintptr_t)coset & 3u) ||
      ((uintptr_t)scale & 3u) || ((uintptr_t)scores & 3u))
    return HQ_EINVAL;
  if (!on_device(q) || !on_device(idx) || !on_device(coset) || !on_device(scale) ||
      !on_device(scores) || !on_device(workspace))
    return HQ_EINVAL;
  ScoreLaunch a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.n_q = n_q;
  a.idx = idx;
  a.coset = coset;
  a.scale = scale;
  a.n_keys = n_keys;
  a.scores = scores;
  a.qr = static_cast<float*>(workspace);
  make_signs(p->rht_seed, p->tile, a.signs);
  a.inv_sqrt_n = 1.0 / sqrt((double)p->tile);
  a.dither = (p->flags & HQ_DITHER) != 0;
  a.dither_seed = p->dither_seed;
  a.dither_base = p->dither_base;
  return launched(launch_scores(a, stream));
}

// Sizes hq_kv_attention takes: every grid below 2^32 work-items (rotation
// and merge: n_heads n_q blocks of 128; attention: ranges x query groups x
// heads blocks of 256).
static bool attn_sizes_ok(int64_t n_heads, int64_t n_q, int64_t n_keys) {
  if (n_heads < 1 || n_heads > 65535 || n_q < 0 || n_q > 65536 || n_keys < 0) return false;
  if (n_heads * n_keys > ((int64_t)1 << 32) || n_heads * n_q >= ((int64_t)1 << 25)) return false;
  if (n_q == 0 || n_keys == 0) return true;
  return attn_blocks(n_heads, n_q, n_keys) * 256 < ((int64_t)1 << 32);
}

size_t hq_kv_attention_workspace_bytes(int64_t n_heads, int64_t n_q, int64_t n_keys) {
  if (!attn_sizes_ok(n_heads, n_q, n_keys) || n_q == 0 || n_keys == 0) return 0;
  return attn_workspace(n_heads, n_q, n_keys);
}

// A K or V cache's parameters for hq_kv_attention.
static hq_status check_cache(const hq_params* p, int64_t n_keys) {
  hq_status st = check_params(p);
  if (st != HQ_OK) return st;
  if (p->lattice != HQ_E8 || p->tile != 128 || idx16(p)) return HQ_EUNSUPPORTED;
  if ((p->flags & HQ_DITHER) && p->dither_base + n_keys > ((int64_t)1 << 32)) return HQ_EINVAL;
  return HQ_OK;
}

hq_status hq_kv_attention(const hq_params* pk, const int8_t* k_idx, const uint32_t* k_coset,
                          const float* k_scale, const hq_params* pv, const int8_t* v_idx,
                          const uint32_t* v_coset, const float* v_scale, int64_t n_heads,
                          int64_t n_keys, const float* q, int64_t n_q, float tau, float* out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!attn_sizes_ok(n_heads, n_q, n_keys) || !isfinite(tau)) {
    if (check_params(pk) != HQ_OK) return check_params(pk);
    return HQ_EINVAL;
  }
  hq_status st = check_cache(pk, n_heads * n_keys);
  if (st != HQ_OK) return st;
  st = check_cache(pv, n_heads * n_keys);
  if (st != HQ_OK) return st;
  if (n_q == 0) return HQ_OK;
  if (n_keys == 0) return HQ_EINVAL;              // softmax over no keys
  if (k_idx == nullptr || k_coset == nullptr || k_scale == nullptr || v_idx == nullptr ||
      v_coset == nullptr || v_scale == nullptr || q == nullptr || out == nullptr ||
      workspace == nullptr)
    return HQ_EINVAL;
  if (workspace_bytes < attn_workspace(n_heads, n_q, n_keys)) return HQ_EINVAL;
  if (!aligned16(q) || !aligned16(k_idx) || !aligned16(v_idx) || !aligned16(workspace) ||
      ((uintptr_t)k_coset & 3u) || ((uintptr_t)k_scale & 3u) || ((uintptr_t)v_coset & 3u) ||
      ((uintptr_t)v_scale & 3u) || ((uintptr_t)out & 3u))
    return HQ_EINVAL;
  if (!on_device(q) || !on_device(k_idx) || !on_device(k_coset) || !on_device(k_scale) ||
      !on_device(v_idx) || !on_device(v_coset) || !on_device(v_scale) || !on_device(out) ||
      !on_device(workspace))
    return HQ_EINVAL;
  AttnLaunch a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.n_q = n_q;
  a.k_idx = k_idx;
  a.k_coset = k_coset;
  a.k_scale = k_scale;
  a.v_idx = v_idx;
  a.v_coset = v_coset;
  a.v_scale = v_scale;
  a.n_keys = n_keys;
  a.n_heads = n_heads;
  a.out = out;
  a.qr = static_cast<float*>(workspace);
  a.part = a.qr + (size_t)(n_heads * n_q) * 128;
  attn_plan(n_heads, n_q, n_keys, a.keys_per_wave, a.n_ranges);
  uint32_t sg[8];
  make_signs(pk->rht_seed, 128, sg);
  memcpy(a.k_signs, sg, sizeof(a.k_signs));
  make_signs(pv->rht_seed, 128, sg);
  memcpy(a.v_signs, sg, sizeof(a.v_signs));
  a.k_dither = (pk->flags & HQ_DITHER) != 0;
  a.v_dither = (pv->flags & HQ_DITHER) != 0;
  a.k_seed = pk->dither_seed;
  a.v_seed = pv->dither_seed;
  a.k_base = pk->dither_base;
  a.v_base = pv->dither_base;
  a.q_scale = (double)tau * 1.4426950408889634 / sqrt(128.0);   // tau log2(e) / sqrt(n)
  return launched(launch_attention(a, stream));
}

int32_t hq_coset_words(const hq_params* p) {
  if (check_params(p) != HQ_OK) return -1;
  return coset_words(p);
}

const char* hq_status_string(hq_status s) {
  switch (s) {
    case HQ_OK: return "ok";
    case HQ_EINVAL: return "invalid argument";
    case HQ_ERANGE: return "auto scale would overflow the indices (int8; int16 with HQ_IDX16)";
    case HQ_EDEVICE: return "HIP call or kernel launch failed";
    case HQ_EUNSUPPORTED: return "unsupported parameter combination";
    case HQ_EIO: return "checkpoint file cannot be opened, written or read";
    case HQ_EFORMAT: return "not a checkpoint file, or a damaged record";
    case HQ_ENOTFOUND: return "no checkpoint record of that name";
    default: return "unknown status";
  }
}

uint64_t hq_splitmix64(uint64_t key) { return splitmix64(key); }

hq_status hq_rht_signs(uint32_t seed, int32_t n, int8_t* out) {
  if (out == nullptr || n <= 0 || n > 256) return HQ_EINVAL;
  for (int j = 0; j < n; ++j)
    out[j] = (splitmix64(((uint64_t)seed << 32) ^ (uint64_t)j) >> 63) ? -1 : 1;
  return HQ_OK;
}

hq_status hq_scale_constant(const hq_params* p, double* out) {
  hq_status st = check_params(p);
  if (st != HQ_OK) return st;
  if (out == nullptr) return HQ_EINVAL;
  *out = scale_constant(p);
  return HQ_OK;
}

int32_t hq_version(void) { return 100; }

}  // extern "C"
