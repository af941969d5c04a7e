// Checkpoint files of packed matrices: the file form of the packed,
// Rice-coded lattice-index format.
//
// Passages: GitHub issue "HyperQuant ... #9", "Additional context" (a
// packed, Rice-coded lattice-index checkpoint format, to be read back);
// [arXiv abstract] item (iii) (the Rice-coded indices are the stored form).
//
// Layout (host byte order, little-endian on every supported host): the
// 8-byte file magic "HQCKPT" 0 1 (format version 1), then records.  A record
// is a 136-byte header -- magic "HQRE", header size, the hq_ckpt_entry
// fields, payload bytes, FNV-1a 64 of the payload -- and its payload:
// scale[n_tiles] fp32, zero padding to 8 bytes, tile_word_offset[n_tiles+1]
// uint64, words[n_words] uint32, zero padding to 8 bytes.  Appending writes
// one record at the end; readers scan the records from the start.
#include <stdio.h>
#include <string.h>
#include <sys/types.h>

#include <string>
#include <vector>

#include "hq.h"

namespace {

const unsigned char kFileMagic[8] = {'H', 'Q', 'C', 'K', 'P', 'T', 0, 1};
const unsigned char kRecMagic[4] = {'H', 'Q', 'R', 'E'};
constexpr uint32_t kRecHeaderBytes = 136;

struct RecHeader {
  unsigned char magic[4];
  uint32_t header_bytes;
  hq_ckpt_entry e;        // 112 bytes
  uint64_t payload_bytes;
  uint64_t checksum;
};
static_assert(sizeof(hq_ckpt_entry) == 112, "entry layout");
static_assert(sizeof(RecHeader) == kRecHeaderBytes, "record header layout");

uint64_t pad8(uint64_t n) { return (n + 7) / 8 * 8; }

uint64_t payload_bytes(const hq_ckpt_entry& e) {
  return pad8((uint64_t)e.n_tiles * 4) + ((uint64_t)e.n_tiles + 1) * 8 + pad8(e.n_words * 4);
}

// FNV-1a, 64-bit (Fowler, Noll, Vo): offset basis and prime of the
// published definition.
struct Fnv {
  uint64_t h = 0xcbf29ce484222325ull;
  void add(const void* p, size_t n) {
    const unsigned char* b = static_cast<const unsigned char*>(p);
    for (size_t i = 0; i < n; ++i) {
      h ^= b[i];
      h *= 0x100000001b3ull;
    }
  }
};

bool name_ok(const char* name) {
  const size_t n = strnlen(name, sizeof(((hq_ckpt_entry*)nullptr)->name));
  return n > 0 && n < sizeof(((hq_ckpt_entry*)nullptr)->name);
}

// The fields an entry must satisfy, with its offsets when given.
hq_status check_entry(const hq_ckpt_entry& e) {
  if (!name_ok(e.name)) return HQ_EINVAL;
  if (e.lattice != HQ_Z && e.lattice != HQ_A2 && e.lattice != HQ_D4 && e.lattice != HQ_E8)
    return HQ_EINVAL;
  if (e.tile != 64 && e.tile != 128 && e.tile != 256 && e.tile != 512) return HQ_EINVAL;
  if (!(e.bps > 0.0f && e.bps <= 8.0f)) return HQ_EINVAL;
  if (e.rows < 0 || e.cols < 0 || e.n_tiles < 0) return HQ_EINVAL;
  // at most 2^48 weights, so the products below stay inside int64
  if (e.rows > 0 && e.cols > ((int64_t)1 << 48) / e.rows) return HQ_EINVAL;
  if (e.n_tiles > ((int64_t)1 << 48) / e.tile) return HQ_EINVAL;
  if (e.rows * e.cols != e.n_tiles * (int64_t)e.tile) return HQ_EINVAL;
  if (e.n_words > ((uint64_t)1 << 40)) return HQ_EINVAL;
  return HQ_OK;
}

hq_status check_offsets(const uint64_t* off, int64_t n_tiles, uint64_t n_words) {
  if (off[0] != 0 || off[n_tiles] != n_words) return HQ_EINVAL;
  for (int64_t t = 0; t < n_tiles; ++t)
    if (off[t + 1] < off[t]) return HQ_EINVAL;
  return HQ_OK;
}

struct File {
  FILE* f = nullptr;
  ~File() {
    if (f) fclose(f);
  }
};

// Reads and checks the file magic.
hq_status open_read(const char* path, File& file) {
  file.f = fopen(path, "rb");
  if (!file.f) return HQ_EIO;
  unsigned char m[8];
  if (fread(m, 1, 8, file.f) != 8) return HQ_EFORMAT;
  if (memcmp(m, kFileMagic, 8) != 0) return HQ_EFORMAT;
  return HQ_OK;
}

// Next record header (HQ_ENOTFOUND at the end of the file); the stream is
// left at the record's payload.
hq_status next_record(File& file, RecHeader& r) {
  const size_t got = fread(&r, 1, sizeof(r), file.f);
  if (got == 0 && feof(file.f)) return HQ_ENOTFOUND;
  if (got != sizeof(r)) return HQ_EFORMAT;
  if (memcmp(r.magic, kRecMagic, 4) != 0 || r.header_bytes != kRecHeaderBytes) return HQ_EFORMAT;
  if (check_entry(r.e) != HQ_OK || r.payload_bytes != payload_bytes(r.e)) return HQ_EFORMAT;
  return HQ_OK;
}

hq_status skip_payload(File& file, const RecHeader& r) {
  return fseeko(file.f, (off_t)r.payload_bytes, SEEK_CUR) == 0 ? HQ_OK : HQ_EFORMAT;
}

// Finds the record named `name`; the stream is left at its payload.
hq_status find(File& file, const char* name, RecHeader& r) {
  for (;;) {
    hq_status st = next_record(file, r);
    if (st != HQ_OK) return st;
    if (strncmp(r.e.name, name, sizeof(r.e.name)) == 0) return HQ_OK;
    st = skip_payload(file, r);
    if (st != HQ_OK) return st;
  }
}

}  // namespace

extern "C" {

hq_status hq_ckpt_append(const char* path, const hq_ckpt_entry* e, const float* scale,
                         const uint64_t* tile_word_offset, const uint32_t* words) {
  if (path == nullptr || e == nullptr) return HQ_EINVAL;
  hq_status st = check_entry(*e);
  if (st != HQ_OK) return st;
  if ((e->n_tiles > 0 && scale == nullptr) || tile_word_offset == nullptr ||
      (e->n_words > 0 && words == nullptr))
    return HQ_EINVAL;
  st = check_offsets(tile_word_offset, e->n_tiles, e->n_words);
  if (st != HQ_OK) return st;
  // a new file gets the magic; an existing one must be a checkpoint without
  // a record of this name
  {
    File probe;
    st = open_read(path, probe);
    if (st == HQ_OK) {
      RecHeader r;
      st = find(probe, e->name, r);
      if (st == HQ_OK) return HQ_EINVAL;        // name taken
      if (st != HQ_ENOTFOUND) return st;
    } else if (st == HQ_EFORMAT) {
      return st;
    }
  }
  File out;
  out.f = fopen(path, "ab");
  if (!out.f) return HQ_EIO;
  if (fseeko(out.f, 0, SEEK_END) != 0) return HQ_EIO;
  if (ftello(out.f) == 0 && fwrite(kFileMagic, 1, 8, out.f) != 8) return HQ_EIO;

  RecHeader r;
  memset(&r, 0, sizeof(r));
  memcpy(r.magic, kRecMagic, 4);
  r.header_bytes = kRecHeaderBytes;
  r.e = *e;
  // the name's unused bytes are written as zeros
  const size_t nlen = strnlen(e->name, sizeof(r.e.name));
  memset(r.e.name + nlen, 0, sizeof(r.e.name) - nlen);
  r.payload_bytes = payload_bytes(*e);
  const unsigned char zeros[8] = {0};
  const uint64_t sb = (uint64_t)e->n_tiles * 4, wb = e->n_words * 4;
  Fnv fnv;
  fnv.add(scale, sb);
  fnv.add(zeros, pad8(sb) - sb);
  fnv.add(tile_word_offset, ((uint64_t)e->n_tiles + 1) * 8);
  fnv.add(words, wb);
  fnv.add(zeros, pad8(wb) - wb);
  r.checksum = fnv.h;
  bool ok = fwrite(&r, 1, sizeof(r), out.f) == sizeof(r);
  ok = ok && fwrite(scale, 1, sb, out.f) == sb;
  ok = ok && fwrite(zeros, 1, pad8(sb) - sb, out.f) == pad8(sb) - sb;
  ok = ok && fwrite(tile_word_offset, 8, (size_t)e->n_tiles + 1, out.f) == (size_t)e->n_tiles + 1;
  ok = ok && fwrite(words, 1, wb, out.f) == wb;
  ok = ok && fwrite(zeros, 1, pad8(wb) - wb, out.f) == pad8(wb) - wb;
  ok = ok && fflush(out.f) == 0;
  return ok ? HQ_OK : HQ_EIO;
}

hq_status hq_ckpt_count(const char* path, int32_t* count) {
  if (path == nullptr || count == nullptr) return HQ_EINVAL;
  File file;
  hq_status st = open_read(path, file);
  if (st != HQ_OK) return st;
  int32_t n = 0;
  for (;;) {
    RecHeader r;
    st = next_record(file, r);
    if (st == HQ_ENOTFOUND) break;
    if (st != HQ_OK) return st;
    st = skip_payload(file, r);
    if (st != HQ_OK) return st;
    ++n;
  }
  *count = n;
  return HQ_OK;
}

hq_status hq_ckpt_entry_at(const char* path, int32_t i, hq_ckpt_entry* e) {
  if (path == nullptr || e == nullptr || i < 0) return HQ_EINVAL;
  File file;
  hq_status st = open_read(path, file);
  if (st != HQ_OK) return st;
  for (int32_t k = 0;; ++k) {
    RecHeader r;
    st = next_record(file, r);
    if (st != HQ_OK) return st;
    if (k == i) {
      *e = r.e;
      return HQ_OK;
    }
    st = skip_payload(file, r);
    if (st != HQ_OK) return st;
  }
}

hq_status hq_ckpt_read(const char* path, const char* name, hq_ckpt_entry* e, float* scale,
                       uint64_t* tile_word_offset, uint32_t* words, int64_t capacity_tiles,
                       uint64_t capacity_words) {
  if (path == nullptr || name == nullptr || e == nullptr || !name_ok(name)) return HQ_EINVAL;
  File file;
  hq_status st = open_read(path, file);
  if (st != HQ_OK) return st;
  RecHeader r;
  st = find(file, name, r);
  if (st != HQ_OK) return st;
  if (capacity_tiles < r.e.n_tiles || capacity_words < r.e.n_words) return HQ_EINVAL;
  if ((r.e.n_tiles > 0 && scale == nullptr) || tile_word_offset == nullptr ||
      (r.e.n_words > 0 && words == nullptr))
    return HQ_EINVAL;
  const uint64_t sb = (uint64_t)r.e.n_tiles * 4, wb = r.e.n_words * 4;
  unsigned char pad[8];
  Fnv fnv;
  bool ok = fread(scale, 1, sb, file.f) == sb;
  ok = ok && fread(pad, 1, pad8(sb) - sb, file.f) == pad8(sb) - sb;
  if (ok) {
    fnv.add(scale, sb);
    fnv.add(pad, pad8(sb) - sb);
  }
  ok = ok && fread(tile_word_offset, 8, (size_t)r.e.n_tiles + 1, file.f) == (size_t)r.e.n_tiles + 1;
  if (ok) fnv.add(tile_word_offset, ((uint64_t)r.e.n_tiles + 1) * 8);
  ok = ok && fread(words, 1, wb, file.f) == wb;
  ok = ok && fread(pad, 1, pad8(wb) - wb, file.f) == pad8(wb) - wb;
  if (ok) {
    fnv.add(words, wb);
    fnv.add(pad, pad8(wb) - wb);
  }
  if (!ok || fnv.h != r.checksum) return HQ_EFORMAT;
  if (check_offsets(tile_word_offset, r.e.n_tiles, r.e.n_words) != HQ_OK) return HQ_EFORMAT;
  *e = r.e;
  return HQ_OK;
}

}  // extern "C"
