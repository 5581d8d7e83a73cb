// Rotation files: the calibrated per-layer, per-KV-head rotations (and
// optionally their eigenvalues) of one model, stored once and loaded at start
// instead of recalibrating.  The pages describe calibration as an offline,
// once-per-model step whose results ship with the method for supported models
// (P1 gen-hub.ru «Открытый код — это серьёзно»; P2 encorp.ai «OSCAR има
// значение…»; P4 aiforradalom.hu «OSCAR: figyelem-tudatos és bevetésre kész»);
// they fix no file layout, so this one is the library's own (all integers
// little endian):
//   [ 0,  8)  magic "OSCARROT"
//   [ 8, 12)  u32 format version (1)
//   [12, 16)  u32 header bytes (64)
//   [16, 20)  u32 head_dim (128)
//   [20, 24)  u32 n_layers
//   [24, 28)  u32 n_kv_heads
//   [28, 32)  u32 group_size the rotations were calibrated for (128, 64, 32)
//   [32, 36)  u32 flags: bit 0 = eigenvalues present
//   [36, 40)  u32 zero
//   [40, 48)  u64 payload bytes
//   [48, 52)  u32 CRC-32 of the payload
//   [52, 56)  u32 CRC-32 of bytes [0, 52)
//   [56, 64)  zero
// Payload, layer by layer: R_K bf16 [Hkv][128][128], R_V bf16 [Hkv][128][128],
// then, with flag bit 0, eig_K and eig_V float64 [Hkv][128].
// CRC-32 is the reflected polynomial 0xEDB88320 with initial value and final
// xor 0xFFFFFFFF (the checksum of zip and PNG).
#include <cstdio>
#include <cstring>
#include <vector>

#include "common.h"

namespace {

constexpr char kMagic[8] = {'O', 'S', 'C', 'A', 'R', 'R', 'O', 'T'};
constexpr uint32_t kVersion = 1, kHeader = 64;

struct Crc32 {
  uint32_t table[256];
  Crc32() {
    for (uint32_t i = 0; i < 256; ++i) {
      uint32_t c = i;
      for (int k = 0; k < 8; ++k) c = (c & 1u) ? 0xEDB88320u ^ (c >> 1) : c >> 1;
      table[i] = c;
    }
  }
  uint32_t update(uint32_t crc, const uint8_t* p, size_t n) const {  // crc: running value before the final xor
    for (size_t i = 0; i < n; ++i) crc = table[(crc ^ p[i]) & 0xffu] ^ (crc >> 8);
    return crc;
  }
};
const Crc32& crc_table() {
  static const Crc32 t;
  return t;
}

void put32(uint8_t* p, uint32_t v) {
  for (int i = 0; i < 4; ++i) p[i] = (uint8_t)(v >> (8 * i));
}
void put64(uint8_t* p, uint64_t v) {
  for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(v >> (8 * i));
}
uint32_t get32(const uint8_t* p) {
  uint32_t v = 0;
  for (int i = 0; i < 4; ++i) v |= (uint32_t)p[i] << (8 * i);
  return v;
}
uint64_t get64(const uint8_t* p) {
  uint64_t v = 0;
  for (int i = 0; i < 8; ++i) v |= (uint64_t)p[i] << (8 * i);
  return v;
}

size_t layer_bytes(int hkv, bool eig) {
  return (size_t)hkv * oscar::kD * oscar::kD * 2 * 2 + (eig ? (size_t)hkv * oscar::kD * 8 * 2 : 0);
}

struct Info {
  uint32_t n_layers, hkv, group, flags;
  uint64_t payload;
  uint32_t crc_payload;
};

// Reads and checks the header.  OSCAR_EIO: cannot read; OSCAR_EFORMAT: not a
// rotation file of this version, inconsistent sizes or a damaged header.
int read_header(FILE* f, Info& info) {
  uint8_t h[kHeader];
  if (std::fread(h, 1, kHeader, f) != kHeader) return OSCAR_EFORMAT;
  if (std::memcmp(h, kMagic, 8) != 0) return OSCAR_EFORMAT;
  uint32_t crc = crc_table().update(0xFFFFFFFFu, h, 52) ^ 0xFFFFFFFFu;
  if (crc != get32(h + 52)) return OSCAR_EFORMAT;
  if (get32(h + 8) != kVersion || get32(h + 12) != kHeader || get32(h + 16) != (uint32_t)oscar::kD)
    return OSCAR_EFORMAT;
  // reserved: u32 at 36 and the 8 bytes after the header checksum are zero
  if (get32(h + 36) != 0 || get64(h + 56) != 0) return OSCAR_EFORMAT;
  info.n_layers = get32(h + 20);
  info.hkv = get32(h + 24);
  info.group = get32(h + 28);
  info.flags = get32(h + 32);
  info.payload = get64(h + 40);
  info.crc_payload = get32(h + 48);
  if (info.n_layers < 1 || info.hkv < 1 || info.hkv > 4096 || info.n_layers > 65536 || (info.flags & ~1u))
    return OSCAR_EFORMAT;
  if (info.group != 32 && info.group != 64 && info.group != (uint32_t)oscar::kD) return OSCAR_EFORMAT;
  if (info.payload != (uint64_t)info.n_layers * layer_bytes((int)info.hkv, info.flags & 1u)) return OSCAR_EFORMAT;
  return OSCAR_OK;
}

}  // namespace

extern "C" size_t oscar_rotation_file_bytes(int32_t n_layers, int32_t n_kv_heads, int32_t with_eigenvalues) {
  if (n_layers < 1 || n_kv_heads < 1) return 0;
  return kHeader + (size_t)n_layers * layer_bytes(n_kv_heads, with_eigenvalues != 0);
}

extern "C" int oscar_rotation_write(const char* path, const oscar_shape* shape, int32_t n_layers,
                                    const uint16_t* r_k, const uint16_t* r_v, const double* eig_k,
                                    const double* eig_v) {
  int st = oscar::check_shape(shape);
  if (st != OSCAR_OK) return st;
  if (!path || !r_k || !r_v || n_layers < 1 || (!eig_k) != (!eig_v)) return OSCAR_EINVAL;
  const int hkv = shape->n_kv_heads;
  const bool eig = eig_k != nullptr;
  const size_t rot = (size_t)hkv * oscar::kD * oscar::kD, ev = (size_t)hkv * oscar::kD;
  // payload in memory, layer by layer (little-endian host)
  std::vector<uint8_t> body(layer_bytes(hkv, eig) * (size_t)n_layers);
  uint8_t* o = body.data();
  for (int l = 0; l < n_layers; ++l) {
    std::memcpy(o, r_k + l * rot, rot * 2), o += rot * 2;
    std::memcpy(o, r_v + l * rot, rot * 2), o += rot * 2;
    if (eig) {
      std::memcpy(o, eig_k + l * ev, ev * 8), o += ev * 8;
      std::memcpy(o, eig_v + l * ev, ev * 8), o += ev * 8;
    }
  }
  uint8_t h[kHeader] = {};
  std::memcpy(h, kMagic, 8);
  put32(h + 8, kVersion);
  put32(h + 12, kHeader);
  put32(h + 16, (uint32_t)oscar::kD);
  put32(h + 20, (uint32_t)n_layers);
  put32(h + 24, (uint32_t)hkv);
  put32(h + 28, (uint32_t)shape->group_size);
  put32(h + 32, eig ? 1u : 0u);
  put64(h + 40, (uint64_t)body.size());
  put32(h + 48, crc_table().update(0xFFFFFFFFu, body.data(), body.size()) ^ 0xFFFFFFFFu);
  put32(h + 52, crc_table().update(0xFFFFFFFFu, h, 52) ^ 0xFFFFFFFFu);
  FILE* f = std::fopen(path, "wb");
  if (!f) return OSCAR_EIO;
  bool ok = std::fwrite(h, 1, kHeader, f) == kHeader && std::fwrite(body.data(), 1, body.size(), f) == body.size();
  ok = (std::fclose(f) == 0) && ok;
  return ok ? OSCAR_OK : OSCAR_EIO;
}

extern "C" int oscar_rotation_read_info(const char* path, int32_t* n_layers, int32_t* n_kv_heads,
                                        int32_t* group_size, int32_t* has_eigenvalues) {
  if (!path) return OSCAR_EINVAL;
  FILE* f = std::fopen(path, "rb");
  if (!f) return OSCAR_EIO;
  Info info;
  int st = read_header(f, info);
  std::fclose(f);
  if (st != OSCAR_OK) return st;
  if (n_layers) *n_layers = (int32_t)info.n_layers;
  if (n_kv_heads) *n_kv_heads = (int32_t)info.hkv;
  if (group_size) *group_size = (int32_t)info.group;
  if (has_eigenvalues) *has_eigenvalues = (int32_t)(info.flags & 1u);
  return OSCAR_OK;
}

extern "C" int oscar_rotation_read(const char* path, const oscar_shape* shape, int32_t n_layers, uint16_t* r_k,
                                   uint16_t* r_v, double* eig_k, double* eig_v) {
  int st = oscar::check_shape(shape);
  if (st != OSCAR_OK) return st;
  if (!path || !r_k || !r_v || n_layers < 1 || (!eig_k) != (!eig_v)) return OSCAR_EINVAL;
  FILE* f = std::fopen(path, "rb");
  if (!f) return OSCAR_EIO;
  Info info;
  st = read_header(f, info);
  if (st != OSCAR_OK) {
    std::fclose(f);
    return st;
  }
  // the caller's shape must be the file's
  if (info.n_layers != (uint32_t)n_layers || info.hkv != (uint32_t)shape->n_kv_heads ||
      info.group != (uint32_t)shape->group_size || (eig_k && !(info.flags & 1u))) {
    std::fclose(f);
    return OSCAR_EFORMAT;
  }
  std::vector<uint8_t> body(info.payload);
  const bool whole = std::fread(body.data(), 1, body.size(), f) == body.size() && std::fgetc(f) == EOF;
  std::fclose(f);
  if (!whole) return OSCAR_EFORMAT;  // truncated, or trailing bytes
  if ((crc_table().update(0xFFFFFFFFu, body.data(), body.size()) ^ 0xFFFFFFFFu) != info.crc_payload)
    return OSCAR_EFORMAT;
  const int hkv = shape->n_kv_heads;
  const bool eig = info.flags & 1u;
  const size_t rot = (size_t)hkv * oscar::kD * oscar::kD, ev = (size_t)hkv * oscar::kD;
  const uint8_t* p = body.data();
  for (int l = 0; l < n_layers; ++l) {
    std::memcpy(r_k + l * rot, p, rot * 2), p += rot * 2;
    std::memcpy(r_v + l * rot, p, rot * 2), p += rot * 2;
    if (eig) {
      if (eig_k) std::memcpy(eig_k + l * ev, p, ev * 8);
      p += ev * 8;
      if (eig_v) std::memcpy(eig_v + l * ev, p, ev * 8);
      p += ev * 8;
    }
  }
  return OSCAR_OK;
}
