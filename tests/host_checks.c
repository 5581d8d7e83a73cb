/*
 * Host-side driver of the library's C ABI, built together with the library's
 * sources under AddressSanitizer and UndefinedBehaviorSanitizer (host code
 * only) by tests/test_host_sanitizers.py.  No GPU is needed: it only reaches
 * the host paths (argument validation, calibration, rotation files).
 *
 *   host_checks validate
 *       every host-detectable argument error of every entry point returns its
 *       documented status before anything is launched
 *   host_checks calibrate IN OUT
 *       IN: int32 hkv, n_q, n_kv, then float q [hkv][n_q][128], k, v
 *       [hkv][n_kv][128]; runs oscar_calibrate, and oscar_calibrate_layers on
 *       two layers (the inputs, then the same inputs again); OUT: the single
 *       call's r_k, r_v (uint16 [hkv][128][128]), eig_k, eig_v (double
 *       [hkv][128]), then a byte that is 1 when both layers of the layered call
 *       equal the single call bit for bit
 *   host_checks rotfile ROT FILE
 *       ROT: the calibrate output (hkv given as argv[4]); writes the two-layer
 *       file FILE (layer 1 = layer 0), reads it back, and checks that flipped,
 *       truncated, extended and mismatched copies are refused
 * Exit status 0 when every check holds; each failure is printed.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oscar.h"

static int failures = 0;

#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);   \
      ++failures;                                                 \
    }                                                             \
  } while (0)

static oscar_shape shape_of(int hq, int hkv, int window, int n_sink, int group) {
  oscar_shape s;
  memset(&s, 0, sizeof s);
  s.n_q_heads = hq;
  s.n_kv_heads = hkv;
  s.head_dim = OSCAR_HEAD_DIM;
  s.group_size = group;
  s.page_size = OSCAR_PAGE_SIZE;
  s.window = window;
  s.n_sink = n_sink;
  return s;
}

static int validate(void) {
  void* f = (void*)(uintptr_t)256; /* aligned, never dereferenced: every call below fails its checks first */
  void* mis = (void*)(uintptr_t)258;
  oscar_shape good = shape_of(32, 8, 128, 0, 128);
  oscar_shape bad[9];
  bad[0] = shape_of(32, 8, 128, 0, 128); bad[0].head_dim = 64;
  bad[1] = shape_of(32, 8, 128, 0, 16);
  bad[2] = shape_of(32, 8, 128, 0, 48);
  bad[3] = shape_of(32, 8, 128, 0, 0);
  bad[4] = shape_of(32, 8, 128, 0, 128); bad[4].page_size = 32;
  bad[5] = shape_of(24, 8, 128, 0, 128);
  bad[6] = shape_of(32, 8, 4096, 0, 128);
  bad[7] = shape_of(32, 8, 128, -1, 128);
  bad[8] = shape_of(32, 8, 128, 2048, 128);
  for (int i = 0; i < 9; ++i) {
    int st = oscar_quantize_append(&bad[i], 0, 0, 0, 0, 1, 0, 0, 1, 0, 1, 0, 0, 1, 0, 0, 0);
    EXPECT(st == OSCAR_EINVAL || st == OSCAR_EUNSUPPORTED);
    EXPECT(oscar_decode_workspace_bytes(&bad[i], 1, 100) == 0);
    EXPECT(oscar_decode_layers_workspace_bytes(&bad[i], 2, 1, 100) == 0);
  }
  EXPECT(oscar_quantize_append(NULL, f, f, f, f, 1, f, f, 1, f, 1, f, f, 1, f, f, 0) == OSCAR_EINVAL);
  EXPECT(oscar_quantize_append(&good, 0, 0, 0, 0, 5, 0, 0, 1, 0, 1, 0, 0, 1, 0, 0, 0) == OSCAR_EINVAL);
  EXPECT(oscar_quantize_append(&good, 0, 0, 0, 0, 0, 0, 0, 1, 0, 1, 0, 0, 1, 0, 0, 0) == OSCAR_OK);
  EXPECT(oscar_quantize_append(&good, f, f, mis, f, 1, f, f, 1, f, 1, f, f, 1, f, f, 0) == OSCAR_EINVAL);
  size_t ws = oscar_decode_workspace_bytes(&good, 8, 100000);
  EXPECT(ws > 8u * 32u * 128u * 4u);
  EXPECT(oscar_decode_attn(&good, f, f, f, 8, f, 100000, f, 100000 / 16 + 1, f, 1, f, f, f, f, ws - 1, 0) ==
         OSCAR_ENOSPACE);
  EXPECT(oscar_decode_attn(&good, f, f, f, 8, f, 100000, f, 100, f, 1, f, f, f, f, ws, 0) == OSCAR_ENOSPACE);
  EXPECT(oscar_decode_attn(&good, mis, f, f, 8, f, 100000, f, 100000 / 16 + 1, f, 1, f, f, f, f, ws, 0) ==
         OSCAR_EINVAL);
  EXPECT(oscar_decode_attn(&good, f, f, mis, 8, f, 100000, f, 100000 / 16 + 1, f, 1, f, f, f, f, ws, 0) ==
         OSCAR_EINVAL);
  EXPECT(oscar_decode_attn(&good, 0, 0, 0, 8, 0, 10, 0, 1, 0, 1, 0, 0, 0, 0, 0, 0) == OSCAR_EINVAL);
  EXPECT(oscar_decode_attn(&good, f, f, f, 8, f, -1, f, 1, f, 1, f, f, f, f, ws, 0) == OSCAR_EINVAL);
  EXPECT(oscar_decode_attn(&good, f, f, f, 0, f, 10, f, 1, f, 1, f, f, f, f, ws, 0) == OSCAR_EINVAL);
  /* timed forms: the two events go together */
  EXPECT(oscar_decode_attn_timed(&good, f, f, f, 8, f, 10, f, 1, f, 1, f, f, f, f, ws, 0, f, 0) == OSCAR_EINVAL);
  EXPECT(oscar_quantize_append_timed(&good, f, f, f, f, 1, f, f, 1, f, 1, f, f, 1, f, f, 0, 0, f) == OSCAR_EINVAL);
  EXPECT(oscar_bf16_decode_attn_timed(&good, f, 8, f, 10, f, 1, f, 1, f, f, ws, 0, f, 0) == OSCAR_EINVAL);
  /* the fused decode step: new-token rows required and aligned, then the decode's checks */
  EXPECT(oscar_decode_step(&good, f, f, 0, f, f, 8, f, 10, f, 1, f, 1, f, f, f, f, ws, 0) == OSCAR_EINVAL);
  EXPECT(oscar_decode_step(&good, f, f, f, 0, f, 8, f, 10, f, 1, f, 1, f, f, f, f, ws, 0) == OSCAR_EINVAL);
  EXPECT(oscar_decode_step(&good, f, f, mis, f, f, 8, f, 100000, f, 100000 / 16 + 1, f, 1, f, f, f, f, ws, 0) ==
         OSCAR_EINVAL);
  EXPECT(oscar_decode_step(&good, f, f, f, f, f, 8, f, 100000, f, 100000 / 16 + 1, f, 1, f, f, f, f, ws - 1, 0) ==
         OSCAR_ENOSPACE);
  EXPECT(oscar_decode_step(&good, f, f, f, f, f, 0, f, 10, f, 1, f, 1, f, f, f, f, ws, 0) == OSCAR_EINVAL);
  EXPECT(oscar_decode_step_timed(&good, f, f, f, f, f, 8, f, 10, f, 1, f, 1, f, f, f, f, ws, 0, f, 0) ==
         OSCAR_EINVAL);
  /* sinks without a window still need the ring */
  oscar_shape sink_only = shape_of(32, 8, 0, 4, 128);
  EXPECT(oscar_decode_attn(&sink_only, f, f, f, 8, f, 10, f, 1, f, 1, 0, 0, f, f, (size_t)1 << 30, 0) ==
         OSCAR_EINVAL);
  EXPECT(oscar_quantize_append(&sink_only, f, f, f, f, 1, f, f, 1, f, 1, f, f, 1, 0, 0, 0) == OSCAR_EINVAL);
  /* layer-batched forms */
  EXPECT(oscar_decode_layers_workspace_bytes(&good, 1, 8, 100000) == ws);
  EXPECT(oscar_decode_layers_workspace_bytes(&good, 4, 8, 100000) > ws);
  EXPECT(oscar_decode_attn_layers(&good, 0, f, f, f, 8, f, 100, f, 16, f, 1, f, f, f, f, (size_t)1 << 30, 0) ==
         OSCAR_EINVAL);
  EXPECT(oscar_decode_attn_layers(&good, 4096, f, f, f, 32, f, 100, f, 16, f, 1, f, f, f, f, (size_t)1 << 40, 0) ==
         OSCAR_EINVAL);
  EXPECT(oscar_decode_attn_layers(&good, 4, f, f, f, 8, f, 100000, f, 100000 / 16 + 1, f, 1, f, f, f, f, ws, 0) ==
         OSCAR_ENOSPACE);
  EXPECT(oscar_quantize_append_layers(&good, -1, f, f, f, f, 1, f, f, 1, f, 1, f, f, 1, f, f, 0) == OSCAR_EINVAL);
  /* bf16 comparator */
  EXPECT(oscar_bf16_append(&good, 0, 0, 5, 0, 0, 1, 0, 1, 0, 1, 0) == OSCAR_EINVAL);
  EXPECT(oscar_bf16_append(&good, f, mis, 5, f, f, 1, f, 1, f, 1, 0) == OSCAR_EINVAL);
  EXPECT(oscar_bf16_decode_attn(&good, f, 8, f, 100000, f, 100000 / 16 + 1, f, 1, f, f, 16, 0) == OSCAR_ENOSPACE);
  /* measurement helpers */
  EXPECT(oscar_hbm_copy(f, f, 17, 0) == OSCAR_EINVAL);
  EXPECT(oscar_hbm_copy(mis, f, 16, 0) == OSCAR_EINVAL);
  EXPECT(oscar_hbm_read(f, 1000, 0, 1, f, 0, 0) == OSCAR_EINVAL);
  EXPECT(oscar_hbm_read(f, 1152, 0, 1, 0, 0, 0) == OSCAR_EINVAL);
  EXPECT(oscar_hbm_read(f, 1152, 0, 1, f, OSCAR_READ_MAX_WORKGROUPS + 1, 0) == OSCAR_EINVAL);
  EXPECT(oscar_hbm_read(f, 1152, 0, 0, f, 0, 0) == OSCAR_OK);
  EXPECT(oscar_gpu_wait(-1, 0) == OSCAR_EINVAL);
  EXPECT(oscar_gpu_wait(0, 0) == OSCAR_OK);
  EXPECT(oscar_event_create(0) == OSCAR_EINVAL);
  EXPECT(oscar_event_destroy(0) == OSCAR_EINVAL);
  EXPECT(oscar_event_elapsed_ms(0, 0, 0) == OSCAR_EINVAL);
  /* calibration */
  float x[128];
  memset(x, 0, sizeof x);
  uint16_t r[128 * 128];
  EXPECT(oscar_calibrate(&good, 0, 1, x, x, 1, r, r, 0, 0) == OSCAR_EINVAL);
  EXPECT(oscar_calibrate(&good, x, 0, x, x, 1, r, r, 0, 0) == OSCAR_EINVAL);
  EXPECT(oscar_calibrate(&bad[0], x, 1, x, x, 1, r, r, 0, 0) == OSCAR_EUNSUPPORTED);
  EXPECT(oscar_calibrate_layers(&good, 0, x, 1, x, x, 1, r, r, 0, 0) == OSCAR_EINVAL);
  /* rotation files */
  EXPECT(oscar_rotation_file_bytes(0, 8, 1) == 0);
  EXPECT(oscar_rotation_file_bytes(2, 8, 1) == 64u + 2u * (8u * 128u * 128u * 2u * 2u + 8u * 128u * 8u * 2u));
  EXPECT(oscar_rotation_write(0, &good, 1, r, r, 0, 0) == OSCAR_EINVAL);
  EXPECT(oscar_rotation_read_info(0, 0, 0, 0, 0) == OSCAR_EINVAL);
  EXPECT(strcmp(oscar_strerror(OSCAR_OK), "ok") == 0);
  EXPECT(strcmp(oscar_strerror(12345), "unknown status") == 0);
  return failures;
}

static void* read_all(const char* path, size_t* n) {
  FILE* fp = fopen(path, "rb");
  if (!fp) return NULL;
  fseek(fp, 0, SEEK_END);
  long len = ftell(fp);
  fseek(fp, 0, SEEK_SET);
  void* buf = malloc(len > 0 ? (size_t)len : 1);
  size_t got = fread(buf, 1, (size_t)len, fp);
  fclose(fp);
  *n = got;
  return buf;
}

static int write_all(const char* path, const void* buf, size_t n) {
  FILE* fp = fopen(path, "wb");
  if (!fp) return -1;
  size_t put = fwrite(buf, 1, n, fp);
  return fclose(fp) == 0 && put == n ? 0 : -1;
}

static int calibrate(const char* in, const char* out) {
  size_t n = 0;
  uint8_t* buf = read_all(in, &n);
  if (!buf || n < 12) return 2;
  int32_t hdr[3];
  memcpy(hdr, buf, sizeof hdr);
  const int hkv = hdr[0], nq = hdr[1], nkv = hdr[2];
  const size_t q_el = (size_t)hkv * nq * 128, kv_el = (size_t)hkv * nkv * 128;
  if (n != 12 + 4 * (q_el + 2 * kv_el)) return 3;
  const float* q = (const float*)(buf + 12);
  const float* k = q + q_el;
  const float* v = k + kv_el;
  oscar_shape s = shape_of(4 * hkv, hkv, 128, 0, 128);
  const size_t rot = (size_t)hkv * 128 * 128, ev = (size_t)hkv * 128;
  uint16_t* rk = malloc(rot * 2 * 3);
  uint16_t* rv = malloc(rot * 2 * 3);
  double* ek = malloc(ev * 8 * 3);
  double* evv = malloc(ev * 8 * 3);
  EXPECT(oscar_calibrate(&s, q, nq, k, v, nkv, rk, rv, ek, evv) == OSCAR_OK);
  /* two layers: the same inputs twice, laid out layer-major */
  float* q2 = malloc(4 * q_el * 2);
  float* k2 = malloc(4 * kv_el * 2);
  float* v2 = malloc(4 * kv_el * 2);
  memcpy(q2, q, 4 * q_el), memcpy(q2 + q_el, q, 4 * q_el);
  memcpy(k2, k, 4 * kv_el), memcpy(k2 + kv_el, k, 4 * kv_el);
  memcpy(v2, v, 4 * kv_el), memcpy(v2 + kv_el, v, 4 * kv_el);
  EXPECT(oscar_calibrate_layers(&s, 2, q2, nq, k2, v2, nkv, rk + rot, rv + rot, ek + ev, evv + ev) == OSCAR_OK);
  uint8_t same = 1;
  for (int l = 1; l <= 2; ++l) {
    same &= memcmp(rk, rk + l * rot, rot * 2) == 0 && memcmp(rv, rv + l * rot, rot * 2) == 0;
    same &= memcmp(ek, ek + l * ev, ev * 8) == 0 && memcmp(evv, evv + l * ev, ev * 8) == 0;
  }
  FILE* fp = fopen(out, "wb");
  if (!fp) return 4;
  fwrite(rk, 2, rot, fp);
  fwrite(rv, 2, rot, fp);
  fwrite(ek, 8, ev, fp);
  fwrite(evv, 8, ev, fp);
  fwrite(&same, 1, 1, fp);
  fclose(fp);
  free(rk), free(rv), free(ek), free(evv), free(q2), free(k2), free(v2), free(buf);
  return failures;
}

static int rotfile(const char* rot_path, const char* file, int hkv) {
  size_t n = 0;
  uint8_t* buf = read_all(rot_path, &n);
  const size_t rot = (size_t)hkv * 128 * 128, ev = (size_t)hkv * 128;
  if (!buf || n != rot * 4 + ev * 16 + 1) return 2;
  oscar_shape s = shape_of(4 * hkv, hkv, 128, 0, 128);
  uint16_t* rk = malloc(rot * 4);
  uint16_t* rv = malloc(rot * 4);
  double* ek = malloc(ev * 16);
  double* evv = malloc(ev * 16);
  for (int l = 0; l < 2; ++l) {
    memcpy(rk + l * rot, buf, rot * 2);
    memcpy(rv + l * rot, buf + rot * 2, rot * 2);
    memcpy(ek + l * ev, buf + rot * 4, ev * 8);
    memcpy(evv + l * ev, buf + rot * 4 + ev * 8, ev * 8);
  }
  EXPECT(oscar_rotation_write(file, &s, 2, rk, rv, ek, evv) == OSCAR_OK);
  int32_t nl = 0, nh = 0, g = 0, he = 0;
  EXPECT(oscar_rotation_read_info(file, &nl, &nh, &g, &he) == OSCAR_OK);
  EXPECT(nl == 2 && nh == hkv && g == 128 && he == 1);
  uint16_t* rk2 = calloc(rot * 2, 2);
  uint16_t* rv2 = calloc(rot * 2, 2);
  double* ek2 = calloc(ev * 2, 8);
  double* ev2 = calloc(ev * 2, 8);
  EXPECT(oscar_rotation_read(file, &s, 2, rk2, rv2, ek2, ev2) == OSCAR_OK);
  EXPECT(memcmp(rk, rk2, rot * 4) == 0 && memcmp(rv, rv2, rot * 4) == 0);
  EXPECT(memcmp(ek, ek2, ev * 16) == 0 && memcmp(evv, ev2, ev * 16) == 0);
  EXPECT(oscar_rotation_read(file, &s, 1, rk2, rv2, 0, 0) == OSCAR_EFORMAT);  /* layer count */
  oscar_shape other = shape_of(4 * hkv, hkv, 128, 0, 64);
  EXPECT(oscar_rotation_read(file, &other, 2, rk2, rv2, 0, 0) == OSCAR_EFORMAT);  /* group size */
  /* damaged copies */
  size_t fn = 0;
  uint8_t* img = read_all(file, &fn);
  char tmp[4096];
  snprintf(tmp, sizeof tmp, "%s.bad", file);
  const size_t flips[3] = {9, 60, fn - 1};  /* header field, header padding, last payload byte */
  for (int i = 0; i < 3; ++i) {
    img[flips[i]] ^= 0x10;
    write_all(tmp, img, fn);
    EXPECT(oscar_rotation_read(tmp, &s, 2, rk2, rv2, 0, 0) == OSCAR_EFORMAT);
    img[flips[i]] ^= 0x10;
  }
  write_all(tmp, img, fn - 1);
  EXPECT(oscar_rotation_read(tmp, &s, 2, rk2, rv2, 0, 0) == OSCAR_EFORMAT);  /* truncated */
  uint8_t* longer = malloc(fn + 1);
  memcpy(longer, img, fn);
  longer[fn] = 0;
  write_all(tmp, longer, fn + 1);
  EXPECT(oscar_rotation_read(tmp, &s, 2, rk2, rv2, 0, 0) == OSCAR_EFORMAT);  /* trailing byte */
  write_all(tmp, img, 20);
  EXPECT(oscar_rotation_read_info(tmp, 0, 0, 0, 0) == OSCAR_EFORMAT);  /* short header */
  snprintf(tmp, sizeof tmp, "%s.missing", file);
  EXPECT(oscar_rotation_read(tmp, &s, 2, rk2, rv2, 0, 0) == OSCAR_EIO);
  free(longer), free(img), free(buf), free(rk), free(rv), free(ek), free(evv), free(rk2), free(rv2), free(ek2),
      free(ev2);
  return failures;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "validate") == 0) return validate() ? 1 : 0;
  if (argc >= 4 && strcmp(argv[1], "calibrate") == 0) return calibrate(argv[2], argv[3]) ? 1 : 0;
  if (argc >= 5 && strcmp(argv[1], "rotfile") == 0) return rotfile(argv[2], argv[3], atoi(argv[4])) ? 1 : 0;
  fprintf(stderr, "usage: host_checks validate | calibrate IN OUT | rotfile ROT FILE HKV\n");
  return 2;
}
