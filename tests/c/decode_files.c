/* A plain C99 caller of libmla: no Python, no torch. Reads a bf16 latent
 * cache and bf16 queries and weights from a directory, runs mla_decode on
 * the default stream with an fp32 output, checks the device status word
 * and writes the output back. Exit status 0 on success; the failing call is
 * printed otherwise.
 *
 * Directory layout (little-endian, written by the test that drives this):
 *   meta.bin     int32 B, H, n_rows, row_stride; float softmax_scale
 *   lens.bin     int32 [B]  cached tokens per sequence (host copy)
 *   start.bin    int32 [B]  first row of each sequence
 *   cap.bin      int32 [B]  rows reserved per sequence
 *   rows.bin     uint8 [n_rows, row_stride]
 *   q_nope.bin   bf16 [B, H, 128]     q_rope.bin  bf16 [B, H, 64]
 *   w_uk.bin     bf16 [H, 128, 512]   w_uv.bin    bf16 [H, 128, 512]
 * Output: o.bin, fp32 [B, H, 128]. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mla.h"

static const char *g_dir;

static void *read_all(const char *name, size_t *n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    exit(2);
  }
  fseek(f, 0, SEEK_END);
  const long len = ftell(f);
  fseek(f, 0, SEEK_SET);
  void *p = malloc(len > 0 ? (size_t)len : 1);
  if (!p || fread(p, 1, (size_t)len, f) != (size_t)len) {
    fprintf(stderr, "cannot read %s\n", path);
    exit(2);
  }
  fclose(f);
  *n = (size_t)len;
  return p;
}

static void *upload(const char *name, size_t want) {
  size_t n = 0;
  void *h = read_all(name, &n);
  if (n != want) {
    fprintf(stderr, "%s: %zu bytes, expected %zu\n", name, n, want);
    exit(2);
  }
  void *d = NULL;
  if (hipMalloc(&d, n) != hipSuccess || hipMemcpy(d, h, n, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "%s: device copy failed\n", name);
    exit(3);
  }
  free(h);
  return d;
}

#define CHECK(call)                                                        \
  do {                                                                     \
    const mla_status st_ = (call);                                         \
    if (st_ != MLA_OK) {                                                   \
      fprintf(stderr, "%s -> %s\n", #call, mla_status_str(st_));           \
      return 4;                                                            \
    }                                                                      \
  } while (0)

int main(int argc, char **argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 1;
  }
  g_dir = argv[1];
  size_t n = 0;
  char *meta = (char *)read_all("meta.bin", &n);
  if (n != 5 * 4) return 2;
  int32_t hdr[4];
  float scale;
  memcpy(hdr, meta, sizeof hdr);
  memcpy(&scale, meta + 16, sizeof scale);
  free(meta);
  const int32_t B = hdr[0], H = hdr[1];
  const int64_t n_rows = hdr[2], row_stride = hdr[3];
  int32_t *lens = (int32_t *)read_all("lens.bin", &n);
  if (n != (size_t)B * 4) return 2;

  const mla_dims d = {H, 512, 64, 128, 128, 0, scale, 10000.0f};
  mla_cache c;
  memset(&c, 0, sizeof c);
  c.latent_dtype = MLA_BF16;
  c.rope_dtype = MLA_BF16;
  c.rows = upload("rows.bin", (size_t)(n_rows * row_stride));
  c.row_stride = row_stride;
  c.n_rows = n_rows;
  c.batch = B;
  c.seq_start = (const int32_t *)upload("start.bin", (size_t)B * 4);
  c.seq_cap = (const int32_t *)upload("cap.bin", (size_t)B * 4);
  c.seq_len = (int32_t *)upload("lens.bin", (size_t)B * 4);
  const size_t q = (size_t)B * H;
  void *q_nope = upload("q_nope.bin", q * 128 * 2);
  void *q_rope = upload("q_rope.bin", q * 64 * 2);
  void *w_uk = upload("w_uk.bin", (size_t)H * 128 * 512 * 2);
  void *w_uv = upload("w_uv.bin", (size_t)H * 128 * 512 * 2);

  mla_plan *plan = NULL;
  CHECK(mla_plan_create(&d, lens, B, 0, &plan));
  const size_t ws_bytes = mla_decode_workspace_bytes(&d, plan);
  void *ws = NULL, *o = NULL;
  if (ws_bytes == 0 || hipMalloc(&ws, ws_bytes) != hipSuccess || hipMalloc(&o, q * 128 * 4) != hipSuccess) {
    fprintf(stderr, "workspace or output allocation failed\n");
    return 3;
  }
  CHECK(mla_workspace_init(ws, ws_bytes, NULL));
  CHECK(mla_decode(&d, &c, plan, q_nope, q_rope, NULL, w_uk, w_uv, MLA_BF16, o, MLA_F32, ws, ws_bytes, NULL));
  int32_t code = -1;
  CHECK(mla_device_error(ws, NULL, &code, 1));
  if (code != MLA_OK) {
    fprintf(stderr, "device status %s\n", mla_status_str((mla_status)code));
    return 5;
  }
  float *host_o = (float *)malloc(q * 128 * 4);
  if (!host_o || hipMemcpy(host_o, o, q * 128 * 4, hipMemcpyDeviceToHost) != hipSuccess) return 3;
  char path[4096];
  snprintf(path, sizeof path, "%s/o.bin", g_dir);
  FILE *f = fopen(path, "wb");
  if (!f || fwrite(host_o, 4, q * 128, f) != q * 128) return 2;
  fclose(f);
  printf("decode_files ok: %d sequences, %d heads, %d work items\n", B, H, (int)mla_plan_num_items(plan));
  mla_plan_destroy(plan);
  free(host_o);
  free(lens);
  return 0;
}
