/*
 * ra_client -- one rank's ring-attention training step driven from plain C
 * through the C ABI of include/ra.h (no C++ or Python): the double-buffered
 * forward walk on a compute stream and a copy stream, then the backward walk.
 *
 *   ra_client IN OUT
 *
 * IN (little-endian): int32 B, H, H_kv, P, C, d, rank, causal; float32
 * scale; then bf16 q [B,H,C,d], the P key chunks [B,H_kv,C,d], the P value
 * chunks, dO [B,H,C,d].  OUT: float32 o [B,H,C,d], lse [B,H,C], dq
 * [B,H,C,d], the P dk chunks [B,H_kv,C,d], the P dv chunks.  Chunk j holds
 * global tokens [j*C, (j+1)*C).  Exit status 0 on success, 1 on any error
 * (reported on stderr with the library's message), 2 on bad usage.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ra.h"

#define MAX_CHUNKS 64

static int hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return 1;
  fprintf(stderr, "ra_client: %s: %s\n", what, hipGetErrorString(e));
  return 0;
}

static int ra_ok(int st, const char* what) {
  if (st == RA_OK) return 1;
  fprintf(stderr, "ra_client: %s: %s (%s)\n", what, ra_status_string(st), ra_last_error());
  return 0;
}

/* n bytes from f into a new device buffer. */
static void* upload(FILE* f, size_t n) {
  void* host = malloc(n);
  void* dev = NULL;
  if (!host || fread(host, 1, n, f) != n) {
    fprintf(stderr, "ra_client: short input file\n");
    free(host);
    return NULL;
  }
  if (!hip_ok(hipMalloc(&dev, n), "hipMalloc") || !hip_ok(hipMemcpy(dev, host, n, hipMemcpyHostToDevice), "upload"))
    dev = NULL;
  free(host);
  return dev;
}

/* n bytes of a device buffer appended to f. */
static int download(FILE* f, const void* dev, size_t n) {
  void* host = malloc(n);
  int ok = host && hip_ok(hipMemcpy(host, dev, n, hipMemcpyDeviceToHost), "download") && fwrite(host, 1, n, f) == n;
  free(host);
  return ok;
}

static void* zeroed(size_t n) {
  void* dev = NULL;
  if (!hip_ok(hipMalloc(&dev, n), "hipMalloc") || !hip_ok(hipMemset(dev, 0, n), "hipMemset")) return NULL;
  return dev;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: ra_client IN OUT (library version %d)\n", RA_VERSION);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    fprintf(stderr, "ra_client: cannot open %s\n", argv[1]);
    return 1;
  }
  int hdr[8];
  float scale;
  if (fread(hdr, sizeof(int), 8, in) != 8 || fread(&scale, sizeof(float), 1, in) != 1) {
    fprintf(stderr, "ra_client: short header\n");
    return 1;
  }
  const int B = hdr[0], H = hdr[1], H_kv = hdr[2], P = hdr[3], C = hdr[4], d = hdr[5], rank = hdr[6];
  const int causal = hdr[7];
  if (P < 1 || P > MAX_CHUNKS || B < 1 || H < 1 || H_kv < 1 || C < 1 || d < 1) {
    fprintf(stderr, "ra_client: bad header\n");
    return 1;
  }
  const size_t q_elems = (size_t)B * H * C * d, kv_elems = (size_t)B * H_kv * C * d, rows = (size_t)B * H * C;

  void* q = upload(in, q_elems * 2);
  const void* k[MAX_CHUNKS];
  const void* v[MAX_CHUNKS];
  float* dk[MAX_CHUNKS];
  float* dv[MAX_CHUNKS];
  int ok = q != NULL;
  for (int j = 0; ok && j < P; ++j) ok = (k[j] = upload(in, kv_elems * 2)) != NULL;
  for (int j = 0; ok && j < P; ++j) ok = (v[j] = upload(in, kv_elems * 2)) != NULL;
  void* dO = ok ? upload(in, q_elems * 2) : NULL;
  fclose(in);
  ok = ok && dO != NULL;

  float *o = NULL, *lse = NULL, *dq = NULL;
  ok = ok && hip_ok(hipMalloc((void**)&o, q_elems * 4), "hipMalloc") &&
       hip_ok(hipMalloc((void**)&lse, rows * 4), "hipMalloc") && hip_ok(hipMalloc((void**)&dq, q_elems * 4), "hipMalloc");
  /* The backward accumulates into dk/dv (+=): the caller zeroes them. */
  for (int j = 0; ok && j < P; ++j) ok = (dk[j] = zeroed(kv_elems * 4)) && (dv[j] = zeroed(kv_elems * 4));

  hipStream_t cs = NULL, xs = NULL;
  ok = ok && hip_ok(hipStreamCreate(&cs), "hipStreamCreate") && hip_ok(hipStreamCreate(&xs), "hipStreamCreate");

  const size_t ws_f_bytes = ra_ring_workspace_bytes_gqa(P, B, H, H_kv, C, d, RA_RING_DOUBLE_BUFFER, 0);
  const size_t ws_b_bytes = ra_ring_workspace_bytes_gqa(P, B, H, H_kv, C, d, RA_RING_RESIDENT, 1);
  void *ws_f = NULL, *ws_b = NULL;
  ok = ok && hip_ok(hipMalloc(&ws_f, ws_f_bytes), "hipMalloc") && hip_ok(hipMalloc(&ws_b, ws_b_bytes), "hipMalloc");

  ok = ok && ra_ok(ra_ring_fwd_gqa(q, k, v, P, o, lse, rank, causal, scale, B, H, H_kv, C, d,
                                   RA_RING_DOUBLE_BUFFER, ws_f, ws_f_bytes, cs, xs),
                   "ra_ring_fwd_gqa");
  ok = ok && ra_ok(ra_ring_bwd_gqa(q, k, v, P, o, lse, dO, dq, dk, dv, rank, causal, scale, B, H, H_kv, C, d, ws_b,
                                   ws_b_bytes, cs),
                   "ra_ring_bwd_gqa");
  ok = ok && hip_ok(hipStreamSynchronize(cs), "hipStreamSynchronize");

  FILE* out = ok ? fopen(argv[2], "wb") : NULL;
  if (ok && !out) fprintf(stderr, "ra_client: cannot open %s\n", argv[2]);
  ok = ok && out && download(out, o, q_elems * 4) && download(out, lse, rows * 4) && download(out, dq, q_elems * 4);
  for (int j = 0; ok && j < P; ++j) ok = download(out, dk[j], kv_elems * 4);
  for (int j = 0; ok && j < P; ++j) ok = download(out, dv[j], kv_elems * 4);
  if (out && fclose(out) != 0) ok = 0;
  return ok ? 0 : 1;
}
