/* A plain C11 caller of the libfva C ABI (include/fva.h): one pass of the
 * path, reorder -> route -> block-sparse attention -> inverse reorder, on
 * token-major bf16 Q, K, V read from a file.  Used by tests/test_c_consumer.py.
 *
 *   c_consumer IN OUT T H W bt bh bw B Hh d top_p topk
 *
 * IN holds Q, K, V as consecutive [B, N, Hh, d] bf16 arrays.  OUT receives the
 * attention output [B, N, Hh, d] bf16, then the row counts [rows] int32, then
 * the bitmask [rows, words] uint32.  Exit status 0 on success. */
#include <stdio.h>
#include <stdlib.h>

#include "fva.h"

#define CK(x)                                                            \
  do {                                                                   \
    hipError_t e_ = (x);                                                 \
    if (e_ != hipSuccess) {                                              \
      fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__);   \
      return 2;                                                          \
    }                                                                    \
  } while (0)
#define FV(x)                                                                            \
  do {                                                                                   \
    fva_status s_ = (x);                                                                 \
    if (s_ != FVA_OK) {                                                                  \
      fprintf(stderr, "%s: %s (line %d)\n", fva_status_string(s_), fva_last_error(), __LINE__); \
      return 3;                                                                          \
    }                                                                                    \
  } while (0)

static void* dev(size_t bytes) {
  void* p = NULL;
  return hipMalloc(&p, bytes ? bytes : 1) == hipSuccess ? p : NULL;
}

int main(int argc, char** argv) {
  if (argc != 14) {
    fprintf(stderr, "usage: c_consumer IN OUT T H W bt bh bw B Hh d top_p topk\n");
    return 1;
  }
  fva_grid g;
  g.T = atoi(argv[3]); g.H = atoi(argv[4]); g.W = atoi(argv[5]);
  g.bt = atoi(argv[6]); g.bh = atoi(argv[7]); g.bw = atoi(argv[8]);
  const int B = atoi(argv[9]), Hh = atoi(argv[10]), d = atoi(argv[11]);
  const float top_p = (float)atof(argv[12]);
  const int topk = atoi(argv[13]);

  fva_sizes_t sz;
  FV(fva_sizes(&g, B, Hh, d, &sz));
  const size_t tok = (size_t)B * sz.N * Hh * d * 2;  /* bytes of one token-major tensor */
  const size_t ro = (size_t)B * Hh * sz.Npad * d * 2;
  const size_t rows = (size_t)sz.rows;

  unsigned char* host = (unsigned char*)malloc(3 * tok);
  FILE* f = fopen(argv[1], "rb");
  if (!host || !f || fread(host, 1, 3 * tok, f) != 3 * tok) {
    fprintf(stderr, "cannot read %s\n", argv[1]);
    return 1;
  }
  fclose(f);

  void *q = dev(tok), *k = dev(tok), *v = dev(tok), *out = dev(tok);
  void *qr = dev(ro), *kr = dev(ro), *vt = dev(ro), *orr = dev(ro);
  void *route_ws = dev(sz.route_ws_bytes), *attn_ws = dev(sz.attn_ws_bytes);
  fva_mask m;
  m.scores = (float*)dev(rows * sz.nB * 4);
  m.bitmask = (uint32_t*)dev(rows * sz.words * 4);
  m.row_count = (int32_t*)dev(rows * 4);
  m.col_idx = (int16_t*)dev(rows * sz.nB * 2);
  m.head_count = (int32_t*)dev((size_t)B * Hh * 4);
  m.queue = (int32_t*)dev(rows * 4);
  if (!q || !k || !v || !out || !qr || !kr || !vt || !orr || !route_ws || !attn_ws ||
      !m.scores || !m.bitmask || !m.row_count || !m.col_idx || !m.head_count || !m.queue) {
    fprintf(stderr, "device allocation failed\n");
    return 2;
  }
  CK(hipMemcpy(q, host, tok, hipMemcpyHostToDevice));
  CK(hipMemcpy(k, host + tok, tok, hipMemcpyHostToDevice));
  CK(hipMemcpy(v, host + 2 * tok, tok, hipMemcpyHostToDevice));

  /* token-major [B, N, Hh, d] strides in elements: batch, token, head */
  const int64_t st[3] = {(int64_t)sz.N * Hh * d, (int64_t)Hh * d, (int64_t)d};
  FV(fva_reorder(q, qr, B, Hh, d, &g, st, FVA_FORWARD, FVA_LAYOUT_ROWS, NULL));
  FV(fva_reorder(k, kr, B, Hh, d, &g, st, FVA_FORWARD, FVA_LAYOUT_K64, NULL));
  FV(fva_reorder(v, vt, B, Hh, d, &g, st, FVA_FORWARD, FVA_LAYOUT_V64, NULL));
  fva_route_params prm;
  prm.top_p = top_p;
  prm.topk_floor = topk;
  prm.aug_budget = 0;
  prm.scale = 0.0f;
  prm.reserved = 0;
  FV(fva_route(qr, kr, B, Hh, d, &g, &prm, &m, route_ws, sz.route_ws_bytes, 0, NULL));
  FV(fva_sparse_attn(qr, kr, vt, orr, B, Hh, d, &g, &m, 0.0f, FVA_SCHED_XCD, attn_ws,
                     sz.attn_ws_bytes, NULL, NULL, NULL));
  FV(fva_reorder(orr, out, B, Hh, d, &g, st, FVA_INVERSE, FVA_LAYOUT_ROWS, NULL));
  CK(hipDeviceSynchronize());

  unsigned char* res = (unsigned char*)malloc(tok + rows * 4 + rows * sz.words * 4);
  if (!res) return 1;
  CK(hipMemcpy(res, out, tok, hipMemcpyDeviceToHost));
  CK(hipMemcpy(res + tok, m.row_count, rows * 4, hipMemcpyDeviceToHost));
  CK(hipMemcpy(res + tok + rows * 4, m.bitmask, rows * sz.words * 4, hipMemcpyDeviceToHost));
  f = fopen(argv[2], "wb");
  if (!f || fwrite(res, 1, tok + rows * 4 + rows * sz.words * 4, f) != tok + rows * 4 + rows * sz.words * 4) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(f);
  printf("c consumer: %lld rows, N %lld\n", (long long)sz.rows, (long long)sz.N);
  return 0;
}
