/* A plain C99 consumer of include/segattn.h.  It calls only host-side entry
 * points and error paths that return before any device work, so it runs
 * without a GPU.  Each line it prints is "<name>: <values>" for the test to
 * compare with the Python side. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "segattn.h"

static void print_i64(const char *name, const int64_t *x, int n) {
  int i;
  printf("%s:", name);
  for (i = 0; i < n; ++i) printf(" %lld", (long long)x[i]);
  printf("\n");
}

int main(void) {
  int64_t bounds[5];
  int64_t cu[4] = {0, 5000, 5001, 45001};
  segattn_item items[16];
  int32_t n = 0, st;
  int64_t rows[3] = {3765, 3765, 2116};
  int64_t row_bytes[3] = {16512, 16512, 16512};
  double alpha[3], mem[3], peak = 0.0;
  int64_t moved[3];
  segattn_shape shape;
  size_t ws = 0;
  int i;

  printf("version: %s\n", segattn_version());

  st = segattn_partition(1024, 4, bounds);
  printf("partition_status: %d\n", st);
  print_i64("partition", bounds, 5);

  /* capacity query, then the call */
  st = segattn_partition_varlen(cu, 3, 16384, NULL, 0, &n);
  printf("varlen_query: %d %d\n", st, n);
  st = segattn_partition_varlen(cu, 3, 16384, items, 16, &n);
  printf("varlen_status: %d %d\n", st, n);
  for (i = 0; i < n; ++i) print_i64("varlen_item", &items[i].seq_off, 5);

  {
    int64_t b[3] = {0, 512, 1024};
    st = segattn_ring_items(b, 2, 256, items, 16, &n);
    printf("ring_status: %d %d\n", st, n);
    for (i = 0; i < n; ++i) print_i64("ring_item", &items[i].seq_off, 5);
  }

  st = segattn_offload_plan(rows, row_bytes, 3, 30000000.0, alpha, moved, mem, &peak);
  printf("offload_status: %d\n", st);
  printf("offload_alpha: %.17g %.17g %.17g\n", alpha[0], alpha[1], alpha[2]);
  print_i64("offload_moved", moved, 3);
  printf("offload_peak: %.17g\n", peak);

  /* error paths: no shape; a valid call with too small a workspace */
  st = segattn_fwd(NULL, NULL, NULL, NULL, NULL, 0, NULL, SEGATTN_BF16, NULL, 0u, NULL, 0, NULL);
  printf("fwd_null_shape: %d %s | %s\n", st, segattn_status_string(st), segattn_last_error());
  memset(&shape, 0, sizeof shape);
  shape.tokens = 1024;
  shape.hq = 4;
  shape.hkv = 2;
  shape.d = 128;
  shape.in_dtype = SEGATTN_BF16;
  shape.scale = 0.08838834764831845f;
  {
    segattn_item one;
    static char fake[64] __attribute__((aligned(16)));
    one.seq_off = 0;
    one.q_lo = 0;
    one.q_hi = 1024;
    one.k_lo = 0;
    one.k_hi = 1024;
    st = segattn_fwd_workspace(&shape, &one, 1, &ws);
    printf("fwd_workspace: %d %s\n", st, ws > 0 ? "positive" : "zero");
    st = segattn_fwd(&shape, fake, fake, fake, &one, 1, fake, SEGATTN_F32, (float *)fake, 0u, fake, 16, NULL);
    printf("fwd_small_workspace: %d %s\n", st, segattn_status_string(st));
  }
  return 0;
}
