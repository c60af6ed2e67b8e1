/* Plain-C client of libpg_attn: plans the tiny three-group batch of
 * tests/golden/grouped_visibility_tiny.txt with pg_pack_host (no GPU) and
 * prints what a caller derives from the descriptor, for the test to compare
 * with the hand-written fixture: the position ids, the pair counts and the
 * visibility matrix given by the descriptor's rule (query row q of group g
 * sees key rows [group start, min(prefix end, q + 1)) and [row_lo[q], q]).
 * Then one invalid description, which must fail with PG_ERR_INVALID_ARG and
 * a message.  Only C99 and the header: no C++ and no Python. */
#include <stdio.h>
#include <stdlib.h>

#include "pg_attn.h"

int main(void) {
  const int32_t prefix_len[3] = {3, 0, 1};
  const int32_t num_resp[3] = {3, 2, 2};
  const int32_t resp_len[7] = {2, 0, 1, 2, 1, 1, 1};
  pg_groups g = {3, prefix_len, num_resp, resp_len, 2, 1, 64};
  const size_t bytes = pg_pack_buffer_size(&g);
  if (bytes == 0) {
    fprintf(stderr, "pg_pack_buffer_size: %s\n", pg_last_error());
    return 1;
  }
  /* 16-byte aligned host buffer for the plan */
  void *buf = NULL;
  if (posix_memalign(&buf, 16, bytes) != 0) return 1;
  int32_t pos[64];
  pg_desc d;
  pg_status st = pg_pack_host(&g, buf, bytes, pos, &d);
  if (st != PG_OK) {
    fprintf(stderr, "pg_pack_host: %d %s\n", (int)st, pg_last_error());
    return 1;
  }
  const int T = d.total_rows;
  printf("version %s\n", pg_version());
  printf("rows %d\n", T);
  printf("positions:");
  for (int q = 0; q < T; ++q) printf(" %d", pos[q]);
  printf("\npairs: %lld %lld\nvisible:\n", (long long)d.pairs, (long long)d.baseline_pairs);
  for (int q = 0; q < T; ++q) {
    int gi = 0;
    while (q >= d.group_start[gi + 1]) ++gi;
    const int g0 = d.group_start[gi], pe = d.prefix_end[gi];
    for (int k = 0; k < T; ++k) {
      const int prefix_seen = k >= g0 && k < pe && k <= q;
      const int own_seen = k >= d.row_lo[q] && k <= q;
      putchar(prefix_seen || own_seen ? '1' : '0');
    }
    putchar('\n');
  }
  /* every key row k is seen by exactly the query rows [k, row_hi[k]) */
  printf("row_hi:");
  for (int k = 0; k < T; ++k) printf(" %d", d.row_hi[k]);
  printf("\n");

  const int32_t bad_prefix[1] = {-1};
  const int32_t one[1] = {1};
  pg_groups bad = {1, bad_prefix, one, one, 2, 1, 64};
  st = pg_pack_host(&bad, buf, bytes, pos, &d);
  printf("invalid: %d %s\n", (int)st, pg_last_error());
  free(buf);
  return st == PG_ERR_INVALID_ARG ? 0 : 2;
}
