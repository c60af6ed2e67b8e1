// Randomised check of the host planner (pg_pack_buffer_size / pg_pack_host),
// meant to run under AddressSanitizer: seeded random batches (empty prefixes,
// empty responses, one-row and multi-tile groups, several head layouts) are
// planned, and every descriptor is checked against what the batch alone
// fixes:
//   * the packed offsets and the baseline position ids (prefix row i -> i,
//     response row j -> P + j);
//   * the visibility rule: row_lo / row_hi of every row, and the pair counts
//     (grouped: P(P+1)/2 + sum_i (R_i P + R_i(R_i+1)/2) per group; baseline:
//     sum_i (P+R_i)(P+R_i+1)/2), recomputed by brute force over rows;
//   * the forward / dQ tiles cover every query row once, inside one group;
//   * the dK/dV work list covers every (key tile, query row) range once:
//     uncut tiles walk [k0, q_end), cut tiles' pieces are consecutive 32-row
//     aligned ranges whose parts are numbered consecutively;
//   * the scored entries (every response row but the first of a response in
//     an empty-prefix group) and their predicting rows.
// Invalid batches (a negative length, a group without responses, a bad head
// layout) must be refused with a message.  Prints "ok <planned> <refused>".
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <utility>
#include <random>
#include <vector>

#include "pg_attn.h"

#define CHECK(c, ...)                                   \
  do {                                                  \
    if (!(c)) {                                         \
      std::fprintf(stderr, "case %d: ", iter);          \
      std::fprintf(stderr, __VA_ARGS__);                \
      std::fprintf(stderr, " [%s]\n", #c);              \
      return 1;                                         \
    }                                                   \
  } while (0)

int main(int argc, char **argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 1000;
  std::mt19937 rng(20240611u);
  long planned = 0, refused = 0;
  for (int iter = 0; iter < iters; ++iter) {
    const int G = 1 + int(rng() % 5);
    const bool make_invalid = rng() % 25 == 0;
    std::vector<int32_t> P(G), NR(G), RL;
    for (int g = 0; g < G; ++g) {
      const int kind = int(rng() % 4);
      P[g] = kind == 0 ? 0 : kind == 1 ? 1 + int(rng() % 4) : int(rng() % (kind == 3 ? 2500 : 400));
      NR[g] = 1 + int(rng() % 24);
      for (int r = 0; r < NR[g]; ++r)
        RL.push_back(rng() % 6 == 0 ? 0 : int(rng() % (kind == 3 ? 1500 : 200)));
    }
    const int reps[] = {1, 2, 3, 4, 8};
    int hkv = 1 + int(rng() % 8), hq = hkv * reps[rng() % 5];
    const int d = rng() % 2 ? 64 : 128;
    int invalid_kind = -1;
    if (make_invalid) {
      invalid_kind = int(rng() % 3);
      if (invalid_kind == 0) RL[rng() % RL.size()] = -1 - int(rng() % 5);
      if (invalid_kind == 1) NR[rng() % G] = 0;
      if (invalid_kind == 2) hkv = hq + 1;  // more kv heads than query heads
    }
    // an invalid num_resp shortens the response list the planner reads
    pg_groups grp = {G, P.data(), NR.data(), RL.data(), hq, hkv, d};
    const size_t bytes = pg_pack_buffer_size(&grp);
    if (make_invalid) {
      CHECK(bytes == 0, "invalid batch (kind %d) was accepted", invalid_kind);
      CHECK(std::strlen(pg_last_error()) > 0, "refusal without a message");
      ++refused;
      continue;
    }
    CHECK(bytes > 0, "valid batch refused: %s", pg_last_error());

    // expected layout
    int64_t T = 0, pairs = 0, base_pairs = 0, scored = 0;
    std::vector<int32_t> gstart(G + 1), pend(G), lo, hi, pos;
    size_t ri = 0;
    for (int g = 0; g < G; ++g) {
      gstart[g] = int32_t(T);
      const int32_t p = P[g];
      for (int i = 0; i < p; ++i) {
        lo.push_back(int32_t(T));
        pos.push_back(i);
      }
      pend[g] = int32_t(T + p);
      pairs += int64_t(p) * (p + 1) / 2;
      int64_t t = T + p;
      std::vector<int32_t> rend;
      for (int r = 0; r < NR[g]; ++r) {
        const int32_t R = RL[ri++];
        for (int j = 0; j < R; ++j) {
          lo.push_back(int32_t(t));
          pos.push_back(p + j);
        }
        pairs += int64_t(R) * p + int64_t(R) * (R + 1) / 2;
        base_pairs += int64_t(p + R) * (p + R + 1) / 2;
        scored += R > 0 ? R - (p == 0 ? 1 : 0) : 0;
        t += R;
        rend.push_back(int32_t(t));
      }
      T = t;
      gstart[g + 1] = int32_t(T);
      for (int i = 0; i < p; ++i) hi.push_back(int32_t(T));
      int64_t u = pend[g];
      for (int r = 0; r < NR[g]; ++r)
        for (; u < rend[r]; ++u) hi.push_back(rend[r]);
    }

    std::vector<char> raw(bytes + 64);
    void *buf = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(raw.data()) + 15) & ~uintptr_t(15));
    std::vector<int32_t> got_pos(T > 0 ? T : 1, -7);
    pg_desc D;
    const pg_status st = pg_pack_host(&grp, buf, bytes, got_pos.data(), &D);
    CHECK(st == PG_OK, "pg_pack_host: %s", pg_last_error());
    ++planned;
    CHECK(D.total_rows == T, "total_rows %d vs %lld", D.total_rows, (long long)T);
    CHECK(D.pairs == pairs, "pairs %lld vs %lld", (long long)D.pairs, (long long)pairs);
    CHECK(D.baseline_pairs == base_pairs, "baseline pairs");
    CHECK(D.num_scored == scored, "scored %d vs %lld", D.num_scored, (long long)scored);
    for (int g = 0; g <= G; ++g) CHECK(D.group_start[g] == gstart[g], "group_start[%d]", g);
    for (int g = 0; g < G; ++g) CHECK(D.prefix_end[g] == pend[g], "prefix_end[%d]", g);
    int64_t vis = 0;
    for (int64_t q = 0; q < T; ++q) {
      CHECK(got_pos[q] == pos[q], "position id of row %lld", (long long)q);
      CHECK(D.row_lo[q] == lo[q], "row_lo[%lld]", (long long)q);
      CHECK(D.row_hi[q] == hi[q], "row_hi[%lld]", (long long)q);
      vis += hi[q] - q;  // key row q is seen by the query rows [q, row_hi)
    }
    CHECK(vis == pairs, "row_hi sums to %lld pairs, not %lld", (long long)vis, (long long)pairs);

    // forward / dQ tiles: every row once, inside one group
    std::vector<int> seen(T, 0);
    for (int i = 0; i < D.num_q_tiles; ++i) {
      const int32_t *t4 = D.q_tiles + 4 * i;
      CHECK(t4[0] < t4[1] && t4[1] - t4[0] <= PG_TILE_Q, "q tile %d size", i);
      CHECK(t4[2] <= t4[0] && t4[1] <= T, "q tile %d range", i);
      int g = 0;
      while (gstart[g + 1] <= t4[0]) ++g;
      CHECK(t4[2] == gstart[g] && t4[3] == pend[g] && t4[1] <= gstart[g + 1], "q tile %d group", i);
      for (int32_t q = t4[0]; q < t4[1]; ++q) ++seen[q];
    }
    for (int64_t q = 0; q < T; ++q) CHECK(seen[q] == 1, "row %lld in %d q tiles", (long long)q, seen[q]);

    // dK/dV work list: per key tile, whole walk or consecutive aligned pieces
    std::vector<int> kseen(T, 0);
    int32_t parts_seen = 0;
    for (int i = 0; i < D.num_kv_tiles; ++i) {
      const int32_t *t4 = D.kv_tiles + 4 * i;
      const int32_t k0 = t4[0], k1 = t4[1], qend = t4[2];
      CHECK(k0 < k1 && k1 - k0 <= PG_TILE_KV, "kv tile %d size", i);
      int32_t want = 0;
      for (int32_t k = k0; k < k1; ++k) {
        want = want > hi[k] ? want : hi[k];
        ++kseen[k];
      }
      CHECK(qend == want, "kv tile %d q_end %d vs %d", i, qend, want);
      std::vector<std::pair<int32_t, int32_t>> ranges;
      int32_t part_lo = 1 << 30, part_hi = -1, cut = 0;
      for (int j = 0; j < D.num_kv_items; ++j) {
        const int32_t *it = D.kv_items + 8 * j;
        if (it[0] != k0) continue;
        CHECK(it[1] == k1, "item %d key range", j);
        ranges.push_back({it[2], it[3]});
        if (it[4] >= 0) {
          ++cut;
          part_lo = part_lo < it[4] ? part_lo : it[4];
          part_hi = part_hi > it[4] ? part_hi : it[4];
          CHECK((it[2] - k0) % 32 == 0, "piece start not block aligned");
        }
      }
      CHECK(!ranges.empty(), "kv tile %d has no work item", i);
      std::sort(ranges.begin(), ranges.end());
      CHECK(ranges.front().first == k0 && ranges.back().second == qend, "kv tile %d walk ends", i);
      for (size_t j = 1; j < ranges.size(); ++j)
        CHECK(ranges[j].first == ranges[j - 1].second, "kv tile %d pieces not consecutive", i);
      if (ranges.size() > 1) {
        CHECK(cut == int(ranges.size()) && part_hi - part_lo + 1 == cut, "kv tile %d parts", i);
        bool found = false;
        for (int s = 0; s < D.num_kv_sums; ++s) {
          const int32_t *s4 = D.kv_sums + 4 * s;
          if (s4[0] == k0) found = s4[1] == k1 && s4[2] == part_lo && s4[3] == cut;
        }
        CHECK(found, "kv tile %d cut without a matching sum entry", i);
        parts_seen += cut;
      } else {
        CHECK(cut == 0, "uncut tile %d with a part index", i);
      }
    }
    CHECK(parts_seen == D.num_kv_parts, "parts %d vs %d", parts_seen, D.num_kv_parts);
    for (int64_t k = 0; k < T; ++k) CHECK(kseen[k] == 1, "key row %lld in %d kv tiles", (long long)k, kseen[k]);

    // scored entries: packed order, each predicted by the previous baseline position
    int32_t e = 0;
    for (int g = 0; g < G; ++g) {
      for (int64_t q = pend[g]; q < gstart[g + 1]; ++q) {
        const bool first = lo[q] == q;
        if (first && P[g] == 0) continue;
        CHECK(e < D.num_scored && D.scored_row[e] == q, "scored entry %d row", e);
        const int32_t pred = first ? pend[g] - 1 : int32_t(q - 1);
        CHECK(D.scored_pred[e] == pred, "scored entry %d predictor", e);
        ++e;
      }
    }
    CHECK(e == D.num_scored, "scored entries %d vs %d", e, D.num_scored);
  }
  std::printf("ok %ld %ld\n", planned, refused);
  return 0;
}
