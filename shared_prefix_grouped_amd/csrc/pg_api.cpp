// Host side of libpg_attn: argument validation, the packed-batch planner
// (pg_pack) and kernel launches.  See include/pg_attn.h for the contract.
//
// The planner turns per-group lengths into the packed row layout
// [P; R_1; ...; R_G] (skillsmp.com "prefix-grouper-grpo", "Step 3: Restructure
// Input Format", here without padding) and into per-row visibility bounds:
// query row q sees key rows [group start, prefix end) and [row_lo[q], q]
// (Pith review of Prefix Grouper, "What carries the argument": a response
// token sees the whole prefix and its own response up to itself).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <map>
#include <mutex>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "pg_attn.h"
#include "pg_internal.h"

namespace {

thread_local std::string g_last_error;

pg_status fail(pg_status st, const std::string &msg) {
  g_last_error = msg;
  return st;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

// Byte offsets of each array inside the descriptor buffer.
struct Layout {
  size_t row_lo, row_hi, q_tiles, kv_tiles, kv_items, kv_sums, group_start, prefix_end,
      prefix_before, resp_start, resp_len, resp_group, scored_row, scored_pred, scored_resp,
      pred_start, pred_list, total;
};

Layout make_layout(int64_t T, int64_t n_groups, int64_t n_resp, int64_t n_qt, int64_t n_kvt,
                   int64_t n_items, int64_t n_sums, int64_t n_scored) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t &field, int64_t n_int32) {
    field = off;
    off = align16(off + size_t(n_int32) * 4);
  };
  take(L.row_lo, T);
  take(L.row_hi, T);
  take(L.q_tiles, 4 * n_qt);
  take(L.kv_tiles, 4 * n_kvt);
  take(L.kv_items, 8 * n_items);
  take(L.kv_sums, 4 * n_sums);
  take(L.group_start, n_groups + 1);
  take(L.prefix_end, n_groups);
  take(L.prefix_before, n_groups + 1);
  take(L.resp_start, n_resp);
  take(L.resp_len, n_resp);
  take(L.resp_group, n_resp);
  take(L.scored_row, n_scored);
  take(L.scored_pred, n_scored);
  take(L.scored_resp, n_scored);
  take(L.pred_start, T + 1);
  take(L.pred_list, n_scored);
  L.total = std::max<size_t>(off, 16);
  return L;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Validate a pg_groups and compute the total row count.
pg_status check_groups(const pg_groups *g, int64_t *T_out, int64_t *n_resp_out) {
  if (!g) return fail(PG_ERR_INVALID_ARG, "pg_groups is NULL");
  if (g->num_groups < 0) return fail(PG_ERR_INVALID_ARG, "num_groups < 0");
  if (g->num_groups > 0 && (!g->prefix_len || !g->num_resp || !g->resp_len))
    return fail(PG_ERR_INVALID_ARG, "prefix_len, num_resp and resp_len must not be NULL");
  if (g->num_q_heads <= 0 || g->num_kv_heads <= 0)
    return fail(PG_ERR_INVALID_ARG, "head counts must be positive");
  if (g->num_q_heads % g->num_kv_heads)
    return fail(PG_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (g->head_dim != 64 && g->head_dim != 128)
    return fail(PG_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  int64_t T = 0, n_resp = 0;
  for (int32_t i = 0; i < g->num_groups; ++i) {
    if (g->prefix_len[i] < 0) return fail(PG_ERR_INVALID_ARG, "prefix_len < 0 in group " + std::to_string(i));
    if (g->num_resp[i] < 1) return fail(PG_ERR_INVALID_ARG, "num_resp < 1 in group " + std::to_string(i));
    int64_t rows = g->prefix_len[i];
    for (int32_t r = 0; r < g->num_resp[i]; ++r) {
      int32_t len = g->resp_len[n_resp + r];
      if (len < 0) return fail(PG_ERR_INVALID_ARG, "resp_len < 0 in group " + std::to_string(i));
      rows += len;
    }
    n_resp += g->num_resp[i];
    T += rows;
    if (T > INT32_MAX / 2) return fail(PG_ERR_INVALID_ARG, "total rows exceed the int32 range");
  }
  if (T * int64_t(g->num_q_heads) * g->head_dim > (int64_t(1) << 40))
    return fail(PG_ERR_INVALID_ARG, "tensor too large");
  *T_out = T;
  *n_resp_out = n_resp;
  return PG_OK;
}

struct Tile {
  int32_t a, b, c, d;
  int64_t cost;
  int64_t order;
};

// One dK/dV work item: key rows [k0, k1) against query rows [qa, qb).
struct KvItem {
  int32_t k0, k1, qa, qb, part;
  int64_t cost;
  int64_t order;
};

// Splitting of long dK/dV walks.  A key tile is seen by every query row from
// its own rows to the end of its visibility range; for a prefix tile that is
// the rest of the prefix and every response of the group, so a short prefix
// with many responses leaves a few key tiles with nearly all the work.  Such a
// tile is cut into pieces of whole 32-row query blocks, each its own
// workgroup, whose float partial sums a second kernel adds in piece order.
// A tile is cut when its work exceeds the mean per workgroup slot (one dK/dV
// workgroup is resident per compute unit; an MI355X has 256), into pieces of
// at least kMinPieceSteps (query head, 32-row block) steps so that the fixed
// cost of a piece (its K/V rows, pipeline fill, partial write and re-read)
// stays small beside its walk.
constexpr int64_t kDkdvSlots = 256;
constexpr int kMinPieceSteps = 32;
constexpr int kQueryBlock = 32;

// The complete plan in host memory, before it is laid out in one buffer.
struct HostPlan {
  int64_t T = 0, n_resp = 0, pairs = 0, base_pairs = 0;
  int32_t n_parts = 0, max_walk = 0;
  std::vector<int32_t> row_lo, row_hi, pos, gstart, pend, pbefore, rstart, rlen, rgroup;
  // scored response rows (log-probability head): target row, predicting row,
  // response index; and per packed row the scored entries it predicts (CSR)
  std::vector<int32_t> sc_row, sc_pred, sc_resp, pred_start, pred_list;
  std::vector<Tile> qt, kvt;
  std::vector<KvItem> items;
  std::vector<int32_t> sums;  // 4 per split tile
};

pg_status plan_batch(const pg_groups *g, HostPlan &hp) {
  pg_status st = check_groups(g, &hp.T, &hp.n_resp);
  if (st != PG_OK) return st;
  const int64_t T = hp.T;
  hp.row_lo.assign(T, 0);
  hp.row_hi.assign(T, 0);
  hp.pos.assign(T, 0);
  hp.gstart.assign(g->num_groups + 1, 0);
  hp.pend.assign(g->num_groups, 0);
  hp.pbefore.assign(g->num_groups + 1, 0);
  hp.rstart.assign(hp.n_resp, 0);
  hp.rlen.assign(hp.n_resp, 0);
  hp.rgroup.assign(hp.n_resp, 0);
  int32_t *row_lo = hp.row_lo.data(), *row_hi = hp.row_hi.data();
  std::vector<Tile> &qt = hp.qt, &kvt = hp.kvt;
  int32_t t = 0, ri = 0;
  for (int32_t gi = 0; gi < g->num_groups; ++gi) {
    const int32_t P = g->prefix_len[gi];
    const int32_t g0 = t, pe = t + P;
    hp.gstart[gi] = g0;
    hp.pend[gi] = pe;
    hp.pbefore[gi + 1] = hp.pbefore[gi] + P;
    int32_t gend = pe;
    for (int32_t r = 0; r < g->num_resp[gi]; ++r) gend += g->resp_len[ri + r];
    // prefix rows: own segment is the prefix itself; seen by every later row of the group
    for (int32_t x = g0; x < pe; ++x) {
      row_lo[x] = g0;
      row_hi[x] = gend;
      hp.pos[x] = x - g0;
    }
    hp.pairs += int64_t(P) * (P + 1) / 2;
    int32_t s = pe;
    for (int32_t r = 0; r < g->num_resp[gi]; ++r, ++ri) {
      const int32_t R = g->resp_len[ri];
      hp.rstart[ri] = s;
      hp.rlen[ri] = R;
      hp.rgroup[ri] = gi;
      for (int32_t x = s; x < s + R; ++x) {
        row_lo[x] = s;
        row_hi[x] = s + R;
        hp.pos[x] = P + (x - s);
        // the token at baseline position P + j is scored by position P + j - 1:
        // the previous response row, or for j = 0 the group's last prefix row
        if (x > s || P > 0) {
          hp.sc_row.push_back(x);
          hp.sc_pred.push_back(x > s ? x - 1 : pe - 1);
          hp.sc_resp.push_back(ri);
        }
      }
      hp.pairs += int64_t(R) * P + int64_t(R) * (R + 1) / 2;
      const int64_t Lb = int64_t(P) + R;
      hp.base_pairs += Lb * (Lb + 1) / 2;
      s += R;
    }
    // query tiles, ordered by run time: the K/V chunks the forward / dQ work
    // item streams (prefix keys up to the tile's end, then the keys from its
    // first row's response start), its waves running side by side; ties by
    // the visible keys summed over the tile's rows.  (Ordered by visible keys
    // alone, a short tile at a group's end -- few rows, but every prefix
    // chunk -- would start last and run alone at the end of the launch.)
    for (int32_t q0 = g0; q0 < gend; q0 += PG_TILE_Q) {
      const int32_t q1 = std::min(gend, q0 + PG_TILE_Q);
      int64_t keys = 0;
      for (int32_t x = q0; x < q1; ++x)
        keys += (x < pe) ? (x - g0 + 1) : (int64_t(P) + (x - row_lo[x] + 1));
      const int64_t a_rows = std::min(pe, q1) - g0;
      const int64_t b_rows = q1 - std::max(pe, row_lo[q0]);
      const int64_t chunks = (a_rows > 0 ? ceil_div(a_rows, pg::kKvChunk) : 0) +
                             (b_rows > 0 ? ceil_div(b_rows, pg::kKvChunk) : 0);
      // chunks first: keys <= PG_TILE_Q * T < 2^37 and chunks < 2^25 (T < 2^30)
      qt.push_back({q0, q1, g0, pe, (chunks << 37) + keys, int64_t(qt.size())});
    }
    // key tiles: cost = number of query rows seeing each key, summed
    for (int32_t k0 = g0; k0 < gend; k0 += PG_TILE_KV) {
      const int32_t k1 = std::min(gend, k0 + PG_TILE_KV);
      int64_t cost = 0;
      int32_t qend = 0;
      for (int32_t x = k0; x < k1; ++x) {
        cost += row_hi[x] - x;
        qend = std::max(qend, row_hi[x]);
      }
      kvt.push_back({k0, k1, qend, pe, cost, int64_t(kvt.size())});
    }
    t = gend;
  }
  hp.gstart[g->num_groups] = t;
  // predicting row -> scored entries, in entry order
  hp.pred_start.assign(T + 1, 0);
  for (int32_t p : hp.sc_pred) ++hp.pred_start[p + 1];
  for (int64_t x = 0; x < T; ++x) hp.pred_start[x + 1] += hp.pred_start[x];
  hp.pred_list.assign(hp.sc_pred.size(), 0);
  {
    std::vector<int32_t> fill(hp.pred_start.begin(), hp.pred_start.end() - (T > 0 ? 1 : 0));
    for (size_t k = 0; k < hp.sc_pred.size(); ++k) hp.pred_list[fill[hp.sc_pred[k]]++] = int32_t(k);
  }

  // dK/dV work items (packed order), cutting the tiles whose walk is too long
  int64_t total = 0;
  for (const Tile &k : kvt) total += k.cost;
  const int rep = g->num_q_heads / g->num_kv_heads;
  const int64_t cap = std::max<int64_t>(1, ceil_div(total * g->num_kv_heads, kDkdvSlots));
  const int64_t min_blocks = ceil_div(kMinPieceSteps, rep);
  for (const Tile &k : kvt) {
    const int32_t k0 = k.a, k1 = k.b, qend = k.c;
    const int64_t nblk = ceil_div(qend - k0, kQueryBlock);
    int64_t pieces = 1;
    if (k.cost > cap) pieces = std::max<int64_t>(1, std::min(ceil_div(k.cost, cap), nblk / min_blocks));
    if (pieces == 1) {
      hp.items.push_back({k0, k1, k0, qend, -1, k.cost, 0});
      continue;
    }
    hp.sums.insert(hp.sums.end(), {k0, k1, hp.n_parts, int32_t(pieces)});
    for (int64_t j = 0; j < pieces; ++j) {
      const int32_t qa = k0 + int32_t(j * nblk / pieces) * kQueryBlock;
      const int32_t qb = (j + 1 == pieces) ? qend : k0 + int32_t((j + 1) * nblk / pieces) * kQueryBlock;
      int64_t cost = 0;  // pairs of the piece: key x is seen by queries [x, row_hi[x])
      for (int32_t x = k0; x < k1; ++x)
        cost += std::max<int64_t>(0, int64_t(std::min(row_hi[x], qb)) - std::max(x, qa));
      hp.items.push_back({k0, k1, qa, qb, hp.n_parts++, cost, 0});
    }
  }
  for (size_t i = 0; i < hp.items.size(); ++i) {
    hp.items[i].order = int64_t(i);
    hp.max_walk = std::max(hp.max_walk, hp.items[i].qb - hp.items[i].qa);
  }
  // A dK/dV work item runs one barrier step per (query head, 32-row block) of
  // its walk, so it is ordered by its block count first, then by its pairs
  // (blocks < 2^25 and pairs <= PG_TILE_KV * T < 2^37 for T < 2^30).
  for (KvItem &it : hp.items)
    it.cost = (ceil_div(it.qb - it.qa, kQueryBlock) << 37) + it.cost;

  // longest-processing-time-first order; ties keep packed order
  auto by_cost = [](const auto &x, const auto &y) {
    return x.cost != y.cost ? x.cost > y.cost : x.order < y.order;
  };
  std::sort(qt.begin(), qt.end(), by_cost);
  std::sort(kvt.begin(), kvt.end(), by_cost);
  std::sort(hp.items.begin(), hp.items.end(), by_cost);
  return PG_OK;
}

Layout layout_of(const pg_groups *g, const HostPlan &hp) {
  return make_layout(hp.T, g->num_groups, hp.n_resp, int64_t(hp.qt.size()), int64_t(hp.kvt.size()),
                     int64_t(hp.items.size()), int64_t(hp.sums.size() / 4),
                     int64_t(hp.sc_row.size()));
}

// Lay the plan out in `buf` (host memory of at least L.total bytes).
void serialize(const pg_groups *g, const HostPlan &hp, const Layout &L, char *buf,
               int32_t *pos_ids, pg_desc *out) {
  std::memset(buf, 0, L.total);
  auto put = [&](size_t off, const std::vector<int32_t> &v) {
    if (!v.empty()) std::memcpy(buf + off, v.data(), v.size() * 4);
  };
  put(L.row_lo, hp.row_lo);
  put(L.row_hi, hp.row_hi);
  put(L.kv_sums, hp.sums);
  put(L.group_start, hp.gstart);
  put(L.prefix_end, hp.pend);
  put(L.prefix_before, hp.pbefore);
  put(L.resp_start, hp.rstart);
  put(L.resp_len, hp.rlen);
  put(L.resp_group, hp.rgroup);
  put(L.scored_row, hp.sc_row);
  put(L.scored_pred, hp.sc_pred);
  put(L.scored_resp, hp.sc_resp);
  put(L.pred_start, hp.pred_start);
  put(L.pred_list, hp.pred_list);
  if (pos_ids && hp.T > 0) std::memcpy(pos_ids, hp.pos.data(), size_t(hp.T) * 4);
  auto arr = [&](size_t off) { return reinterpret_cast<int32_t *>(buf + off); };
  int32_t *qa = arr(L.q_tiles), *ka = arr(L.kv_tiles), *ia = arr(L.kv_items);
  for (size_t i = 0; i < hp.qt.size(); ++i) {
    const Tile &x = hp.qt[i];
    qa[4 * i + 0] = x.a;
    qa[4 * i + 1] = x.b;
    qa[4 * i + 2] = x.c;
    qa[4 * i + 3] = x.d;
  }
  for (size_t i = 0; i < hp.kvt.size(); ++i) {
    const Tile &x = hp.kvt[i];
    ka[4 * i + 0] = x.a;
    ka[4 * i + 1] = x.b;
    ka[4 * i + 2] = x.c;
    ka[4 * i + 3] = x.d;
  }
  for (size_t i = 0; i < hp.items.size(); ++i) {
    const KvItem &x = hp.items[i];
    int32_t *e = ia + 8 * i;
    e[0] = x.k0;
    e[1] = x.k1;
    e[2] = x.qa;
    e[3] = x.qb;
    e[4] = x.part;
  }
  pg_desc d{};
  d.num_groups = g->num_groups;
  d.num_resp = int32_t(hp.n_resp);
  d.total_rows = int32_t(hp.T);
  d.num_q_heads = g->num_q_heads;
  d.num_kv_heads = g->num_kv_heads;
  d.head_dim = g->head_dim;
  d.num_q_tiles = int32_t(hp.qt.size());
  d.num_kv_tiles = int32_t(hp.kvt.size());
  d.num_kv_items = int32_t(hp.items.size());
  d.num_kv_sums = int32_t(hp.sums.size() / 4);
  d.num_kv_parts = hp.n_parts;
  d.total_prefix_rows = hp.pbefore[g->num_groups];
  d.num_scored = int32_t(hp.sc_row.size());
  d.max_walk_rows = hp.max_walk;
  d.pairs = hp.pairs;
  d.baseline_pairs = hp.base_pairs;
  d.buf_bytes = L.total;
  *out = d;
}

void point_into(pg_desc *d, const Layout &L, const char *base) {
  auto p = [&](size_t off) { return reinterpret_cast<const int32_t *>(base + off); };
  d->row_lo = p(L.row_lo);
  d->row_hi = p(L.row_hi);
  d->q_tiles = p(L.q_tiles);
  d->kv_tiles = p(L.kv_tiles);
  d->kv_items = p(L.kv_items);
  d->kv_sums = p(L.kv_sums);
  d->group_start = p(L.group_start);
  d->prefix_end = p(L.prefix_end);
  d->prefix_before = p(L.prefix_before);
  d->resp_start = p(L.resp_start);
  d->resp_len = p(L.resp_len);
  d->resp_group = p(L.resp_group);
  d->scored_row = p(L.scored_row);
  d->scored_pred = p(L.scored_pred);
  d->scored_resp = p(L.scored_resp);
  d->pred_start = p(L.pred_start);
  d->pred_list = p(L.pred_list);
}

pg_status check_desc(const pg_desc *d) {
  if (!d) return fail(PG_ERR_INVALID_ARG, "pg_desc is NULL");
  if (d->total_rows < 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 ||
      d->num_q_heads % d->num_kv_heads || d->num_q_tiles < 0 || d->num_kv_tiles < 0 ||
      d->num_kv_items < 0 || d->num_kv_sums < 0 || d->num_kv_parts < 0)
    return fail(PG_ERR_INVALID_ARG, "descriptor is not one filled by pg_pack");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(PG_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (d->total_rows > 0 &&
      (!d->row_lo || !d->row_hi || !d->q_tiles || !d->kv_tiles || !d->kv_items || !d->kv_sums))
    return fail(PG_ERR_INVALID_ARG, "descriptor arrays are NULL");
  return PG_OK;
}

pg_status check_dtype(pg_dtype t) {
  if (t != PG_F32 && t != PG_BF16) return fail(PG_ERR_UNSUPPORTED, "dtype must be PG_F32 or PG_BF16");
  return PG_OK;
}

pg_status check_ptrs(std::initializer_list<std::pair<const void *, const char *>> ptrs) {
  for (auto &pr : ptrs) {
    if (!pr.first) return fail(PG_ERR_INVALID_ARG, std::string(pr.second) + " is NULL");
    if (!aligned16(pr.first))
      return fail(PG_ERR_INVALID_ARG, std::string(pr.second) + " is not 16-byte aligned");
  }
  return PG_OK;
}

pg::Plan plan_of(const pg_desc *d) {
  pg::Plan p;
  p.T = d->total_rows;
  p.Hq = d->num_q_heads;
  p.Hkv = d->num_kv_heads;
  p.D = d->head_dim;
  p.n_q_tiles = d->num_q_tiles;
  p.n_kv_tiles = d->num_kv_tiles;
  p.row_lo = d->row_lo;
  p.row_hi = d->row_hi;
  p.q_tiles = d->q_tiles;
  p.kv_tiles = d->kv_tiles;
  p.n_kv_items = d->num_kv_items;
  p.n_kv_sums = d->num_kv_sums;
  p.n_kv_parts = d->num_kv_parts;
  p.kv_items = d->kv_items;
  p.kv_sums = d->kv_sums;
  p.n_groups = d->num_groups;
  p.group_start = d->group_start;
  p.prefix_end = d->prefix_end;
  p.prefix_before = d->prefix_before;
  return p;
}

pg_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return PG_OK;
  return fail(PG_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

float resolve_scale(float s, int D) { return s > 0.f ? s : 1.0f / std::sqrt(float(D)); }

// ---------------------------------------------------------------- kernel timing
const char *const kKernelNames[PG_KERNEL_COUNT] = {
    "fwd", "bwd_pre", "bwd_dkdv", "bwd_dq", "rope", "rows", "head_fwd", "head_bwd", "grpo_loss"};

struct TimedLaunch {
  int id;
  hipEvent_t start, stop;
};

struct Timing {
  std::mutex mu;
  bool enabled = false;
  std::vector<TimedLaunch> pending;
  std::vector<hipEvent_t> pool;
  int64_t launches[PG_KERNEL_COUNT] = {};
  double total_ms[PG_KERNEL_COUNT] = {};
  // first error met by a non-waiting drain inside a launch, reported by the
  // next timing query (the launch that triggered the drain is not at fault)
  hipError_t deferred = hipSuccess;
};

Timing &timing() {
  static Timing t;
  return t;
}

hipEvent_t take_event(Timing &t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Folds finished launches into the totals; waits for them if `wait`.
hipError_t drain(Timing &t, bool wait) {
  hipError_t err = hipSuccess;
  std::vector<TimedLaunch> keep;
  for (auto &l : t.pending) {
    hipError_t q = wait ? hipEventSynchronize(l.stop) : hipEventQuery(l.stop);
    if (q == hipErrorNotReady) {
      keep.push_back(l);
      continue;
    }
    float ms = 0.f;
    if (q == hipSuccess) q = hipEventElapsedTime(&ms, l.start, l.stop);
    if (q != hipSuccess && err == hipSuccess) err = q;
    t.launches[l.id] += 1;
    t.total_ms[l.id] += ms;
    t.pool.push_back(l.start);
    t.pool.push_back(l.stop);
  }
  t.pending.swap(keep);
  return err;
}

// Runs `launch` on stream s, bracketed by events when timing is enabled.
template <typename F>
hipError_t timed(int id, hipStream_t s, F &&launch) {
  Timing &t = timing();
  std::unique_lock<std::mutex> lock(t.mu);
  if (!t.enabled) {
    lock.unlock();
    return launch();
  }
  hipEvent_t a = take_event(t), b = take_event(t);
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, s);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(b, s);
  if (e != hipSuccess) {
    t.pool.push_back(a);
    t.pool.push_back(b);
    return e;
  }
  t.pending.push_back({id, a, b});
  if (t.pending.size() > 4096) {
    const hipError_t q = drain(t, false);
    if (q != hipSuccess && t.deferred == hipSuccess) t.deferred = q;
  }
  return hipSuccess;
}

// Shared checks of pg_pack_rows / pg_unpack_rows; the prefix (response)
// buffer may be NULL when the batch has no prefix (response) rows.
pg_status check_rows(const pg_desc *d, const void *packed, const void *pre, const void *resp,
                     size_t row_bytes) {
  pg_status st = check_desc(d);
  if (st != PG_OK) return st;
  if (row_bytes == 0 || row_bytes % 4)
    return fail(PG_ERR_INVALID_ARG, "row_bytes must be a positive multiple of 4");
  if (d->num_groups > 0 && (!d->group_start || !d->prefix_end || !d->prefix_before))
    return fail(PG_ERR_INVALID_ARG, "descriptor arrays are NULL");
  if (d->total_rows == 0) return PG_OK;
  if (size_t(d->total_rows) * row_bytes / row_bytes != size_t(d->total_rows) ||
      size_t(d->total_rows) * row_bytes > (size_t(1) << 46))
    return fail(PG_ERR_INVALID_ARG, "rows too large");
  const size_t align = row_bytes % 16 == 0 ? 16 : 4;
  auto ok = [&](const void *ptr, const char *name, bool needed) -> pg_status {
    if (!needed) return PG_OK;
    if (!ptr) return fail(PG_ERR_INVALID_ARG, std::string(name) + " is NULL");
    if (reinterpret_cast<uintptr_t>(ptr) % align)
      return fail(PG_ERR_INVALID_ARG, std::string(name) + " is not " + std::to_string(align) +
                                          "-byte aligned");
    return PG_OK;
  };
  const bool any_prefix = d->total_prefix_rows > 0, any_resp = d->total_rows > d->total_prefix_rows;
  if ((st = ok(packed, "packed_rows", true)) != PG_OK) return st;
  if ((st = ok(pre, "prefix_rows", any_prefix)) != PG_OK) return st;
  return ok(resp, "resp_rows", any_resp);
}

pg_status rows_call(const pg_desc *d, bool pack, void *packed, void *pre, void *resp,
                    size_t row_bytes, void *stream) {
  pg_status st = check_rows(d, packed, pre, resp, row_bytes);
  if (st != PG_OK || d->total_rows == 0) return st;
  pg::Plan p = plan_of(d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(timed(PG_KERNEL_ROWS, s,
                          [&] { return pg::launch_rows(p, pack, packed, pre, resp, row_bytes, s); }),
                    pack ? "pg_pack_rows launch" : "pg_unpack_rows launch");
}

// ---------------------------------------------------------------- log-prob head
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace of the head: the gradient of the loss with respect to the logits
// as G [n, V64] and G^T [V, n64] bf16 (V64, n64: rounded up to multiples of
// 64, so that rows start on 128-byte lines), H_pred [n, dm] and H_pred^T
// [dm, n64] bf16, W^T [dm, V64] bf16, dH_pred [n, dm] fp32, and the forward's
// per-vocab-tile row max and sum ([nvt, n] fp32 each).  The logits
// themselves are never stored.
struct HeadWs {
  size_t g, gt, hp, hpt, wt, dhp, pm, ps, total;
};
HeadWs head_ws(int64_t n, int64_t V, int64_t dm) {
  HeadWs w{};
  const size_t nvt = size_t(pg::head_vocab_tiles(int(V)));
  const size_t n64 = size_t(pg::round64(int(n))), V64 = size_t(pg::round64(int(V)));
  w.g = 0;
  w.gt = align256(w.g + size_t(n) * V64 * 2);
  w.hp = align256(w.gt + size_t(V) * n64 * 2);
  w.hpt = align256(w.hp + size_t(n) * dm * 2);
  w.wt = align256(w.hpt + size_t(dm) * n64 * 2);
  w.dhp = align256(w.wt + size_t(dm) * V64 * 2);
  w.pm = align256(w.dhp + size_t(n) * dm * 4);
  w.ps = align256(w.pm + nvt * size_t(n) * 4);
  w.total = std::max<size_t>(256, align256(w.ps + nvt * size_t(n) * 4));
  return w;
}

pg_status check_head(const pg_desc *d, int32_t vocab, int32_t d_model) {
  pg_status st = check_desc(d);
  if (st != PG_OK) return st;
  if (vocab < 1 || d_model < 8 || d_model % 8)
    return fail(PG_ERR_INVALID_ARG, "vocab must be >= 1 and d_model a positive multiple of 8");
  // the tile kernels address each operand with 32-bit byte offsets: W,
  // H_pred and the logit gradient G (and their transposes) must each be
  // under 4 GiB
  const int64_t n64 = (int64_t(d->num_scored) + 63) & ~int64_t(63);
  const int64_t V64 = (int64_t(vocab) + 63) & ~int64_t(63);
  const int64_t lim = int64_t(1) << 32;
  if (V64 * d_model * 2 >= lim || n64 * d_model * 2 >= lim || n64 * V64 * 2 >= lim)
    return fail(PG_ERR_UNSUPPORTED,
                "weight, scored hidden rows and their logit gradient must each be under 4 GiB");
  if (d->num_scored < 0 || d->num_resp < 0)
    return fail(PG_ERR_INVALID_ARG, "descriptor is not one filled by pg_pack");
  if (d->num_scored > 0 && (!d->scored_row || !d->scored_pred || !d->scored_resp ||
                            !d->pred_start || !d->pred_list))
    return fail(PG_ERR_INVALID_ARG, "descriptor arrays are NULL");
  return PG_OK;
}

// ---------------------------------------------------------------- plan upload staging
// pg_pack writes the plan into a pinned, device-mapped host buffer that the
// library owns, and a kernel on the caller's stream copies it into the
// caller's device buffer, reading it over the bus: the call does not wait for
// the GPU, and in stream order the upload is one more kernel, with no hand-off
// to a copy engine.  The buffers are coherent (the GPU does not cache them),
// reused once the event recorded after their copy has completed, and never
// freed: they live until the process ends.  When kMaxStaging buffers exist and
// none is free, the call waits for the oldest large enough one.
struct Staging {
  char *host = nullptr;
  void *dev = nullptr;  // its device address
  size_t cap = 0;
  hipEvent_t done = nullptr;
  bool busy = false;  // being filled by a caller (the event then says nothing)
  uint64_t seq = 0;   // order of the last upload
};

struct StagingPool {
  std::mutex mu;
  std::vector<Staging> bufs;
  uint64_t next_seq = 1;
};

StagingPool &staging_pool() {
  static StagingPool p;
  return p;
}

constexpr size_t kMaxStaging = 64;

// A free pinned buffer of at least `bytes`, marked busy; its index in *idx.
hipError_t take_staging(size_t bytes, size_t *idx) {
  StagingPool &p = staging_pool();
  std::lock_guard<std::mutex> lock(p.mu);
  size_t best = SIZE_MAX, oldest = SIZE_MAX;
  for (size_t i = 0; i < p.bufs.size(); ++i) {
    Staging &b = p.bufs[i];
    if (b.busy || b.cap < bytes) continue;
    if (oldest == SIZE_MAX || b.seq < p.bufs[oldest].seq) oldest = i;
    if (hipEventQuery(b.done) == hipSuccess && (best == SIZE_MAX || b.cap < p.bufs[best].cap))
      best = i;
  }
  if (best == SIZE_MAX && p.bufs.size() >= kMaxStaging && oldest != SIZE_MAX) {
    // too many uploads in flight: wait for the oldest large enough buffer
    hipError_t e = hipEventSynchronize(p.bufs[oldest].done);
    if (e != hipSuccess) return e;
    best = oldest;
  }
  if (best == SIZE_MAX) {
    Staging b;
    size_t cap = 4096;
    while (cap < bytes) cap *= 2;
    void *h = nullptr;
    hipError_t e = hipHostMalloc(&h, cap, hipHostMallocMapped | hipHostMallocCoherent);
    if (e != hipSuccess) return e;
    e = hipHostGetDevicePointer(&b.dev, h, 0);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&b.done, hipEventDisableTiming);
    if (e != hipSuccess) {
      (void)hipHostFree(h);  // never read by a kernel
      return e;
    }
    b.host = static_cast<char *>(h);
    b.cap = cap;
    p.bufs.push_back(b);
    best = p.bufs.size() - 1;
  }
  p.bufs[best].busy = true;
  *idx = best;
  return hipSuccess;
}

// After the copies from buffer idx were enqueued on s (or failed): record the
// event that frees it and release it to the pool.
hipError_t release_staging(size_t idx, hipStream_t s, bool enqueued) {
  StagingPool &p = staging_pool();
  std::lock_guard<std::mutex> lock(p.mu);
  Staging &b = p.bufs[idx];
  hipError_t e = enqueued ? hipEventRecord(b.done, s) : hipSuccess;
  if (e != hipSuccess) e = hipStreamSynchronize(s);  // the event is unusable: drain instead
  b.busy = false;
  b.seq = p.next_seq++;
  return e;
}

// ---------------------------------------------------------------- no-alloc backward scratch
// pg_attn_bwd_noalloc keeps the backward's workspace (delta, the base-2
// logsumexp and the partial dK/dV sums of cut key tiles) in this file-scope
// device array instead of a caller buffer.  Each device that loads the
// library holds its own copy until the process ends.  In host code the name
// `scratch` is only a host-side stand-in for the symbol: its device address
// is looked up once per device (with that device current) and kept here, and
// only that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[PG_NOALLOC_SCRATCH_BYTES];

struct ScratchAddr {
  std::mutex mu;
  std::map<int, void *> ptr;  // device ordinal -> device address of `scratch`
};
ScratchAddr &scratch_addr() {
  static ScratchAddr a;
  return a;
}

// Device address of this device's scratch array (the current device).
pg_status scratch_for_current_device(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  ScratchAddr &a = scratch_addr();
  std::lock_guard<std::mutex> lock(a.mu);
  auto it = a.ptr.find(dev);
  if (it == a.ptr.end()) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(PG_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    it = a.ptr.emplace(dev, p).first;
  }
  *out = it->second;
  return PG_OK;
}

// The backward of pg_attn_bwd and pg_attn_bwd_noalloc (same kernels); with
// `timing` false nothing but the launches is enqueued (no timing events).
pg_status attn_bwd(const pg_desc *d, pg_dtype t, float softmax_scale, const void *q, const void *k,
                   const void *v, const void *o, const float *lse, const void *dout, void *dq,
                   void *dk, void *dv, void *workspace, hipStream_t s, bool timing) {
  pg::Plan p = plan_of(d);
  const float scale = resolve_scale(softmax_scale, p.D);
  auto run = [&](int id, auto &&launch) -> hipError_t {
    return timing ? timed(id, s, launch) : launch();
  };
  float *delta = static_cast<float *>(workspace);
  const size_t rows = align16(size_t(p.Hq) * size_t(p.T) * 4);
  float *lse2 = reinterpret_cast<float *>(static_cast<char *>(workspace) + rows);
  float *partial = reinterpret_cast<float *>(static_cast<char *>(workspace) + 2 * rows);
  hipError_t e;
  if (t == PG_BF16) {
    // dQ first: it also writes delta and the base-2 logsumexp of its rows,
    // which the dK/dV kernel reads
    e = run(PG_KERNEL_BWD_DQ, [&] {
      return pg::launch_bwd_dq_bf16(p, scale, q, k, v, o, lse, lse2, delta, dout, dq, s);
    });
    if (e == hipSuccess)
      e = run(PG_KERNEL_BWD_DKDV, [&] {
        return pg::launch_bwd_dkdv_bf16(p, scale, q, k, v, lse2, delta, dout, dk, dv, partial, s);
      });
    return hip_status(e, "pg_attn_bwd launch");
  }
  // float32: one launch (dK/dV and dQ workgroups), timed as the dK/dV kernel
  e = run(PG_KERNEL_BWD_DKDV, [&] {
    return pg::launch_bwd_f32(p, scale, q, k, v, o, lse, dout, dq, dk, dv, s);
  });
  return hip_status(e, "pg_attn_bwd launch");
}

// Argument checks shared by both backward entry points.
pg_status check_bwd(const pg_desc *d, pg_dtype t, const void *q, const void *k, const void *v,
                    const void *o, const float *lse, const void *dout, const void *dq,
                    const void *dk, const void *dv) {
  pg_status st = check_desc(d);
  if (st != PG_OK) return st;
  if ((st = check_dtype(t)) != PG_OK) return st;
  if (d->total_rows == 0) return PG_OK;
  if ((st = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {o, "o"}, {lse, "lse"}, {dout, "dout"},
                        {dq, "dq"}, {dk, "dk"}, {dv, "dv"}})) != PG_OK)
    return st;
  if (t == PG_BF16) {
    if (d->max_walk_rows < 0 || d->max_walk_rows > d->total_rows)
      return fail(PG_ERR_INVALID_ARG, "descriptor is not one filled by pg_pack");
    if ((size_t(d->max_walk_rows) + 32) * size_t(d->num_q_heads) * size_t(d->head_dim) * 2 >
        size_t(UINT32_MAX))
      return fail(PG_ERR_UNSUPPORTED,
                  "bf16 backward: the query rows of one dK/dV work item (at most one group) "
                  "must be under 4 GiB of q (32-bit buffer offsets from the item's first row)");
    if (size_t(d->num_q_heads) * size_t(d->total_rows) * 4 >= (size_t(1) << 31))
      return fail(PG_ERR_UNSUPPORTED, "bf16 backward: Hq * T * 4 must be under 2^31");
  }
  return PG_OK;
}

}  // namespace

extern "C" {

size_t pg_pack_buffer_size(const pg_groups *g) {
  HostPlan hp;
  if (plan_batch(g, hp) != PG_OK) return 0;
  return layout_of(g, hp).total;
}

pg_status pg_pack_host(const pg_groups *g, void *h_buf, size_t buf_bytes, int32_t *h_pos_ids,
                       pg_desc *out) {
  if (!h_buf || !out) return fail(PG_ERR_INVALID_ARG, "h_buf and out must not be NULL");
  HostPlan hp;
  pg_status st = plan_batch(g, hp);
  if (st != PG_OK) return st;
  const Layout L = layout_of(g, hp);
  if (buf_bytes < L.total)
    return fail(PG_ERR_WORKSPACE, "descriptor buffer too small: need " + std::to_string(L.total) +
                                      " bytes, got " + std::to_string(buf_bytes));
  pg_desc d;
  serialize(g, hp, L, static_cast<char *>(h_buf), h_pos_ids, &d);
  point_into(&d, L, static_cast<const char *>(h_buf));
  *out = d;
  return PG_OK;
}

pg_status pg_pack(const pg_groups *g, void *d_buf, size_t buf_bytes, int32_t *d_pos_ids,
                  pg_desc *out, void *stream) {
  if (!d_buf || !out) return fail(PG_ERR_INVALID_ARG, "d_buf and out must not be NULL");
  if (!aligned16(d_buf)) return fail(PG_ERR_INVALID_ARG, "d_buf is not 16-byte aligned");
  HostPlan hp;
  pg_status st = plan_batch(g, hp);
  if (st != PG_OK) return st;
  const Layout L = layout_of(g, hp);
  if (buf_bytes < L.total)
    return fail(PG_ERR_WORKSPACE, "descriptor buffer too small: need " + std::to_string(L.total) +
                                      " bytes, got " + std::to_string(buf_bytes));
  const int64_t T = hp.T;
  const size_t pos_off = align16(L.total);
  const size_t need = pos_off + (d_pos_ids ? size_t(T) * 4 : 0);
  size_t slot = 0;
  hipError_t e = take_staging(need, &slot);
  if (e != hipSuccess) return hip_status(e, "pg_pack staging buffer");
  // the pool only appends, and a busy buffer is not touched by other calls
  char *host;
  char *dev;
  {
    StagingPool &pool = staging_pool();
    std::lock_guard<std::mutex> lock(pool.mu);
    host = pool.bufs[slot].host;
    dev = static_cast<char *>(pool.bufs[slot].dev);
  }
  pg_desc d;
  serialize(g, hp, L, host, nullptr, &d);
  const bool with_pos = d_pos_ids && T > 0;
  if (with_pos) std::memcpy(host + pos_off, hp.pos.data(), size_t(T) * 4);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // L.total is a multiple of 16 (every array of the layout is 16-byte aligned)
  e = pg::launch_upload(dev, d_buf, L.total, dev + pos_off, d_pos_ids,
                        with_pos ? size_t(T) : 0, s);
  // the buffer is reused only after the upload kernel has run (or right away
  // if nothing was enqueued)
  const hipError_t r = release_staging(slot, s, e == hipSuccess);
  if (e == hipSuccess) e = r;
  if (e != hipSuccess) return hip_status(e, "pg_pack copy");
  point_into(&d, L, static_cast<const char *>(d_buf));
  *out = d;
  return PG_OK;
}

pg_status pg_attn_fwd(const pg_desc *d, pg_dtype t, float softmax_scale, const void *q,
                      const void *k, const void *v, void *o, float *lse, void *stream) {
  pg_status st = check_desc(d);
  if (st != PG_OK) return st;
  if ((st = check_dtype(t)) != PG_OK) return st;
  if (d->total_rows == 0) return PG_OK;
  if ((st = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {o, "o"}})) != PG_OK) return st;
  if (lse != nullptr && (st = check_ptrs({{lse, "lse"}})) != PG_OK) return st;
  pg::Plan p = plan_of(d);
  const float scale = resolve_scale(softmax_scale, p.D);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed(PG_KERNEL_FWD, s, [&] {
    return (t == PG_BF16) ? pg::launch_fwd_bf16(p, scale, q, k, v, o, lse, s)
                          : pg::launch_fwd_f32(p, scale, q, k, v, o, lse, s);
  });
  return hip_status(e, "pg_attn_fwd launch");
}

size_t pg_attn_bwd_workspace_size(const pg_desc *d, pg_dtype t) {
  if (check_desc(d) != PG_OK) return 0;
  // float32: the backward computes delta and the logsumexp where it uses them
  // and keeps its partial sums on chip
  if (t != PG_BF16) return 16;
  // bf16: delta and the base-2 logsumexp, float [Hq, T] each, and the float
  // dK/dV partial sums of the split key tiles
  const size_t rows = align16(size_t(d->num_q_heads) * size_t(d->total_rows) * 4);
  const size_t parts = size_t(d->num_kv_parts) * size_t(d->num_kv_heads) * 2 * PG_TILE_KV *
                       size_t(d->head_dim) * 4;
  return std::max<size_t>(16, 2 * rows + parts);
}

pg_status pg_attn_bwd(const pg_desc *d, pg_dtype t, float softmax_scale, const void *q,
                      const void *k, const void *v, const void *o, const float *lse,
                      const void *dout, void *dq, void *dk, void *dv, void *workspace,
                      size_t ws_bytes, void *stream) {
  pg_status st = check_bwd(d, t, q, k, v, o, lse, dout, dq, dk, dv);
  if (st != PG_OK || d->total_rows == 0) return st;
  if ((st = check_ptrs({{workspace, "workspace"}})) != PG_OK) return st;
  const size_t need = pg_attn_bwd_workspace_size(d, t);
  if (ws_bytes < need)
    return fail(PG_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) +
                                      " bytes, got " + std::to_string(ws_bytes));
  return attn_bwd(d, t, softmax_scale, q, k, v, o, lse, dout, dq, dk, dv, workspace,
                  static_cast<hipStream_t>(stream), true);
}

pg_status pg_attn_bwd_noalloc(const pg_desc *d, pg_dtype t, float softmax_scale, const void *q,
                              const void *k, const void *v, const void *o, const float *lse,
                              const void *dout, void *dq, void *dk, void *dv, void *stream) {
  pg_status st = check_bwd(d, t, q, k, v, o, lse, dout, dq, dk, dv);
  if (st != PG_OK || d->total_rows == 0) return st;
  const size_t need = pg_attn_bwd_workspace_size(d, t);
  if (need > size_t(PG_NOALLOC_SCRATCH_BYTES))
    return fail(PG_ERR_WORKSPACE,
                "pg_attn_bwd_noalloc: this batch needs " + std::to_string(need) +
                    " bytes of scratch, more than the library's fixed " +
                    std::to_string(size_t(PG_NOALLOC_SCRATCH_BYTES)) +
                    "; use pg_attn_bwd with a caller workspace");
  void *ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != PG_OK) return st;
  return attn_bwd(d, t, softmax_scale, q, k, v, o, lse, dout, dq, dk, dv, ws,
                  static_cast<hipStream_t>(stream), false);
}

pg_status pg_rope(const pg_desc *d, pg_dtype t, void *x, int32_t num_heads, int32_t head_dim,
                  const int32_t *pos_ids, float theta, int32_t inverse, void *stream) {
  pg_status st = check_desc(d);
  if (st != PG_OK) return st;
  if ((st = check_dtype(t)) != PG_OK) return st;
  if (num_heads <= 0 || head_dim <= 0 || (head_dim & 1))
    return fail(PG_ERR_INVALID_ARG, "num_heads must be > 0 and head_dim even and > 0");
  if (!(theta > 1.0f)) return fail(PG_ERR_INVALID_ARG, "theta must be > 1");
  if (d->total_rows == 0) return PG_OK;
  if ((st = check_ptrs({{x, "x"}, {pos_ids, "pos_ids"}})) != PG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(timed(PG_KERNEL_ROPE, s, [&] {
                      return pg::launch_rope(d->total_rows, num_heads, head_dim, t, x, pos_ids,
                                             theta, inverse, s);
                    }),
                    "pg_rope launch");
}

pg_status pg_pack_rows(const pg_desc *d, const void *prefix_rows, const void *resp_rows,
                       void *packed_rows, size_t row_bytes, void *stream) {
  return rows_call(d, true, packed_rows, const_cast<void *>(prefix_rows),
                   const_cast<void *>(resp_rows), row_bytes, stream);
}

pg_status pg_unpack_rows(const pg_desc *d, const void *packed_rows, void *prefix_rows,
                         void *resp_rows, size_t row_bytes, void *stream) {
  return rows_call(d, false, const_cast<void *>(packed_rows), prefix_rows, resp_rows, row_bytes,
                   stream);
}

size_t pg_logprob_workspace_size(const pg_desc *d, int32_t vocab, int32_t d_model) {
  if (check_head(d, vocab, d_model) != PG_OK) return 0;
  return head_ws(d->num_scored, vocab, d_model).total;
}

pg_status pg_logprob_fwd(const pg_desc *d, const void *hidden, const void *weight, int32_t vocab,
                         int32_t d_model, const int32_t *tokens, float *logp, float *lse,
                         void *workspace, size_t ws_bytes, void *stream) {
  pg_status st = check_head(d, vocab, d_model);
  if (st != PG_OK) return st;
  const int n = d->num_scored;
  if (n == 0) return PG_OK;
  if ((st = check_ptrs({{hidden, "hidden"}, {weight, "weight"}, {tokens, "tokens"}, {logp, "logp"},
                        {lse, "lse"}, {workspace, "workspace"}})) != PG_OK)
    return st;
  const HeadWs w = head_ws(n, vocab, d_model);
  if (ws_bytes < w.total)
    return fail(PG_ERR_WORKSPACE, "workspace too small: need " + std::to_string(w.total) +
                                      " bytes, got " + std::to_string(ws_bytes));
  char *ws = static_cast<char *>(workspace);
  void *hp = ws + w.hp;
  float *pm = reinterpret_cast<float *>(ws + w.pm), *ps = reinterpret_cast<float *>(ws + w.ps);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed(PG_KERNEL_HEAD_FWD, s, [&] {
    hipError_t r = pg::launch_gather_rows(d->scored_pred, hidden, hp, n, d_model, s);
    if (r != hipSuccess) return r;
    return pg::launch_head_logprob(hp, weight, d->scored_row, tokens, pm, ps, logp, lse, n,
                                   vocab, d_model, s);
  });
  return hip_status(e, "pg_logprob_fwd launch");
}

pg_status pg_grpo_loss(const pg_desc *d, const float *logp, const float *advantages, float *loss,
                       float *dlogp, void *stream) {
  pg_status st = check_desc(d);
  if (st != PG_OK) return st;
  if (d->num_scored > 0 && !d->scored_resp)
    return fail(PG_ERR_INVALID_ARG, "descriptor arrays are NULL");
  if (d->num_resp == 0) return fail(PG_ERR_INVALID_ARG, "the batch has no responses");
  if ((st = check_ptrs({{advantages, "advantages"}, {loss, "loss"}})) != PG_OK) return st;
  if (d->num_scored > 0 && (st = check_ptrs({{logp, "logp"}, {dlogp, "dlogp"}})) != PG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(timed(PG_KERNEL_LOSS, s, [&] {
                      return pg::launch_grpo_loss(logp, d->scored_resp, advantages, loss, dlogp,
                                                  d->num_scored, d->num_resp, s);
                    }),
                    "pg_grpo_loss launch");
}

pg_status pg_logprob_bwd(const pg_desc *d, const void *hidden, const void *weight, int32_t vocab,
                         int32_t d_model, const int32_t *tokens, const float *lse,
                         const float *dlogp, float *dhidden, float *dweight, void *workspace,
                         size_t ws_bytes, void *stream) {
  pg_status st = check_head(d, vocab, d_model);
  if (st != PG_OK) return st;
  const int n = d->num_scored;
  if ((st = check_ptrs({{hidden, "hidden"}, {weight, "weight"}, {dweight, "dweight"},
                        {workspace, "workspace"}})) != PG_OK)
    return st;
  if (d->total_rows > 0 && (st = check_ptrs({{dhidden, "dhidden"}})) != PG_OK) return st;
  if (n > 0 && (st = check_ptrs({{tokens, "tokens"}, {lse, "lse"}, {dlogp, "dlogp"}})) != PG_OK)
    return st;
  const HeadWs w = head_ws(n, vocab, d_model);
  if (ws_bytes < w.total)
    return fail(PG_ERR_WORKSPACE, "workspace too small: need " + std::to_string(w.total) +
                                      " bytes, got " + std::to_string(ws_bytes));
  char *ws = static_cast<char *>(workspace);
  void *g = ws + w.g, *gt = ws + w.gt, *hp = ws + w.hp, *hpt = ws + w.hpt, *wt = ws + w.wt;
  float *dhp = reinterpret_cast<float *>(ws + w.dhp);
  // contraction lengths (multiples of 8) and row strides (multiples of 64)
  const int n8 = pg::round8(n), V8 = pg::round8(vocab);
  const int n64 = pg::round64(n), V64 = pg::round64(vocab);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed(PG_KERNEL_HEAD_BWD, s, [&] {
    hipError_t r = hipSuccess;
    if (n > 0) {
      // operands of the two products, each contiguous along its contraction
      if ((r = pg::launch_gather_rows(d->scored_pred, hidden, hp, n, d_model, s)) != hipSuccess)
        return r;
      if ((r = pg::launch_transpose_pad(hidden, d->scored_pred, n, d_model, hpt, n64, s)) !=
          hipSuccess)
        return r;
      if ((r = pg::launch_transpose_pad(weight, nullptr, vocab, d_model, wt, V64, s)) !=
          hipSuccess)
        return r;
      if ((r = pg::launch_head_grad(hp, weight, d->scored_row, tokens, lse, dlogp, g, gt, n, vocab,
                                    d_model, s)) != hipSuccess)
        return r;
      // dH_pred [n, dm] = G W = G [n, V64] (W^T [dm, V64])^T over V8 entries
      if ((r = pg::launch_nt_f32(g, wt, n, d_model, V8, V64, V64, dhp, d_model, s)) != hipSuccess)
        return r;
    }
    // dW [V, dm] = G^T H_pred = G^T [V, n64] (H_pred^T [dm, n64])^T over n8
    // entries; zeros when nothing is scored (an empty contraction)
    if ((r = pg::launch_nt_f32(gt, hpt, vocab, d_model, n8, n64, n64, dweight, d_model, s)) !=
        hipSuccess)
      return r;
    return pg::launch_scatter_rows(d->pred_start, d->pred_list, dhp, dhidden, d->total_rows,
                                   d_model, s);
  });
  return hip_status(e, "pg_logprob_bwd launch");
}

pg_status pg_kernel_timing(int32_t enable) {
  Timing &t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  hipError_t e = drain(t, true);
  if (e == hipSuccess) e = t.deferred;
  t.deferred = hipSuccess;
  for (int i = 0; i < PG_KERNEL_COUNT; ++i) {
    t.launches[i] = 0;
    t.total_ms[i] = 0.0;
  }
  t.enabled = enable != 0;
  return hip_status(e, "pg_kernel_timing");
}

pg_status pg_kernel_times(int32_t kernel_id, int64_t *launches, double *total_ms) {
  if (kernel_id < 0 || kernel_id >= PG_KERNEL_COUNT || !launches || !total_ms)
    return fail(PG_ERR_INVALID_ARG, "unknown kernel id or NULL output");
  Timing &t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  hipError_t e = drain(t, true);
  if (e == hipSuccess) e = t.deferred;
  t.deferred = hipSuccess;
  *launches = t.launches[kernel_id];
  *total_ms = t.total_ms[kernel_id];
  return hip_status(e, "pg_kernel_times");
}

const char *pg_kernel_name(int32_t kernel_id) {
  return (kernel_id >= 0 && kernel_id < PG_KERNEL_COUNT) ? kKernelNames[kernel_id] : nullptr;
}

const char *pg_last_error(void) { return g_last_error.c_str(); }

const char *pg_version(void) { return "pg_attn 0.1 (gfx950)"; }

}  // extern "C"
