// Host-side validation and slice planner (no HIP calls; unit-tested on the CPU).
//
// Turns the slice list of the MagiAttention FFA interface (quickstart page,
// "Single-GPU Flex-Flash-Attention": q_ranges, k_ranges, attn_type_map) into
// the worklist described in ffa_internal.h:
//
//  1. q segments: the query axis is cut at every slice boundary, so inside a
//     segment each row is covered by the same set of slices.
//  2. q tiles: a segment is cut into tiles of rows_per_item rows, aligned to
//     the segment start (the last tile may be short).
//  3. key runs: for each slice covering a tile, the visible end of a row is
//     ke (full) or ke - (qe - 1 - i) (causal, bottom-right aligned; the
//     kv-interval formula of the MagiAttention blog page "Calculate KV Interval
//     Boundaries for Mask Types").  It is nondecreasing in i, so the first and
//     last rows of the tile bound it: tiles of BN keys from ks up to the last
//     row's end are needed, those ending before the first row's end need no
//     mask, and a slice the last row cannot see is skipped.
//  4. split-K: long items are cut into chunks of key tiles that write float32
//     partial (out, lse); the combine kernel merges them with a global
//     logsumexp (FlagAttention user guide, "Split-KV and paged attention").
//     The automatic rule picks the split by occupancy, as FlagAttention picks
//     its split-KV path: it estimates the time of the plan without a split and
//     with chunks of 1/2, 1 and 2 fair shares (dispatch makespan of the items
//     in longest-first order on the resident workgroup slots, plus the combine
//     pass for a split) and keeps the cheapest.  The constants are measured on
//     MI355X (per-tile and per-item time of the main kernel, combine launch and
//     HBM rate).
//  5. order: longest items first, so the hardware dispatcher fills the device
//     with long work and ends on short work.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <functional>
#include <numeric>
#include <string>
#include <vector>

#include "ffa_internal.h"

namespace ffa {

namespace {
thread_local std::string g_last_error;

// A slice as a band: row i (qs <= i < qe) sees keys
// [max(ks, i + lo_base), min(ke, i + edge_base)); lo_base = -kNoEdge and
// edge_base = kNoEdge stand for "no bound".  The mask types of the interface
// are the cases lo_base = ks - qs (bit 1 of the type) and edge_base = ke - qe + 1
// (bit 0): the kv-interval formula of the MagiAttention blog page "Calculate
// KV Interval Boundaries for Mask Types".  The transpose of a band (keys as
// rows) is again a band, which is how the key-major backward worklist is made.
struct Slice {
  int32_t qs, qe, ks, ke, type, id;
  int32_t lo_base, edge_base;
  bool has_lo() const { return lo_base != -kNoEdge; }
  bool has_hi() const { return edge_base != kNoEdge; }
};

Slice make_slice(int32_t qs, int32_t qe, int32_t ks, int32_t ke, int32_t type, int32_t id) {
  Slice s{qs, qe, ks, ke, type, id, -kNoEdge, kNoEdge};
  if (type & 2) s.lo_base = ks - qs;
  if (type & 1) s.edge_base = ke - qe + 1;
  return s;
}

// Key j is visible from row i iff i + lo <= j < i + hi; with the key j as the
// row, i runs over [j + 1 - hi, j + 1 - lo).
Slice transpose(const Slice& s) {
  Slice t{s.ks, s.ke, s.qs, s.qe, -1, s.id, -kNoEdge, kNoEdge};
  if (s.has_hi()) t.lo_base = 1 - s.edge_base;
  if (s.has_lo()) t.edge_base = 1 - s.lo_base;
  return t;
}

// Keys row i sees through slice s: [row_start, row_end), clamped to [ks, ke]
// (the interval may be empty).  Both are nondecreasing in i.
inline int64_t row_start(const Slice& s, int64_t i) {
  return s.has_lo() ? std::max<int64_t>(s.ks, i + s.lo_base) : (int64_t)s.ks;
}
inline int64_t row_end(const Slice& s, int64_t i) {
  return s.has_hi() ? std::min<int64_t>(s.ke, i + s.edge_base) : (int64_t)s.ke;
}

int64_t slice_visible_pairs(const Slice& s) {
  const int64_t M = s.qe - s.qs, N = s.ke - s.ks;
  if (M <= 0 || N <= 0) return 0;
  if (s.type == FFA_MASK_FULL) return M * N;
  if (s.type == FFA_MASK_BICAUSAL) return M * std::max<int64_t>(0, N - M + 1);  // a band of N - M + 1 keys
  // causal: local row m sees clamp(N - M + 1 + m, 0, N) keys; inverse causal is
  // the same count with the rows in reverse order
  const int64_t c = N - M + 1;
  const int64_t m0 = std::max<int64_t>(0, 1 - c);
  if (m0 >= M) return 0;
  return (c + m0 + N) * (M - m0) / 2;
}

// Rows where a piecewise-linear row function built from the slices' bounds can
// turn: where a bound that moves with the row (slope 1, i + c) meets a fixed
// one (a range end); with the ends of [r0, r1] and their neighbours.
void kink_rows(const Slice* const* sl, int n, int64_t r0, int64_t r1, std::vector<int64_t>& out) {
  out.assign({r0, r1});
  std::vector<int64_t> moving, fixed;
  for (int x = 0; x < n; ++x) {
    if (sl[x]->has_lo()) moving.push_back(sl[x]->lo_base);
    if (sl[x]->has_hi()) moving.push_back(sl[x]->edge_base);
    fixed.push_back(sl[x]->ks);
    fixed.push_back(sl[x]->ke);
  }
  for (int64_t c : moving)
    for (int64_t f : fixed)
      for (int64_t d = -1; d <= 1; ++d) out.push_back(std::min(r1, std::max(r0, f - c + d)));
}

// Largest number of keys two slices share on one row over the rows both cover
// (0: disjoint).  The shared count min(ends) - max(starts) is concave and
// piecewise linear in the row (slopes 0 / 1), so its maximum lies at an end of
// the shared rows or where a moving bound meets a fixed one.
int64_t max_shared_keys(const Slice& a, const Slice& b) {
  const int64_t r0 = std::max(a.qs, b.qs), r1 = std::min(a.qe, b.qe) - 1;
  if (r1 < r0) return 0;
  const Slice* both[2] = {&a, &b};
  std::vector<int64_t> cand;
  kink_rows(both, 2, r0, r1, cand);
  int64_t best = 0;
  for (int64_t i : cand)
    best = std::max(best, std::min(row_end(a, i), row_end(b, i)) - std::max(row_start(a, i), row_start(b, i)));
  return best;
}

// Largest number of keys one row of [r0, r1] sees through s (concave in the row).
int64_t max_row_width(const Slice& s, int64_t r0, int64_t r1) {
  const Slice* one[1] = {&s};
  std::vector<int64_t> cand;
  kink_rows(one, 1, r0, r1, cand);
  int64_t best = 0;
  for (int64_t i : cand) best = std::max(best, row_end(s, i) - row_start(s, i));
  return best;
}

struct TileRun {
  int32_t k0, n_tiles, n_full, k_hi, edge_base, n_lead, lo_base;
};

struct QTile {
  int32_t q0, nrows;
  std::vector<TileRun> runs;
  int64_t tiles = 0;
};

constexpr int32_t kMinChunkTiles = 16;   // never split below 1024 keys per chunk
constexpr int32_t kItemOverhead = 3;     // prologue / epilogue cost of an item, in tiles (measured)
constexpr int32_t kResidentPerCu = 2;    // main-kernel workgroups resident per CU
// Split cost model (measured on MI355X, D = 128; D = 64 tiles take about 0.6x):
constexpr double kTileUs128 = 1.8;         // one key tile of one item, per resident slot
constexpr double kCombineFixedUs = 6.0;    // combine launch and its own tail
constexpr double kCombineBytesPerUs = 4.0e6;  // effective HBM rate of partial writes + combine (4 TB/s)
constexpr double kSplitImbalance = 1.1;    // only consider a split when the makespan exceeds the mean by 10%

// Longest-first greedy makespan of item costs on `slots` identical slots (what
// the hardware dispatcher does with an item list in longest-first order).
double lpt_makespan(std::vector<int64_t>& costs, int64_t slots) {
  if (costs.empty()) return 0.0;
  std::sort(costs.begin(), costs.end(), std::greater<int64_t>());
  if ((int64_t)costs.size() <= slots) return (double)costs.front();
  std::vector<int64_t> heap(slots, 0);  // min-heap of slot loads
  for (int64_t c : costs) {
    std::pop_heap(heap.begin(), heap.end(), std::greater<int64_t>());
    heap.back() += c;
    std::push_heap(heap.begin(), heap.end(), std::greater<int64_t>());
  }
  return (double)*std::max_element(heap.begin(), heap.end());
}
// Largest token count of either axis.  It keeps every bound a slice can produce
// (edge_base = ke - qe + 1 <= kMaxTokens, lo_base = ks - qs >= 1 - kMaxTokens, and
// the same for the transposed slices) strictly inside (-kNoEdge, kNoEdge), so a real
// bound never reads as "no bound", and row + bound stays inside int32 on the device.
constexpr int64_t kMaxTokens = ((int64_t)1 << 30) - 2;

// Steps 1-3: q segments, q tiles of rows_per_item rows and their key runs.
std::vector<QTile> make_tiles(const std::vector<Slice>& slices, int32_t total_rows, int32_t rows_per_item) {
  std::vector<int32_t> bounds = {0, total_rows};
  for (const Slice& s : slices) {
    bounds.push_back(s.qs);
    bounds.push_back(s.qe);
  }
  std::sort(bounds.begin(), bounds.end());
  bounds.erase(std::unique(bounds.begin(), bounds.end()), bounds.end());

  std::vector<int> by_qs(slices.size());
  std::iota(by_qs.begin(), by_qs.end(), 0);
  std::sort(by_qs.begin(), by_qs.end(), [&](int a, int b) { return slices[a].qs < slices[b].qs; });

  std::vector<QTile> tiles;
  std::vector<int> active;
  size_t next_slice = 0;
  for (size_t bi = 0; bi + 1 < bounds.size(); ++bi) {
    const int32_t a = bounds[bi], b = bounds[bi + 1];
    if (b <= a) continue;
    while (next_slice < by_qs.size() && slices[by_qs[next_slice]].qs <= a) active.push_back(by_qs[next_slice++]);
    active.erase(std::remove_if(active.begin(), active.end(), [&](int s) { return slices[s].qe <= a; }),
                 active.end());
    for (int32_t r0 = a; r0 < b; r0 += rows_per_item) {
      QTile t;
      t.q0 = r0;
      t.nrows = std::min(rows_per_item, b - r0);
      const int64_t r_last = (int64_t)r0 + t.nrows - 1;
      for (int si : active) {
        const Slice& s = slices[si];
        // starts and ends are nondecreasing in the row: the tile sees
        // [lo_first, e_last) in total and every row of it sees [lo_last, e_first)
        if (max_row_width(s, r0, r_last) <= 0) continue;  // no row sees this slice
        const int64_t lo_first = row_start(s, r0), lo_last = row_start(s, r_last);
        const int64_t e_first = row_end(s, r0), e_last = row_end(s, r_last);
        const int64_t t_first = (lo_first - s.ks) / kBlockN;  // tiles aligned to ks
        const int64_t k0 = s.ks + t_first * kBlockN;
        TileRun run;
        run.k0 = (int32_t)k0;
        run.n_tiles = (int32_t)((e_last - k0 + kBlockN - 1) / kBlockN);
        run.n_lead = (int32_t)std::min<int64_t>(run.n_tiles, (std::max<int64_t>(lo_last - k0, 0) + kBlockN - 1) / kBlockN);
        run.n_full = (int32_t)std::max<int64_t>(0, std::min<int64_t>(run.n_tiles, (e_first - k0) / kBlockN) - run.n_lead);
        run.k_hi = s.ke;
        run.edge_base = s.edge_base;
        run.lo_base = s.lo_base;
        t.runs.push_back(run);
        t.tiles += run.n_tiles;
      }
      std::sort(t.runs.begin(), t.runs.end(), [](const TileRun& x, const TileRun& y) { return x.k0 < y.k0; });
      tiles.push_back(std::move(t));
    }
  }
  return tiles;
}

}  // namespace

ffa_status set_error(ffa_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}
void clear_error() { g_last_error.clear(); }

ffa_status check_extras(const ffa_attn_extras* ex, bool has_rows) {
  if (!ex) return FFA_OK;
  if (!(ex->softcap >= 0.0f) || !std::isfinite(ex->softcap))
    return set_error(FFA_ERR_ARG, "softcap must be finite and >= 0 (0: off)");
  if (ex->n_sink < 0) return set_error(FFA_ERR_ARG, "n_sink must be >= 0");
  if (ex->dtype != FFA_DTYPE_BF16 && ex->dtype != FFA_DTYPE_F16)
    return set_error(FFA_ERR_ARG, "dtype must be FFA_DTYPE_BF16 or FFA_DTYPE_F16");
  if (ex->n_sink > 65536) return set_error(FFA_ERR_ARG, "n_sink must be at most 65536");
  if (ex->flags & ~FFA_EXTRAS_ROUNDED_NORM) return set_error(FFA_ERR_ARG, "unknown bits in extras flags");
  if (ex->n_sink > 0 && has_rows && !ex->sink) return set_error(FFA_ERR_NULL, "n_sink > 0 but sink is NULL");
  return FFA_OK;
}
const char* last_error() { return g_last_error.c_str(); }

ffa_status build_plan(const int32_t* q_ranges, const int32_t* k_ranges, const int32_t* mask_types,
                      int32_t num_slices, int32_t total_q, int32_t total_k, int32_t heads_q,
                      int32_t heads_kv, int32_t head_dim, int32_t split_tiles, int32_t max_splits,
                      int32_t num_cus, uint32_t flags, Plan* plan) {
  // ---------------------------------------------------------------- validation
  if (!plan) return set_error(FFA_ERR_NULL, "plan output pointer is NULL");
  if (num_slices < 0) return set_error(FFA_ERR_ARG, "num_slices < 0");
  if (num_slices > 0 && (!q_ranges || !k_ranges || !mask_types))
    return set_error(FFA_ERR_NULL, "q_ranges, k_ranges and mask_types must be non-NULL when num_slices > 0");
  if (total_q < 0 || total_k < 0 || total_q > kMaxTokens || total_k > kMaxTokens)
    return set_error(FFA_ERR_SHAPE, "total_q and total_k must be in [0, 2^30 - 2]");
  if (heads_q <= 0 || heads_kv <= 0) return set_error(FFA_ERR_SHAPE, "head counts must be positive");
  if (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128)
    return set_error(FFA_ERR_SHAPE, "head_dim must be 16, 32, 64 or 128, got " + std::to_string(head_dim));
  if (heads_q % heads_kv != 0)
    return set_error(FFA_ERR_GQA, "heads_q (" + std::to_string(heads_q) + ") must be a multiple of heads_kv (" +
                                      std::to_string(heads_kv) + ")");
  if (num_cus <= 0) return set_error(FFA_ERR_ARG, "num_cus must be positive");
  if (max_splits <= 0) max_splits = 64;

  std::vector<Slice> slices;
  slices.reserve(num_slices);
  int64_t visible = 0;
  for (int32_t s = 0; s < num_slices; ++s) {
    const Slice x = make_slice(q_ranges[2 * s], q_ranges[2 * s + 1], k_ranges[2 * s], k_ranges[2 * s + 1],
                               mask_types[s], s);
    if (x.qs < 0 || x.qe > total_q || x.qs > x.qe)
      return set_error(FFA_ERR_RANGE, "slice " + std::to_string(s) + ": q_range [" + std::to_string(x.qs) + ", " +
                                          std::to_string(x.qe) + ") outside [0, " + std::to_string(total_q) + "]");
    if (x.ks < 0 || x.ke > total_k || x.ks > x.ke)
      return set_error(FFA_ERR_RANGE, "slice " + std::to_string(s) + ": k_range [" + std::to_string(x.ks) + ", " +
                                          std::to_string(x.ke) + ") outside [0, " + std::to_string(total_k) + "]");
    if (x.type < FFA_MASK_FULL || x.type > FFA_MASK_BICAUSAL)
      return set_error(FFA_ERR_MASK_TYPE, "slice " + std::to_string(s) + ": mask type " + std::to_string(x.type) +
                                              " (supported: 0 full, 1 causal, 2 inverse causal, 3 bi-causal)");
    const int64_t vp = slice_visible_pairs(x);
    if (vp == 0) continue;  // a slice that makes nothing visible is a no-op
    visible += vp;
    slices.push_back(x);
  }

  // overlap: two slices share a visible pair iff some row both cover sees a
  // common key (max_shared_keys evaluates the shared count where it can peak).
  {
    std::vector<int> ord(slices.size());
    std::iota(ord.begin(), ord.end(), 0);
    std::sort(ord.begin(), ord.end(), [&](int a, int b) { return slices[a].qs < slices[b].qs; });
    for (size_t ia = 0; ia < ord.size(); ++ia) {
      const Slice& a = slices[ord[ia]];
      for (size_t ib = ia + 1; ib < ord.size(); ++ib) {
        const Slice& b = slices[ord[ib]];
        if (b.qs >= a.qe) break;
        if (b.ks >= a.ke || a.ks >= b.ke) continue;  // key ranges apart: nothing shared
        if (max_shared_keys(a, b) > 0)
          return set_error(FFA_ERR_OVERLAP, "slices " + std::to_string(a.id) + " and " + std::to_string(b.id) +
                                                " overlap");
      }
    }
  }

  // ---------------------------------------------------------------- shape of a workgroup
  const int32_t ratio = heads_q / heads_kv;
  int32_t G = 1;
  for (int32_t g : {4, 2}) {
    if (ratio % g == 0) {
      G = g;
      break;
    }
  }
  const int32_t rows_per_item = kSlotsPerItem / G;
  const int32_t n_groups = heads_q / G;
  // The groups of a q tile are emitted kv head by kv head within each round j of the
  // ratio / G groups that share a kv head: group g reads kv head g / (ratio / G), and
  // the hardware hands consecutive workgroups to the 8 XCDs in turn, so with 8 kv heads
  // every group of a kv head lands on the same XCD (and its L2) instead of two or more.
  std::vector<int32_t> group_order;
  group_order.reserve(n_groups);
  {
    const int32_t per_kv = ratio / G;
    for (int32_t j = 0; j < per_kv; ++j)
      for (int32_t kv = 0; kv < heads_kv; ++kv) group_order.push_back(kv * per_kv + j);
  }

  // ---------------------------------------------------------------- segments and q tiles
  const std::vector<QTile> tiles = make_tiles(slices, total_q, rows_per_item);

  // ---------------------------------------------------------------- split-K decision
  // number of chunks of a q tile for a chunk target (0: no split)
  auto n_chunks_of = [&](int64_t tiles, int64_t target) -> int64_t {
    if (target <= 0 || tiles <= target) return 1;
    return std::min<int64_t>({(int64_t)max_splits, (tiles + target - 1) / target, tiles});
  };
  int64_t chunk_target = 0;  // 0: no split
  if (split_tiles > 0) {
    chunk_target = split_tiles;
  } else if (split_tiles == 0) {
    const int64_t slots = (int64_t)num_cus * kResidentPerCu;
    const double tile_us = head_dim == 128 ? kTileUs128 : 0.6 * kTileUs128;
    // estimated time (us) of the plan for a chunk target
    auto estimate = [&](int64_t target) -> double {
      std::vector<int64_t> costs;
      double comb_bytes = 0.0;
      for (const QTile& t : tiles) {
        const int64_t n = n_chunks_of(t.tiles, target);
        for (int64_t c = 0; c < n; ++c) {
          const int64_t ct = (c + 1) * t.tiles / n - c * t.tiles / n;
          const int64_t cost = ct + (t.runs.empty() ? 1 : kItemOverhead);
          for (int32_t g = 0; g < n_groups; ++g) costs.push_back(cost);
        }
        if (n > 1)  // partials written and read back, out written by the combine
          comb_bytes += (double)n_groups * t.nrows * G * ((2.0 * n) * (4.0 * head_dim + 4.0) + 2.0 * head_dim + 4.0);
      }
      const double t_main = lpt_makespan(costs, slots) * tile_us;
      return comb_bytes > 0.0 ? t_main + kCombineFixedUs + comb_bytes / kCombineBytesPerUs : t_main;
    };
    int64_t total_cost = 0;
    for (const QTile& t : tiles) total_cost += (t.tiles + (t.runs.empty() ? 1 : kItemOverhead)) * n_groups;
    const double mean = (double)total_cost / (double)slots;
    double best = estimate(0);
    if (best > kSplitImbalance * mean * (head_dim == 128 ? kTileUs128 : 0.6 * kTileUs128)) {
      const int64_t fair = std::max<int64_t>(1, (int64_t)std::ceil(mean));
      for (int64_t target : {fair / 2, fair, 2 * fair}) {
        const int64_t tgt = std::max<int64_t>(kMinChunkTiles, target);
        const double e = estimate(tgt);
        if (e < best) {
          best = e;
          chunk_target = tgt;
        }
      }
    }
  }

  // ---------------------------------------------------------------- emit
  struct ItemRec {
    int32_t q0, nrows, h0, run_off, n_runs, slot, tiles;
  };
  // The first wave fills two slots per CU, and the dispatcher puts workgroup i and
  // workgroup i + (number of CUs) on the same CU.  Reversing the second half of the
  // first wave of a longest-first list (in whole q-tile blocks of n_groups items, which
  // keeps each block's kv heads on their XCDs) pairs the k-th longest item with the k-th
  // shortest of the wave, so the CUs start with about equal work.  This matters when the
  // items about fill the slots once (rect_causal_gqa: 512 items of 33-64 tiles, +1.8%
  // measured on the forward); with many more items the longest-first dispatch after the
  // first wave balances by itself.  Used for the lists of kernels that run two
  // workgroups per CU (the forward and the query-major backward).
  auto pair_first_wave = [&](std::vector<ItemRec>& its) {
    if (flags & 1u) return;
    const size_t half = (size_t)num_cus, nb = (size_t)n_groups;
    if (half % nb != 0 || its.size() <= half) return;
    const size_t end = std::min(its.size(), 2 * half) / nb * nb;
    std::vector<ItemRec> seg(its.begin() + half, its.begin() + end);
    const size_t nblk = seg.size() / nb;
    for (size_t k = 0; k < nblk; ++k)
      std::copy(seg.begin() + (nblk - 1 - k) * nb, seg.begin() + (nblk - k) * nb, its.begin() + half + k * nb);
  };
  std::vector<ItemRec> items;
  std::vector<int32_t> runs;      // flattened run records (kRec each)
  std::vector<int32_t> combine;   // flattened combine records
  int32_t n_slots = 0, n_split_items = 0;
  int64_t computed = 0, all_tiles = 0;
  auto push_run = [&](int32_t k0, int32_t nt, int32_t nl, int32_t nf, const TileRun& r) {
    const int32_t rec[kRec] = {k0, nt, nf, r.k_hi, r.edge_base, nl, r.lo_base, 0};
    runs.insert(runs.end(), rec, rec + kRec);
  };

  for (const QTile& t : tiles) {
    computed += (int64_t)rows_per_item * t.tiles * kBlockN;
    all_tiles += t.tiles * n_groups;
    const int64_t n_chunks = n_chunks_of(t.tiles, chunk_target);
    if (n_chunks <= 1) {
      const int32_t off = (int32_t)(runs.size() / kRec);
      for (const TileRun& r : t.runs) push_run(r.k0, r.n_tiles, r.n_lead, r.n_full, r);
      for (const int32_t g : group_order)
        items.push_back({t.q0, t.nrows, g * G, off, (int32_t)t.runs.size(), -1, (int32_t)t.tiles});
      continue;
    }
    // split: chunk c covers item tiles [c*T/n, (c+1)*T/n) across the runs in order
    std::vector<int32_t> chunk_off(n_chunks), chunk_nruns(n_chunks), chunk_tiles(n_chunks);
    for (int64_t c = 0; c < n_chunks; ++c) {
      const int64_t ta = c * t.tiles / n_chunks, tb = (c + 1) * t.tiles / n_chunks;
      chunk_off[c] = (int32_t)(runs.size() / kRec);
      chunk_tiles[c] = (int32_t)(tb - ta);
      int32_t nr = 0;
      int64_t cs = 0;
      for (const TileRun& r : t.runs) {
        const int64_t a = std::max(ta, cs), b = std::min(tb, cs + r.n_tiles);
        if (b > a) {
          const int32_t skip = (int32_t)(a - cs);
          const int32_t nt = (int32_t)(b - a);
          // the chunk's tiles [skip, skip + nt) of the run: lead edge tiles, then
          // the full ones, then trailing edge tiles, as in the run itself
          const int32_t nl = std::max(0, std::min(nt, r.n_lead - skip));
          const int32_t fa = std::max(skip, r.n_lead), fb = std::min(skip + nt, r.n_lead + r.n_full);
          push_run(r.k0 + skip * kBlockN, nt, nl, std::max(0, fb - fa), r);
          ++nr;
        }
        cs += r.n_tiles;
      }
      chunk_nruns[c] = nr;
    }
    for (const int32_t g : group_order) {
      const int32_t slot0 = n_slots;
      n_slots += (int32_t)n_chunks * kSlotsPerItem;
      for (int64_t c = 0; c < n_chunks; ++c) {
        items.push_back({t.q0, t.nrows, g * G, chunk_off[c], chunk_nruns[c], slot0 + (int32_t)c * kSlotsPerItem,
                         chunk_tiles[c]});
        ++n_split_items;
      }
      const int32_t rec[kRec] = {t.q0, t.nrows, g * G, (int32_t)n_chunks, slot0, 0, 0, 0};
      combine.insert(combine.end(), rec, rec + kRec);
    }
  }

  if (!(flags & 1u)) {
    std::stable_sort(items.begin(), items.end(), [](const ItemRec& x, const ItemRec& y) {
      const int32_t cx = x.tiles + (x.n_runs ? kItemOverhead : 1), cy = y.tiles + (y.n_runs ? kItemOverhead : 1);
      return cx > cy;
    });
    if (n_split_items == 0) pair_first_wave(items);
  }

  // ---------------------------------------------------------------- backward worklists
  // dQ: the query-major tiles of the forward without split (a row's dQ sums
  // over all its keys inside one workgroup).  dK / dV: the same construction on
  // the transposed slices, one item per (key block, kv head); the item visits
  // its query tiles once for each query head that shares the kv head.
  std::vector<ItemRec> dq_items, kv_items;
  std::vector<int32_t> dq_runs, kv_runs;
  int64_t dq_tiles = 0, kv_tiles = 0;
  const bool want_bwd = (flags & FFA_PLAN_BACKWARD) != 0;
  if (want_bwd) {
    auto emit = [&](const std::vector<QTile>& ts, int32_t n_heads, int32_t head_step, std::vector<ItemRec>& its,
                    std::vector<int32_t>& rs, int64_t& total) {
      for (const QTile& t : ts) {
        const int32_t off = (int32_t)(rs.size() / kRec);
        for (const TileRun& r : t.runs) {
          const int32_t rec[kRec] = {r.k0, r.n_tiles, r.n_full, r.k_hi, r.edge_base, r.n_lead, r.lo_base, 0};
          rs.insert(rs.end(), rec, rec + kRec);
        }
        for (int32_t g = 0; g < n_heads; ++g)
          its.push_back({t.q0, t.nrows, g * head_step, off, (int32_t)t.runs.size(), -1, (int32_t)t.tiles});
        total += t.tiles * n_heads;
      }
      if (!(flags & 1u))
        std::stable_sort(its.begin(), its.end(), [](const ItemRec& x, const ItemRec& y) { return x.tiles > y.tiles; });
    };
    emit(tiles, n_groups, G, dq_items, dq_runs, dq_tiles);
    pair_first_wave(dq_items);
    std::vector<Slice> tr;
    tr.reserve(slices.size());
    for (const Slice& s : slices) tr.push_back(transpose(s));
    emit(make_tiles(tr, total_k, kKvRowsPerItem), heads_kv, 1, kv_items, kv_runs, kv_tiles);
    kv_tiles *= ratio;
    // a key-major item walks its tiles once per query head of its kv head (int32 step count)
    for (const ItemRec& it : kv_items)
      if ((int64_t)it.tiles * ratio > INT32_MAX) return set_error(FFA_ERR_ARG, "plan too large (key-major item)");
  }

  if (items.size() > (size_t)INT32_MAX / kItemRec || runs.size() > (size_t)INT32_MAX ||
      dq_items.size() + kv_items.size() > (size_t)INT32_MAX / kItemRec ||
      dq_runs.size() + kv_runs.size() > (size_t)INT32_MAX)
    return set_error(FFA_ERR_ARG, "plan too large");

  Plan p;
  p.total_q = total_q;
  p.total_k = total_k;
  p.heads_q = heads_q;
  p.heads_kv = heads_kv;
  p.head_dim = head_dim;
  p.heads_per_item = G;
  p.rows_per_item = rows_per_item;
  p.num_items = (int32_t)items.size();
  p.num_runs = (int32_t)(runs.size() / kRec);
  p.num_combine = (int32_t)(combine.size() / kRec);
  p.num_split_items = n_split_items;
  p.num_slots = n_slots;
  p.visible_pairs = visible;
  p.computed_pairs = computed;
  p.total_tiles = all_tiles;
  int32_t max_item = 0;
  for (const ItemRec& it : items) max_item = std::max(max_item, it.tiles);
  p.max_item_tiles = max_item;

  const size_t fwd_size = kHdr + items.size() * kItemRec + runs.size() + combine.size();
  const size_t bwd_size =
      want_bwd ? kBwdHdr + (dq_items.size() + kv_items.size()) * kItemRec + dq_runs.size() + kv_runs.size() : 0;
  if (fwd_size + bwd_size > (size_t)INT32_MAX) return set_error(FFA_ERR_ARG, "plan too large");
  try {
    p.meta.assign(fwd_size + bwd_size, 0);
  } catch (...) {
    return set_error(FFA_ERR_HOST_OOM, "host allocation of the plan failed");
  }
  int32_t* h = p.meta.data();
  h[kHdrMagic] = kMagic;
  h[kHdrVersion] = FFA_ABI_VERSION;
  h[kHdrItems] = p.num_items;
  h[kHdrRuns] = p.num_runs;
  h[kHdrCombine] = p.num_combine;
  h[kHdrHeadsPerItem] = G;
  h[kHdrRowsPerItem] = rows_per_item;
  h[kHdrBlockN] = kBlockN;
  h[kHdrHeadDim] = head_dim;
  h[kHdrHeadsQ] = heads_q;
  h[kHdrHeadsKv] = heads_kv;
  h[kHdrTotalQ] = total_q;
  h[kHdrTotalK] = total_k;
  h[kHdrSlots] = n_slots;
  int32_t* w = h + kHdr;
  // items (with the inline copy of their first run), then their runs
  auto put_items = [&](const std::vector<ItemRec>& its, const std::vector<int32_t>& rs) {
    for (const ItemRec& it : its) {
      int32_t rec[kItemRec] = {it.q0, it.nrows, it.h0, it.run_off, it.n_runs, it.slot, it.tiles, 0};
      if (it.n_runs > 0) std::memcpy(rec + 8, rs.data() + (size_t)it.run_off * kRec, kRec * 4);
      std::memcpy(w, rec, sizeof(rec));
      w += kItemRec;
    }
    if (!rs.empty()) std::memcpy(w, rs.data(), rs.size() * 4);
    w += rs.size();
  };
  put_items(items, runs);
  if (!combine.empty()) std::memcpy(w, combine.data(), combine.size() * 4);
  w += combine.size();
  if (want_bwd) {
    p.bwd_off = (int32_t)fwd_size;
    p.num_dq_items = (int32_t)dq_items.size();
    p.num_dq_runs = (int32_t)(dq_runs.size() / kRec);
    p.num_kv_items = (int32_t)kv_items.size();
    p.num_kv_runs = (int32_t)(kv_runs.size() / kRec);
    p.dq_tiles = dq_tiles;
    p.kv_tiles = kv_tiles;
    h[kHdrBwd] = p.bwd_off;
    const int32_t bh[kBwdHdr] = {p.num_dq_items, p.num_dq_runs, p.num_kv_items, p.num_kv_runs, kKvRowsPerItem, G, 0, 0};
    std::memcpy(w, bh, sizeof(bh));
    w += kBwdHdr;
    put_items(dq_items, dq_runs);
    put_items(kv_items, kv_runs);
  }
  *plan = std::move(p);
  return FFA_OK;
}

}  // namespace ffa
