// C ABI of libmla.so: argument validation, the host split-KV planner, and
// the launch sequence (attention kernel, then the split combine kernel).
//
// The planner is the counterpart of the host planning step the pages
// describe: FlashMLA's "get_mla_metadata" (tile-scheduler metadata derived
// from cache_seqlens once before the decode loop, reused across layers) and
// FlashInfer's "batch_mla_decode_with_paged_kv_cache" (host reads seq_lens /
// qo_indptr to derive plan bounds; capture-safe callers pre-plan).  Its
// contents are our own: a static per-workgroup list of work items that
// balances key tokens across compute units, cutting requests into key
// chunks where needed.  Partial results of cut requests are merged by the
// log-sum-exp identity ("mla_decoding_single_batch": exp_sum / qk_max
// statistics used for split-K reduction).
#include "../../include/mla.h"

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <utility>
#include <vector>

#include "mla_internal.h"

using mla::SplitGroup;
using mla::WorkItem;

struct mla_plan {
  mla_plan_desc d;
  int32_t tile_mode = 0;       // resolved: MLA_TILE_WIDE, _NARROW or _QUAD
  int32_t rows_per_block = 0;  // rows one workgroup holds
  int32_t num_wgs = 0;         // work lists (per workgroup; per sibling group in quad mode)
  int32_t grid = 0;            // workgroups launched
  int32_t group_size = 1;      // quad mode: sibling workgroups per work list
  int32_t xcd_map = 0;         // quad mode: siblings share blockIdx.x mod 8
  int32_t num_slots = 0;       // partial-result slots
  std::vector<int32_t> kv_indptr;  // [batch + 1] host copy of the page offsets the plan was made for
  std::vector<int32_t> qo_indptr;  // [batch + 1] prefill: host copy of the query offsets (empty for capacity plans)
  int32_t capacity = 0;            // a capacity plan (desc.max_kv_len > 0): runs take live lengths
  int32_t max_q = 1;               // query tokens per request a capacity plan allows
  int32_t lse_sq = 0;              // > 0: lse laid out [batch, H, lse_sq]
  std::vector<int32_t> wg_ptr;  // [num_wgs + 1] item range of each workgroup
  std::vector<WorkItem> items;
  std::vector<SplitGroup> groups;
  std::vector<int32_t> blob;    // uploaded image: wg_ptr | items | groups
  size_t off_items = 0, off_groups = 0, off_part_lse = 0, off_part_o = 0, ws_bytes = 0;
  // uploaded copies of the plan's kv_indptr / qo_indptr and the status word of
  // the validate checks
  size_t off_plan_kv = 0, off_plan_qo = 0, off_status = 0;
  // token-sparse plans: entries per list, and the workspace regions of the
  // compacted lists [batch][topk], their counts [batch], page offsets
  // [batch + 1] and the partial maxima [slots][rows_per_block]
  int32_t topk = 0;
  size_t off_sp_list = 0, off_sp_count = 0, off_sp_indptr = 0, off_part_max = 0;
};

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

int32_t ilog2(int32_t x) {
  int32_t s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

// Fixed per-item cost in key-token units: loading Q, the epilogue, and the
// pipeline fill.  Used only to balance the schedule.
constexpr int64_t kItemOverhead = 256;
// Smallest key chunk worth a separate work item (unless it is a remainder).
constexpr int64_t kMinChunk = 128;
// Modeled slowdown accepted for gang packing (see build_schedule).
constexpr double kGangSlack = 1.10;

struct Unit {
  int32_t b, row0, nrows, vis, kv_len, q_len;
};

// Greedy packing of units into workgroups with `budget` key-token units
// each: a unit is cut into pieces (multiples of the stage size) where a
// workgroup's budget runs out; a cut unit becomes a split group whose
// pieces own consecutive partial-result slots.
void pack_units(mla_plan* p, const std::vector<Unit>& units, int64_t budget) {
  const mla_plan_desc& d = p->d;
  const int64_t stage = mla::kStageTokens;
  p->items.clear();
  p->groups.clear();
  p->wg_ptr.assign(1, 0);
  p->num_slots = 0;
  auto close_wg = [&]() { p->wg_ptr.push_back((int32_t)p->items.size()); };
  auto wg_open = [&]() { return p->items.size() > (size_t)p->wg_ptr.back(); };
  int64_t left = budget;  // budget left on the current workgroup
  for (const Unit& u : units) {
    size_t first = p->items.size();
    if (d.force_splits > 0) {
      // exactly min(force_splits, stages) pieces, stages spread evenly
      const int64_t nchunks = std::max<int64_t>(1, (u.vis + stage - 1) / stage);
      const int64_t s = std::min<int64_t>(d.force_splits, nchunks);
      int64_t t = 0;
      for (int64_t k = 0; k < s; ++k) {
        const int64_t n = nchunks / s + (k < nchunks % s ? 1 : 0);
        const int64_t e = std::min<int64_t>(u.vis, t + n * stage);
        if (left < kItemOverhead + kMinChunk && wg_open()) {
          close_wg();
          left = budget;
        }
        p->items.push_back({u.b, u.row0, u.nrows, (int32_t)t, (int32_t)e, u.kv_len, u.q_len, -1});
        left -= (e - t) + kItemOverhead;
        t = e;
      }
    } else {
      int64_t t = 0;
      int32_t npieces = 0;
      do {
        const int64_t rest = u.vis - t;
        if (left < kItemOverhead + std::min<int64_t>(kMinChunk, rest) && wg_open()) {
          close_wg();
          left = budget;
        }
        int64_t take = std::max<int64_t>(left - kItemOverhead, stage) / stage * stage;
        // never leave a remainder smaller than a minimum chunk behind: take
        // less (the next workgroup gets a minimum chunk) rather than overrun
        // this workgroup's budget, unless the whole rest is small
        if (rest > take && rest - take < kMinChunk) {
          const int64_t shorter = (rest - kMinChunk) / stage * stage;
          take = shorter >= stage ? shorter : rest;
        }
        if (d.max_splits > 0 && npieces + 1 >= d.max_splits) take = rest;
        take = std::min<int64_t>(take, rest);
        p->items.push_back({u.b, u.row0, u.nrows, (int32_t)t, (int32_t)(t + take), u.kv_len, u.q_len, -1});
        ++npieces;
        left -= take + kItemOverhead;
        t += take;
      } while (t < u.vis);
    }
    const int32_t n = (int32_t)(p->items.size() - first);
    if (n > 1) {
      SplitGroup g{u.b, u.row0, u.nrows, n, p->num_slots, u.q_len, {0, 0}};
      for (int32_t k = 0; k < n; ++k) p->items[first + k].slot = p->num_slots + k;
      p->num_slots += n;
      p->groups.push_back(g);
    }
  }
  if (wg_open()) close_wg();
  p->num_wgs = (int32_t)p->wg_ptr.size() - 1;
  p->grid = p->num_wgs;
}

// Modeled cost of the longest list of a packing, in key-token units: each
// item costs its stages plus the fixed per-item cost.
int64_t max_list_cost(const mla_plan* p) {
  int64_t worst = 0;
  for (size_t w = 0; w + 1 < p->wg_ptr.size(); ++w) {
    int64_t c = 0;
    for (int32_t i = p->wg_ptr[w]; i < p->wg_ptr[w + 1]; ++i) {
      const WorkItem& it = p->items[i];
      c += kItemOverhead + (it.tok1 - it.tok0 + mla::kStageTokens - 1) / mla::kStageTokens * mla::kStageTokens;
    }
    worst = std::max(worst, c);
  }
  return worst;
}

// One item per list: every unit is cut into the fewest pieces of at most
// `k` stages, its stages spread evenly over them, and each piece is a list of
// its own (units in order, so a unit's pieces sit on neighbouring lists).
// All lists then start at once and no list pays two item costs; the units of
// one request that see the same keys (its query tokens) walk them at the
// same time on neighbouring lists, which share an XCD and its L2.
void pack_even(mla_plan* p, const std::vector<Unit>& units, int64_t k) {
  const int64_t stage = mla::kStageTokens;
  p->items.clear();
  p->groups.clear();
  p->wg_ptr.assign(1, 0);
  p->num_slots = 0;
  for (const Unit& u : units) {
    const int64_t ns = std::max<int64_t>(1, (u.vis + stage - 1) / stage);
    const int64_t n = (ns + k - 1) / k;
    int64_t t = 0;
    for (int64_t j = 0; j < n; ++j) {
      const int64_t e = std::min<int64_t>(u.vis, t + (ns / n + (j < ns % n ? 1 : 0)) * stage);
      p->items.push_back({u.b, u.row0, u.nrows, (int32_t)t, (int32_t)e, u.kv_len, u.q_len,
                          n > 1 ? p->num_slots + (int32_t)j : -1});
      p->wg_ptr.push_back((int32_t)p->items.size());
      t = e;
    }
    if (n > 1) {
      p->groups.push_back({u.b, u.row0, u.nrows, (int32_t)n, p->num_slots, u.q_len, {0, 0}});
      p->num_slots += (int32_t)n;
    }
  }
  p->num_wgs = (int32_t)p->wg_ptr.size() - 1;
  p->grid = p->num_wgs;
}

// Gang packing for requests with several row blocks that see (almost) the
// same keys: the query tokens of a prefill request.  Requests are grouped by
// their number of row blocks w; each group is packed greedily (pack_units)
// into lists of pieces as if each request were one unit, and each such list
// becomes w real lists, one per row block, with the same pieces.  The w
// lists of a request then walk the same key ranges at the same time on
// neighbouring workgroups, which share an XCD: its L2 serves the keys to w
// workgroups from one HBM read.  Gangs wider than `cap` are cut into
// sub-gangs of at most `cap` blocks (fewer widths pack with less waste).
// Returns false (p untouched) when no request has two row blocks with
// visible key counts within one stage of each other.
bool pack_gangs(mla_plan* p, const std::vector<Unit>& units, int64_t cus, int32_t cap) {
  const int64_t stage = mla::kStageTokens;
  // gangs: runs of units of one request whose visible key counts differ by
  // less than a stage; anything else is a gang of one
  struct Gang { int32_t first, w, vis; };
  std::vector<Gang> gangs;
  int32_t widest = 1;
  for (int32_t i = 0; i < (int32_t)units.size();) {
    int32_t j = i + 1, lo = units[i].vis, hi = units[i].vis;
    while (j < (int32_t)units.size() && units[j].b == units[i].b) {
      const int32_t l2 = std::min(lo, units[j].vis), h2 = std::max(hi, units[j].vis);
      if (h2 - l2 >= stage) break;
      lo = l2, hi = h2, ++j;
    }
    const int32_t n = (j - i + cap - 1) / cap;  // sub-gangs of near-equal width
    for (int32_t k = 0, f = i; k < n; ++k) {
      const int32_t w = (j - i) / n + (k < (j - i) % n ? 1 : 0);
      int32_t v = 0;
      for (int32_t m = f; m < f + w; ++m) v = std::max(v, units[m].vis);
      gangs.push_back({f, w, v});
      widest = std::max(widest, w);
      f += w;
    }
    i = j;
  }
  if (widest < 2) return false;
  std::vector<std::vector<Unit>> cls(widest + 1);  // per width: one stand-in unit per gang
  std::vector<std::vector<int32_t>> cls_gang(widest + 1);
  int64_t total = 0;
  for (int32_t g = 0; g < (int32_t)gangs.size(); ++g) {
    const Unit& u = units[gangs[g].first];
    cls[gangs[g].w].push_back({(int32_t)g, u.row0, u.nrows, gangs[g].vis, u.kv_len, u.q_len});
    cls_gang[gangs[g].w].push_back(g);
    total += (int64_t)gangs[g].w * (gangs[g].vis + kItemOverhead);
  }
  mla_plan tmp;
  tmp.d = p->d;
  std::vector<std::vector<std::vector<WorkItem>>> packed(widest + 1);  // [w][gang list] -> pieces
  // Smallest budget whose packing fits in `cus` lists.  With one gang list
  // per width class the count is the sum of the widths present; if even that
  // does not fit, there is no gang packing.  Small steps first, then
  // doubling ones, as in build_schedule, so the search always ends.
  int64_t budget = std::max<int64_t>((total + cus - 1) / cus, kItemOverhead + kMinChunk);
  for (int iter = 0;; ++iter) {
    int64_t lists = 0;
    bool single = true;  // every class packed into one gang list
    for (int32_t w = 1; w <= widest; ++w) {
      packed[w].clear();
      if (cls[w].empty()) continue;
      pack_units(&tmp, cls[w], budget);
      for (int32_t l = 0; l < tmp.num_wgs; ++l)
        packed[w].emplace_back(tmp.items.begin() + tmp.wg_ptr[l], tmp.items.begin() + tmp.wg_ptr[l + 1]);
      lists += (int64_t)w * tmp.num_wgs;
      single = single && tmp.num_wgs == 1;
    }
    if (lists <= cus) break;
    if (single) return false;
    budget += iter < 400 ? std::max<int64_t>(16, budget / 256) : budget;
  }
  // expand: gang list -> w real lists; item.b holds the gang index until here
  p->items.clear();
  p->groups.clear();
  p->wg_ptr.assign(1, 0);
  p->num_slots = 0;
  for (int32_t w = widest; w >= 1; --w) {
    for (const auto& gl : packed[w]) {
      for (int32_t j = 0; j < w; ++j) {
        for (const WorkItem& pc : gl) {
          const Unit& u = units[gangs[pc.b].first + j];
          const int32_t t0 = std::min(pc.tok0, u.vis), t1 = std::min(pc.tok1, u.vis);
          p->items.push_back({u.b, u.row0, u.nrows, t0, t1, u.kv_len, u.q_len, -1});
        }
        p->wg_ptr.push_back((int32_t)p->items.size());
      }
    }
  }
  // split groups: every unit cut into several pieces, its pieces in list order
  std::vector<std::vector<int32_t>> of_unit(units.size());
  {
    // a request's units are consecutive, one per rows_per_block rows
    std::vector<int32_t> first_unit(p->d.batch + 1, 0);
    for (int32_t i = (int32_t)units.size() - 1; i >= 0; --i) first_unit[units[i].b] = i;
    for (int32_t i = 0; i < (int32_t)p->items.size(); ++i) {
      const WorkItem& it = p->items[i];
      of_unit[first_unit[it.b] + it.row0 / p->rows_per_block].push_back(i);
    }
  }
  for (size_t k = 0; k < units.size(); ++k) {
    const int32_t n = (int32_t)of_unit[k].size();
    if (n < 2) continue;
    const Unit& u = units[k];
    p->groups.push_back({u.b, u.row0, u.nrows, n, p->num_slots, u.q_len, {0, 0}});
    for (int32_t m = 0; m < n; ++m) p->items[of_unit[k][m]].slot = p->num_slots + m;
    p->num_slots += n;
  }
  p->num_wgs = (int32_t)p->wg_ptr.size() - 1;
  p->grid = p->num_wgs;
  return true;
}

mla_status build_schedule(mla_plan* p, const std::vector<int32_t>& kv_len,
                          const std::vector<int32_t>& q_len, int32_t num_cus) {
  const mla_plan_desc& d = p->d;
  const int32_t H = d.num_qo_heads;
  int64_t max_rows = 0;
  for (int32_t b = 0; b < d.batch; ++b) max_rows = std::max<int64_t>(max_rows, (int64_t)q_len[b] * H);
  int32_t mode = d.tile_mode;
  // Automatic choice: the 128-row tile once a request holds at least half
  // of one (its key stream then feeds 4 waves' MFMAs from one LDS copy),
  // otherwise the 16-row tile, which splits keys across waves.
  if (mode == MLA_TILE_AUTO) mode = (max_rows >= mla::kWideRows / 2) ? MLA_TILE_WIDE : MLA_TILE_NARROW;
  p->tile_mode = mode;
  int32_t RB = (mode == MLA_TILE_WIDE) ? mla::kWideRows : mla::kNarrowRows;
  int64_t lists = std::max<int32_t>(1, num_cus);
  p->group_size = 1;
  p->xcd_map = 0;
  if (mode == MLA_TILE_QUAD) {
    // G sibling workgroups (one 32-row slice each) per row group; siblings
    // share an XCD when the grid is a multiple of 8 G.
    const int32_t G = std::min<int32_t>(4, std::max<int32_t>(1, (H + mla::kQuadRowsPerWg - 1) / mla::kQuadRowsPerWg));
    p->group_size = G;
    RB = G * mla::kQuadRowsPerWg;
    if (num_cus >= 8 * G) {
      lists = (num_cus / (8 * G)) * 8;
      p->xcd_map = 1;
    } else {
      lists = std::max<int32_t>(1, num_cus / G);
    }
  }
  p->rows_per_block = RB;

  // Units: (request, row block) with the keys the block can see.
  std::vector<Unit> units;
  for (int32_t b = 0; b < d.batch; ++b) {
    const int64_t rows = (int64_t)q_len[b] * H;
    for (int64_t r0 = 0; r0 < rows; r0 += RB) {
      const int32_t nr = (int32_t)std::min<int64_t>(RB, rows - r0);
      int32_t vis = kv_len[b];
      // capacity plans are not trimmed: the live counts move the causal bound
      if (d.kind == MLA_KIND_PREFILL && d.causal && !p->capacity) {
        const int32_t last_q = (int32_t)((r0 + nr - 1) / H);  // query token of the block's last row
        vis = kv_len[b] - q_len[b] + last_q + 1;
      }
      units.push_back({b, (int32_t)r0, nr, vis, kv_len[b], q_len[b]});
    }
  }

  int64_t total = 0;
  for (const Unit& u : units) total += u.vis + kItemOverhead;
  const int64_t cus = lists;
  // Smallest per-workgroup budget whose packing needs at most `cus`
  // workgroups: one persistent workgroup per compute unit.
  // The search always ends: once the budget covers every piece and its
  // overhead, the packing is one list.  Small steps first (tight balance),
  // then doubling steps (forced splits add an overhead per piece that the
  // first budget does not count, and can need several times it).
  int64_t budget = std::max<int64_t>((total + cus - 1) / cus, kItemOverhead + kMinChunk);
  for (int iter = 0;; ++iter) {
    pack_units(p, units, budget);
    if (p->num_wgs <= cus) break;
    budget += iter < 400 ? std::max<int64_t>(16, budget / 256) : budget;
  }
  if (p->num_wgs > cus) return MLA_ERR_INVALID_ARGUMENT;  // unreachable: the loop exits only when they fit
  // The one-item-per-list packing with the smallest piece bound that fits,
  // when its longest list is modeled no longer than the greedy packing's.
  if (d.force_splits == 0) {
    int64_t k = 1;
    for (const Unit& u : units) k = std::max<int64_t>(k, (u.vis + mla::kStageTokens - 1) / mla::kStageTokens);
    auto pieces = [&](int64_t kk) {
      int64_t n = 0, most = 0;
      for (const Unit& u : units) {
        const int64_t ns = std::max<int64_t>(1, (u.vis + mla::kStageTokens - 1) / mla::kStageTokens);
        n += (ns + kk - 1) / kk;
        most = std::max<int64_t>(most, (ns + kk - 1) / kk);
      }
      return std::make_pair(n, most);
    };
    if (pieces(k).first <= cus) {
      // pieces(kk).first only grows as kk shrinks: bisect for the smallest kk that fits
      int64_t lo = 0, hi = k;  // pieces(hi) fits; lo does not (or is 0)
      while (hi - lo > 1) {
        const int64_t mid = (lo + hi) / 2;
        if (pieces(mid).first <= cus) hi = mid; else lo = mid;
      }
      const bool splits_ok = d.max_splits <= 0 || pieces(hi).second <= d.max_splits;
      if (splits_ok && kItemOverhead + hi * mla::kStageTokens < max_list_cost(p)) pack_even(p, units, hi);
    }
  }
  // Gang packing (prefill): the widest gang width cap (the most query tokens
  // sharing each key stage through L2) whose modeled longest list is within
  // kGangSlack of the packing chosen so far.  Lists that share their keys
  // through L2 ran their stages about 14% faster on the 128-head causal
  // prefill than the model, which counts HBM-fed stages, assumes.
  if (d.kind == MLA_KIND_PREFILL && d.force_splits == 0 && d.max_splits == 0 && mode == MLA_TILE_WIDE) {
    const double limit = kGangSlack * (double)max_list_cost(p);
    for (int32_t cap = 8; cap >= 2; --cap) {
      mla_plan alt;
      alt.d = p->d;
      alt.rows_per_block = p->rows_per_block;
      if (!pack_gangs(&alt, units, cus, cap)) break;
      if ((double)max_list_cost(&alt) > limit) continue;
      p->items.swap(alt.items);
      p->groups.swap(alt.groups);
      p->wg_ptr.swap(alt.wg_ptr);
      p->num_slots = alt.num_slots;
      p->num_wgs = alt.num_wgs;
      p->grid = alt.grid;
      break;
    }
  }
  if (p->tile_mode == MLA_TILE_QUAD) {
    p->grid = p->xcd_map ? (int32_t)cus * p->group_size : p->num_wgs * p->group_size;
  }

  // Workspace layout: [wg_ptr | items | groups | plan kv_indptr | plan
  // qo_indptr] [status] [part_lse] [part_o]
  const size_t n_ptr = align_up((size_t)(p->num_wgs + 1) * 4, 32);
  p->off_items = n_ptr;
  p->off_groups = p->off_items + p->items.size() * sizeof(WorkItem);
  p->off_plan_kv = p->off_groups + p->groups.size() * sizeof(SplitGroup);
  p->off_plan_qo = p->off_plan_kv + p->kv_indptr.size() * 4;
  const size_t blob_bytes = p->off_plan_qo + p->qo_indptr.size() * 4;
  p->off_status = align_up(blob_bytes, mla::kWsAlign);
  p->off_part_lse = align_up(p->off_status + 4, mla::kWsAlign);
  p->off_part_o = align_up(p->off_part_lse + (size_t)p->num_slots * RB * 4, mla::kWsAlign);
  p->ws_bytes = align_up(p->off_part_o + (size_t)p->num_slots * RB * mla::kDimCkv * 2, mla::kWsAlign);
  if (d.kind == MLA_KIND_SPARSE_DECODE) {
    p->off_sp_list = p->ws_bytes;
    p->off_sp_count = align_up(p->off_sp_list + (size_t)d.batch * p->topk * 4, mla::kWsAlign);
    p->off_sp_indptr = align_up(p->off_sp_count + (size_t)d.batch * 4, mla::kWsAlign);
    p->off_part_max = align_up(p->off_sp_indptr + (size_t)(d.batch + 1) * 4, mla::kWsAlign);
    p->ws_bytes = align_up(p->off_part_max + (size_t)p->num_slots * RB * 4, mla::kWsAlign);
  }
  p->blob.assign(blob_bytes / 4, 0);
  std::memcpy(p->blob.data(), p->wg_ptr.data(), p->wg_ptr.size() * 4);
  std::memcpy((char*)p->blob.data() + p->off_items, p->items.data(), p->items.size() * sizeof(WorkItem));
  std::memcpy((char*)p->blob.data() + p->off_groups, p->groups.data(), p->groups.size() * sizeof(SplitGroup));
  std::memcpy((char*)p->blob.data() + p->off_plan_kv, p->kv_indptr.data(), p->kv_indptr.size() * 4);
  if (!p->qo_indptr.empty())
    std::memcpy((char*)p->blob.data() + p->off_plan_qo, p->qo_indptr.data(), p->qo_indptr.size() * 4);
  return MLA_OK;
}

mla_status device_cus(int32_t* num_cus) {
  if (*num_cus != 0) return MLA_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_DEVICE;
  if (hipDeviceGetAttribute(num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MLA_ERR_DEVICE;
  return MLA_OK;
}

// A capacity plan ("batch_mla_decode_with_paged_kv_cache": max_kv_len, the
// static K/V length bound; max_seq_len_q, the per-request packed-query
// capacity): every request planned at max_kv_len keys and max_q query
// tokens, with no causal trimming; run calls clip the work to the live
// counts they are given on the device.
mla_status create_capacity_plan(mla_plan** out, const mla_plan_desc* d, const int32_t* qo_indptr_host) {
  int32_t max_q = 1;
  if (d->kind == MLA_KIND_PREFILL) {
    max_q = d->max_seq_len_q;
    if (max_q == 0) {
      if (d->batch > 0 && !qo_indptr_host) return MLA_ERR_INVALID_ARGUMENT;
      for (int32_t b = 0; b < d->batch; ++b) {
        const int64_t n = (int64_t)qo_indptr_host[b + 1] - qo_indptr_host[b];
        if (n < 0 || (b == 0 && qo_indptr_host[0] != 0)) return MLA_ERR_INVALID_ARGUMENT;
        max_q = (int32_t)std::max<int64_t>(max_q, n);
      }
      max_q = std::max(max_q, 1);
    }
    if (d->causal && max_q > d->max_kv_len) return MLA_ERR_INVALID_ARGUMENT;
  } else if (d->max_seq_len_q > 1) {
    return MLA_ERR_INVALID_ARGUMENT;  // decode has one query token per request
  }
  if ((int64_t)max_q * d->num_qo_heads > ((int64_t)1 << 30)) return MLA_ERR_INVALID_ARGUMENT;
  int32_t num_cus = d->num_cus;
  mla_status st = device_cus(&num_cus);
  if (st != MLA_OK) return st;
  mla_plan* p = new (std::nothrow) mla_plan();
  if (!p) return MLA_ERR_INVALID_ARGUMENT;
  p->d = *d;
  p->capacity = 1;
  p->max_q = max_q;
  // the bound's page layout (used by the block-table adapter's width check)
  const int32_t pages = (d->max_kv_len + d->page_size - 1) / d->page_size;
  p->kv_indptr.resize((size_t)d->batch + 1);
  for (int32_t b = 0; b <= d->batch; ++b) p->kv_indptr[b] = b * pages;
  if (d->lse_layout == MLA_LSE_HEADS_FIRST) p->lse_sq = max_q;
  std::vector<int32_t> kv_len(d->batch, d->max_kv_len), q_len(d->batch, max_q);
  st = build_schedule(p, kv_len, q_len, num_cus);
  if (st != MLA_OK) {
    delete p;
    return st;
  }
  *out = p;
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_str(int32_t s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported";
    case MLA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MLA_ERR_PLAN_MISMATCH: return "plan does not match this call";
    case MLA_ERR_DEVICE: return "HIP device error";
    default: return "unknown status";
  }
}

mla_status mla_plan_create(mla_plan** out, const mla_plan_desc* d, const int32_t* kv_len_host,
                           const int32_t* kv_indptr_host, const int32_t* qo_indptr_host) {
  if (!out || !d) return MLA_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (d->kind != MLA_KIND_DECODE && d->kind != MLA_KIND_PREFILL) return MLA_ERR_INVALID_ARGUMENT;
  if (d->batch < 0 || d->num_qo_heads < 1 || d->num_pages < 1) return MLA_ERR_INVALID_ARGUMENT;
  if (d->head_dim_ckv != mla::kDimCkv || d->head_dim_kpe != mla::kDimKpe) return MLA_ERR_UNSUPPORTED;
  if (!is_pow2(d->page_size) || d->page_size > 4096) return MLA_ERR_UNSUPPORTED;
  if (d->kv_format != MLA_KV_BF16 && d->kv_format != MLA_KV_FP8_E4M3_T128 && d->kv_format != MLA_KV_FP8_MODEL1)
    return MLA_ERR_UNSUPPORTED;
  if (d->kv_format != MLA_KV_BF16 && d->kind != MLA_KIND_DECODE) return MLA_ERR_UNSUPPORTED;
  if (d->tile_mode < MLA_TILE_AUTO || d->tile_mode > MLA_TILE_QUAD) return MLA_ERR_INVALID_ARGUMENT;
  if (d->kv_format != MLA_KV_BF16 && d->tile_mode == MLA_TILE_QUAD) return MLA_ERR_UNSUPPORTED;
  if (d->max_splits < 0 || d->force_splits < 0 || d->num_cus < 0) return MLA_ERR_INVALID_ARGUMENT;
  if (d->validate != 0 && d->validate != 1) return MLA_ERR_INVALID_ARGUMENT;
  if (d->lse_layout != MLA_LSE_ROWS && d->lse_layout != MLA_LSE_HEADS_FIRST) return MLA_ERR_INVALID_ARGUMENT;
  if (d->max_kv_len < 0 || d->max_seq_len_q < 0 || d->max_kv_len > (1 << 30)) return MLA_ERR_INVALID_ARGUMENT;
  const bool cap = d->max_kv_len > 0;
  if (!cap && d->max_seq_len_q > 0) return MLA_ERR_INVALID_ARGUMENT;
  if (cap && d->kv_format != MLA_KV_BF16) return MLA_ERR_UNSUPPORTED;
  if (d->kind == MLA_KIND_DECODE && qo_indptr_host) return MLA_ERR_INVALID_ARGUMENT;
  if (cap) return create_capacity_plan(out, d, qo_indptr_host);
  if (d->batch > 0 && !kv_indptr_host) return MLA_ERR_INVALID_ARGUMENT;
  if (d->kind == MLA_KIND_PREFILL && d->batch > 0 && !qo_indptr_host) return MLA_ERR_INVALID_ARGUMENT;

  std::vector<int32_t> kv_len(d->batch), q_len(d->batch, 1);
  if (d->batch > 0 && kv_indptr_host[0] != 0) return MLA_ERR_INVALID_ARGUMENT;
  for (int32_t b = 0; b < d->batch; ++b) {
    const int64_t np = (int64_t)kv_indptr_host[b + 1] - kv_indptr_host[b];
    if (np < 0) return MLA_ERR_INVALID_ARGUMENT;
    const int64_t L = kv_len_host ? kv_len_host[b] : np * d->page_size;
    if (L < 0 || L > (int64_t)1 << 30) return MLA_ERR_INVALID_ARGUMENT;
    if ((L + d->page_size - 1) / d->page_size != np) return MLA_ERR_INVALID_ARGUMENT;
    kv_len[b] = (int32_t)L;
    if (d->kind == MLA_KIND_PREFILL) {
      if (b == 0 && qo_indptr_host[0] != 0) return MLA_ERR_INVALID_ARGUMENT;
      const int64_t n = (int64_t)qo_indptr_host[b + 1] - qo_indptr_host[b];
      if (n < 0) return MLA_ERR_INVALID_ARGUMENT;
      if (d->causal && n > L) return MLA_ERR_INVALID_ARGUMENT;
      q_len[b] = (int32_t)n;
    }
  }
  if (d->lse_layout == MLA_LSE_HEADS_FIRST)
    for (int32_t b = 1; b < d->batch; ++b)
      if (q_len[b] != q_len[0]) return MLA_ERR_INVALID_ARGUMENT;

  int32_t num_cus = d->num_cus;
  const mla_status cus_st = device_cus(&num_cus);
  if (cus_st != MLA_OK) return cus_st;

  mla_plan* p = new (std::nothrow) mla_plan();
  if (!p) return MLA_ERR_INVALID_ARGUMENT;
  p->d = *d;
  p->kv_indptr.assign(kv_indptr_host ? kv_indptr_host : nullptr, kv_indptr_host ? kv_indptr_host + d->batch + 1 : nullptr);
  if (p->kv_indptr.empty()) p->kv_indptr.assign(1, 0);
  if (d->kind == MLA_KIND_PREFILL && qo_indptr_host) p->qo_indptr.assign(qo_indptr_host, qo_indptr_host + d->batch + 1);
  if (d->lse_layout == MLA_LSE_HEADS_FIRST) p->lse_sq = d->batch > 0 ? q_len[0] : 1;
  mla_status st = build_schedule(p, kv_len, q_len, num_cus);
  if (st != MLA_OK) {
    delete p;
    return st;
  }
  *out = p;
  return MLA_OK;
}

mla_status mla_sparse_plan_create(mla_plan** out, int32_t num_tokens, int32_t num_heads, int32_t num_slots,
                                  int32_t topk, int32_t kv_format, int32_t num_cus, int32_t force_splits) {
  if (!out) return MLA_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (num_tokens < 0 || num_heads < 1 || num_slots < 1 || topk < 1 || num_cus < 0 || force_splits < 0)
    return MLA_ERR_INVALID_ARGUMENT;
  if (kv_format != MLA_KV_BF16 && kv_format != MLA_KV_FP8_E4M3_T128 && kv_format != MLA_KV_FP8_MODEL1)
    return MLA_ERR_UNSUPPORTED;
  if ((int64_t)num_tokens * topk > ((int64_t)1 << 31) - 1) return MLA_ERR_INVALID_ARGUMENT;
  if (num_cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_DEVICE;
    if (hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return MLA_ERR_DEVICE;
  }
  mla_plan* p = new (std::nothrow) mla_plan();
  if (!p) return MLA_ERR_INVALID_ARGUMENT;
  // Each query token is a request of one query row block whose "pages" are
  // the topk single-token slots of its list (page size 1).
  mla_plan_desc& d = p->d;
  d.kind = MLA_KIND_SPARSE_DECODE;
  d.batch = num_tokens;
  d.num_qo_heads = num_heads;
  d.head_dim_ckv = mla::kDimCkv;
  d.head_dim_kpe = mla::kDimKpe;
  d.page_size = 1;
  d.num_pages = num_slots;
  d.kv_format = kv_format;
  d.num_cus = num_cus;
  d.force_splits = force_splits;
  d.tile_mode = MLA_TILE_WIDE;
  p->topk = topk;
  std::vector<int32_t> kv_len(num_tokens, topk), q_len(num_tokens, 1);
  p->kv_indptr.resize((size_t)num_tokens + 1);
  for (int32_t t = 0; t <= num_tokens; ++t) p->kv_indptr[t] = t * topk;
  mla_status st = build_schedule(p, kv_len, q_len, num_cus);
  if (st != MLA_OK) {
    delete p;
    return st;
  }
  *out = p;
  return MLA_OK;
}

void mla_plan_destroy(mla_plan* p) { delete p; }

size_t mla_plan_workspace_bytes(const mla_plan* p) { return p ? p->ws_bytes : 0; }
int32_t mla_plan_num_work_items(const mla_plan* p) { return p ? (int32_t)p->items.size() : -1; }
int32_t mla_plan_num_split_groups(const mla_plan* p) { return p ? (int32_t)p->groups.size() : -1; }

int32_t mla_plan_num_workgroups(const mla_plan* p) { return p ? p->num_wgs : -1; }
int32_t mla_plan_group_size(const mla_plan* p) { return p ? p->group_size : -1; }

mla_status mla_plan_get_workgroup_ptr(const mla_plan* p, int32_t* out, size_t capacity) {
  if (!p || !out || capacity < p->wg_ptr.size()) return MLA_ERR_INVALID_ARGUMENT;
  std::memcpy(out, p->wg_ptr.data(), p->wg_ptr.size() * 4);
  return MLA_OK;
}

mla_status mla_plan_get_work_items(const mla_plan* p, int32_t* items_host, size_t capacity) {
  if (!p || (!items_host && !p->items.empty())) return MLA_ERR_INVALID_ARGUMENT;
  if (capacity < p->items.size()) return MLA_ERR_INVALID_ARGUMENT;
  if (!p->items.empty()) std::memcpy(items_host, p->items.data(), p->items.size() * sizeof(WorkItem));
  return MLA_OK;
}

mla_status mla_plan_upload(const mla_plan* p, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!p) return MLA_ERR_INVALID_ARGUMENT;
  if (p->blob.empty()) return MLA_OK;
  if (!ws || ws_bytes < p->ws_bytes || ((uintptr_t)ws % mla::kWsAlign) != 0) return MLA_ERR_WORKSPACE;
  if (hipMemcpyAsync(ws, p->blob.data(), p->blob.size() * 4, hipMemcpyHostToDevice, stream) != hipSuccess)
    return MLA_ERR_DEVICE;
  return MLA_OK;
}

}  // extern "C"

namespace {

thread_local hipEvent_t t_ev_before = nullptr;
thread_local hipEvent_t t_ev_after = nullptr;

// Row strides of the two bf16 layouts: split ckv / kpe tensors and q_nope /
// q_pe, or one concatenated 576-wide row per token (latent then rope).
struct Layout {
  int32_t ckv_stride, kpe_stride, q_stride, qpe_stride;
};
constexpr Layout kSplit{mla::kDimCkv * 2, mla::kDimKpe * 2, mla::kDimCkv, mla::kDimKpe};
constexpr Layout kPacked{(mla::kDimCkv + mla::kDimKpe) * 2, (mla::kDimCkv + mla::kDimKpe) * 2,
                         mla::kDimCkv + mla::kDimKpe, mla::kDimCkv + mla::kDimKpe};
// MODEL1 queries: one 512-wide row per (token, head), 448 NoPE dims then 64 RoPE dims.
constexpr int kM1Nope = 448;
constexpr Layout kModel1Q{0, 0, kM1Nope + mla::kDimKpe, kM1Nope + mla::kDimKpe};

// Inputs of the token-sparse decode beyond the dense ones.
struct Sparse {
  const int32_t* indices = nullptr;
  const int32_t* topk_length = nullptr;
  const float* attn_sink = nullptr;
  float* max_logits = nullptr;
};

// The opt-in device-array checks (desc.validate = 1): one small kernel, then
// the stream is synchronised and its result read back, before anything
// reads through the arrays.
mla_status validate_arrays(const mla_plan* p, char* w, const int32_t* qo_indptr, const int32_t* kv_indptr,
                           const int32_t* kv_indices, const int32_t* live_kv_len, hipStream_t stream) {
  mla::ValidateArgs v{};
  v.kv_indptr = kv_indptr;
  v.kv_indices = kv_indices;
  v.qo_indptr = p->d.kind == MLA_KIND_PREFILL ? qo_indptr : nullptr;
  v.live_kv_len = live_kv_len;
  v.plan_kv_indptr = (const int32_t*)(w + p->off_plan_kv);
  v.plan_qo_indptr = p->qo_indptr.empty() ? nullptr : (const int32_t*)(w + p->off_plan_qo);
  v.batch = p->d.batch;
  v.page_size = p->d.page_size;
  v.num_pages = p->d.num_pages;
  v.max_kv_len = p->d.max_kv_len;
  v.max_q = p->max_q;
  v.causal = p->d.kind == MLA_KIND_PREFILL ? p->d.causal : 0;
  v.status = (int32_t*)(w + p->off_status);
  if (mla::launch_validate(v, stream) != hipSuccess) return MLA_ERR_DEVICE;
  int32_t flags = -1;
  if (hipMemcpyAsync(&flags, v.status, 4, hipMemcpyDeviceToHost, stream) != hipSuccess) return MLA_ERR_DEVICE;
  if (hipStreamSynchronize(stream) != hipSuccess) return MLA_ERR_DEVICE;
  return flags == 0 ? MLA_OK : MLA_ERR_INVALID_ARGUMENT;
}

mla_status run(const mla_plan* p, int32_t want_kind, int32_t want_format, const void* q_nope,
               const void* q_pe, const void* ckv, const void* kpe, const void* kv_fp8,
               const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
               float sm_scale, void* out, int32_t out_dtype, float* lse, void* ws, size_t ws_bytes,
               hipStream_t stream, const Layout& lay = kSplit, float out_scale = 1.f,
               const Sparse* sparse = nullptr, bool q8 = false, const int32_t* live_kv_len = nullptr,
               bool live = false) {
  if (!p) return MLA_ERR_INVALID_ARGUMENT;
  if (p->d.kind != want_kind || p->d.kv_format != want_format) return MLA_ERR_PLAN_MISMATCH;
  if ((p->capacity != 0) != live) return MLA_ERR_PLAN_MISMATCH;
  if (live && !live_kv_len) return MLA_ERR_INVALID_ARGUMENT;
  if (out_dtype != MLA_DTYPE_BF16 && out_dtype != MLA_DTYPE_FP32) return MLA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(sm_scale) || !std::isfinite(out_scale)) return MLA_ERR_INVALID_ARGUMENT;
  if (p->items.empty()) return MLA_OK;  // nothing to compute (batch 0 or no rows)
  if (!q_nope || !q_pe || !out || !lse) return MLA_ERR_INVALID_ARGUMENT;
  if (sparse ? !sparse->indices : (!kv_indptr || !kv_indices)) return MLA_ERR_INVALID_ARGUMENT;
  if (want_format == MLA_KV_BF16 && (!ckv || !kpe)) return MLA_ERR_INVALID_ARGUMENT;
  if (want_format != MLA_KV_BF16 && !kv_fp8) return MLA_ERR_INVALID_ARGUMENT;
  if (want_kind == MLA_KIND_PREFILL && !qo_indptr) return MLA_ERR_INVALID_ARGUMENT;
  if (!ws || ws_bytes < p->ws_bytes || ((uintptr_t)ws % mla::kWsAlign) != 0) return MLA_ERR_WORKSPACE;
  if (q8 && p->tile_mode != MLA_TILE_WIDE) return MLA_ERR_UNSUPPORTED;
  char* w = (char*)ws;
  if (p->d.validate && !sparse) {
    const mla_status vs = validate_arrays(p, w, qo_indptr, kv_indptr, kv_indices, live_kv_len, stream);
    if (vs != MLA_OK) return vs;
  }
  if (sparse) {
    // the lists are compacted into the workspace first; the attention kernel
    // then reads them as page lists of page size 1
    int32_t* list = (int32_t*)(w + p->off_sp_list);
    int32_t* count = (int32_t*)(w + p->off_sp_count);
    int32_t* indptr = (int32_t*)(w + p->off_sp_indptr);
    if (mla::launch_sparse_lists(sparse->indices, p->d.batch, p->topk, sparse->topk_length,
                                 (int64_t)p->d.num_pages * p->d.page_size, list, count, indptr,
                                 stream) != hipSuccess)
      return MLA_ERR_DEVICE;
    kv_indptr = indptr;
    kv_indices = list;
  }

  mla::AttnArgs a{};
  a.q_nope = q_nope;
  a.q_pe = q_pe;
  a.ckv = ckv;
  a.kpe = kpe;
  a.kv_fp8 = kv_fp8;
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.qo_indptr = (want_kind == MLA_KIND_PREFILL) ? qo_indptr : nullptr;
  a.wg_ptr = (const int32_t*)w;
  a.items = (const WorkItem*)(w + p->off_items);
  a.groups = (const SplitGroup*)(w + p->off_groups);
  a.out = out;
  a.lse = lse;
  a.part_o = (__bf16*)(w + p->off_part_o);
  a.part_lse = (float*)(w + p->off_part_lse);
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.num_heads = p->d.num_qo_heads;
  a.page_shift = ilog2(p->d.page_size);
  a.out_bf16 = out_dtype == MLA_DTYPE_BF16;
  a.causal = (want_kind == MLA_KIND_PREFILL) ? p->d.causal : 0;
  a.rows_per_block = p->rows_per_block;
  a.num_wgs = p->num_wgs;
  a.grid = p->grid;
  a.group_size = p->group_size;
  a.xcd_map = p->xcd_map;
  a.num_items = (int32_t)p->items.size();
  a.num_groups = (int32_t)p->groups.size();
  a.ckv_stride = lay.ckv_stride;
  a.kpe_stride = lay.kpe_stride;
  a.q_stride = lay.q_stride;
  a.qpe_stride = lay.qpe_stride;
  a.out_scale = out_scale;
  a.live_kv_len = live_kv_len;
  a.live_q = (live && want_kind == MLA_KIND_PREFILL) ? 1 : 0;
  a.lse_sq = p->lse_sq;
  if (sparse) {
    a.sparse_len = (const int32_t*)(w + p->off_sp_count);
    a.attn_sink = sparse->attn_sink;
    a.max_logits = sparse->max_logits;
    a.part_max = (float*)(w + p->off_part_max);
  }
  hipEvent_t ev0 = t_ev_before, ev1 = t_ev_after;
  t_ev_before = t_ev_after = nullptr;
  hipError_t e = sparse ? mla::launch_sparse_attention(a, stream, ev0, ev1, want_format == MLA_KV_FP8_MODEL1)
                 : q8     ? mla::launch_attention_q8(a, stream, ev0, ev1)
                          : mla::launch_attention(a, p->tile_mode, want_format, stream, ev0, ev1);
  if (e != hipSuccess) return MLA_ERR_DEVICE;
  if (!p->groups.empty()) {
    e = mla::launch_combine(a, stream);
    if (e != hipSuccess) return MLA_ERR_DEVICE;
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_record_attention_events(hipEvent_t before, hipEvent_t after) {
  if ((before == nullptr) != (after == nullptr)) return MLA_ERR_INVALID_ARGUMENT;
  t_ev_before = before;
  t_ev_after = after;
  return MLA_OK;
}

mla_status mla_decode(const mla_plan* p, const void* q_nope, const void* q_pe, const void* ckv,
                      const void* kpe, const int32_t* kv_indptr, const int32_t* kv_indices,
                      float sm_scale, void* out, int32_t out_dtype, float* lse, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  return run(p, MLA_KIND_DECODE, MLA_KV_BF16, q_nope, q_pe, ckv, kpe, nullptr, nullptr, kv_indptr,
             kv_indices, sm_scale, out, out_dtype, lse, ws, ws_bytes, stream);
}

mla_status mla_prefill(const mla_plan* p, const void* q_nope, const void* q_pe, const void* ckv,
                       const void* kpe, const int32_t* qo_indptr, const int32_t* kv_indptr,
                       const int32_t* kv_indices, float sm_scale, void* out, int32_t out_dtype,
                       float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return run(p, MLA_KIND_PREFILL, MLA_KV_BF16, q_nope, q_pe, ckv, kpe, nullptr, qo_indptr, kv_indptr,
             kv_indices, sm_scale, out, out_dtype, lse, ws, ws_bytes, stream);
}

mla_status mla_decode_live(const mla_plan* p, const void* q_nope, const void* q_pe, const void* ckv,
                           const void* kpe, const int32_t* kv_len, const int32_t* kv_indptr,
                           const int32_t* kv_indices, float sm_scale, void* out, int32_t out_dtype, float* lse,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  return run(p, MLA_KIND_DECODE, MLA_KV_BF16, q_nope, q_pe, ckv, kpe, nullptr, nullptr, kv_indptr, kv_indices,
             sm_scale, out, out_dtype, lse, ws, ws_bytes, stream, kSplit, 1.f, nullptr, false, kv_len, true);
}

mla_status mla_prefill_live(const mla_plan* p, const void* q_nope, const void* q_pe, const void* ckv,
                            const void* kpe, const int32_t* qo_indptr, const int32_t* kv_len,
                            const int32_t* kv_indptr, const int32_t* kv_indices, float sm_scale, void* out,
                            int32_t out_dtype, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return run(p, MLA_KIND_PREFILL, MLA_KV_BF16, q_nope, q_pe, ckv, kpe, nullptr, qo_indptr, kv_indptr, kv_indices,
             sm_scale, out, out_dtype, lse, ws, ws_bytes, stream, kSplit, 1.f, nullptr, false, kv_len, true);
}

mla_status mla_decode_fp8(const mla_plan* p, const void* q_nope, const void* q_pe, const void* kv,
                          const int32_t* kv_indptr, const int32_t* kv_indices, float sm_scale,
                          void* out, int32_t out_dtype, float* lse, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  return run(p, MLA_KIND_DECODE, MLA_KV_FP8_E4M3_T128, q_nope, q_pe, nullptr, nullptr, kv, nullptr,
             kv_indptr, kv_indices, sm_scale, out, out_dtype, lse, ws, ws_bytes, stream);
}

mla_status mla_decode_fp8_q8(const mla_plan* p, const void* q, const void* kv, const int32_t* kv_indptr,
                             const int32_t* kv_indices, float sm_scale, void* out, int32_t out_dtype, float* lse,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* qb = (const char*)q;
  // q rows are 576 one-byte codes: the concatenated layout's element strides
  return run(p, MLA_KIND_DECODE, MLA_KV_FP8_E4M3_T128, q, q ? qb + mla::kDimCkv : nullptr, nullptr, nullptr, kv,
             nullptr, kv_indptr, kv_indices, sm_scale, out, out_dtype, lse, ws, ws_bytes, stream, kPacked, 1.f, nullptr,
             true);
}

mla_status mla_decode_packed(const mla_plan* p, const void* q, const void* kv_cache, const int32_t* kv_indptr,
                             const int32_t* kv_indices, float sm_scale, float out_scale, void* out,
                             int32_t out_dtype, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* qb = (const char*)q;
  const char* kb = (const char*)kv_cache;
  return run(p, MLA_KIND_DECODE, MLA_KV_BF16, q, q ? qb + mla::kDimCkv * 2 : nullptr, kv_cache,
             kv_cache ? kb + mla::kDimCkv * 2 : nullptr, nullptr, nullptr, kv_indptr, kv_indices, sm_scale, out,
             out_dtype, lse, ws, ws_bytes, stream, kPacked, out_scale);
}

mla_status mla_prefill_packed(const mla_plan* p, const void* q, const void* kv_cache, const int32_t* qo_indptr,
                              const int32_t* kv_indptr, const int32_t* kv_indices, float sm_scale, float out_scale,
                              void* out, int32_t out_dtype, float* lse, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  const char* qb = (const char*)q;
  const char* kb = (const char*)kv_cache;
  return run(p, MLA_KIND_PREFILL, MLA_KV_BF16, q, q ? qb + mla::kDimCkv * 2 : nullptr, kv_cache,
             kv_cache ? kb + mla::kDimCkv * 2 : nullptr, nullptr, qo_indptr, kv_indptr, kv_indices, sm_scale, out,
             out_dtype, lse, ws, ws_bytes, stream, kPacked, out_scale);
}

mla_status mla_sparse_decode_fp8(const mla_plan* p, const void* q, const void* kv_cache, const int32_t* indices,
                                 const int32_t* topk_length, const float* attn_sink, float sm_scale, void* out,
                                 int32_t out_dtype, float* lse, float* max_logits, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  Sparse sp;
  sp.indices = indices;
  sp.topk_length = topk_length;
  sp.attn_sink = attn_sink;
  sp.max_logits = max_logits;
  const char* qb = (const char*)q;
  return run(p, MLA_KIND_SPARSE_DECODE, MLA_KV_FP8_E4M3_T128, q, q ? qb + mla::kDimCkv * 2 : nullptr, nullptr, nullptr,
             kv_cache, nullptr, nullptr, nullptr, sm_scale, out, out_dtype, lse, ws, ws_bytes, stream, kPacked, 1.f,
             &sp);
}

mla_status mla_decode_model1(const mla_plan* p, const void* q, const void* kv_cache, const int32_t* kv_indptr,
                             const int32_t* kv_indices, float sm_scale, void* out, int32_t out_dtype, float* lse,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* qb = (const char*)q;
  return run(p, MLA_KIND_DECODE, MLA_KV_FP8_MODEL1, q, q ? qb + kM1Nope * 2 : nullptr, nullptr, nullptr, kv_cache,
             nullptr, kv_indptr, kv_indices, sm_scale, out, out_dtype, lse, ws, ws_bytes, stream, kModel1Q);
}

mla_status mla_sparse_decode_model1(const mla_plan* p, const void* q, const void* kv_cache, const int32_t* indices,
                                    const int32_t* topk_length, const float* attn_sink, float sm_scale, void* out,
                                    int32_t out_dtype, float* lse, float* max_logits, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  Sparse sp;
  sp.indices = indices;
  sp.topk_length = topk_length;
  sp.attn_sink = attn_sink;
  sp.max_logits = max_logits;
  const char* qb = (const char*)q;
  return run(p, MLA_KIND_SPARSE_DECODE, MLA_KV_FP8_MODEL1, q, q ? qb + kM1Nope * 2 : nullptr, nullptr, nullptr,
             kv_cache, nullptr, nullptr, nullptr, sm_scale, out, out_dtype, lse, ws, ws_bytes, stream, kModel1Q, 1.f,
             &sp);
}

mla_status mla_sparse_prefill(const mla_plan* p, const void* q, const void* kv, const int32_t* indices,
                              const int32_t* topk_length, const float* attn_sink, float sm_scale, void* out,
                              int32_t out_dtype, float* lse, float* max_logits, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  Sparse sp;
  sp.indices = indices;
  sp.topk_length = topk_length;
  sp.attn_sink = attn_sink;
  sp.max_logits = max_logits;
  const char* qb = (const char*)q;
  const char* kb = (const char*)kv;
  return run(p, MLA_KIND_SPARSE_DECODE, MLA_KV_BF16, q, q ? qb + mla::kDimCkv * 2 : nullptr, kv,
             kv ? kb + mla::kDimCkv * 2 : nullptr, nullptr, nullptr, nullptr, nullptr, sm_scale, out, out_dtype, lse,
             ws, ws_bytes, stream, kPacked, 1.f, &sp);
}

mla_status mla_block_table_to_indices(const mla_plan* p, const int32_t* block_table, int32_t max_blocks,
                                      const int32_t* kv_indptr, int32_t* kv_indices, hipStream_t stream) {
  if (!p || max_blocks < 0) return MLA_ERR_INVALID_ARGUMENT;
  if (p->d.batch == 0) return MLA_OK;
  for (int32_t b = 0; b < p->d.batch; ++b)
    if (p->kv_indptr[b + 1] - p->kv_indptr[b] > max_blocks) return MLA_ERR_INVALID_ARGUMENT;
  if (!block_table || !kv_indptr || (!kv_indices && p->kv_indptr[p->d.batch] > 0)) return MLA_ERR_INVALID_ARGUMENT;
  if (mla::launch_block_table(block_table, p->d.batch, max_blocks, kv_indptr, kv_indices, stream) != hipSuccess)
    return MLA_ERR_DEVICE;
  return MLA_OK;
}

mla_status mla_model1_expand_records(const uint8_t* records, int64_t num_tokens, void* rows, hipStream_t stream) {
  if (num_tokens < 0) return MLA_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return MLA_OK;
  if (!records || !rows || ((uintptr_t)records % 4) != 0 || ((uintptr_t)rows % 16) != 0)
    return MLA_ERR_INVALID_ARGUMENT;
  if (mla::launch_model1_records(records, num_tokens, (__bf16*)rows, stream) != hipSuccess) return MLA_ERR_DEVICE;
  return MLA_OK;
}

mla_status mla_model1_expand_q(const void* q, int64_t num_rows, void* q576, hipStream_t stream) {
  if (num_rows < 0) return MLA_ERR_INVALID_ARGUMENT;
  if (num_rows == 0) return MLA_OK;
  if (!q || !q576 || ((uintptr_t)q % 16) != 0 || ((uintptr_t)q576 % 16) != 0) return MLA_ERR_INVALID_ARGUMENT;
  if (mla::launch_model1_q((const __bf16*)q, num_rows, (__bf16*)q576, stream) != hipSuccess) return MLA_ERR_DEVICE;
  return MLA_OK;
}

}  // extern "C"
