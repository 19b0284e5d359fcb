// Host-side slice validation and block-sparse planning.  See planner.hpp.
#include "planner.hpp"

#include <algorithm>
#include <numeric>
#include <map>
#include <limits>
#include <tuple>

namespace ffa {

std::string check_slice(int64_t Tq, int64_t Tk, const int32_t* q_ranges, const int32_t* k_ranges,
                        const int32_t* types, int r) {
  const int64_t qs = q_ranges[2 * r], qe = q_ranges[2 * r + 1];
  const int64_t ks = k_ranges[2 * r], ke = k_ranges[2 * r + 1];
  const int32_t t = types[r];
  if (qs < 0 || qe < qs || qe > Tq)
    return "slice " + std::to_string(r) + ": q range [" + std::to_string(qs) + ", " +
           std::to_string(qe) + ") is not inside [0, " + std::to_string(Tq) + ")";
  if (ks < 0 || ke < ks || ke > Tk)
    return "slice " + std::to_string(r) + ": k range [" + std::to_string(ks) + ", " +
           std::to_string(ke) + ") is not inside [0, " + std::to_string(Tk) + ")";
  if (t != kFull && t != kCausal)
    return "slice " + std::to_string(r) + ": attention type " + std::to_string(t) +
           " is neither FULL (0) nor CAUSAL (1)";
  return "";
}

std::string validate_slices(int64_t Tq, int64_t Tk, const int32_t* q_ranges,
                            const int32_t* k_ranges, const int32_t* types, int R,
                            std::vector<Slice>* out) {
  out->clear();
  if (R < 0) return "R must be >= 0";
  if (R > 0 && (!q_ranges || !k_ranges || !types)) return "slice arrays must not be NULL when R > 0";
  out->reserve(static_cast<size_t>(R));
  for (int r = 0; r < R; ++r) {
    std::string m = check_slice(Tq, Tk, q_ranges, k_ranges, types, r);
    if (!m.empty()) return m;
    const int64_t qs = q_ranges[2 * r], qe = q_ranges[2 * r + 1];
    const int64_t ks = k_ranges[2 * r], ke = k_ranges[2 * r + 1];
    const int32_t t = types[r];
    // a zero-length range on either axis covers no cell: drop it
    if (qs == qe || ks == ke) continue;
    out->push_back(Slice{static_cast<int32_t>(qs), static_cast<int32_t>(qe),
                         static_cast<int32_t>(ks), static_cast<int32_t>(ke), t, r});
  }
  return "";
}

namespace {

// Visible columns of row i under slice s, as [lo, hi) (empty when hi <= lo).
inline void row_span(const Slice& s, int64_t i, int64_t* lo, int64_t* hi) {
  *lo = s.ks;
  *hi = s.ke;
  if (s.type == kCausal) *hi = std::min<int64_t>(s.ke, i + 1 + (int64_t(s.ke) - s.qe));
}

}  // namespace

std::string check_disjoint(const std::vector<Slice>& s) {
  for (size_t a = 0; a < s.size(); ++a) {
    for (size_t b = a + 1; b < s.size(); ++b) {
      const int64_t r0 = std::max(s[a].qs, s[b].qs), r1 = std::min(s[a].qe, s[b].qe);
      const int64_t c0 = std::max(s[a].ks, s[b].ks), c1 = std::min(s[a].ke, s[b].ke);
      if (r0 >= r1 || c0 >= c1) continue;
      // rectangles meet; the slices share a cell iff some row's spans meet.
      // Both spans start at their ks, so per row the overlap is
      // [c0, min(hi_a, hi_b)); that is monotone in the row, so the last
      // common row decides.
      int64_t la, ha, lb, hb;
      row_span(s[a], r1 - 1, &la, &ha);
      row_span(s[b], r1 - 1, &lb, &hb);
      if (std::min(ha, hb) > c0)
        return "slices " + std::to_string(s[a].r) + " and " + std::to_string(s[b].r) +
               " cover the same cells";
    }
  }
  return "";
}

void build_plan(const std::vector<Slice>& slices, int64_t Tq, int64_t Tk, int bm, int bn,
                bool transpose, Plan* plan) {
  const int64_t nqt = (Tq + bm - 1) / bm;
  const int64_t nkt = (Tk + bn - 1) / bn;
  struct Item {
    int64_t tile, other;
    int32_t slice, kind;
  };
  std::vector<Item> items;

  for (size_t si = 0; si < slices.size(); ++si) {
    const Slice& s = slices[si];
    const int64_t diag = int64_t(s.ke) - s.qe;  // CAUSAL: row i sees j <= i + diag
    for (int64_t qt = s.qs / bm; qt <= (int64_t(s.qe) - 1) / bm; ++qt) {
      const int64_t r0 = qt * bm, r1 = r0 + bm;
      int64_t a = std::max<int64_t>(r0, s.qs);
      const int64_t b = std::min<int64_t>(r1, s.qe);
      int64_t col_end = s.ke;  // exclusive bound on visible columns in these rows
      if (s.type == kCausal) {
        a = std::max<int64_t>(a, int64_t(s.ks) - diag);  // first row that sees a key
        col_end = std::min<int64_t>(s.ke, b + diag);     // last row sees the most
      }
      if (a >= b || col_end <= s.ks) continue;
      const bool rows_full = (r0 >= s.qs) && (r1 <= s.qe);
      for (int64_t kt = s.ks / bn; kt <= (col_end - 1) / bn; ++kt) {
        const int64_t c0 = kt * bn, c1 = c0 + bn;
        bool full = rows_full && c0 >= s.ks && c1 <= s.ke;
        // CAUSAL: the tile's top-right cell is the last one to become visible
        if (full && s.type == kCausal) full = (c1 - 1) <= (r0 + diag);
        const int32_t kind = full ? kEntryFull : kEntryPartial;
        if (transpose)
          items.push_back(Item{kt, qt, static_cast<int32_t>(si), kind});
        else
          items.push_back(Item{qt, kt, static_cast<int32_t>(si), kind});
      }
    }
  }

  // canonical order: by tile, then other tile, then the slice's bounds
  std::sort(items.begin(), items.end(), [&](const Item& x, const Item& y) {
    const Slice& sx = slices[x.slice];
    const Slice& sy = slices[y.slice];
    return std::make_tuple(x.tile, x.other, sx.qs, sx.qe, sx.ks, sx.ke, sx.type, sx.r) <
           std::make_tuple(y.tile, y.other, sy.qs, sy.qe, sy.ks, sy.ke, sy.type, sy.r);
  });

  plan->n_tiles = transpose ? nkt : nqt;
  plan->row_ptr.assign(static_cast<size_t>(plan->n_tiles + 1), 0);
  plan->entries.resize(items.size());
  for (size_t e = 0; e < items.size(); ++e) {
    plan->row_ptr[static_cast<size_t>(items[e].tile) + 1]++;
    plan->entries[e] = PlanEntry{static_cast<int32_t>(items[e].other), items[e].slice, items[e].kind};
  }
  for (int64_t t = 0; t < plan->n_tiles; ++t) plan->row_ptr[t + 1] += plan->row_ptr[t];

  // Order of tiles.  Tiles are grouped by the first query row of the slices
  // their lists meet (for a packed batch: one document), groups go by their
  // longest list, tiles inside a group by their own length (ties: lower tile
  // first).  Longest-first keeps the kernels' tail short; keeping a
  // document's tiles together means the workgroups resident on one XCD at the
  // same time walk the same K/V (or Q/dO) tiles and share them in L2.
  const int64_t nt = plan->n_tiles;
  std::vector<int64_t> key(static_cast<size_t>(nt), std::numeric_limits<int64_t>::max());
  std::vector<int32_t> len(static_cast<size_t>(nt));
  for (int64_t t = 0; t < nt; ++t) {
    len[t] = plan->row_ptr[t + 1] - plan->row_ptr[t];
    for (int32_t e = plan->row_ptr[t]; e < plan->row_ptr[t + 1]; ++e)
      key[t] = std::min<int64_t>(key[t], slices[plan->entries[e].slice].qs);
  }
  std::map<int64_t, int32_t> group_len;  // key -> longest list in the group
  for (int64_t t = 0; t < nt; ++t) {
    int32_t& m = group_len[key[t]];
    m = std::max(m, len[t]);
  }
  plan->order.resize(static_cast<size_t>(nt));
  std::iota(plan->order.begin(), plan->order.end(), 0);
  std::sort(plan->order.begin(), plan->order.end(), [&](int32_t x, int32_t y) {
    const int32_t gx = group_len[key[x]], gy = group_len[key[y]];
    return std::make_tuple(-gx, key[x], -len[x], x) < std::make_tuple(-gy, key[y], -len[y], y);
  });
}

std::string block_slices(int64_t Tq, int64_t Tk, int block_q, int block_k, const int32_t* num,
                         const int32_t* idx, int width, std::vector<RangePair>* out) {
  out->clear();
  if (Tq < 0 || Tk < 0) return "Tq and Tk must be >= 0";
  if (block_q <= 0 || block_k <= 0) return "block sizes must be positive";
  if (width < 0) return "max_blocks must be >= 0";
  const int64_t n_qb = (Tq + block_q - 1) / block_q, n_kb = (Tk + block_k - 1) / block_k;
  if (n_qb > 0 && (!num || (width > 0 && !idx))) return "block arrays must not be NULL";
  // key ranges open from an earlier query block: (ks, ke) -> first row
  std::map<std::pair<int64_t, int64_t>, int64_t> open;
  auto emit = [&](int64_t qs, int64_t qe, int64_t ks, int64_t ke) {
    out->push_back(RangePair{static_cast<int32_t>(qs), static_cast<int32_t>(qe), static_cast<int32_t>(ks),
                             static_cast<int32_t>(ke)});
  };
  std::vector<int64_t> kb;
  for (int64_t b = 0; b < n_qb; ++b) {
    const int64_t n = num[b];
    if (n < 0 || n > width)
      return "query block " + std::to_string(b) + ": count " + std::to_string(n) + " is not in [0, " +
             std::to_string(width) + "]";
    kb.assign(idx + b * width, idx + b * width + n);
    std::sort(kb.begin(), kb.end());
    for (size_t i = 0; i < kb.size(); ++i) {
      if (kb[i] < 0 || kb[i] >= n_kb)
        return "query block " + std::to_string(b) + ": key block " + std::to_string(kb[i]) +
               " is not in [0, " + std::to_string(n_kb) + ")";
      if (i > 0 && kb[i] == kb[i - 1])
        return "query block " + std::to_string(b) + ": key block " + std::to_string(kb[i]) + " listed twice";
    }
    // this block's key ranges: runs of adjacent key blocks
    std::map<std::pair<int64_t, int64_t>, int64_t> now;
    for (size_t i = 0; i < kb.size();) {
      size_t j = i + 1;
      while (j < kb.size() && kb[j] == kb[j - 1] + 1) ++j;
      const int64_t ks = kb[i] * block_k, ke = std::min<int64_t>(Tk, (kb[j - 1] + 1) * block_k);
      auto it = open.find({ks, ke});
      now[{ks, ke}] = it != open.end() ? it->second : b * block_q;
      i = j;
    }
    for (const auto& o : open)
      if (!now.count(o.first)) emit(o.second, b * block_q, o.first.first, o.first.second);
    open.swap(now);
  }
  for (const auto& o : open) emit(o.second, Tq, o.first.first, o.first.second);
  std::sort(out->begin(), out->end(), [](const RangePair& x, const RangePair& y) {
    return std::tie(x.qs, x.ks) < std::tie(y.qs, y.ks);
  });
  return "";
}

}  // namespace ffa
