// Tile scheduler: integer index math shared by host and device.
//
// A work item is one (batch, query head, query tile).  For each item the
// scheduler gives the query rows it owns and the range of key tiles it must
// visit, already clipped to what the mask can allow:
//   - causal: keys at global positions <= the last query position of the tile
//     (Ring Attention summary, Summary: a host's query block against one
//     key/value block per step, chunk offset k_pos0 = global position);
//   - S2-Attn: keys of the same group of rolled positions, up to the tile's
//     last rolled position (LongLoRA summary, Summary: groups, half of the heads
//     shifted by half a group).  Rolled position r of a shifted head is original
//     row (r + G/2) mod S; tiles never straddle the wrap because the tile sizes
//     divide G/2, so every tile is one contiguous run of original rows.
// Masks are evaluated in "coordinate positions": global positions for plain
// causal attention, rolled positions for S2.
#pragma once

#include "ba_common.h"

namespace ba {

struct Sched {
  int64_t Sq, Sk, q_pos0, k_pos0;
  int32_t causal;
  int32_t s2_group;  // 0: no S2
  int32_t s2_shift;  // rows of roll for this head (0 or group/2)
  int32_t BM, BN;
};

struct QTile {
  int64_t row0;      // original row of the tile's first query
  int64_t rows;      // valid query rows in the tile (<= BM)
  int64_t cpos0;     // coordinate position of the first query
  int64_t kt_begin;  // first key tile to visit
  int64_t kt_end;    // one past the last key tile to visit
};

struct KTile {
  int64_t row0;   // original row (into the key chunk) of the first key
  int64_t rows;   // valid keys in the tile (<= BN)
  int64_t cpos0;  // coordinate position of the first key
};

BA_HD int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

BA_HD int64_t num_qtiles(const Sched& s) { return ceil_div(s.Sq, s.BM); }

BA_HD QTile make_qtile(const Sched& s, int64_t qt) {
  QTile t;
  if (s.s2_group > 0) {
    const int64_t r0 = qt * s.BM;  // rolled position of the first query
    t.row0 = r0 + s.s2_shift >= s.Sq ? r0 + s.s2_shift - s.Sq : r0 + s.s2_shift;
    t.rows = s.BM;
    t.cpos0 = r0;
    const int64_t g0 = (r0 / s.s2_group) * s.s2_group;
    t.kt_begin = g0 / s.BN;
    t.kt_end = ceil_div(r0 + s.BM, s.BN);
    return t;
  }
  t.row0 = qt * s.BM;
  t.rows = s.Sq - t.row0 < s.BM ? s.Sq - t.row0 : s.BM;
  t.cpos0 = s.q_pos0 + t.row0;
  t.kt_begin = 0;
  const int64_t nkt = ceil_div(s.Sk, s.BN);
  if (!s.causal) {
    t.kt_end = nkt;
  } else {
    // last key index j with k_pos0 + j <= q_pos0 + row0 + rows - 1
    const int64_t last = s.q_pos0 + t.row0 + t.rows - 1 - s.k_pos0;
    t.kt_end = last < 0 ? 0 : (last / s.BN + 1 < nkt ? last / s.BN + 1 : nkt);
  }
  return t;
}

BA_HD KTile make_ktile(const Sched& s, int64_t kt) {
  KTile k;
  if (s.s2_group > 0) {
    const int64_t r0 = kt * s.BN;
    k.row0 = r0 + s.s2_shift >= s.Sk ? r0 + s.s2_shift - s.Sk : r0 + s.s2_shift;
    k.rows = s.BN;
    k.cpos0 = r0;
    return k;
  }
  k.row0 = kt * s.BN;
  k.rows = s.Sk - k.row0 < s.BN ? s.Sk - k.row0 : s.BN;
  k.cpos0 = s.k_pos0 + k.row0;
  return k;
}

// Visiting order inside one (batch, head): the w-th item is the query tile with
// the most work first, so that the grid drains with the lightest tiles last.
BA_HD int64_t qtile_of_rank(const Sched& s, int64_t nq, int64_t w) {
  if (s.s2_group > 0) {
    const int64_t per_group = s.s2_group / s.BM;
    const int64_t ngroups = nq / per_group;
    const int64_t pos = per_group - 1 - w / ngroups;
    const int64_t g = w % ngroups;
    return g * per_group + pos;
  }
  return nq - 1 - w;
}

// Key/value-stationary items (backward dK/dV): one item owns BN keys starting
// at key tile kt; the query tiles (of BM rows) it must visit are those holding
// at least one query the mask allows for some key of the item.
struct KVItem {
  int64_t krow0, krows, kcpos0;  // as KTile
  int64_t qt_begin, qt_end;      // query tiles to visit
};

BA_HD KVItem make_kv_item(const Sched& s, int64_t kt) {
  KVItem it;
  const int64_t nq = num_qtiles(s);
  if (s.s2_group > 0) {
    const int64_t r0 = kt * s.BN;
    it.krow0 = r0 + s.s2_shift >= s.Sk ? r0 + s.s2_shift - s.Sk : r0 + s.s2_shift;
    it.krows = s.BN;
    it.kcpos0 = r0;
    const int64_t gend = (r0 / s.s2_group + 1) * s.s2_group;  // end of the key's group (rolled)
    it.qt_begin = r0 / s.BM;
    it.qt_end = gend / s.BM;
    return it;
  }
  it.krow0 = kt * s.BN;
  it.krows = s.Sk - it.krow0 < s.BN ? s.Sk - it.krow0 : s.BN;
  it.kcpos0 = s.k_pos0 + it.krow0;
  it.qt_end = nq;
  if (!s.causal) {
    it.qt_begin = 0;
  } else {
    // first query row i with q_pos0 + i >= kcpos0
    const int64_t first = it.kcpos0 - s.q_pos0;
    it.qt_begin = first <= 0 ? 0 : (first >= s.Sq ? nq : first / s.BM);
  }
  return it;
}

BA_HD int64_t num_ktiles(const Sched& s) { return ceil_div(s.Sk, s.BN); }

// Visiting order of key tiles inside one (batch, key/value head): most query
// tiles first.
BA_HD int64_t ktile_of_rank(const Sched& s, int64_t nk, int64_t w) {
  if (s.s2_group > 0) {
    const int64_t per_group = s.s2_group / s.BN;
    const int64_t ngroups = nk / per_group;
    const int64_t pos = w / ngroups;      // position inside the group, ascending
    const int64_t g = w % ngroups;
    return g * per_group + pos;
  }
  // causal: a later key tile never sees more query tiles than an earlier one,
  // so ascending order is longest first (and any order is, without a mask)
  return w;
}

// Workgroups are handed to the 8 XCDs round-robin (block i -> XCD i % 8).  The
// remap gives XCD x the contiguous logical range [x*per, (x+1)*per), so the
// query tiles of one head (which read the same keys and values) share one L2.
BA_HD int64_t xcd_remap(int64_t pid, int64_t n) {
  const int64_t per = n / 8;
  const int64_t full = per * 8;
  return pid < full ? (pid % 8) * per + pid / 8 : pid;
}

// (batch*head, rank) of logical item pid of a query-stationary launch with
// n_ranks tiles per (batch, head).  Head-major by default: an XCD's slots work
// through one head's tiles (longest first) before the next head's, so the
// key/value rows they share stay in its L2.  When a launch has few ranks per
// head (an XCD's 64 slots would see only a round or two of one head's tiles)
// and its heads split evenly over the XCDs, the XCD's heads are taken in groups
// of hx, each group rank-major: every head of the group starts its longest tile
// first, so the launch is not left waiting on a late head's longest tile, while
// only hx heads' keys and values are live in the XCD at a time.
BA_HD void qitem_of_pid(int64_t pid, int64_t n_ranks, int64_t hx, int64_t& bh, int64_t& w) {
  if (hx > 1) {
    const int64_t per = hx * n_ranks;  // items of one group
    const int64_t j = pid % per;
    bh = (pid / per) * hx + j % hx;
    w = j / hx;
  } else {
    bh = pid / n_ranks;
    w = pid % n_ranks;
  }
}

// Group size hx for qitem_of_pid, or 0 for head-major order: enough heads for two
// rounds of an XCD's workgroup slots (256 CUs in 8 XCDs; slots = workgroups an XCD
// runs at once), a divisor of the heads each XCD takes.
inline int64_t interleave_heads(int64_t n_bh, int64_t n_ranks, int64_t slots) {
  if (n_ranks <= 0 || n_ranks >= 2 * slots || n_bh % 8 != 0) return 0;
  const int64_t per_xcd = n_bh / 8;
  int64_t g = (2 * slots + n_ranks - 1) / n_ranks;
  if (g > per_xcd) g = per_xcd;
  while (per_xcd % g != 0) --g;
  return g;
}

}  // namespace ba
