// fa_prefill_plan.h -- the work plan of the chunked prefill against a paged cache.
//
// The plan turns the per-sequence lengths (known only on the device) into work items for a
// persistent kernel, in the order that balances the chip.  It is plain integer arithmetic with
// no GPU types, so the same functions run in the plan kernel and, compiled for the host, in a
// CPU check of the plan's invariants (every output row written exactly once, every visible key
// of a row in exactly one piece, every index inside its buffer).
//
// Vocabulary.  A sequence b has L_b keys in the cache and a chunk of its newest Q_b tokens as
// queries, at key positions off_b = L_b - Q_b .. L_b - 1 (causal with that offset).  Its
// Hkv * hgk "units" are (kv head, head subset) pairs: a work item of a unit covers RPH query rows
// of each of the HP query heads of the subset (NW waves of 32 rows: RPH = 32 NW / HP), so the
// heads that share a kv head read each key/value tile once.  The unit's query blocks
// qb = 0 .. ceil(Q_b / RPH) - 1 each need the key tiles 0 .. n_kt(b, qb) - 1 (64 keys per tile);
// blocks past the chunk (up to ceil(max_q / RPH)) are "zero" items that only write the padding
// output.  A block whose key loop is longer than T tiles is split into np = ceil(n_kt / T)
// pieces of at most T tiles each ("Split-KV"): the pieces run as separate items and write partial
// results, merged exactly afterwards as the online softmax merges any two blocks of keys
// ("FlashAttention优化" §3.2.2).
//
// T = max(kMinPieceTiles, ceil(W / (2 R))), W the total key tiles of all query blocks and R the
// number of resident workgroups: no item is longer than twice the average share of a workgroup,
// and the split pieces number at most 4 R (a block with n > T tiles gives ceil(n / T) < 2 n / T
// pieces, and the sum of n over those blocks is at most W <= 2 R T), which bounds the partials
// workspace independently of the lengths.
//
// Order.  Units are ranked by key length L_b (longest first: a unit's items cost up to L_b key
// tiles each), and dealt to the 8 XCDs in a snake (0..7, 7..0, ...), each XCD keeping a list: a
// unit's items sit together in one list, pieces-major (piece p of every query block, then piece
// p + 1), so the items running side by side on one XCD read the same key tiles through its L2.
// Each list holds its units' real items first and their zero items last.
//
// Placement.  The attention kernel runs one workgroup per item, and workgroup w runs on XCD
// w mod 8 (workgroups are dealt round-robin over the XCDs), so item k of list x goes to
// position 8 k + x of one dense array: each XCD meets its list in order, and the hardware
// dispatcher hands the next item to whichever slot frees first.  The lists are first evened
// out: with c* = ceil(total / 8), the items of a list past position c* (the tail: zero items,
// or the lightest real ones) fill the positions c_x' .. c* - 1 of the shorter lists.  At most 7
// positions below 8 c* stay empty; workgroups at or past 8 c* exit at once.
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#define FA_PLAN_FN __host__ __device__ inline
#else
#define FA_PLAN_FN inline
#endif

namespace fa {
namespace plan {

constexpr int kTileKeys = 64;        // keys per tile of the forward kernel
constexpr int kXcds = 8;             // accelerator complex dies of an MI355X
constexpr int kMinPieceTiles = 16;   // shortest split piece (1024 keys)
constexpr int kItemInts = 8;         // ints per work item
constexpr int kMergeInts = 8;        // ints per merge entry
constexpr int kPageRows = 16;        // tokens per physical block of the cache
constexpr int kDirect = -1;          // item slot value: unsplit, writes O and LSE itself
constexpr int kZeroItem = -2;        // item slot value: padding rows only
constexpr int kBadItem = -3;         // item slot value: never produced (a bound was exceeded)

// Work item: {b, hg (unit index within the sequence), qb, t0, t1, slot, 0, 0}; slot >= 0 is the
// partials slot of a split piece; b = -1 marks an empty position.  Merge entry:
// {b, hg, qb, slot0, np, 0, 0, 0}.
// Header (ints): count[8] (list lengths), excess_base[8], deficit_base[8] (prefix sums of the
// lists' surplus over c* and shortfall below it), n_merge, T, items, ok, c*, positions (8 c*).
constexpr int kHdrCount = 0, kHdrExcess = 8, kHdrDeficit = 16, kHdrMerge = 24, kHdrT = 25,
              kHdrItems = 26, kHdrOk = 27, kHdrCstar = 28, kHdrPositions = 29, kHdrInts = 64;

struct Shape {
  int S;          // sequences
  int max_q;      // query rows per (sequence, head) in q and o
  int Hkv;        // kv heads
  int hgk;        // head subsets per kv head (group / HP)
  int rph;        // query rows per head of a work item (pairs / HP)
  int pairs;      // (head, row) pairs of one work item = one partials slot (32 rows per wave)
  int max_keys;   // max_blocks_per_seq * 16: the longest sequence the block table can hold
  int R;          // resident workgroups of the attention kernel
};

FA_PLAN_FN int imin(int a, int b) { return a < b ? a : b; }
FA_PLAN_FN int imax(int a, int b) { return a > b ? a : b; }

FA_PLAN_FN int units_per_seq(const Shape& s) { return s.Hkv * s.hgk; }
FA_PLAN_FN int blocks_per_unit(const Shape& s) { return (s.max_q + s.rph - 1) / s.rph; }

// Clamped lengths of a sequence: L in [0, max_keys], Q in [0, min(L, max_q)].
FA_PLAN_FN int seq_keys(const Shape& s, int L_raw) { return imin(imax(L_raw, 0), s.max_keys); }
FA_PLAN_FN int seq_queries(const Shape& s, int L, int Q_raw) {
  return imin(imax(Q_raw, 0), imin(L, s.max_q));
}
FA_PLAN_FN int real_blocks(const Shape& s, int Q) { return (Q + s.rph - 1) / s.rph; }

// Key tiles query block qb of a sequence needs: keys 0 .. min(L, off + (qb + 1) * RPH) - 1.
FA_PLAN_FN int key_tiles(const Shape& s, int L, int Q, int qb) {
  const long long end = (long long)(L - Q) + (long long)(qb + 1) * s.rph;
  const int kv_end = end < L ? (int)end : L;
  return (kv_end + kTileKeys - 1) / kTileKeys;
}

FA_PLAN_FN int pieces(int tiles, int T) { return tiles <= T ? 1 : (tiles + T - 1) / T; }

// Piece p of np over n tiles: [t0, t1), every piece non-empty and at most T tiles long.
FA_PLAN_FN void piece_range(int n, int np, int p, int* t0, int* t1) {
  const int per = (n + np - 1) / np;
  *t0 = imin(p * per, n);
  *t1 = imin(*t0 + per, n);
}

FA_PLAN_FN int split_tiles(long long W, int R) {
  const long long t = (W + 2LL * R - 1) / (2LL * R);
  return t < kMinPieceTiles ? kMinPieceTiles : (t > (1 << 30) ? (1 << 30) : (int)t);
}

// XCD of the unit at global rank position u (snake order; u < 2^31 by the size checks).
FA_PLAN_FN int unit_xcd(int u) {
  const int r = u & (kXcds - 1);
  return ((u / kXcds) & 1) ? kXcds - 1 - r : r;
}

// Units u' < n with unit_xcd(u') == x: each period of 16 holds two (x and 15 - x).
FA_PLAN_FN int units_below_on_xcd(int n, int x) {
  const int m = n & (2 * kXcds - 1);
  return 2 * (n / (2 * kXcds)) + (m > x) + (m > 2 * kXcds - 1 - x);
}

// Upper bounds that size the workspace (host) and guard every index (device).
FA_PLAN_FN long long max_split_slots(const Shape& s) { return 4LL * s.R; }
FA_PLAN_FN long long max_merge_entries(const Shape& s) { return 2LL * s.R; }
FA_PLAN_FN long long max_items(const Shape& s) {
  return (long long)s.S * units_per_seq(s) * blocks_per_unit(s) + max_split_slots(s);
}
// Positions of the dense item array (and workgroups of the attention grid): 8 c* <= this.
FA_PLAN_FN long long max_positions(const Shape& s) { return (max_items(s) + kXcds - 1) / kXcds * kXcds; }

// Per-sequence totals for the split length T.
struct SeqCounts {
  int items;    // real items of one unit (sum of pieces over its query blocks)
  int zeros;    // zero items of one unit
  int slots;    // partials slots of one unit (pieces of its split blocks)
  int entries;  // merge entries of one unit (its split blocks)
};

FA_PLAN_FN long long seq_tiles(const Shape& s, int L, int Q) {
  long long t = 0;
  const int nb = real_blocks(s, Q);
  for (int qb = 0; qb < nb; ++qb) t += key_tiles(s, L, Q, qb);
  return t;
}

FA_PLAN_FN SeqCounts seq_counts(const Shape& s, int L, int Q, int T) {
  SeqCounts c = {0, 0, 0, 0};
  const int nb = real_blocks(s, Q);
  for (int qb = 0; qb < nb; ++qb) {
    const int np = pieces(key_tiles(s, L, Q, qb), T);
    c.items += np;
    if (np > 1) {
      c.slots += np;
      c.entries += 1;
    }
  }
  c.zeros = blocks_per_unit(s) - nb;
  return c;
}

// Index of unit j of the sequence at rank r among that sequence's units on XCD x.
FA_PLAN_FN int unit_rank_on_xcd(int nu, int r, int j) {
  const int u0 = r * nu;
  const int x = unit_xcd(u0 + j);
  return units_below_on_xcd(u0 + j, x) - units_below_on_xcd(u0, x);
}

// Units of the sequence at rank r that land on XCD x.
FA_PLAN_FN int units_on_xcd(int nu, int r, int x) {
  return units_below_on_xcd((r + 1) * nu, x) - units_below_on_xcd(r * nu, x);
}


// ---------------------------------------------------------------------------------------------
// Workspace layout (byte offsets, each region 256-byte aligned).  Per-sequence arrays are
// indexed by rank; pos_real / pos_zero by XCD * S + rank.
struct Layout {
  size_t hdr, order, len_k, len_q, n_items, n_zero, n_slots, n_entries, slot_base, entry_base,
      pos_real, pos_zero, items, merge, opart, mpart, lpart, total;
};

FA_PLAN_FN size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

FA_PLAN_FN Layout layout(const Shape& s, int d) {
  Layout l;
  size_t o = 0;
  const size_t S = (size_t)s.S;
  const size_t slots = (size_t)max_split_slots(s);
  l.hdr = o;        o = align256(o + sizeof(int) * kHdrInts);
  l.order = o;      o = align256(o + sizeof(int) * S);
  l.len_k = o;      o = align256(o + sizeof(int) * S);
  l.len_q = o;      o = align256(o + sizeof(int) * S);
  l.n_items = o;    o = align256(o + sizeof(int) * S);
  l.n_zero = o;     o = align256(o + sizeof(int) * S);
  l.n_slots = o;    o = align256(o + sizeof(int) * S);
  l.n_entries = o;  o = align256(o + sizeof(int) * S);
  l.slot_base = o;  o = align256(o + sizeof(int) * S);
  l.entry_base = o; o = align256(o + sizeof(int) * S);
  l.pos_real = o;   o = align256(o + sizeof(int) * S * kXcds);
  l.pos_zero = o;   o = align256(o + sizeof(int) * S * kXcds);
  l.items = o;      o = align256(o + sizeof(int) * kItemInts * (size_t)max_positions(s));
  l.merge = o;      o = align256(o + sizeof(int) * kMergeInts * (size_t)max_merge_entries(s));
  const size_t pairs = (size_t)s.pairs;
  l.opart = o;      o = align256(o + sizeof(float) * slots * pairs * (size_t)d);
  l.mpart = o;      o = align256(o + sizeof(float) * slots * pairs);
  l.lpart = o;      o = align256(o + sizeof(float) * slots * pairs);
  l.total = o;
  return l;
}

// The plan's integer arrays inside the workspace.
struct Bufs {
  int* hdr;
  int* order;
  int* len_k;  // clamped key length L of the sequence at each rank
  int* len_q;  // clamped chunk length Q
  int* n_items;
  int* n_zero;
  int* n_slots;
  int* n_entries;
  int* slot_base;
  int* entry_base;
  int* pos_real;
  int* pos_zero;
  int* items;
  int* merge;
};

FA_PLAN_FN Bufs bufs(unsigned char* ws, const Layout& l) {
  Bufs b;
  b.hdr = (int*)(ws + l.hdr);
  b.order = (int*)(ws + l.order);
  b.len_k = (int*)(ws + l.len_k);
  b.len_q = (int*)(ws + l.len_q);
  b.n_items = (int*)(ws + l.n_items);
  b.n_zero = (int*)(ws + l.n_zero);
  b.n_slots = (int*)(ws + l.n_slots);
  b.n_entries = (int*)(ws + l.n_entries);
  b.slot_base = (int*)(ws + l.slot_base);
  b.entry_base = (int*)(ws + l.entry_base);
  b.pos_real = (int*)(ws + l.pos_real);
  b.pos_zero = (int*)(ws + l.pos_zero);
  b.items = (int*)(ws + l.items);
  b.merge = (int*)(ws + l.merge);
  return b;
}

// ---------------------------------------------------------------------------------------------
// The plan's phases.  The plan kernel runs each one in parallel over its index (one barrier
// between phases); the host check runs them as loops in the same order.

// Sequences ranked by key length only up to this many (an all-pairs count); beyond it the
// natural order is kept.
constexpr int kMaxRanked = 512;

// Phase 1 (per sequence i, S <= kMaxRanked): the rank of sequence i, longest first, ties by
// index.  keys[] holds the clamped key lengths.
FA_PLAN_FN void rank_one(int S, const int* keys, int i, int* order) {
  int r = 0;
  for (int t = 0; t < S; ++t) r += (keys[t] > keys[i]) || (keys[t] == keys[i] && t < i);
  order[r] = i;
}

// Phase 2 (per rank r): the unit counts of the sequence at rank r for split length T.
FA_PLAN_FN void count_one(const Shape& s, const int* seq_lens, const int* q_lens, int T, int r,
                          const Bufs& w) {
  const int b = w.order[r];
  const int L = seq_keys(s, seq_lens[b]);
  const int Q = seq_queries(s, L, q_lens[b]);
  const SeqCounts c = seq_counts(s, L, Q, T);
  w.len_k[r] = L;
  w.len_q[r] = Q;
  w.n_items[r] = c.items;
  w.n_zero[r] = c.zeros;
  w.n_slots[r] = c.slots;
  w.n_entries[r] = c.entries;
}

// Phase 3: running sums over ranks.  Its inputs (per rank r and XCD x): the real and zero
// items the sequence at rank r puts on list x, and its slots and merge entries; its outputs the
// exclusive prefix sums of each over r (pos_real[x * S + r], pos_zero[x * S + r], slot_base[r],
// entry_base[r]) and the totals: tot[x] real and tot[8 + x] zero items of list x, tot[16] slots,
// tot[17] merge entries.  scan_inputs (per rank) writes the inputs in place; the plan kernel
// then scans each array in parallel, the host check with scan_serial.
FA_PLAN_FN void scan_inputs(const Shape& s, int r, const Bufs& w) {
  const int nu = units_per_seq(s);
  for (int x = 0; x < kXcds; ++x) {
    const int k = units_on_xcd(nu, r, x);
    w.pos_real[x * s.S + r] = k * w.n_items[r];
    w.pos_zero[x * s.S + r] = k * w.n_zero[r];
  }
  w.slot_base[r] = nu * w.n_slots[r];
  w.entry_base[r] = nu * w.n_entries[r];
}

// Exclusive prefix sum of v[0 .. n) in place; returns the total.
FA_PLAN_FN long long exclusive_scan_serial(int* v, int n) {
  long long run = 0;
  for (int i = 0; i < n; ++i) {
    const int x = v[i];
    v[i] = (int)run;
    run += x;
  }
  return run;
}

FA_PLAN_FN void scan_serial(const Shape& s, const Bufs& w, long long* tot) {
  for (int x = 0; x < kXcds; ++x) {
    tot[x] = exclusive_scan_serial(w.pos_real + x * s.S, s.S);
    tot[kXcds + x] = exclusive_scan_serial(w.pos_zero + x * s.S, s.S);
  }
  tot[2 * kXcds] = exclusive_scan_serial(w.slot_base, s.S);
  tot[2 * kXcds + 1] = exclusive_scan_serial(w.entry_base, s.S);
}

// Position in the dense array of item k of list x, once the header is written.
FA_PLAN_FN long long position(const int* hdr, int x, long long k) {
  const long long cs = hdr[kHdrCstar];
  if (k < cs) return k * kXcds + x;
  const long long e = hdr[kHdrExcess + x] + (k - cs);  // surplus item number
  for (int xx = 0; xx < kXcds; ++xx) {
    const long long def = cs - hdr[kHdrCount + xx];
    if (def > 0 && e < hdr[kHdrDeficit + xx] + def)
      return (hdr[kHdrCount + xx] + (e - hdr[kHdrDeficit + xx])) * kXcds + xx;
  }
  return -1;  // not reached: the shortfall covers the surplus
}

// Phase 4 (one lane): the header, and the empty markers of the positions no item fills.
// Returns false if a total exceeds its bound (never, by the bounds above; the plan is then
// empty).
FA_PLAN_FN bool header(const Shape& s, int T, const long long* tot, const Bufs& w) {
  long long total = 0;
  for (int x = 0; x < kXcds; ++x) total += tot[x] + tot[kXcds + x];
  const bool ok = tot[2 * kXcds] <= max_split_slots(s) &&
                  tot[2 * kXcds + 1] <= max_merge_entries(s) && total <= max_items(s);
  const long long cs = ok ? (total + kXcds - 1) / kXcds : 0;
  long long excess = 0, deficit = 0;
  for (int x = 0; x < kXcds; ++x) {
    const long long n = ok ? tot[x] + tot[kXcds + x] : 0;
    w.hdr[kHdrCount + x] = (int)n;
    w.hdr[kHdrExcess + x] = (int)excess;
    w.hdr[kHdrDeficit + x] = (int)deficit;
    excess += n > cs ? n - cs : 0;
    deficit += n < cs ? cs - n : 0;
  }
  w.hdr[kHdrMerge] = ok ? (int)tot[2 * kXcds + 1] : 0;
  w.hdr[kHdrT] = T;
  w.hdr[kHdrItems] = (int)(ok ? total : 0);
  w.hdr[kHdrOk] = ok ? 1 : 0;
  w.hdr[kHdrCstar] = (int)cs;
  w.hdr[kHdrPositions] = (int)(cs * kXcds);
  // Shortfall positions past the surplus stay empty (at most 7 of them).
  for (long long e = excess; e < deficit; ++e) {
    for (int xx = 0; xx < kXcds; ++xx) {
      const long long def = cs - w.hdr[kHdrCount + xx];
      if (def > 0 && e < w.hdr[kHdrDeficit + xx] + def) {
        const long long at = (w.hdr[kHdrCount + xx] + (e - w.hdr[kHdrDeficit + xx])) * kXcds + xx;
        if (at >= 0 && at < max_positions(s)) w.items[at * kItemInts] = -1;
        break;
      }
    }
  }
  return ok;
}

// Phase 5a (per task t = unit * blocks_per_unit + qb, unit = rank * nu + j; t < 2^31 by the
// size checks): the zero item of a block past the chunk, and the item of a real block of a
// sequence with no split block.
FA_PLAN_FN void put_item(const Shape& s, const Bufs& w, int x, long long k_list, int b, int j,
                         int qb, int t0, int t1, int slot) {
  const long long at = position(w.hdr, x, k_list);
  if (at < 0 || at >= max_positions(s)) return;
  struct alignas(16) Int4 { int v[4]; };
  Int4* e = reinterpret_cast<Int4*>(w.items + at * kItemInts);
  e[0] = Int4{{b, j, qb, t0}};
  e[1] = Int4{{t1, slot, 0, 0}};
}

FA_PLAN_FN void emit_task(const Shape& s, const long long* tot, int t, const Bufs& w) {
  if (!w.hdr[kHdrOk]) return;  // a bound was exceeded: the plan is empty
  const int nq = blocks_per_unit(s), nu = units_per_seq(s);
  const int u = t / nq;
  const int qb = t - u * nq;
  const int r = u / nu, j = u - r * nu;
  const int L = w.len_k[r], Q = w.len_q[r];
  const int nb = real_blocks(s, Q);
  const int x = unit_xcd(u);
  const int k = unit_rank_on_xcd(nu, r, j);
  if (qb >= nb) {
    const long long zt = tot[x] + w.pos_zero[x * s.S + r] + (long long)k * w.n_zero[r] + (qb - nb);
    put_item(s, w, x, zt, w.order[r], j, qb, 0, 0, kZeroItem);
  } else if (w.n_slots[r] == 0) {  // no block of this sequence is split: item qb is block qb
    const long long it = w.pos_real[x * s.S + r] + (long long)k * w.n_items[r] + qb;
    put_item(s, w, x, it, w.order[r], j, qb, 0, key_tiles(s, L, Q, qb), kDirect);
  }
}

// Phase 5b (per unit u = rank * nu + j, sequences with a split block only): the unit's real
// items, pieces-major, and the merge entries of its split blocks.
FA_PLAN_FN void emit_split(const Shape& s, int T, int u, const Bufs& w) {
  if (!w.hdr[kHdrOk]) return;
  const int nu = units_per_seq(s);
  const int r = u / nu, j = u - r * nu;
  if (w.n_slots[r] == 0) return;
  const int b = w.order[r];
  const int L = w.len_k[r], Q = w.len_q[r];
  const int x = unit_xcd(u);
  const int k = unit_rank_on_xcd(nu, r, j);
  long long it = w.pos_real[x * s.S + r] + (long long)k * w.n_items[r];
  const long long slot0 = w.slot_base[r] + (long long)j * w.n_slots[r];
  long long ent = w.entry_base[r] + (long long)j * w.n_entries[r];
  const int nb = real_blocks(s, Q);
  // Merge entries, in query-block order, and the largest piece count.
  int max_np = 0;
  long long sl = slot0;
  for (int qb = 0; qb < nb; ++qb) {
    const int np = pieces(key_tiles(s, L, Q, qb), T);
    max_np = imax(max_np, np);
    if (np > 1) {
      if (ent < max_merge_entries(s)) {
        int* e = w.merge + ent * kMergeInts;
        e[0] = b;
        e[1] = j;
        e[2] = qb;
        e[3] = (int)sl;
        e[4] = np;
        e[5] = 0;
        e[6] = 0;
        e[7] = 0;
      }
      ++ent;
      sl += np;
    }
  }
  // Items, pieces-major.
  for (int p = 0; p < max_np; ++p) {
    long long sb = slot0;
    for (int qb = 0; qb < nb; ++qb) {
      const int n = key_tiles(s, L, Q, qb);
      const int np = pieces(n, T);
      if (p < np) {
        int t0, t1;
        piece_range(n, np, p, &t0, &t1);
        const long long slot = np > 1 ? sb + p : kDirect;
        put_item(s, w, x, it++, b, j, qb, t0, t1,
                 slot < max_split_slots(s) ? (int)slot : kBadItem);
      }
      if (np > 1) sb += np;
    }
  }
}

}  // namespace plan
}  // namespace fa
