// plan_main.cpp -- host check of the chunked prefill's work plan (fa_prefill_plan.h).
//
// Runs the plan's phases in the order the plan kernel runs them, on the host, for many sequence
// mixes and head layouts, and checks what the attention kernel relies on:
//   * every (sequence, unit, query block) is covered: a block past the chunk by exactly one zero
//     item; a real block by pieces whose key-tile ranges partition [0, n_kt) exactly, each at
//     most T tiles long, unsplit ones writing directly and split ones into distinct partials
//     slots listed by exactly one merge entry;
//   * every field and index lies inside its buffer (the kernels index by them), and the totals
//     stay within the bounds that size the workspace;
//   * a unit's items sit in the list of its XCD, and the lists hold real items before zero items
//     in rank order of the sequences (longest key length first).
// Prints "plan checks hold" when every case passes.  Built with the address and undefined-
// behaviour sanitizers by tests/test_abi_sanitizers.py.
#include <algorithm>
#include <climits>
#include <cstdio>
#include <cstring>
#include <map>
#include <random>
#include <set>
#include <tuple>
#include <vector>

#include "fa_launch.h"
#include "fa_prefill_plan.h"

namespace {

using namespace fa::plan;

int failures = 0;
#define EXPECT(cond, ...)                 \
  do {                                    \
    if (!(cond)) {                        \
      if (failures < 20) {                \
        std::printf("FAIL %s: ", #cond);  \
        std::printf(__VA_ARGS__);         \
        std::printf("\n");                \
      }                                   \
      ++failures;                         \
    }                                     \
  } while (0)

struct Result {
  int T;
  long long items, slots, entries;
};

Result run_case(const char* name, int S, int max_q, int Hq, int Hkv, int max_blocks,
                const std::vector<int>& L_raw, const std::vector<int>& Q_raw) {
  const Shape s = fa::paged_prefill_shape(S, max_q, Hq, Hkv, max_blocks);
  const Layout l = layout(s, 128);
  // The plan touches only the integer regions (everything before the partials).
  std::vector<unsigned char> ws(l.opart, 0xAB);
  const Bufs w = bufs(ws.data(), l);
  const int* sl = L_raw.data();
  const int* ql = Q_raw.data();
  const int nu = units_per_seq(s);

  // The plan kernel's phases, in order.
  if (S <= kMaxRanked) {
    std::vector<int> keys(S);
    for (int i = 0; i < S; ++i) keys[i] = seq_keys(s, sl[i]);
    for (int i = 0; i < S; ++i) rank_one(S, keys.data(), i, w.order);
  } else {
    for (int i = 0; i < S; ++i) w.order[i] = i;
  }
  long long W = 0;
  for (int i = 0; i < S; ++i) {
    const int L = seq_keys(s, sl[i]);
    W += seq_tiles(s, L, seq_queries(s, L, ql[i]));
  }
  const int T = split_tiles(W * nu, s.R);
  for (int r = 0; r < S; ++r) count_one(s, sl, ql, T, r, w);
  long long tot[2 * kXcds + 2];
  for (int r = 0; r < S; ++r) scan_inputs(s, r, w);
  scan_serial(s, w, tot);
  const bool ok = header(s, T, tot, w);
  const int units = S * nu;
  for (int t = 0; t < units * blocks_per_unit(s); ++t) emit_task(s, tot, t, w);
  for (int u = 0; u < units; ++u) emit_split(s, T, u, w);

  EXPECT(ok, "%s: a total exceeds its bound", name);
  EXPECT(w.hdr[kHdrOk] == 1 && w.hdr[kHdrT] == T, "%s: header", name);
  EXPECT(T >= kMinPieceTiles && (long long)2 * s.R * T >= W * nu, "%s: T=%d W=%lld", name, T, W * nu);

  // The order is a permutation, longest first when ranked.
  {
    std::vector<int> seen(S, 0);
    for (int r = 0; r < S; ++r) {
      const int b = w.order[r];
      EXPECT(b >= 0 && b < S, "%s: order[%d]=%d", name, r, b);
      if (b >= 0 && b < S) ++seen[b];
      if (S <= kMaxRanked && r > 0)
        EXPECT(seq_keys(s, sl[w.order[r - 1]]) >= seq_keys(s, sl[b]), "%s: rank %d", name, r);
    }
    for (int b = 0; b < S; ++b) EXPECT(seen[b] == 1, "%s: sequence %d ranked %d times", name, b, seen[b]);
  }

  // Walk the dense item array: 8 c* positions, position p runs on XCD p mod 8.
  std::map<std::tuple<int, int, int>, std::vector<std::tuple<int, int, int>>> pieces_of;  // -> (t0,t1,slot)
  std::map<std::tuple<int, int, int>, int> zeros_of;
  std::set<int> slots_used;
  const long long cs = w.hdr[kHdrCstar], npos = w.hdr[kHdrPositions];
  long long total = 0, surplus = 0;
  for (int x = 0; x < kXcds; ++x) {
    const int c = w.hdr[kHdrCount + x];
    EXPECT(c >= 0, "%s: list %d count %d", name, x, c);
    total += c;
    surplus += c > cs ? c - cs : 0;
  }
  EXPECT(total == w.hdr[kHdrItems] && total <= max_items(s), "%s: item total", name);
  EXPECT(cs == (total + kXcds - 1) / kXcds && npos == cs * kXcds && npos <= max_positions(s),
         "%s: c*=%lld positions=%lld", name, cs, npos);
  long long empties = 0, off_xcd = 0, n_items = 0;
  for (int x = 0; x < kXcds; ++x) {
    int last_rank = -1;
    bool in_zero = false;
    for (long long k = 0; k < cs; ++k) {
      const long long pos = k * kXcds + x;
      const int* e = w.items + (size_t)pos * kItemInts;
      const int b = e[0], j = e[1], qb = e[2], t0 = e[3], t1 = e[4], slot = e[5];
      if (b == -1) {
        ++empties;
        continue;
      }
      ++n_items;
      const bool fields = b >= 0 && b < S && j >= 0 && j < nu && qb >= 0 && qb < blocks_per_unit(s);
      EXPECT(fields, "%s: position %lld fields b=%d j=%d qb=%d", name, pos, b, j, qb);
      if (!fields) continue;
      int r = 0;
      while (r < S && w.order[r] != b) ++r;
      const bool home = unit_xcd(r * nu + j) == x && k < w.hdr[kHdrCount + x];
      off_xcd += !home;
      const int L = seq_keys(s, sl[b]), Q = seq_queries(s, L, ql[b]);
      if (slot == kZeroItem) {
        if (home) in_zero = true;
        EXPECT(qb >= real_blocks(s, Q), "%s: zero item for a real block", name);
        ++zeros_of[{b, j, qb}];
        continue;
      }
      if (home) {
        EXPECT(!in_zero, "%s: real item after zero items on XCD %d", name, x);
        EXPECT(r >= last_rank, "%s: XCD %d out of rank order", name, x);
        last_rank = r;
      }
      EXPECT(qb < real_blocks(s, Q), "%s: real item past the chunk", name);
      EXPECT(slot == kDirect || (slot >= 0 && slot < max_split_slots(s)), "%s: slot %d", name, slot);
      EXPECT(t0 >= 0 && t1 > t0 && t1 - t0 <= T, "%s: piece [%d,%d) T=%d", name, t0, t1, T);
      if (slot >= 0) {
        EXPECT(!slots_used.count(slot), "%s: slot %d used twice", name, slot);
        slots_used.insert(slot);
      }
      pieces_of[{b, j, qb}].push_back({t0, t1, slot});
    }
  }
  EXPECT(n_items == total && empties == npos - total && empties < kXcds,
         "%s: %lld items, %lld empty positions", name, n_items, empties);
  EXPECT(off_xcd <= surplus, "%s: %lld items away from their XCD, surplus %lld", name, off_xcd,
         surplus);

  // Coverage of every block, and the merge entries.
  std::map<std::tuple<int, int, int>, std::pair<int, int>> merge_of;
  const int n_merge = w.hdr[kHdrMerge];
  EXPECT(n_merge >= 0 && n_merge <= max_merge_entries(s), "%s: %d merge entries", name, n_merge);
  for (int m = 0; m < n_merge && m < max_merge_entries(s); ++m) {
    const int* e = w.merge + (size_t)m * kMergeInts;
    EXPECT(!merge_of.count({e[0], e[1], e[2]}), "%s: block merged twice", name);
    merge_of[{e[0], e[1], e[2]}] = {e[3], e[4]};
    EXPECT(e[4] >= 2 && e[3] >= 0 && (long long)e[3] + e[4] <= max_split_slots(s),
           "%s: merge entry slots [%d,+%d)", name, e[3], e[4]);
  }
  long long slots_total = 0;
  for (int b = 0; b < S; ++b) {
    const int L = seq_keys(s, sl[b]), Q = seq_queries(s, L, ql[b]);
    for (int j = 0; j < nu; ++j)
      for (int qb = 0; qb < blocks_per_unit(s); ++qb) {
        const auto key = std::make_tuple(b, j, qb);
        if (qb >= real_blocks(s, Q)) {
          EXPECT(zeros_of[key] == 1 && !pieces_of.count(key), "%s: zero block b=%d qb=%d", name, b, qb);
          continue;
        }
        auto ps = pieces_of[key];
        const int n = key_tiles(s, L, Q, qb);
        EXPECT(!ps.empty(), "%s: block b=%d j=%d qb=%d has no item", name, b, j, qb);
        if (ps.empty()) continue;
        std::sort(ps.begin(), ps.end());
        int at = 0;
        for (auto& p : ps) {
          EXPECT(std::get<0>(p) == at, "%s: gap or overlap at tile %d", name, at);
          at = std::get<1>(p);
        }
        EXPECT(at == n, "%s: pieces end at %d, block needs %d tiles", name, at, n);
        if (ps.size() == 1) {
          EXPECT(std::get<2>(ps[0]) == kDirect && !merge_of.count(key), "%s: unsplit block", name);
        } else {
          EXPECT(merge_of.count(key), "%s: split block without merge entry", name);
          if (!merge_of.count(key)) continue;
          const auto me = merge_of[key];
          EXPECT(me.second == (int)ps.size(), "%s: merge piece count", name);
          for (size_t i = 0; i < ps.size(); ++i)
            EXPECT(std::get<2>(ps[i]) == me.first + (int)i, "%s: piece slot order", name);
          slots_total += (long long)ps.size();
        }
      }
  }
  EXPECT((long long)slots_used.size() == slots_total && slots_total <= max_split_slots(s),
         "%s: slots", name);
  return {T, n_items, slots_total, (long long)n_merge};
}

}  // namespace

int main() {
  // The closed-form XCD counts against a walk over the units.
  for (int nu = 1; nu <= 40; ++nu)
    for (int r = 0; r < 24; ++r) {
      int seen[kXcds] = {0};
      for (int j = 0; j < nu; ++j) {
        const int x = unit_xcd(r * nu + j);
        EXPECT(unit_rank_on_xcd(nu, r, j) == seen[x], "unit rank nu=%d r=%d j=%d", nu, r, j);
        ++seen[x];
      }
      for (int x = 0; x < kXcds; ++x)
        EXPECT(units_on_xcd(nu, r, x) == seen[x], "units on XCD nu=%d r=%d x=%d", nu, r, x);
    }
  // The 16-sequence chunked-prefill mix (contexts U[1024, 32768], chunks U[1, 1024]) and the same
  // contexts with chunks cut to 128 and 48 tokens.
  const std::vector<int> L16 = {10154, 19980, 16752, 26921, 29798, 13176, 13126, 9680,
                                17003, 11432, 3741,  4463,  4169,  31674, 30051, 15306};
  const std::vector<int> Q16 = {605, 566, 1002, 984, 327, 779, 110, 547,
                                373, 277, 94,  94,  346, 48,  905, 408};
  std::vector<int> Q128(Q16), Q48(Q16);
  for (auto& q : Q128) q = q < 128 ? q : 128;
  for (auto& q : Q48) q = q < 48 ? q : 48;
  const Result mix = run_case("mix", 16, 1024, 32, 8, 2048, L16, Q16);
  const Result c128 = run_case("chunks<=128", 16, 1024, 32, 8, 2048, L16, Q128);
  const Result c48 = run_case("chunks<=48", 16, 1024, 32, 8, 2048, L16, Q48);
  std::printf("mix: T=%d items=%lld split slots=%lld; chunks<=128: T=%d slots=%lld; "
              "chunks<=48: T=%d slots=%lld\n",
              mix.T, mix.items, mix.slots, c128.T, c128.slots, c48.T, c48.slots);
  EXPECT(mix.slots == 0, "the mix splits nothing");
  EXPECT(c128.slots > 0 && c48.slots > 0, "short chunks against long contexts are split");

  // Edge mixes.
  run_case("empty", 4, 64, 8, 8, 64, {0, 0, 0, 0}, {0, 0, 0, 0});
  run_case("one token", 1, 1, 1, 1, 1, {1}, {1});
  run_case("chunk = context", 3, 300, 4, 2, 32, {300, 17, 512}, {300, 17, 512});
  run_case("lengths past the table", 2, 64, 8, 2, 4, {10000, -5}, {70, 3});
  run_case("all splits", 2, 32, 32, 8, 4096, {65536, 65536}, {1, 32});

  // Random mixes over head layouts (groups 1, 2, 3, 4, 8, 16) and sizes, some above the ranked
  // limit.
  std::mt19937 gen(7);
  const int layouts[][2] = {{8, 8}, {16, 8}, {12, 4}, {32, 8}, {64, 8}, {32, 2}, {6, 6}};
  for (int c = 0; c < 60; ++c) {
    const int* hl = layouts[c % 7];
    const int S = c == 59 ? 700 : 1 + (int)(gen() % (c < 40 ? 24 : 200));
    const int max_q = 1 + (int)(gen() % 700);
    const int max_blocks = 1 + (int)(gen() % 1200);
    std::vector<int> Ls(S), Qs(S);
    for (int i = 0; i < S; ++i) {
      Ls[i] = (int)(gen() % (max_blocks * 16 + 40)) - 20;
      Qs[i] = (int)(gen() % (max_q + 20)) - 5;
    }
    char name[64];
    std::snprintf(name, sizeof name, "random %d (S=%d Hq=%d Hkv=%d)", c, S, hl[0], hl[1]);
    run_case(name, S, max_q, hl[0], hl[1], max_blocks, Ls, Qs);
  }
  if (failures) {
    std::printf("%d plan check(s) failed\n", failures);
    return 1;
  }
  std::printf("plan checks hold\n");
  return 0;
}
