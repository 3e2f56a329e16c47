// Host build of the decode kernel's work split (the kernel's own
// partition.hpp, compiled for the CPU), checked by brute force: every unit
// has exactly one owner and the owner functions find it, runs are non-empty
// and ordered, row runs start on even blocks, a band's segment count equals
// the workgroups that really meet it, and the partial-sum slots of shared
// bands are distinct and inside the workspace.  Built and called by
// tests/test_partition.py.
#include <stdio.h>
#include <string.h>

#include <set>
#include <utility>
#include <vector>

#include "partition.hpp"

using namespace spear;

static char g_msg[512];

#define REQUIRE(cond, ...)                           \
  do {                                               \
    if (!(cond)) {                                   \
      snprintf(g_msg, sizeof(g_msg), __VA_ARGS__);   \
      return 1;                                      \
    }                                                \
  } while (0)

extern "C" const char* check_message() { return g_msg; }

// FastDiv against the divider for divisors 1 .. dmax and numerators below
// 2^31 (all small ones, then a stride through the range and its top end).
extern "C" int check_fastdiv(uint32_t dmax) {
  g_msg[0] = 0;
  for (uint32_t d = 1; d <= dmax; ++d) {
    const FastDiv f = make_fastdiv(d);
    for (uint32_t n = 0; n < 4096; ++n)
      REQUIRE(fdiv(n, f) == n / d && fmod(n, f) == n % d, "fdiv(%u, %u)", n, d);
    for (uint64_t n = 4096; n < (1ull << 31); n += 7919 * (uint64_t)d + 104729)
      REQUIRE(fdiv((uint32_t)n, f) == (uint32_t)n / d, "fdiv(%llu, %u)", (unsigned long long)n, d);
    for (uint32_t k = 0; k < 64; ++k) {
      const uint32_t n = (1u << 31) - 1 - k;
      REQUIRE(fdiv(n, f) == n / d, "fdiv(%u, %u)", n, d);
    }
  }
  return 0;
}

// 0 = all checks hold; otherwise g_msg says which failed.  stats (may be
// NULL): P, Rw, S, D, max segments of a row band, max segments of a rank
// band, workspace slots, max row units of one workgroup.
extern "C" int check_split(int KB, int RB, int NB, int slots, int max_slots, int shared,
                           long long* stats) {
  g_msg[0] = 0;
  const DecodeSplit d = make_split(KB, RB, NB, slots, shared != 0);
  const int ws_slots = split_workspace_slots(KB, RB, NB, max_slots, shared != 0);
  const long long RU = split_ru(d), WU = split_wu(d);
  REQUIRE(d.KB == KB && d.RB == RB && d.NB == NB, "split fields");
  REQUIRE(d.P >= 1 && d.P <= (slots < 1 ? 1 : slots), "P=%d outside [1, %d]", d.P, slots);
  // rank work: workgroup 0 reduces it and takes no rows, unless it is alone
  REQUIRE(RB == 0 ? d.S == 0 : (d.P == 1 ? d.S == 0 : (d.S == 1 || d.S == d.Rw)),
          "S=%d Rw=%d P=%d", d.S, d.Rw, d.P);
  REQUIRE(shared || RB == 0 || d.P == 1 || d.S == d.Rw, "shared mode when asked for separate");
  REQUIRE(RB == 0 ? d.Rw == 0 : (d.Rw >= 1 && d.Rw <= d.P && d.Rw <= RU), "Rw=%d", d.Rw);
  REQUIRE(d.S < d.P, "no workgroup takes rows (S=%d P=%d)", d.S, d.P);

  // rank runs
  std::vector<int> rown(RU, -1);
  for (int w = 0; w < d.P; ++w) {
    const long long a = rank_begin(d, w), b = rank_begin(d, w + 1);
    REQUIRE(a <= b, "rank runs out of order at w=%d", w);
    REQUIRE(w >= d.Rw ? a == b : a < b, "rank run of w=%d: [%lld, %lld)", w, a, b);
    for (long long u = a; u < b; ++u) {
      REQUIRE(rown[u] == -1, "rank unit %lld twice", u);
      rown[u] = w;
      REQUIRE(rank_owner(d, u) == w, "rank_owner(%lld)=%d, run of %d", u, rank_owner(d, u), w);
    }
  }
  for (long long u = 0; u < RU; ++u) REQUIRE(rown[u] >= 0, "rank unit %lld unowned", u);

  // row runs
  std::vector<int> wown(WU, -1);
  long long maxrun = 0;
  REQUIRE(row_begin(d, 0) == 0 && row_begin(d, d.P) == WU, "row runs do not cover [0, WU)");
  for (int w = 0; w < d.P; ++w) {
    const long long a = row_begin(d, w), b = row_begin(d, w + 1);
    REQUIRE(w < d.S ? (a == 0 && b == 0) || (w + 1 == d.S && a == 0) : a < b,
            "row run of w=%d: [%lld, %lld) (S=%d)", w, a, b, d.S);
    if (a > 0 && a < WU) REQUIRE((a % KB) % 2 == 0, "row run of w=%d starts on odd block %lld", w, a);
    if (b - a > maxrun) maxrun = b - a;
    for (long long u = a; u < b; ++u) {
      REQUIRE(wown[u] == -1, "row unit %lld twice", u);
      wown[u] = w;
    }
  }
  for (long long u = 0; u < WU; ++u) {
    REQUIRE(wown[u] >= 0, "row unit %lld unowned", u);
    REQUIRE(row_owner(d, u) == wown[u], "row_owner(%lld)=%d, run of %d", u, row_owner(d, u), wown[u]);
  }

  // bands: segment counts and slots
  std::set<int> used;
  long long maxseg_row = 0, maxseg_rank = 0;
  for (int rank = 0; rank < 2; ++rank) {
    const int nb = rank ? RB : NB;
    const std::vector<int>& own = rank ? rown : wown;
    for (int band = 0; band < nb; ++band) {
      const long long bb = (long long)band * KB, be = bb + KB;
      std::set<int> meet;
      for (long long u = bb; u < be; ++u) meet.insert(own[u]);
      REQUIRE((long long)d.C < (1LL << 22) && (long long)d.P * d.C < (1LL << 32), "32-bit range");
      const int first = rank ? rank_owner(d, bb) : row_owner(d, bb);
      const int last = rank ? rank_owner(d, be - 1) : row_owner(d, be - 1);
      const int nseg = last - first + 1;
      REQUIRE(nseg == (int)meet.size() && *meet.begin() == first && *meet.rbegin() == last,
              "%s band %d: nseg %d, %zu workgroups meet it", rank ? "rank" : "row", band, nseg,
              meet.size());
      if (rank) { if (nseg > maxseg_rank) maxseg_rank = nseg; }
      else if (nseg > maxseg_row) maxseg_row = nseg;
      if (nseg == 1) continue;  // finished by its only workgroup: no partial
      for (int w : meet) {
        const int s = rank ? rank_slot(d, w, band) : row_slot(d, w, band);
        REQUIRE(s >= (rank ? 2 * d.P : 0) && s < (rank ? 2 * d.P + 2 * d.Rw : 2 * d.P),
                "slot %d of w=%d out of its range", s, w);
        REQUIRE(s < ws_slots, "slot %d beyond the workspace's %d", s, ws_slots);
        REQUIRE(used.insert(s).second, "slot %d used twice (w=%d band %d)", s, w, band);
      }
    }
  }
  if (stats) {
    const long long v[8] = {d.P, d.Rw, d.S, d.D, maxseg_row, maxseg_rank, ws_slots, maxrun};
    memcpy(stats, v, sizeof(v));
  }
  return 0;
}
