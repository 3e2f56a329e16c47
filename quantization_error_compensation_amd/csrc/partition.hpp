// Work split of the decode kernel: which rank units (128-column blocks of
// 64 rows of A) and which row units (128-column blocks of one row band) each
// persistent workgroup takes.  The same functions run in the kernel and on
// the host (the planner, and a host-built check over a grid of shapes).
//
// Units.  Rank units are numbered band-major, [0, RU) with RU = RB * KB; row
// units the same, [0, WU) with WU = NB * KB.
//
// Rank units.  Workgroups [0, Rw) take contiguous, near-equal runs of the
// rank units, rank_begin(w) = floor(w RU / Rw), so the rank-r projection is
// spread over many compute units and is published early (every row band's
// finisher waits for it).  Workgroup 0 sums the partial projections and
// publishes the gated result; it takes no row units (unless it is the only
// workgroup), so that work delays no row stream.
//
// Row units.  Laid out as a stream-K split over a cost axis of C row-unit
// equivalents: workgroup w owns [w C / P', (w + 1) C / P') (P' = P - S, w
// counted from S), and a rank workgroup spends the first D units of its
// range on its rank units ("shared" mode, S = 1: the rank workgroups but the
// first go on to stream rows).  When the rank units would take more than
// half of a workgroup's share (short row runs would cut bands into many
// partial sums), the rank workgroups take no rows at all ("separate" mode,
// S = Rw, D = 0) and the rows are split over the other P - Rw; the caller
// can ask for separate mode outright (the library does for layers with
// per-channel scales, whose shared-mode splits no device test covers).  On
// the cost axis each row band boundary takes X units (row_cost), so a run
// that crosses one carries fewer units.  Where the runs are short (under 32
// units) and the row workgroups take no rank units, the planner launches
// S + M NB workgroups instead, M per row band, with X = 0: every M-th run
// then starts a band and none crosses one.  Row parts start on an even
// block of their band, so the bursts' code loads stay on 128-byte lines;
// every workgroup from S on keeps at least one row unit.
//
// Arithmetic.  Unit counts stay below 2^21 (KB, NB <= 1024, RB <= 2) and the
// cost axis below 2^22, so every numerator here (at most P <= 256 times a
// count) is below 2^31.  The GPU has no integer divider: a division by a
// value known only at run time is a dependent sequence of some thirty
// instructions, and the owner searches take dozens of them before a
// workgroup's first load.  Every divisor here is fixed per call, so the host
// computes a multiplier for each (FastDiv) and a division becomes one
// 32 x 32 -> 64-bit multiply and a shift.
//
// Partial sums.  A band covered by several workgroups is finished by the last
// to arrive.  A workgroup's run meets at most two row bands that it does not
// cover alone (the first and the last of its run), and the same for rank
// bands, so its partial sums have fixed slots: row 2 w + {0: the band of its
// first row unit, 1: any other}, rank 2 P + 2 w + {0, 1} likewise.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spear {

// Division by a fixed d >= 1 for numerators n < 2^31 (the round-up method:
// with l = ceil(log2 d), m = ceil(2^(31+l) / d) <= 2^31 and
// floor(n m / 2^(31+l)) = floor(n / d) for every such n).
struct FastDiv {
  uint32_t d, m, s;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const unsigned long long two = 1ull << (31 + l);
  FastDiv f;
  f.d = d;
  f.m = (uint32_t)((two + d - 1) / d);
  f.s = 31 + l;
  return f;
}
__host__ __device__ inline uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return (uint32_t)(((unsigned long long)n * f.m) >> f.s);
}
__host__ __device__ inline uint32_t fmod(uint32_t n, const FastDiv& f) {
  return n - fdiv(n, f) * f.d;
}

struct DecodeSplit {
  int KB;       // 128-column blocks per row
  int RB;       // rank bands (64 ranks each)
  int NB;       // row bands
  int P;        // workgroups
  int Rw;       // workgroups [0, Rw) take rank units (0 when RB == 0)
  int S;        // workgroups [0, S) take no row units: 1 (shared), Rw (separate), 0 (no
                // rank units, or one workgroup)
  int D;        // row-unit equivalents a rank workgroup's rank units stand for (shared)
  int X;        // cost of a row band boundary on the cost axis (row units)
  int C;        // the row cost axis: WU + X (NB - 1) + (Rw - S) D
  FastDiv by_kb, by_pp, by_rw, by_ru;  // KB, P - S, Rw, RU (1 when zero)
  FastDiv by_c, by_cd;                 // C, C - (P - S) D (the owner estimate)
  FastDiv by_kbx;                      // KB + X
};

__host__ __device__ inline uint32_t split_ru(const DecodeSplit& d) {
  return (uint32_t)d.RB * (uint32_t)d.KB;
}
__host__ __device__ inline uint32_t split_wu(const DecodeSplit& d) {
  return (uint32_t)d.NB * (uint32_t)d.KB;
}

// First rank unit of workgroup w (RU for w >= Rw).
__host__ __device__ inline uint32_t rank_begin(const DecodeSplit& d, int w) {
  const uint32_t RU = split_ru(d);
  return w >= d.Rw ? RU : fdiv((uint32_t)w * RU, d.by_rw);
}
// Workgroup whose rank run holds rank unit u (0 <= u < RU): the largest w
// with rank_begin(w) <= u, i.e. ceil((u + 1) Rw / RU) - 1.
__host__ __device__ inline int rank_owner(const DecodeSplit& d, uint32_t u) {
  const uint32_t RU = split_ru(d);
  return (int)fdiv((u + 1) * (uint32_t)d.Rw + RU - 1, d.by_ru) - 1;
}

// Row units on the cost axis: each band takes KB + X, its units then a gap of
// X, so a run that crosses a band boundary pays X of its share (the arrival
// and the next band's start cost a stream about that much), and a run
// boundary that falls into a gap moves to the next band's start.
__host__ __device__ inline uint32_t row_cost(const DecodeSplit& d, uint32_t u) {
  if (d.X == 0) return u;
  return u + (uint32_t)d.X * fdiv(u, d.by_kb);
}
__host__ __device__ inline uint32_t row_unit_at(const DecodeSplit& d, uint32_t c) {
  if (d.X == 0) return c;
  const uint32_t k = fdiv(c, d.by_kbx);
  const uint32_t off = c - k * (uint32_t)(d.KB + d.X);
  return k * (uint32_t)d.KB + (off < (uint32_t)d.KB ? off : (uint32_t)d.KB);
}
// First row unit of workgroup w, before alignment.
__host__ __device__ inline uint32_t row_begin_raw(const DecodeSplit& d, int w) {
  const uint32_t wp = w > d.S ? (uint32_t)(w - d.S) : 0u;
  const uint32_t Pp = (uint32_t)(d.P - d.S);
  const uint32_t Rp = (uint32_t)(d.Rw - d.S);
  return row_unit_at(d, fdiv(wp * (uint32_t)d.C + Pp - 1, d.by_pp) -
                            (wp < Rp ? wp : Rp) * (uint32_t)d.D);
}
// First row unit of workgroup w (WU for w == P), moved to an even block.
__host__ __device__ inline uint32_t row_begin(const DecodeSplit& d, int w) {
  uint32_t b = row_begin_raw(d, w);
  if (b > 0 && b < split_wu(d) && fmod(b, d.by_kb) % 2 == 1) ++b;
  return b;
}
// Workgroup whose row run holds row unit u: the largest w with
// row_begin(w) <= u (runs from S on are never empty).  Without the
// even-block move, row_begin_raw(S + w') <= u reads, with c = row_cost(u),
// for w' >= Rw - S, w' C / P' <= c + (Rw - S) D, and below,
// w' (C - P' D) / P' <= c (the ceilings drop out against the integer c, and
// row_unit_at(a) <= u exactly when a <= c); the largest such w' is one
// division.  The move adds at most one unit, so the owner is that estimate
// or the workgroup before it.
__host__ __device__ inline int row_owner(const DecodeSplit& d, uint32_t u) {
  const uint32_t Pp = (uint32_t)(d.P - d.S);
  const uint32_t Rp = (uint32_t)(d.Rw - d.S);
  const uint32_t c = row_cost(d, u);
  uint32_t wp = fdiv((c + Rp * (uint32_t)d.D) * Pp, d.by_c);
  if (wp < Rp) wp = fdiv(c * Pp, d.by_cd);
  int w = d.S + (int)(wp < Pp - 1 ? wp : Pp - 1);
  if (w > d.S && row_begin(d, w) > u) --w;
  return w;
}
// The search it replaces, for the host-side check.
inline int row_owner_search(const DecodeSplit& d, uint32_t u) {
  int lo = d.S, hi = d.P - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (row_begin(d, mid) <= u) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Partial-sum slot of workgroup w for row band `band` / rank band `rb`.
__host__ __device__ inline int row_slot(const DecodeSplit& d, int w, int band) {
  return 2 * w + (fdiv(row_begin(d, w), d.by_kb) == (uint32_t)band ? 0 : 1);
}
__host__ __device__ inline int rank_slot(const DecodeSplit& d, int w, int rb) {
  return 2 * d.P + 2 * w + (fdiv(rank_begin(d, w), d.by_kb) == (uint32_t)rb ? 0 : 1);
}
__host__ __device__ inline int split_slots(const DecodeSplit& d) { return 4 * d.P; }

// The planner's constants: rank units per rank workgroup (four bursts;
// workgroup 0 sums one partial per rank workgroup), and what a rank
// workgroup's share of the projection stands for in row units: 1.5 per rank
// unit (16 KB of A against 8 KB of codes, but the rank stream starts at once
// and its loads are wide rows).  Measured on the 28672 x 8192 layer at rank
// 64: 2.5 per unit plus 4 for the hand-off left the rank workgroups' row
// runs ending 5 us before the others; 1.5 gave the shortest call (1 and 2
// measured longer).
constexpr int kRankUnitsPerWg = 8;
constexpr int kRankUnitCost2 = 3;   // twice the row-unit equivalents of one rank unit
constexpr int kRankFixedCost = 0;

inline DecodeSplit with_divisors(DecodeSplit d) {
  const uint32_t RU = split_ru(d);
  d.by_kb = make_fastdiv((uint32_t)d.KB);
  d.by_pp = make_fastdiv((uint32_t)(d.P - d.S));
  d.by_rw = make_fastdiv(d.Rw > 0 ? (uint32_t)d.Rw : 1u);
  d.by_ru = make_fastdiv(RU > 0 ? RU : 1u);
  d.by_c = make_fastdiv(d.C > 0 ? (uint32_t)d.C : 1u);
  d.by_kbx = make_fastdiv((uint32_t)(d.KB + d.X));
  const long long cd = (long long)d.C - (long long)(d.P - d.S) * d.D;
  d.by_cd = make_fastdiv(cd > 0 ? (uint32_t)cd : 1u);
  return d;
}

// What a run's crossing of a row band boundary costs on the cost axis: about
// what a stream covers in the time of the arrival and the next band's start
// (measured: 10 units), at most a quarter of a workgroup's share, so that
// no run's window can fall into a gap whole.
constexpr int kBoundaryCost = 10;
constexpr int kBoundaryShare = 4;
constexpr int kAlignedShare = 32;

// The split for P_max = slots workgroups, before the band boundaries are
// given a cost.  shared = false keeps the rank workgroups off the rows
// (separate mode) whatever the sizes.  Host only.
inline DecodeSplit make_split_flat(int KB, int RB, int NB, int slots, bool shared = true) {
  DecodeSplit d;
  d.X = 0;
  d.KB = KB;
  d.RB = RB;
  d.NB = NB;
  const long long RU = (long long)RB * KB, WU = (long long)NB * KB;
  slots = slots < 1 ? 1 : slots;
  const long long prow = WU / 2 > 0 ? WU / 2 : 1;  // at least two row units per row workgroup
  if (RU == 0) {
    d.Rw = d.S = d.D = 0;
    d.P = (int)(slots < prow ? slots : prow);
    d.C = (int)WU;
    return d;
  }
  long long Rw = (RU + kRankUnitsPerWg - 1) / kRankUnitsPerWg;
  if (Rw > slots) Rw = slots;
  const long long upw = (RU + Rw - 1) / Rw;
  const long long D = (kRankUnitCost2 * upw + 1) / 2 + kRankFixedCost;
  // shared: floor(C / (P - 1)) >= 2 D + 2, so a rank workgroup keeps at
  // least as many row units as its rank units stand for (and two at least)
  long long p_sh = 1 + (WU + (Rw - 1) * D) / (2 * D + 2);
  if (p_sh > slots) p_sh = slots;
  // separate: Rw rank workgroups, then P - Rw >= 1 row workgroups of >= 2
  // units each (fewer rank workgroups if the slots run out)
  if (Rw > slots - 1) Rw = slots - 1;
  long long p_sep = Rw + prow;
  if (p_sep > slots) p_sep = slots;
  const long long rw_sh = (RU + kRankUnitsPerWg - 1) / kRankUnitsPerWg < slots
                              ? (RU + kRankUnitsPerWg - 1) / kRankUnitsPerWg
                              : slots;
  if (shared && p_sh >= rw_sh && p_sh >= 2 && (Rw < 1 || p_sh >= p_sep)) {
    d.S = 1;
    d.P = (int)p_sh;
    d.D = (int)D;
    d.Rw = (int)rw_sh;
    d.C = (int)(WU + (rw_sh - 1) * D);
  } else if (Rw >= 1) {
    d.S = (int)Rw;
    d.Rw = (int)Rw;
    d.P = (int)p_sep;
    d.D = 0;
    d.C = (int)WU;
  } else {  // one workgroup takes everything
    d.S = 0;
    d.P = 1;
    d.Rw = 1;
    d.D = 0;
    d.C = (int)WU;
  }
  return d;
}

// The split with the band boundaries' cost.  Host only.
inline DecodeSplit make_split_plain(int KB, int RB, int NB, int slots, bool shared = true) {
  DecodeSplit d = make_split_flat(KB, RB, NB, slots, shared);
  const int Pp = d.P - d.S;
  const long long share = Pp > 0 ? (long long)d.C / Pp : 0;
  // Short runs, and no rank work on the row workgroups: M row workgroups
  // per band (S + M NB in all) and no boundary cost, so that every M-th run
  // starts a band and no run crosses one (a crossing costs a second arrival
  // and segment start, several times a short run's streaming), as long as
  // that keeps three quarters of the row workgroups busy.  Measured: the
  // 4096 x 4096 layer (runs of 4 units) 16.1 -> 13.4 us at one token and
  // 22.4 -> 19.2 us at 32; 8192 x 8192 (runs of 16-17) -0.4 us at 16 tokens
  // and -0.7 us at 9.
  if (d.S == d.Rw && Pp >= NB && share < kAlignedShare) {
    const int M = Pp / NB;
    if (2 * M <= KB && 4 * NB * M >= 3 * Pp) {
      d.P = d.S + NB * M;
      return d;
    }
  }
  // (runs of a few units, a few microseconds in all, gain nothing from it:
  // measured slower with X = 1 at 4 units per run)
  const long long X = share >= 4 * kBoundaryShare ? share / kBoundaryShare : 0;
  d.X = (int)(X < kBoundaryCost ? X : kBoundaryCost);
  d.C += d.X * (NB - 1);
  return d;
}

inline DecodeSplit make_split(int KB, int RB, int NB, int slots, bool shared = true) {
  return with_divisors(make_split_plain(KB, RB, NB, slots, shared));
}

// Partial-sum slots a workspace holds for a layer: enough for the split at
// any slot count up to max_slots (P and Rw only shrink with fewer slots): two
// per workgroup of the largest split, two per rank workgroup at most.  Host.
inline int split_workspace_slots(int KB, int RB, int NB, int max_slots, bool shared = true) {
  const DecodeSplit big = make_split(KB, RB, NB, max_slots, shared);
  const long long RU = (long long)RB * KB;
  long long rw = (RU + kRankUnitsPerWg - 1) / kRankUnitsPerWg;
  if (rw > max_slots) rw = max_slots;
  if (rw < big.Rw) rw = big.Rw;
  return 2 * big.P + 2 * (int)rw;
}

}  // namespace spear
