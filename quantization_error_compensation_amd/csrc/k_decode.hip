// Decode path (1..32 tokens): one fused, bandwidth-bound kernel.
//
// SPEAR summary, section 2.2 A (phase-aware adaptive kernel fusion): in the
// memory-bound decode phase the compensator is fused into the epilogue of the
// low-bit GEMM, so the whole compensated layer is one kernel.  One launch
// streams the packed weights once, computes the rank-r projection of every
// token once, gates it, and adds alpha * B * v before the single bf16 store.
//
// Work.  A "band" is either BR = 16 x (waves per workgroup) output rows of
// packed codes or 64 rows (ranks) of A; a "unit" is one 128-column block of
// one band.  partition.hpp fixes which units each of the P persistent
// workgroups takes: the rank units in short runs on the first workgroups
// (so the projection every row finisher needs is published early), and the
// row units in a stream-K split in which those workgroups' share starts later
// by the cost of their rank units.  A workgroup walks its runs band segment
// by band segment.  A band covered by several workgroups has its partial sums
// combined by whichever arrives last (in workgroup order, so results are
// deterministic); partial sums move through device-scope stores and loads
// (coherent across XCDs, no L2-wide fence).
//
// Inside a row segment each wave of a workgroup owns one 16-row tile and all
// walk the same K blocks in bursts of NS blocks (tall bands and short bursts:
// x is read from L2 once per BR rows, and few loads queue per compute unit):
//   * every load of a burst (x, codes or A rows, metadata) is issued one
//     burst ahead, into registers, so it is in flight while the previous
//     burst computes (in row segments the second half of the waves issues
//     it after the previous burst's barrier, the first half before);
//   * x of the burst is loaded once per workgroup (4 tokens x 256 B per
//     instruction, full cache lines, spread over the waves: in row segments
//     three per wave of the first half, one per wave of the second), permuted into
//     the matrix-core K order and written to a double-buffered LDS area; one
//     barrier per burst publishes it to all waves;
//   * codes: 16 bytes per lane per block, four consecutive lanes reading a
//     row's 64 contiguous bytes (16 rows x 64 B per instruction: lanes that
//     read 16 different rows slowed the address unit), turned into the
//     matrix-core layout (lane = row) through a wave-private LDS area when
//     the burst computes; bf16 operands 128 + c by byte permutes;
//   * group scales and zero-points: staged per wave in LDS by chunks of 16
//     bursts (one packed word per row and block), one row of the next chunk
//     loaded with each burst;
//   * matrix cores 16x16x32: tokens (padded to 16 or 32) x 16 rows x 32 K;
//     each K step also multiplies x by the exact bf16 -(128 + z), which
//     removes the codes' offset inside the same fp32 chain (block sums of x
//     in vector code cost more than these matrix-core steps: the decode
//     kernel's vector units, not its matrix cores, are the busy ones).
// In a rank segment the waves form W / 4 phases of four 16-rank tiles; phase
// f takes block f of each burst and the phases are summed in LDS at the end.
// The band finisher adds alpha * B * v as a small K = r matrix-core product
// (v split into bf16 high and low parts) and stores y.
//
// The projection.  Each rank workgroup stores its partial projection of a
// rank band in its slot and posts it with an atomic whose result it does not
// wait for, then goes on to its row units.  Workgroup 0, which takes no row
// units, waits for every post of a band, sums the partials in workgroup
// order, gates, publishes alpha * v and raises the count that the row
// finishers wait for.  So the reduction delays no row stream.
//
// Waiting: row finishers wait for that count, and workgroup 0 for the posts.
// Rank units belong to the lowest workgroup indices, which the dispatcher
// starts first, and a rank workgroup posts before it waits for anything;
// with one workgroup per compute unit and no more workgroups than compute
// units every wait ends.  The waits are bounded all the same: one that gives
// up writes NaN (or publishes NaN) and sets an error bit
// (spear_ec_workspace_status).
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace spear {
namespace {

struct DecodeParams {
  const uint16_t* x;       // [T][K] bf16
  const uint32_t* wq;      // [N][K/8]
  const uint16_t* scales;  // [N][G] fp16
  const uint32_t* zeros;   // [N][ZW], or any valid address when has_z == 0
  const uint16_t* A;       // [r][K] bf16
  const uint16_t* B;       // [N][r] bf16
  const float* gv;         // [r]
  const float* bv;         // [r]
  int gh;                  // bottleneck-MLP gate width (0: elementwise gate gv, bv)
  const float* w1;         // [gh][r]
  const float* b1;         // [gh]
  const float* w2;         // [r][gh]
  const float* b2;         // [r]
  float alpha;
  float* part;             // [nslots][BR][T4] partial sums
  float* wv32;             // [T][r] alpha * v
  int* ctr;                // counter words
  void* y;                 // [T][N] bf16 (fp32 with out_f32)
  int out_f32;
  int T, K, N, r, G, ZW, has_z;
  int KB;                  // 128-column blocks per row
  int RB;                  // rank bands (64 ranks each)
  DecodeSplit sp;          // which units each workgroup takes (partition.hpp)
  int nslots;              // partial-sum slots in the workspace
  int s0;                  // SERQ: first salient channel (the correction is x[:, s0 ..] R^T,
                           // R in B's place, no rank bands); -1 otherwise
};

constexpr int W = kDecodeWaves;        // waves per workgroup
constexpr int BR = kDecodeBandRows;    // rows of a row band (16 per wave)
constexpr int PH = W / 4;              // phases of a rank segment (4 tiles of 16 ranks each)
static_assert(W == 8 || W == 16, "a workgroup is 8 or 16 waves");
constexpr int kThreads = 64 * W;

constexpr int XROW = 272;            // LDS row of one token: 256 B + 16 B pad
// Bounded wait: 2^20 polls, each a device-scope load (about a microsecond
// under load) after s_sleep 1 (64 clocks): about a second at most.
constexpr int kSpinLimit = 1 << 20;

// Blocks per burst: 4 in row segments up to 16 tokens (2 above, for
// registers), one per phase in rank segments.  One x buffer holds
// [kMax][16 MT tokens][XROW] of x, then [kMax][16 MT] floats of room that the
// MLP gate's working area and the rank phase sums also use.
template <int MT>
struct Burst {
  static constexpr int kRow = MT == 1 ? 4 : 2;
  static constexpr int kRank = PH;
  static constexpr int kMax = kRow > kRank ? kRow : kRank;
  static constexpr int kBuf = kMax * 16 * MT * (XROW + 4);  // bytes of one x buffer
};

// ------------------------------------------------------------- x staging
// x of blocks [b, b + NS) into an LDS buffer [NS][16*MT tokens][XROW], each
// 16-byte piece already in the matrix-core K order.  The burst is NS x 4MT
// pieces of 4 tokens x 256 B; in rank segments piece e = k W + w (block
// e / 4MT, tokens 4 (e % 4MT) .. +3) is load k of wave w (lane: token +
// l/16, 16 B l%16); row segments split the pieces unevenly (below).
// Every wave issues the same loads whatever T is, so the count of loads in
// flight, and with it every wait, is path-independent: lanes of tokens past
// T, pieces past the burst, blocks past the segment and all lanes when live
// is false load from past the end of the buffer, which reads zeros without a
// memory access.  A block past the segment is then computed with x = 0 (it
// adds nothing): skipping it would leave its registers unwaited on a path
// the compiler cannot rule out, and it then waits for every load at the top
// of the loop instead.
template <int MT, int NS>
struct XStage {
  static constexpr int kPieces = NS * 4 * MT;
  static constexpr int kLoads = (kPieces + W - 1) / W;
  u32x4 g[kLoads];
};

template <int MT, int NS>
__device__ __forceinline__ void x_issue(const DecodeParams& p, int wave, int lane, int b, int hi,
                                        bool live, XStage<MT, NS>& s) {
  using S = XStage<MT, NS>;
  const uint32_t xrowB = (uint32_t)p.K * 2;
  const rsrc_t xr = make_rsrc(p.x, (uint32_t)p.T * xrowB);
  for (int k = 0; k < S::kLoads; ++k) {
    const int e = k * W + wave, i = min(e / (4 * MT), NS - 1);
    const int t = 4 * (e % (4 * MT)) + (lane >> 4);
    const bool ok = live && e < S::kPieces && t < p.T && b + i < hi;
    const uint32_t vo = ok ? (uint32_t)t * xrowB + 16u * (lane & 15) : 0x80000000u;
    // (uniform: readfirstlane keeps the offset scalar, or the compiler loops)
    s.g[k] = bload16(xr, vo, __builtin_amdgcn_readfirstlane((uint32_t)min(b + i, hi - 1) * 256));
  }
}

// Store the burst's x into buf, each 16-byte piece in the matrix-core K
// order.
template <int MT, int NS>
__device__ __forceinline__ void x_store(uint8_t* buf, int wave, int lane,
                                        const XStage<MT, NS>& s) {
  using S = XStage<MT, NS>;
  for (int k = 0; k < S::kLoads; ++k) {
    const int e = k * W + wave, i = e / (4 * MT);
    const int t = 4 * (e % (4 * MT)) + (lane >> 4);
    if (S::kPieces % W == 0 || e < S::kPieces)
      *reinterpret_cast<u32x4*>(buf + (i * 16 * MT + t) * XROW + 16 * (lane & 15)) =
          x_permute8(s.g[k]);
  }
}

// Row segments split the burst's 16 x pieces unevenly: the first half of
// the waves loads three each (pieces 4 j + wave), the second half one each
// (piece 12 + wave - 4).  The second half's waves get the SIMD last in each
// burst's compute; what they load and store before the next barrier is
// what the whole workgroup waits for (measured at 16 tokens on the 28672 x
// 8192 layer: 0.7 us less per call than two pieces each, and 0.5 us less at
// one token on the 4096 and 8192 layers).
template <int H>
struct XRowSplit {
  static constexpr int kLoads = H == 0 ? 3 : 1;
};
__device__ __forceinline__ int x_row_piece(int h, int j, int wave) {
  return h == 0 ? 4 * j + wave : 12 + wave - W / 2;
}
template <int MT>
struct XRowStage {
  u32x4 g[3];
};
template <int MT, int NS, int H>
__device__ __forceinline__ void x_issue_row(const DecodeParams& p, int wave, int lane, int b, int hi,
                                            bool live, XRowStage<MT>& s) {
  static_assert(W == 8 && NS * 4 * MT == 16, "16 pieces over 8 waves");
  const uint32_t xrowB = (uint32_t)p.K * 2;
  const rsrc_t xr = make_rsrc(p.x, (uint32_t)p.T * xrowB);
  for (int j = 0; j < XRowSplit<H>::kLoads; ++j) {
    const int e = x_row_piece(H, j, wave), i = e / (4 * MT);
    const int t = 4 * (e % (4 * MT)) + (lane >> 4);
    const bool ok = live && t < p.T && b + i < hi;
    const uint32_t vo = ok ? (uint32_t)t * xrowB + 16u * (lane & 15) : 0x80000000u;
    s.g[j] = bload16(xr, vo, __builtin_amdgcn_readfirstlane((uint32_t)min(b + i, hi - 1) * 256));
  }
}
template <int MT, int NS, int H>
__device__ __forceinline__ void x_store_row(uint8_t* buf, int wave, int lane, const XRowStage<MT>& s) {
  for (int j = 0; j < XRowSplit<H>::kLoads; ++j) {
    const int e = x_row_piece(H, j, wave), i = e / (4 * MT);
    const int t = 4 * (e % (4 * MT)) + (lane >> 4);
    *reinterpret_cast<u32x4*>(buf + (i * 16 * MT + t) * XROW + 16 * (lane & 15)) =
        x_permute8(s.g[j]);
  }
}

// Fragment (mt, j) of block i for lane (token c16 + 16 mt, K group q): piece
// 4q + j of the token's 256-byte block row (columns 32q + 8j .. +7).
template <int MT>
__device__ __forceinline__ void x_frags(const uint8_t* buf, int i, int lane, u32x4 (&f)[MT][4]) {
  const int q = lane >> 4, c16 = lane & 15;
  for (int mt = 0; mt < MT; ++mt)
    for (int j = 0; j < 4; ++j)
      f[mt][j] = *reinterpret_cast<const u32x4*>(buf + (i * 16 * MT + 16 * mt + c16) * XROW +
                                                 (4 * q + j) * 16);
}

// A wave's code area (4 KB of LDS), where loads made with consecutive lanes
// along a row are turned into the matrix-core layout (one lane per row).
// Row segments: [block of the burst][16 rows][64 B], 16-byte piece q of row
// r at position q ^ code_swz(r); rank segments: [16 rows of A][256 B], piece
// e of row r at position e ^ r.  Both spread the writes (consecutive lanes
// along a row) and the reads (one lane per row) over the banks.
__device__ __forceinline__ int code_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
constexpr int kCodeArea = 4 * 1024;  // bytes per wave: up to four blocks

// The same two stages, with each burst's loads issued inside the previous
// burst's consume, right after its barrier and before its compute.  The
// second half of a workgroup's waves runs its row segments this way.  The
// two waves that share a SIMD compute a burst at the same time and the
// first half gets the SIMD first (it finishes about 0.4 us earlier); a wave
// of the second half then issued its next loads only after its compute,
// where the queue at the memory pipeline held it 0.3-0.4 us on the way to
// the next barrier.  Issued before its compute, that wait overlaps the first
// half's compute; the loads have one compute phase to arrive instead of a
// whole burst, which is enough for the second half's later use.
template <class Stage, class Issue, class Consume>
__device__ __forceinline__ void pipeline2_late(int lo, int hi, int ns, Stage& s0, Stage& s1,
                                               Issue&& issue, Consume&& consume) {
  const int nb = (hi - lo + ns - 1) / ns;
  int b = lo;
  for (int k = 0; k + 1 < nb; k += 2, b += 2 * ns) {
    consume(s0, b, [&] { issue(s1, b + ns); });
    consume(s1, b + ns, [&] { issue(s0, b + 2 * ns); });
  }
  if (nb & 1) consume(s0, b, [&] { issue(s1, b + ns); });
  __builtin_amdgcn_s_waitcnt(0);
}

// ------------------------------------------------------------ rank segment
// A barrier that leaves global loads in flight: only this wave's LDS writes
// are awaited before the workgroup meets.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The burst loop of a segment [lo, hi) in bursts of ns blocks, stage s0
// already issued for the first burst: two register stages in turn, the next
// burst's loads issued before this one computes.  The loop has one exit (at
// the bottom) and every stage that enters it is consumed in it, so the
// compiler's wait counts stay exact; with two exits its merged exit path
// reached the top of the loop with a stage never consumed, and it then waited
// for every load there, on every burst.  The scheduling barriers keep the
// next stage's loads ahead of the work on this one.  The stage issued past
// the last burst (out of range: no memory access, returns at once) is waited
// for at the end, so nothing is left in flight for the code that follows.
template <class Stage, class Issue, class Consume>
__device__ __forceinline__ void pipeline2(int lo, int hi, int ns, Stage& s0, Stage& s1,
                                          Issue&& issue, Consume&& consume) {
  const int nb = (hi - lo + ns - 1) / ns;  // bursts
  int b = lo;
  for (int k = 0; k + 1 < nb; k += 2, b += 2 * ns) {
    issue(s1, b + ns);
    __builtin_amdgcn_sched_barrier(0);
    consume(s0, b);
    issue(s0, b + 2 * ns);
    __builtin_amdgcn_sched_barrier(0);
    consume(s1, b + ns);
  }
  if (nb & 1) {  // last burst in s0
    issue(s1, b + ns);
    __builtin_amdgcn_sched_barrier(0);
    consume(s0, b);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// What one burst of a rank segment takes from memory: x and, per wave, the
// A rows of its tile in its phase's block.
template <int MT, int NS>
struct RankStage {
  XStage<MT, NS> x;
  u32x4 a[4];
};

// Ranks 64 rb + 16 (wave % 4) + c16, blocks [lo, hi): u = x A^T over the
// segment, in the waves of phase 0 (wave < 4) on return.  Loads run one burst
// ahead, in two register stages, as in row segments; phase f = wave / 4
// takes block b + f of the burst starting at b.
template <int MT>
__device__ void rank_segment(const DecodeParams& p, int rb, int lo, int hi, uint8_t* xlds,
                             uint8_t* clds, int& burst, f32x4 (&uo)[MT]) {
  constexpr int NS = Burst<MT>::kRank;
  static_assert(NS == PH, "one block per phase and burst");
  const int lane = threadIdx.x & 63, wave = wave_id(), q = lane >> 4, c16 = lane & 15;
  const int tile = wave & 3, ph = wave >> 2;
  // A tile of ranks j0 .. j0 + 15; a tile past r reads the last tile again
  // (its u columns are never published)
  const int j0 = min(64 * rb + 16 * tile, p.r - 16);
  const uint32_t arowB = (uint32_t)p.K * 2;
  const rsrc_t ar = make_rsrc(p.A + (size_t)j0 * p.K, 16u * arowB);
  // load layout: 16 consecutive lanes read a row's 256 B (rows lane / 16 + 4 j),
  // turned into the matrix-core layout through the wave's code area
  const uint32_t ao = (uint32_t)(lane >> 4) * arowB + 16u * (lane & 15);
  uint8_t* cl = clds + wave * kCodeArea;
  for (int mt = 0; mt < MT; ++mt) uo[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](RankStage<MT, NS>& s, int b) {
    const bool live = b < hi;  // a burst past the segment loads nothing
    x_issue<MT, NS>(p, wave, lane, b, hi, live, s.x);
    const uint32_t av = b + ph < hi ? ao : 0x80000000u;
    for (int j = 0; j < 4; ++j)
      s.a[j] = bload16(ar, av + 4u * j * arowB,
                       __builtin_amdgcn_readfirstlane((uint32_t)min(b + ph, hi - 1) * 256));
  };
  auto consume = [&](RankStage<MT, NS>& s, int b) {
    uint8_t* buf = xlds + (burst & 1) * Burst<MT>::kBuf;
    ++burst;
    x_store<MT, NS>(buf, wave, lane, s.x);
    for (int j = 0; j < 4; ++j) {  // piece e of row r at position e ^ r
      const int r = (lane >> 4) + 4 * j;
      *reinterpret_cast<u32x4*>(cl + r * 256 + (((lane & 15) ^ r) * 16)) = s.a[j];
    }
    lds_barrier();
    {  // a block past the segment has x = 0 and A = 0: it adds nothing
      u32x4 xf[MT][4];
      x_frags<MT>(buf, ph, lane, xf);
      for (int j = 0; j < 4; ++j) {
        const u32x4 araw =
            *reinterpret_cast<const u32x4*>(cl + c16 * 256 + (((4 * q + j) ^ c16) * 16));
        const u32x4 ap = x_permute8(araw);
        for (int mt = 0; mt < MT; ++mt) uo[mt] = mfma16x16x32(xf[mt][j], ap, uo[mt]);
      }
    }
  };

  RankStage<MT, NS> s0, s1;
  __builtin_amdgcn_s_waitcnt(0);  // as in row segments
  issue(s0, lo);
  pipeline2(lo, hi, NS, s0, s1, issue, consume);

  // Phase sums, in phase order, through the x buffer the next burst fills
  // (every wave has passed the barrier after its last read).
  if constexpr (PH > 1) {
    static_assert((PH - 1) * 4 * MT * 64 * 16 <= Burst<MT>::kBuf, "phase sums fit an x buffer");
    f32x4* red = reinterpret_cast<f32x4*>(xlds + (burst & 1) * Burst<MT>::kBuf);
    if (ph > 0)
      for (int mt = 0; mt < MT; ++mt) red[(((ph - 1) * 4 + tile) * MT + mt) * 64 + lane] = uo[mt];
    __syncthreads();
    if (ph == 0)
      for (int f = 1; f < PH; ++f)
        for (int mt = 0; mt < MT; ++mt) uo[mt] += red[(((f - 1) * 4 + tile) * MT + mt) * 64 + lane];
    __syncthreads();
  }
}

// -------------------------------------------------------------- row segment
// Group scales and zero-points of a wave's 16 rows are staged in the wave's
// own LDS area by chunks of C blocks counted from the segment start
// (chunk j: blocks lo + C j .., C = 16 NS), two chunks at a time: slot j % 2
// holds one 32-bit word per (row, block), the scale's fp16 bits in the low
// half and the bf16 bits of -(128 + z) (exact) in the high half, rows C + 4 words
// apart (a burst's NS words are one 8- or 16-byte read).  The first chunk is
// loaded with the segment's first burst; then each burst of chunk j loads
// one row of chunk j + 1 (a scale and its zero-point word per lane), packed
// and written to LDS when the burst computes.  Bursts never straddle a
// chunk, and all loads are issued on every burst.
template <int MT>
struct Meta {
  static constexpr int kChunk = 16 * Burst<MT>::kRow;  // one row of the next chunk per burst
  static constexpr int kStride = kChunk + 4;           // words per row
  static constexpr int kSlot = 16 * kStride;           // words per slot
  static constexpr int kWave = 2 * kSlot * 4;          // bytes per wave
  static_assert(kChunk <= 64, "an entry per lane");
};

// The packed word of one (row, block): fp16 scale bits s in the low half and
// the bf16 bits of -(128 + z) (exact) in the high half, z from the
// zero-point word zw of the block's group of eight (none: z = 8).
__device__ __forceinline__ uint32_t meta_pack(uint32_t s, uint32_t zw, int blk, bool has_z) {
  const uint32_t z = has_z ? (zw >> (4 * (blk & 7))) & 15u : 8u;
  return (s & 0xFFFFu) | ((0xC300u | z) << 16);
}
// A matrix-core operand of eight copies of the bf16 value in the high half
// of w (one K group of one row).
__device__ __forceinline__ u32x4 bf16_splat_hi(uint32_t w) {
  const uint32_t pair = (w & 0xFFFF0000u) | (w >> 16);
  return u32x4{pair, pair, pair, pair};
}

// What one burst of a row segment takes from memory: x (permuted into LDS
// when the burst starts), the codes, and one row of the
// next metadata chunk.  Each burst's loads are issued one burst ahead, so
// they are in flight while the previous burst computes; every load is
// issued on every burst (out of range, with no memory access, past the
// segment), so the compiler's wait counts stay exact.
template <int MT, int NS>
struct RowStage {
  XRowStage<MT> x;
  u32x4 w[NS];
  uint32_t ms, mz;
};

// Rows BR band + 16 wave + c16 (this wave's tile), blocks [lo, hi): partial
// y with the scales applied.  Per block and token the result is s P, P the
// matrix-core chain over the block's K steps of x times the 128 + c
// operands and of x times -(128 + z), that is the sum of (c - z) x.

// mid() runs while the segment's first loads are in flight (scalar work
// that the segment does not need).
template <int MT, bool GROUPED, class Mid>
__device__ void row_segment(const DecodeParams& p, int band, int lo, int hi, uint8_t* xlds,
                            uint8_t* mlds, uint8_t* clds, int& burst, f32x4 (&yo)[MT],
                            Mid&& mid) {
  constexpr int NS = Burst<MT>::kRow;
  constexpr uint32_t kOut = 0x80000000u;
  const int lane = threadIdx.x & 63, wave = wave_id(), q = lane >> 4, c16 = lane & 15;
  // Tile of rows rc .. rc + 15; a tile past N (last band of an N that is not
  // a multiple of BR) reads the last tile again and stores nothing.
  const int rc = min(band * BR + 16 * wave, p.N - 16);
  const uint32_t wrowB = (uint32_t)p.K / 2;
  const rsrc_t wr = make_rsrc(p.wq + (size_t)rc * (p.K / 8), 16u * wrowB);
  // load layout: lane 4 r + j reads piece j of row r
  const int lr = lane >> 2, lj = lane & 3;
  const uint32_t wo = (uint32_t)lr * wrowB + 16u * lj;
  uint8_t* cl = clds + wave * kCodeArea;
  static_assert(NS * 1024 <= kCodeArea, "code area");
  const rsrc_t sr = make_rsrc(p.scales + (size_t)rc * p.G, 16u * p.G * 2);
  const rsrc_t zr = make_rsrc(p.zeros + (size_t)rc * p.ZW, p.has_z ? 16u * p.ZW * 4 : 0u);
  using M = Meta<MT>;
  uint32_t* mw = reinterpret_cast<uint32_t*>(mlds + wave * M::kWave);
  // packed word of row n, block lo + C j + c: slot j & 1, [n][c]
  auto mp_at = [&](int slot, int n, int c) { return mw + slot * M::kSlot + n * M::kStride + c; };
  // this lane's entry of a chunk (lanes past C repeat an entry) and its block
  // (clamped into the segment) in a chunk starting at cb
  const int ment = lane % M::kChunk;
  auto meta_blk = [&](int cb) { return min(cb + ment, hi - 1); };
  // loads of row n (per lane) at block blk: scale bits, zero-point word
  auto meta_scale = [&](int n, int blk) { return bload2(sr, (uint32_t)(n * p.G + blk) * 2, 0); };
  auto meta_zero = [&](int n, int blk) { return bload4(zr, (uint32_t)(n * p.ZW + (blk >> 3)) * 4, 0); };

  // acc: the grouped result; per-channel: one product accumulator per block
  // of a burst (accb), summed at the end
  f32x4 acc[MT], accb[NS][MT];
  for (int mt = 0; mt < MT; ++mt) {
    acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < NS; ++i) accb[i][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Per-channel: the row's -(128 + z) operand and scale, read before the loop.
  u32x4 nzrow = u32x4{0u, 0u, 0u, 0u};
  float scrow = 0.f;
  if constexpr (!GROUPED) {
    const int n = rc + c16;
    const uint32_t z = p.has_z ? p.zeros[(size_t)n * p.ZW] & 15u : 8u;
    nzrow = bf16_splat_hi((0xC300u | z) << 16);
    scrow = half_bits_to_f32(p.scales[n]);
  }

  auto issue = [&](RowStage<MT, NS>& s, int b, auto half) {
    const bool live = b < hi;  // a burst past the segment loads nothing
    x_issue_row<MT, NS, decltype(half)::value>(p, wave, lane, b, hi, live, s.x);
    const uint32_t wv = live ? wo : kOut;
    for (int i = 0; i < NS; ++i)
      s.w[i] = bload16(wr, wv, __builtin_amdgcn_readfirstlane((uint32_t)min(b + i, hi - 1) * 64));
    if constexpr (GROUPED) {
      const int k = (b - lo) / NS;  // burst index: row k % 16 of chunk k / 16 + 1
      const int blk = meta_blk(lo + M::kChunk * (k / 16 + 1));
      s.ms = meta_scale(k & 15, blk);
      s.mz = meta_zero(k & 15, blk);
    }
  };

  // after(): the next burst's loads on the waves that issue them past the
  // barrier (nothing on the others).  The scheduling barriers keep this
  // burst's LDS stores from moving up into the previous burst's compute and
  // the next burst's loads from moving past this one's start.
  auto consume = [&](RowStage<MT, NS>& s, int b, auto&& after, auto half) {
    __builtin_amdgcn_sched_barrier(0);
    uint8_t* buf = xlds + (burst & 1) * Burst<MT>::kBuf;
    ++burst;
    x_store_row<MT, NS, decltype(half)::value>(buf, wave, lane, s.x);
    for (int i = 0; i < NS; ++i)
      *reinterpret_cast<u32x4*>(cl + i * 1024 + lr * 64 + ((lj ^ code_swz(lr)) * 16)) = s.w[i];
    lds_barrier();
    after();
    __builtin_amdgcn_sched_barrier(0);
    const int k = (b - lo) / NS, j = k / 16;  // this burst's chunk
    uint32_t meta[NS];  // packed words of blocks b .. b + NS - 1 for row c16
    if constexpr (GROUPED) {
      if constexpr (NS == 4) {
        const u32x4 m = *reinterpret_cast<const u32x4*>(mp_at(j & 1, c16, NS * (k & 15)));
        for (int i = 0; i < NS; ++i) meta[i] = m[i];
      } else {
        const u32x2 m = *reinterpret_cast<const u32x2*>(mp_at(j & 1, c16, NS * (k & 15)));
        for (int i = 0; i < NS; ++i) meta[i] = m[i];
      }
    }
    // All blocks' operands first, then their matrix-core chains interleaved
    // (independent chains hide each other's latency), then the per-block
    // scale fold.  The +128 offset of the code operands comes out in the
    // matrix cores too: each K step also multiplies x by -(128 + z) (exact
    // in bf16), so a chain sums (c - z) x directly.  A block past the
    // segment has x = 0: it adds nothing.
    u32x4 xf[NS][MT][4], wb[NS][4], nzb[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      x_frags<MT>(buf, i, lane, xf[i]);
      if constexpr (GROUPED) nzb[i] = bf16_splat_hi(meta[i]);
      else nzb[i] = nzrow;
      const u32x4 cw =
          *reinterpret_cast<const u32x4*>(cl + i * 1024 + c16 * 64 + ((q ^ code_swz(c16)) * 16));
      wb[i][0] = codes_to_bf16_offset(cw.x);
      wb[i][1] = codes_to_bf16_offset(cw.y);
      wb[i][2] = codes_to_bf16_offset(cw.z);
      wb[i][3] = codes_to_bf16_offset(cw.w);
    }
    if constexpr (GROUPED) {
      f32x4 P[NS][MT];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        for (int i = 0; i < NS; ++i)
          for (int mt = 0; mt < MT; ++mt) {
            P[i][mt] = mfma16x16x32(xf[i][mt][jj], wb[i][jj],
                                    jj == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : P[i][mt]);
            P[i][mt] = mfma16x16x32(xf[i][mt][jj], nzb[i], P[i][mt]);
          }
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const float sc = half_bits_to_f32((uint16_t)meta[i]);
        for (int mt = 0; mt < MT; ++mt)
          for (int v = 0; v < 4; ++v) acc[mt][v] = fmaf(sc, P[i][mt][v], acc[mt][v]);
      }
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        for (int i = 0; i < NS; ++i)
          for (int mt = 0; mt < MT; ++mt) {
            accb[i][mt] = mfma16x16x32(xf[i][mt][jj], wb[i][jj], accb[i][mt]);
            accb[i][mt] = mfma16x16x32(xf[i][mt][jj], nzb[i], accb[i][mt]);
          }
    }
    // Row k % 16 of the next chunk (read from burst 16 (j + 1) on).
    if constexpr (GROUPED)
      *mp_at((j + 1) & 1, k & 15, ment) =
          meta_pack(s.ms, s.mz, meta_blk(lo + M::kChunk * (j + 1)), p.has_z);
  };

  // Two stages in turn: while one burst computes, the next one loads.  The
  // stage past the segment's last burst is issued too, with its loads out of
  // range (no memory access): the number of loads in flight is then the same
  // on every path, so the waits on each stage stay exact.  The first chunk's
  // metadata is requested with the first stage and stored in LDS before the
  // loop.
  RowStage<MT, NS> s0, s1;
  // Nothing from before may be in flight when the loop starts: the compiler
  // would otherwise guard the loop's first register writes with a wait for
  // every load, on every burst.
  __builtin_amdgcn_s_waitcnt(0);
  auto run = [&](auto half, auto&& loop) {
    auto iss = [&](RowStage<MT, NS>& s, int b) { issue(s, b, half); };
    if constexpr (GROUPED) {
      uint32_t m0s[16], m0z[16];  // row n, this lane's entry
      const int blk = meta_blk(lo);
      for (int n = 0; n < 16; ++n) m0s[n] = meta_scale(n, blk);
      for (int n = 0; n < 16; ++n) m0z[n] = meta_zero(n, blk);
      iss(s0, lo);
      mid();
      for (int n = 0; n < 16; ++n) *mp_at(0, n, ment) = meta_pack(m0s[n], m0z[n], blk, p.has_z);
    } else {
      iss(s0, lo);
      mid();
    }
    loop(iss);
  };
  if (wave < W / 2) {
    run(std::integral_constant<int, 0>{}, [&](auto& iss) {
      auto consume0 = [&](RowStage<MT, NS>& s, int b) {
        consume(s, b, [] {}, std::integral_constant<int, 0>{});
      };
      pipeline2(lo, hi, NS, s0, s1, iss, consume0);
    });
  } else {
    run(std::integral_constant<int, 1>{}, [&](auto& iss) {
      auto consume1 = [&](RowStage<MT, NS>& s, int b, auto&& after) {
        consume(s, b, after, std::integral_constant<int, 1>{});
      };
      pipeline2_late(lo, hi, NS, s0, s1, iss, consume1);
    });
  }

  if constexpr (!GROUPED) {  // per-channel: one scale per row
    for (int mt = 0; mt < MT; ++mt)
      for (int i = 0; i < NS; ++i) acc[mt] += accb[i][mt];
    for (int mt = 0; mt < MT; ++mt)
      for (int v = 0; v < 4; ++v) acc[mt][v] = scrow * acc[mt][v];
  }
  for (int mt = 0; mt < MT; ++mt) yo[mt] = acc[mt];
}

// ------------------------------------------------------------ partial sums
// [nslots][BR columns][T4] floats (T4: T rounded up to a multiple of 4),
// written and read at device scope; a lane's four tokens of one column form
// one 16-byte word, and words holding no token below T are neither stored
// nor loaded.  Column c of a partial is row BR band + c of a row band, or
// rank 64 rb + c (c < 64) of a rank band.  The slot of workgroup w's partial
// of a band is fixed by the split (row_slot, rank_slot).
__device__ __forceinline__ int tokens4(const DecodeParams& p) { return (p.T + 3) & ~3; }
__device__ __forceinline__ rsrc_t part_rsrc(const DecodeParams& p) {
  return make_rsrc(p.part, (uint32_t)p.nslots * BR * tokens4(p) * 4);
}
__device__ __forceinline__ uint32_t part_off(const DecodeParams& p, int slot, int col, int t) {
  return (uint32_t)(((slot * BR + col) * tokens4(p) + t) * 4);
}
__device__ __forceinline__ int slot_of(const DecodeParams& p, bool rank, int w, int band) {
  return rank ? rank_slot(p.sp, w, band) : row_slot(p.sp, w, band);
}

template <int MT>
__device__ __forceinline__ void put_part(const DecodeParams& p, int slot, int col,
                                         const f32x4 (&v)[MT]) {
  const int q = (threadIdx.x & 63) >> 4;
  const rsrc_t r = part_rsrc(p);
  for (int mt = 0; mt < MT; ++mt) {
    const int t = 16 * mt + 4 * q;
    if (t < p.T) bstore16_dev(r, part_off(p, slot, col, t), 0, v[mt]);
  }
}

// The partials of workgroups first .. first + nseg - 1 for one band, summed
// in workgroup order; 16 / MT partials are in flight at a time.
template <int MT>
__device__ __forceinline__ void sum_parts(const DecodeParams& p, bool rank, int band, int first,
                                          int nseg, int col, f32x4 (&v)[MT]) {
  constexpr int CH = 16 / MT;
  const int q = (threadIdx.x & 63) >> 4;
  const rsrc_t r = part_rsrc(p);
  for (int mt = 0; mt < MT; ++mt) v[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < nseg; k0 += CH) {
    const int n = min(CH, nseg - k0);
    u32x4 w[CH][MT];
    for (int kk = 0; kk < CH; ++kk) {
      const int slot = kk < n ? slot_of(p, rank, first + k0 + kk, band) : 0;
      for (int mt = 0; mt < MT; ++mt) {
        const int t = 16 * mt + 4 * q;
        w[kk][mt] = kk < n && t < p.T ? bload16_dev(r, part_off(p, slot, col, t), 0)
                                      : u32x4{0u, 0u, 0u, 0u};
      }
    }
    for (int kk = 0; kk < CH; ++kk)
      if (kk < n)
        for (int mt = 0; mt < MT; ++mt) v[mt] += __builtin_bit_cast(f32x4, w[kk][mt]);
  }
}

// Finish a rank band: gate and publish alpha * v for this wave's 16 ranks
// (with the MLP gate, which needs every rank of a token, publish u itself).
template <int MT>
__device__ void finish_rank(const DecodeParams& p, int j, float g, float b, const f32x4 (&u)[MT]) {
  const int lane = threadIdx.x & 63, q = lane >> 4;
  if (j >= p.r) return;
  const rsrc_t wr = make_rsrc(p.wv32, (uint32_t)p.T * p.r * 4);
  for (int mt = 0; mt < MT; ++mt)
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * mt + 4 * q + i;
      if (t < p.T) {
        const float uu = u[mt][i];
        bstore_dev(wr, (uint32_t)(t * p.r + j) * 4, 0,
                   p.gh > 0 ? uu : p.alpha * (sigmoidf_safe(fmaf(g, uu, b)) * uu));
      }
    }
}

// n floats from src (plain or device-scope loads) into LDS, eight loads in
// flight per thread so the copy costs about one memory round trip.
template <bool DEV>
__device__ __forceinline__ void copy_to_lds(const float* src, float* dst, int n) {
  const rsrc_t r = make_rsrc(src, (uint32_t)n * 4);
  for (int e0 = threadIdx.x; e0 < n; e0 += 8 * kThreads) {
    float v[8];
    for (int i = 0; i < 8; ++i) {
      const uint32_t off = (uint32_t)(e0 + kThreads * i) * 4;  // past n: zero, not stored
      v[i] = DEV ? bload_dev(r, off, 0) : __builtin_bit_cast(float, bload4(r, off, 0));
    }
    for (int i = 0; i < 8; ++i)
      if (e0 + kThreads * i < n) dst[e0 + kThreads * i] = v[i];
  }
}

// The bottleneck-MLP gate (SPEAR summary, section 2.1 A), run once by the
// workgroup that publishes the last rank band: every token's u (published
// by the rank bands) goes to LDS, then
//     h[t,k]       = relu(b1[k] + sum_i W1[k,i] u[t,i])
//     alpha v[t,j] = alpha * sigmoid(b2[j] + sum_k W2[j,k] h[t,k]) * u[t,j]
// in fp32 (sums in index order), written over u, and the gate counter is
// raised.  W1 and W2 pass through LDS in chunks of whole rows.  lds: lds_floats
// floats free for this workgroup, at least T (r + gh) + max(r, gh).
__device__ void gate_mlp(const DecodeParams& p, uint8_t* lds, int lds_floats) {
  const int tid = threadIdx.x, T = p.T, r = p.r, h = p.gh;
  float* su = reinterpret_cast<float*>(lds);  // [T][r]
  float* sh = su + T * r;                     // [T][h]
  float* sw = sh + T * h;                     // weight rows
  const int cap = lds_floats - T * (r + h);
  const int c1 = min(h, cap / r), c2 = min(r, cap / h);  // rows per chunk of W1, W2
  copy_to_lds<true>(p.wv32, su, T * r);
  for (int k0 = 0; k0 < h; k0 += c1) {
    const int nk = min(c1, h - k0);
    copy_to_lds<false>(p.w1 + (size_t)k0 * r, sw, nk * r);
    __syncthreads();
    for (int e = tid; e < T * nk; e += kThreads) {
      const int t = e / nk, k = e - t * nk;
      float a = p.b1[k0 + k];
      for (int i = 0; i < r; ++i) a = fmaf(sw[k * r + i], su[t * r + i], a);
      sh[t * h + k0 + k] = fmaxf(a, 0.f);
    }
    __syncthreads();
  }
  const rsrc_t wr = make_rsrc(p.wv32, (uint32_t)T * r * 4);
  for (int j0 = 0; j0 < r; j0 += c2) {
    const int nj = min(c2, r - j0);
    copy_to_lds<false>(p.w2 + (size_t)j0 * h, sw, nj * h);
    __syncthreads();
    for (int e = tid; e < T * nj; e += kThreads) {
      const int t = e / nj, j = e - t * nj;
      float a = p.b2[j0 + j];
      for (int k = 0; k < h; ++k) a = fmaf(sw[j * h + k], sh[t * h + k], a);
      bstore_dev(wr, (uint32_t)(t * r + j0 + j) * 4, 0,
                 p.alpha * (sigmoidf_safe(a) * su[t * r + j0 + j]));
    }
    __syncthreads();
  }
  wait_vmem();
  __syncthreads();
  if (tid == 0) atomicAdd(&p.ctr[kCtrGateDone], 1);
  __syncthreads();  // the LDS is the caller's again
}

// Wait (bounded) until alpha * v of every rank is published: every rank band
// (elementwise gate) or the MLP gate's pass.  Returns false for the whole
// workgroup if the wait gave up; the error word then has
// SPEAR_EC_WS_WAIT_TIMEOUT (1) set.
__device__ __forceinline__ bool wait_ranks(const DecodeParams& p, int* s_flag) {
  if (threadIdx.x == 0) {
    int spins = 0, ok = 1;
    const int* ctr = p.gh > 0 ? &p.ctr[kCtrGateDone] : &p.ctr[kCtrRankDone];
    const int target = p.gh > 0 ? 1 : p.RB;
    while (load_dev(ctr) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        atomicOr(&p.ctr[kCtrError], 1);
        ok = 0;
        break;
      }
    }
    *s_flag = ok;
  }
  __syncthreads();
  const bool ok = *s_flag != 0;
  __syncthreads();
  return ok;
}

// alpha * v of this lane's tokens as matrix-core operands: for each K = 32
// rank step k, the bf16 high part and the bf16 remainder of 8 ranks.  Every
// word of all steps is requested before the first is used.
constexpr int kRankSteps = 4;  // r <= 128
template <int MT>
__device__ __forceinline__ void alpha_v_operands(const DecodeParams& p, u32x4 (&hi)[kRankSteps][MT],
                                                 u32x4 (&lo)[kRankSteps][MT]) {
  const int lane = threadIdx.x & 63, q = lane >> 4, c16 = lane & 15;
  // Offsets past a buffer's end read as zero: ranks past r contribute nothing.
  constexpr uint32_t kOut = 0x80000000u;
  const rsrc_t wr = make_rsrc(p.wv32, (uint32_t)p.T * p.r * 4);
  u32x4 wv[kRankSteps][MT][2];
  for (int k = 0; k < kRankSteps; ++k) {
    const int jj = 32 * k + 8 * q;  // this lane's 8 ranks of step k
    for (int mt = 0; mt < MT; ++mt) {
      const int t = min(16 * mt + c16, p.T - 1);
      const uint32_t src = jj < p.r ? (uint32_t)(t * p.r + jj) * 4 : kOut;
      wv[k][mt][0] = bload16_dev(wr, src, 0);
      wv[k][mt][1] = bload16_dev(wr, src + 16, 0);
    }
  }
  for (int k = 0; k < kRankSteps; ++k)
    for (int mt = 0; mt < MT; ++mt) {
      // steps past r are skipped by add_correction: no conversion (at
      // MT = 2 the conversions of four steps took about 1.5 us)
      if (32 * k >= p.r) {
        hi[k][mt] = lo[k][mt] = u32x4{0u, 0u, 0u, 0u};
        continue;
      }
      uint32_t h[8], l[8];
      for (int e = 0; e < 8; ++e) {
        const float v = __uint_as_float(wv[k][mt][e >> 2][e & 3]);
        h[e] = f32_to_bf16_rne(v);
        l[e] = f32_to_bf16_rne(v - __uint_as_float(h[e] << 16));
      }
      hi[k][mt] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                        h[6] | (h[7] << 16)};
      lo[k][mt] = u32x4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16),
                        l[6] | (l[7] << 16)};
    }
}

// SERQ's operands: the salient channels x[t, s0 + 32 k + 8 q ..] of this
// lane's tokens, already bf16 (SERQ summary: one extra product with the
// salient activations, no intermediate quantization).
template <int MT>
__device__ __forceinline__ void serq_operands(const DecodeParams& p, u32x4 (&hi)[kRankSteps][MT]) {
  const int lane = threadIdx.x & 63, q = lane >> 4, c16 = lane & 15;
  constexpr uint32_t kOut = 0x80000000u;
  const rsrc_t xr = make_rsrc(p.x, (uint32_t)p.T * p.K * 2);
  for (int k = 0; k < kRankSteps; ++k) {
    const int jj = 32 * k + 8 * q;
    for (int mt = 0; mt < MT; ++mt) {
      const int t = 16 * mt + c16;
      hi[k][mt] = bload16(xr, jj < p.r && t < p.T ? (uint32_t)(t * p.K + p.s0 + jj) * 2 : kOut, 0);
    }
  }
}

// B fragments of the 16 rows of this wave's tile of a row band: for each
// K = 32 rank step, 8 ranks of the lane's row (zero past r).
__device__ __forceinline__ void b_fragments(const DecodeParams& p, int band,
                                            u32x4 (&bfr)[kRankSteps]) {
  const int lane = threadIdx.x & 63, wave = wave_id(), q = lane >> 4, c16 = lane & 15;
  const int nrow = band * BR + 16 * wave + c16;
  constexpr uint32_t kOut = 0x80000000u;
  const rsrc_t bs = make_rsrc(p.B, (uint32_t)p.N * p.r * 2);
  const uint32_t bro = (uint32_t)min(nrow, p.N - 1) * p.r * 2;
  for (int k = 0; k < kRankSteps; ++k) {
    const int jj = 32 * k + 8 * q;
    bfr[k] = bload16(bs, jj < p.r ? bro + 2 * jj : kOut, 0);
  }
}

// yv += alpha * v B^T for the 16 rows of this wave's tile of a row band, as
// K = r matrix-core products (v split into bf16 high and low parts).
template <int MT>
__device__ __forceinline__ void add_correction(const DecodeParams& p, const u32x4 (&bfr)[kRankSteps],
                                               const u32x4 (&hi)[kRankSteps][MT],
                                               const u32x4 (&lo)[kRankSteps][MT], f32x4 (&yv)[MT]) {
  for (int k = 0; k < kRankSteps; ++k) {
    if (32 * k >= p.r) break;
    for (int mt = 0; mt < MT; ++mt) {
      yv[mt] = mfma16x16x32(hi[k][mt], bfr[k], yv[mt]);
      yv[mt] = mfma16x16x32(lo[k][mt], bfr[k], yv[mt]);
    }
  }
}

// Store y for this wave's tile of a finished row band (bf16, or fp32 with
// out_f32).
template <int MT>
__device__ __forceinline__ void store_row(const DecodeParams& p, int band, const f32x4 (&yv)[MT]) {
  const int lane = threadIdx.x & 63, wave = wave_id(), q = lane >> 4, c16 = lane & 15;
  const int nrow = band * BR + 16 * wave + c16;
  if (nrow < p.N)
    for (int mt = 0; mt < MT; ++mt)
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * mt + 4 * q + i;
        if (t >= p.T) continue;
        if (p.out_f32) static_cast<float*>(p.y)[(size_t)t * p.N + nrow] = yv[mt][i];
        else static_cast<uint16_t*>(p.y)[(size_t)t * p.N + nrow] = (uint16_t)f32_to_bf16_rne(yv[mt][i]);
      }
}

// Add this workgroup's partial sum of row band `band` (shared by workgroups
// first .. first + nseg - 1) and report whether it arrived last; the last one
// gets the sum of all partials in workgroup order in v and clears the band's
// counter.
template <int MT>
__device__ __forceinline__ bool arrive(const DecodeParams& p, int band, int first, int nseg,
                                       int* s_last, f32x4 (&v)[MT]) {
  const int tid = threadIdx.x, col = 16 * wave_id() + (tid & 15);
  int* ctr = &p.ctr[kCtrBand + p.RB + band];
  put_part<MT>(p, slot_of(p, false, blockIdx.x, band), col, v);
  wait_vmem();
  __syncthreads();
  if (tid == 0) *s_last = atomicAdd(ctr, 1) == nseg - 1;
  __syncthreads();
  const bool last = *s_last;
  if (last) {
    sum_parts<MT>(p, false, band, first, nseg, col, v);
    if (tid == 0) store_dev(ctr, 0);
  }
  return last;
}

// A rank workgroup's partial projection of rank band rb: stored in its slot
// (the 64 columns are in waves 0-3), then counted on the band's counter with
// an atomic whose result is not awaited.
template <int MT>
__device__ __forceinline__ void post_rank_part(const DecodeParams& p, int rb, const f32x4 (&v)[MT]) {
  const int tid = threadIdx.x, col = 16 * wave_id() + (tid & 15);
  if (wave_id() < 4) put_part<MT>(p, slot_of(p, true, blockIdx.x, rb), col, v);
  wait_vmem();
  __syncthreads();
  if (tid == 0)
    __hip_atomic_fetch_add(&p.ctr[kCtrBand + rb], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup 0: wait (bounded) until every rank workgroup has posted, sum each
// rank band's partials in workgroup order (the two bands of r > 64 at once,
// one per half of the workgroup), gate and publish alpha v (the MLP gate: u,
// then the gate pass over all ranks), and raise the count the row finishers
// wait for.  A wait that gives up publishes NaN and sets the error word.
template <int MT>
__device__ void reduce_ranks(const DecodeParams& p, uint8_t* xlds, int* s_flag) {
  const DecodeSplit& sp = p.sp;
  const int tid = threadIdx.x, wave = wave_id();
  // With two rank bands each half of the workgroup reduces one, at the same
  // time; with one, the first four waves do.  Lane: rank j of band rb.
  const int rb = p.RB > 1 ? wave >> 2 : 0;
  const bool active = p.RB > 1 || wave < 4;
  const int col = 16 * (wave & 3) + (tid & 15);
  const int j = 64 * rb + col;
  // the gate's parameters, requested before the wait
  float g = 0.f, b = 0.f;
  if (p.gh == 0 && active && j < p.r) {
    g = p.gv[j];
    b = p.bv[j];
  }
  if (tid == 0) {
    int spins = 0, ok = 1;
    for (int k = 0; k < p.RB && ok; ++k) {
      const uint32_t bbeg = (uint32_t)k * p.KB;
      const int nseg = rank_owner(sp, bbeg + p.KB - 1) - rank_owner(sp, bbeg) + 1;
      while (load_dev(&p.ctr[kCtrBand + k]) < nseg) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
          atomicOr(&p.ctr[kCtrError], 1);
          ok = 0;
          break;
        }
      }
    }
    *s_flag = ok;
  }
  __syncthreads();
  const bool ok = *s_flag != 0;
  __syncthreads();
  if (active) {
    const uint32_t bbeg = (uint32_t)rb * p.KB;
    const int first = rank_owner(sp, bbeg);
    const int nseg = rank_owner(sp, bbeg + p.KB - 1) - first + 1;
    f32x4 v[MT];
    sum_parts<MT>(p, true, rb, first, nseg, col, v);
    if (!ok)
      for (int mt = 0; mt < MT; ++mt) v[mt] = f32x4{NAN, NAN, NAN, NAN};
    finish_rank<MT>(p, j, g, b, v);
  }
  if (tid == 0)
    for (int k = 0; k < p.RB; ++k) store_dev(&p.ctr[kCtrBand + k], 0);
  wait_vmem();
  __syncthreads();
  if (p.gh > 0) {
    gate_mlp(p, xlds, 2 * Burst<MT>::kBuf / 4);
  } else if (tid == 0) {
    __hip_atomic_fetch_add(&p.ctr[kCtrRankDone], p.RB, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Second bound: waves per SIMD (one workgroup of W waves per compute unit),
// which gives a wave 256 registers: a burst's operands and both register
// stages stay in registers.
template <int MT, bool GROUPED>
__global__ __launch_bounds__(kThreads, W * kDecodeOccupancy / 4) void decode_kernel(DecodeParams p) {
  warm_kernel_args<sizeof(DecodeParams)>();
  // x buffers (also the MLP gate's working area, T (r + h) + max(r, h) floats)
  static_assert(2 * Burst<MT>::kBuf / 4 >= 16 * MT * 256 + 128, "MLP gate LDS");
  __shared__ __attribute__((aligned(16))) uint8_t xlds[2 * Burst<MT>::kBuf];
  __shared__ __attribute__((aligned(16))) uint8_t mlds[GROUPED ? W * Meta<MT>::kWave : 16];
  __shared__ __attribute__((aligned(16))) uint8_t clds[W * kCodeArea];
  __shared__ int s_last, s_wait;
  const int tid = threadIdx.x;
  const int wg = blockIdx.x;
  const DecodeSplit& sp = p.sp;
  int burst = 0;

  // Rank runs (workgroups below sp.Rw): each partial projection goes to its
  // slot and is posted without waiting for the count; workgroup 0 then sums
  // every rank band, gates and publishes alpha v.
  {
    const uint32_t u1 = rank_begin(sp, wg + 1);
    for (uint32_t u = rank_begin(sp, wg); u < u1;) {
      const int band = (int)fdiv(u, sp.by_kb);
      const uint32_t bbeg = (uint32_t)band * p.KB, bend = bbeg + p.KB;
      const int lo = (int)(u - bbeg);
      const int hi = (int)(min(u1, bend) - bbeg);
      u = min(u1, bend);
      f32x4 v[MT];
      rank_segment<MT>(p, band, lo, hi, xlds, clds, burst, v);
      post_rank_part<MT>(p, band, v);
    }
    if (wg == 0 && p.RB > 0) reduce_ranks<MT>(p, xlds, &s_wait);
  }

  // Row runs.
  const uint32_t u1 = row_begin(sp, wg + 1);
  for (uint32_t u = row_begin(sp, wg); u < u1;) {
    const int band = (int)fdiv(u, sp.by_kb);
    const uint32_t bbeg = (uint32_t)band * p.KB, bend = bbeg + p.KB;
    const int lo = (int)(u - bbeg);
    const int hi = (int)(min(u1, bend) - bbeg);
    u = min(u1, bend);
    // the owners of the band's first and last units (a search over the
    // split) while the segment's first loads are in flight
    int first = 0, nseg = 1;
    auto owners = [&]() {
      first = row_owner(sp, bbeg);
      nseg = row_owner(sp, bend - 1) - first + 1;
    };

    f32x4 v[MT];
    row_segment<MT, GROUPED>(p, band, lo, hi, xlds, mlds, clds, burst, v, owners);
    if (nseg > 1 && !arrive<MT>(p, band, first, nseg, &s_last, v)) continue;
    if (p.r > 0) {
      u32x4 bfr[kRankSteps];
      b_fragments(p, band, bfr);
      u32x4 vhi[kRankSteps][MT], vlo[kRankSteps][MT];
      if (p.s0 >= 0) {  // SERQ: x's salient channels, nothing to wait for
        serq_operands<MT>(p, vhi);
        for (int k = 0; k < kRankSteps; ++k)
          for (int mt = 0; mt < MT; ++mt) vlo[k][mt] = u32x4{0u, 0u, 0u, 0u};
      } else if (wait_ranks(p, &s_wait)) {
        alpha_v_operands<MT>(p, vhi, vlo);
      } else {  // gave up waiting: no plausible-looking output
        for (int mt = 0; mt < MT; ++mt) v[mt] = f32x4{NAN, NAN, NAN, NAN};
        for (int k = 0; k < kRankSteps; ++k)
          for (int mt = 0; mt < MT; ++mt) vhi[k][mt] = vlo[k][mt] = u32x4{0u, 0u, 0u, 0u};
      }
      add_correction<MT>(p, bfr, vhi, vlo, v);
    }
    store_row<MT>(p, band, v);
  }

  if (p.RB > 0 && tid == 0) {
    wait_vmem();
    if (atomicAdd(&p.ctr[kCtrExit], 1) == sp.P - 1) {
      store_dev(&p.ctr[kCtrRankDone], 0);
      store_dev(&p.ctr[kCtrGateDone], 0);
      store_dev(&p.ctr[kCtrExit], 0);
    }
  }
}

template <int MT, bool GROUPED>
hipError_t go(const DecodeParams& p, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<MT, GROUPED>), dim3(p.sp.P), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace

// Compute units of the current device.
static int compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

hipError_t launch_decode(const Shape& s, const LayerArgs& a, const WsPtrs& w, hipStream_t st) {
  const DecodePlan pl = plan_decode(s, compute_units() * kDecodeOccupancy);
  DecodeParams p;
  p.x = static_cast<const uint16_t*>(a.x);
  p.wq = a.wq;
  p.scales = a.scales;
  p.has_z = a.zeros != nullptr;
  p.zeros = a.zeros ? a.zeros : reinterpret_cast<const uint32_t*>(a.scales);
  p.A = static_cast<const uint16_t*>(a.A);
  p.B = static_cast<const uint16_t*>(a.B);
  p.gv = a.gv;
  p.bv = a.bv;
  p.gh = a.gh;
  p.w1 = a.w1;
  p.b1 = a.b1;
  p.w2 = a.w2;
  p.b2 = a.b2;
  p.alpha = a.alpha;
  p.part = w.ypart;
  p.wv32 = w.wv32;
  p.ctr = w.counters;
  p.y = a.y;
  p.out_f32 = a.out_f32 ? 1 : 0;
  p.T = s.T;
  p.K = s.K;
  p.N = s.N;
  p.r = s.r;
  p.G = s.K / s.g;
  p.ZW = (p.G + 7) / 8;
  p.KB = s.KB();
  p.RB = pl.rank_bands;
  p.sp = pl.split;
  p.nslots = pl.slots;
  p.s0 = a.s0;
  if (s.T <= 16) return s.grouped ? go<1, true>(p, st) : go<1, false>(p, st);
  return s.grouped ? go<2, true>(p, st) : go<2, false>(p, st);
}

}  // namespace spear
