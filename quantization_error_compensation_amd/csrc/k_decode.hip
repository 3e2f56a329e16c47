// Decode path (1..32 tokens): one fused, bandwidth-bound kernel.
//
// SPEAR summary, section 2.2 A (phase-aware adaptive kernel fusion): in the
// memory-bound decode phase the compensator is fused into the epilogue of the
// low-bit GEMM, so the whole compensated layer is one kernel.  One launch
// streams the packed weights once, computes the rank-r projection of every
// token once, gates it, and adds alpha * B * v before the single bf16 store.
//
// Work.  A "band" is either 64 output rows of packed codes or 64 rows (ranks)
// of A; a "unit" is one 128-column block of one band.  Rank bands come first
// in the unit order.  A unit of a rank band moves 16 KB of bf16, a row unit
// 4 KB of codes, so units carry a cost and the P persistent workgroups each
// take a contiguous run of units of equal cost (stream-K).  A workgroup walks
// its run band segment by band segment.  A band covered by several
// workgroups has its partial sums combined by whichever arrives last (in
// segment order, so results are deterministic); partial sums move through
// device-scope stores and loads (coherent across XCDs, no L2-wide fence).
//
// Inside a segment the four waves of a workgroup own one 16-row tile each
// and walk the same K blocks in bursts of NS blocks:
//   * every load of a burst (x, codes or A rows, metadata) is issued one
//     burst ahead, into registers, so it is in flight while the previous
//     burst computes;
//   * x of the burst is loaded once per workgroup (each wave 4 tokens x
//     256 B per instruction, full cache lines), permuted into the
//     matrix-core K order and written to a double-buffered LDS area; one
//     barrier per burst publishes it to all four waves;
//   * codes: 16 bytes per lane per block (16 rows x 64 B per instruction),
//     all NS blocks issued back to back; bf16 operands 128 + c by byte
//     permutes;
//   * group scales and zero-points: staged per 32-block chunk in each wave's
//     LDS area with loads that cover whole runs of a row's metadata;
//   * matrix cores 16x16x32: tokens (padded to 16 or 32) x 16 rows x 32 K; a
//     ones-operand product gives the block sums of x that remove the offset.
// The band finisher adds alpha * B * v as a small K = r matrix-core product
// (v split into bf16 high and low parts) and stores y.
//
// Waiting: finishers of row bands wait for the rank bands to publish.  Rank
// units are the first units, owned by the lowest workgroup indices, which the
// dispatcher starts first, so they run before anyone waits; rank units are
// costed above their byte count so those workgroups finish early.  The wait
// is bounded and raises an error word instead of hanging.
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
  float* part;             // [bands][maxseg][64][T4] partial sums
  float* wv32;             // [T][r] alpha * v
  int* ctr;                // counter words
  uint16_t* y;             // [T][N] bf16
  int T, K, N, r, G, ZW, has_z;
  int KB;                  // 128-column blocks per row
  int RB;                  // rank bands (64 ranks each)
  int NB;                  // row bands (64 rows each)
  int P;                   // workgroups
  int rank_cost;           // cost of a rank unit; a row unit costs 1
  long long ctot;          // total cost of all units
  int maxseg;              // bound on the partial sums of one band
  int cw;                  // correction workgroups (the first cw, whose runs hold rank
                           // units only): each adds alpha v B^T to up to
                           // kCorrBands / MT row bands as one more partial
};

constexpr int XROW = 272;            // LDS row of one token: 256 B + 16 B pad
constexpr int kSpinLimit = 1 << 20;  // bounded wait (about a second)

// Blocks per burst: 8 (row bands) / 4 (rank bands) up to 16 tokens, half that
// up to 32 tokens, so one LDS buffer of x always holds 128 token-blocks.
template <int MT>
struct Burst {
  static constexpr int kRow = MT == 1 ? 8 : 4;
  static constexpr int kRank = kRow / 2;
  static constexpr int kBuf = kRow * 16 * MT * XROW;  // bytes of one x buffer
};

// ------------------------------------------------------------- partition
// Cost of the first u units, and the first unit of workgroup w: the smallest
// u with S(u) * P >= w * ctot.  owner_of(u) is the workgroup whose run holds
// unit u.
__device__ __forceinline__ long long cost_prefix(const DecodeParams& p, long long u) {
  const long long ru = (long long)p.RB * p.KB;
  return u <= ru ? u * p.rank_cost : ru * p.rank_cost + (u - ru);
}
__device__ __forceinline__ long long unit_begin(const DecodeParams& p, int w) {
  const long long X = (long long)w * p.ctot;
  const long long ru = (long long)p.RB * p.KB;
  const long long rc = (long long)p.rank_cost * p.P;
  if (X <= ru * rc) return (X + rc - 1) / rc;
  return ru + (X - ru * rc + p.P - 1) / p.P;
}
__device__ __forceinline__ int owner_of(const DecodeParams& p, long long u) {
  return (int)(cost_prefix(p, u) * p.P / p.ctot);
}

// ------------------------------------------------------------- x staging
// x of blocks [b, b + NS) into an LDS buffer [NS][16*MT tokens][XROW], each
// 16-byte piece already in the matrix-core K order.  Wave w loads tokens
// 4w + 16m .. +3 (lane: token 4w + 16m + l/16, piece l%16).  Every wave
// issues the same loads whatever T is, so the count of loads in flight, and
// with it every wait, is path-independent: lanes of tokens past T, and all
// lanes when live is false, load from past the end of the buffer, which
// reads zeros without a memory access.
template <int MT, int NS>
struct XStage {
  u32x4 g[NS][MT];
};

template <int MT, int NS>
__device__ __forceinline__ void x_issue(const DecodeParams& p, int wave, int lane, int b, int hi,
                                        bool live, XStage<MT, NS>& s) {
  const uint32_t xrowB = (uint32_t)p.K * 2;
  const rsrc_t xr = make_rsrc(p.x, (uint32_t)p.T * xrowB);
  for (int m = 0; m < MT; ++m) {
    const int t = 4 * wave + 16 * m + (lane >> 4);
    const uint32_t vo = live && t < p.T ? (uint32_t)t * xrowB + 16u * (lane & 15) : 0x80000000u;
    for (int i = 0; i < NS; ++i) s.g[i][m] = bload16(xr, vo, (uint32_t)min(b + i, hi - 1) * 256);
  }
}

template <int MT, int NS>
__device__ __forceinline__ void x_store(uint8_t* buf, int wave, int lane,
                                        const XStage<MT, NS>& s) {
  for (int i = 0; i < NS; ++i)
    for (int m = 0; m < MT; ++m) {
      const int t = 4 * wave + 16 * m + (lane >> 4);
      *reinterpret_cast<u32x4*>(buf + (i * 16 * MT + t) * XROW + 16 * (lane & 15)) =
          x_permute8(s.g[i][m]);
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

// ------------------------------------------------------------ rank segment
// A barrier that leaves global loads in flight: only this wave's LDS writes
// are awaited before the workgroup meets.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// What one burst of a rank segment takes from memory: x and the A rows.
template <int MT, int NS>
struct RankStage {
  XStage<MT, NS> x;
  u32x4 a[NS][4];
};

// Ranks 64 rb + 16 wave + c16, blocks [lo, hi): u = x A^T over the segment.
// Loads run one burst ahead, in two register stages, as in row segments.
template <int MT>
__device__ void rank_segment(const DecodeParams& p, int rb, int lo, int hi, uint8_t* xlds,
                             int& burst, f32x4 (&uo)[MT]) {
  constexpr int NS = Burst<MT>::kRank;
  const int lane = threadIdx.x & 63, wave = wave_id(), q = lane >> 4, c16 = lane & 15;
  // A tile of ranks j0 .. j0 + 15; a wave past r reads the last tile again
  // (its u columns are never published)
  const int j0 = min(64 * rb + 16 * wave, p.r - 16);
  const uint32_t arowB = (uint32_t)p.K * 2;
  const rsrc_t ar = make_rsrc(p.A + (size_t)j0 * p.K, 16u * arowB);
  const uint32_t ao = (uint32_t)c16 * arowB + 64u * q;  // pieces 4q .. 4q + 3 of row c16
  for (int mt = 0; mt < MT; ++mt) uo[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](RankStage<MT, NS>& s, int b) {
    const bool live = b < hi;  // a burst past the segment loads nothing
    x_issue<MT, NS>(p, wave, lane, b, hi, live, s.x);
    const uint32_t av = live ? ao : 0x80000000u;
    for (int i = 0; i < NS; ++i)
      for (int j = 0; j < 4; ++j)
        s.a[i][j] = bload16(ar, av + 16 * j, (uint32_t)min(b + i, hi - 1) * 256);
  };
  auto consume = [&](RankStage<MT, NS>& s, int b) {
    uint8_t* buf = xlds + (burst & 1) * Burst<MT>::kBuf;
    ++burst;
    x_store<MT, NS>(buf, wave, lane, s.x);
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (b + i < hi) {
        u32x4 xf[MT][4];
        x_frags<MT>(buf, i, lane, xf);
        for (int j = 0; j < 4; ++j) {
          const u32x4 ap = x_permute8(s.a[i][j]);
          for (int mt = 0; mt < MT; ++mt) uo[mt] = mfma16x16x32(xf[mt][j], ap, uo[mt]);
        }
      }
    }
  };

  RankStage<MT, NS> s0, s1;
  issue(s0, lo);
  for (int b = lo;; b += 2 * NS) {
    issue(s1, b + NS);
    consume(s0, b);
    if (b + NS >= hi) break;
    issue(s0, b + 2 * NS);
    consume(s1, b + NS);
    if (b + 2 * NS >= hi) break;
  }
}

// -------------------------------------------------------------- row segment
// Group scales and zero-points of a wave's 16 rows are staged per chunk of
// kMetaChunk blocks in the wave's own LDS area: ms[16][kMetaChunk] fp16 bits
// and mz[16][8] zero-point words (word w0 + k holds blocks 8(w0 + k) ..).
// Each staging load covers 2 rows x 32 consecutive scales (or 16 rows x 4
// words), so a row's metadata costs a few cache-line requests per chunk
// rather than one per burst.
constexpr int kMetaChunk = 32;
constexpr int kMetaWave = 16 * kMetaChunk * 2 + 16 * 8 * 4;  // bytes per wave

// What one burst of a row segment takes from memory: x (permuted into LDS
// when the burst starts), the codes, and at the start of a metadata chunk the
// chunk's scales and zero-points.  Each burst's loads are issued one burst
// ahead, so they are in flight while the previous burst computes.
template <int MT, int NS>
struct RowStage {
  XStage<MT, NS> x;
  u32x4 w[NS];
  uint32_t sv[8], zv[2];
};

// Rows 64 band + 16 wave + c16 (this wave's tile), blocks [lo, hi): partial
// y with the scales applied.
template <int MT, bool GROUPED>
__device__ void row_segment(const DecodeParams& p, int band, int lo, int hi, uint8_t* xlds,
                            uint8_t* mlds, int& burst, f32x4 (&yo)[MT]) {
  constexpr int NS = Burst<MT>::kRow;
  const int lane = threadIdx.x & 63, wave = wave_id(), q = lane >> 4, c16 = lane & 15;
  // Tile of rows rc .. rc + 15; a tile past N (last band of an N that is not
  // a multiple of 64) reads the last tile again and stores nothing.
  const int rc = min(band * 64 + 16 * wave, p.N - 16);
  const uint32_t wrowB = (uint32_t)p.K / 2;
  const rsrc_t wr = make_rsrc(p.wq + (size_t)rc * (p.K / 8), 16u * wrowB);
  const uint32_t wo = (uint32_t)c16 * wrowB + 16u * q;
  const uint16_t* St = p.scales + (size_t)rc * p.G;
  const uint32_t* Zt = p.zeros + (size_t)rc * p.ZW;
  const u32x4 ones = {kBf16One, kBf16One, kBf16One, kBf16One};
  uint16_t* ms = reinterpret_cast<uint16_t*>(mlds + wave * kMetaWave);
  uint32_t* mz = reinterpret_cast<uint32_t*>(mlds + wave * kMetaWave + 16 * kMetaChunk * 2);
  int c0 = lo, w0 = lo >> 3;  // first block and first zero-point word of the staged chunk

  f32x4 acc[MT], ssum[MT];
  for (int mt = 0; mt < MT; ++mt) acc[mt] = ssum[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](RowStage<MT, NS>& s, int b) {
    if (GROUPED && (b - lo) % kMetaChunk == 0) {
      const int c1 = min(b + kMetaChunk, hi);
      const int blk = min(b + (lane & 31), c1 - 1);
      for (int k = 0; k < 8; ++k)
        s.sv[k] = gload2(St, (uint32_t)((2 * k + (lane >> 5)) * p.G + blk) * 2);
      for (int e = 0; e < 2; ++e) {
        const int wd = min((b >> 3) + (lane & 3) + 4 * e, (c1 - 1) >> 3);
        s.zv[e] = p.has_z ? gload4(Zt, (uint32_t)((lane >> 2) * p.ZW + wd) * 4) : 0x88888888u;
      }
    }
    const bool live = b < hi;  // a burst past the segment loads nothing
    x_issue<MT, NS>(p, wave, lane, b, hi, live, s.x);
    const uint32_t wv = live ? wo : 0x80000000u;
    for (int i = 0; i < NS; ++i) s.w[i] = bload16(wr, wv, (uint32_t)min(b + i, hi - 1) * 64);
  };

  auto consume = [&](RowStage<MT, NS>& s, int b) {
    uint8_t* buf = xlds + (burst & 1) * Burst<MT>::kBuf;
    ++burst;
    if (GROUPED && (b - lo) % kMetaChunk == 0) {
      c0 = b;
      w0 = b >> 3;
      for (int k = 0; k < 8; ++k)
        ms[(2 * k + (lane >> 5)) * kMetaChunk + (lane & 31)] = (uint16_t)s.sv[k];
      for (int e = 0; e < 2; ++e) mz[(lane >> 2) * 8 + (lane & 3) + 4 * e] = s.zv[e];
    }
    x_store<MT, NS>(buf, wave, lane, s.x);
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (b + i >= hi) continue;
      u32x4 xf[MT][4];
      x_frags<MT>(buf, i, lane, xf);
      u32x4 wb[4];
      wb[0] = codes_to_bf16_offset(s.w[i].x);
      wb[1] = codes_to_bf16_offset(s.w[i].y);
      wb[2] = codes_to_bf16_offset(s.w[i].z);
      wb[3] = codes_to_bf16_offset(s.w[i].w);
      if constexpr (GROUPED) {
        const int blk = b + i;
        const float sc = half_bits_to_f32(ms[c16 * kMetaChunk + (blk - c0)]);
        const uint32_t z = (mz[c16 * 8 + ((blk >> 3) - w0)] >> (4 * (blk & 7))) & 15u;
        const float nz = -(float)(128u + z);
        for (int mt = 0; mt < MT; ++mt) {
          f32x4 sb = mfma16x16x32(xf[mt][0], ones, f32x4{0.f, 0.f, 0.f, 0.f});
          f32x4 P = mfma16x16x32(xf[mt][0], wb[0], f32x4{0.f, 0.f, 0.f, 0.f});
          for (int j = 1; j < 4; ++j) {
            sb = mfma16x16x32(xf[mt][j], ones, sb);
            P = mfma16x16x32(xf[mt][j], wb[j], P);
          }
          for (int v = 0; v < 4; ++v) acc[mt][v] = fmaf(sc, fmaf(nz, sb[v], P[v]), acc[mt][v]);
        }
      } else {
        for (int mt = 0; mt < MT; ++mt)
          for (int j = 0; j < 4; ++j) {
            ssum[mt] = mfma16x16x32(xf[mt][j], ones, ssum[mt]);
            acc[mt] = mfma16x16x32(xf[mt][j], wb[j], acc[mt]);
          }
      }
    }
  };

  // Two stages in turn: while one burst computes, the next one loads.  The
  // stage past the segment's last burst is issued too, with its loads out of
  // range (no memory access): the number of loads in flight is then the same
  // on every path, so the waits on each stage stay exact.
  RowStage<MT, NS> s0, s1;
  issue(s0, lo);
  for (int b = lo;; b += 2 * NS) {
    issue(s1, b + NS);
    consume(s0, b);
    if (b + NS >= hi) break;
    issue(s0, b + 2 * NS);
    consume(s1, b + NS);
    if (b + 2 * NS >= hi) break;
  }

  if constexpr (!GROUPED) {  // per-channel: one scale and one offset correction per row
    const int n = rc + c16;
    const float sc = half_bits_to_f32(p.scales[n]);
    const int z = p.has_z ? (int)(p.zeros[(size_t)n * p.ZW] & 15u) : 8;
    const float mz = -(float)(128 + z);
    for (int mt = 0; mt < MT; ++mt)
      for (int v = 0; v < 4; ++v) acc[mt][v] = sc * fmaf(mz, ssum[mt][v], acc[mt][v]);
  }
  for (int mt = 0; mt < MT; ++mt) yo[mt] = acc[mt];
}

// ------------------------------------------------------------ partial sums
// [maxseg][64 columns][T4] floats per band (T4: T rounded up to a multiple
// of 4), written and read at device scope; a lane's four tokens of one
// column form one 16-byte word, and words holding no token below T are
// neither stored nor loaded.  Column c of a partial is row 64 band + c of a
// row band, or rank 64 rb + c.
__device__ __forceinline__ int tokens4(const DecodeParams& p) { return (p.T + 3) & ~3; }
__device__ __forceinline__ rsrc_t part_rsrc(const DecodeParams& p, int band) {
  const uint32_t seg = 64u * tokens4(p);  // floats of one partial
  return make_rsrc(p.part + (size_t)band * p.maxseg * seg, (uint32_t)p.maxseg * seg * 4);
}
__device__ __forceinline__ uint32_t part_off(const DecodeParams& p, int sidx, int col, int t) {
  return (uint32_t)(((sidx * 64 + col) * tokens4(p) + t) * 4);
}

template <int MT>
__device__ __forceinline__ void put_part(const DecodeParams& p, int band, int sidx, int col,
                                         const f32x4 (&v)[MT]) {
  const int q = (threadIdx.x & 63) >> 4;
  const rsrc_t r = part_rsrc(p, band);
  for (int mt = 0; mt < MT; ++mt) {
    const int t = 16 * mt + 4 * q;
    if (t < p.T) bstore16_dev(r, part_off(p, sidx, col, t), 0, v[mt]);
  }
}

// The band's nseg partials summed in segment order; 16 / MT partials are in
// flight at a time.
template <int MT>
__device__ __forceinline__ void sum_parts(const DecodeParams& p, int band, int nseg, int col,
                                          f32x4 (&v)[MT]) {
  constexpr int CH = 16 / MT;
  const int q = (threadIdx.x & 63) >> 4;
  const rsrc_t r = part_rsrc(p, band);
  for (int mt = 0; mt < MT; ++mt) v[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < nseg; k0 += CH) {
    const int n = min(CH, nseg - k0);
    u32x4 w[CH][MT];
    for (int kk = 0; kk < CH; ++kk)
      for (int mt = 0; mt < MT; ++mt) {
        const int t = 16 * mt + 4 * q;
        w[kk][mt] = kk < n && t < p.T ? bload16_dev(r, part_off(p, k0 + kk, col, t), 0)
                                      : u32x4{0u, 0u, 0u, 0u};
      }
    for (int kk = 0; kk < CH; ++kk)
      if (kk < n)
        for (int mt = 0; mt < MT; ++mt) v[mt] += __builtin_bit_cast(f32x4, w[kk][mt]);
  }
}

// Finish a rank band: gate and publish alpha * v for this wave's 16 ranks
// (with the MLP gate, which needs every rank of a token, publish u itself).
template <int MT>
__device__ void finish_rank(const DecodeParams& p, int rb, const f32x4 (&u)[MT]) {
  const int lane = threadIdx.x & 63, wave = wave_id(), q = lane >> 4, c16 = lane & 15;
  const int j = 64 * rb + 16 * wave + c16;
  if (j >= p.r) return;
  const float g = p.gh > 0 ? 0.f : p.gv[j], b = p.gh > 0 ? 0.f : p.bv[j];
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
  for (int e0 = threadIdx.x; e0 < n; e0 += 8 * 256) {
    float v[8];
    for (int i = 0; i < 8; ++i) {
      const uint32_t off = (uint32_t)(e0 + 256 * i) * 4;  // past n: zero, not stored
      v[i] = DEV ? bload_dev(r, off, 0) : __builtin_bit_cast(float, bload4(r, off, 0));
    }
    for (int i = 0; i < 8; ++i)
      if (e0 + 256 * i < n) dst[e0 + 256 * i] = v[i];
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
    for (int e = tid; e < T * nk; e += 256) {
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
    for (int e = tid; e < T * nj; e += 256) {
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

// Row bands whose correction a correction workgroup adds (as an extra
// partial); kCorrBands / MT bands per correction workgroup.
constexpr int kCorrBands = 8;
template <int MT>
__device__ __forceinline__ bool corrected(const DecodeParams& p, int nb) {
  return nb < p.cw * (kCorrBands / MT);
}

// Wait (bounded, error word on timeout) until alpha * v of every rank is
// published: every rank band (elementwise gate) or the MLP gate's pass.
__device__ __forceinline__ void wait_ranks(const DecodeParams& p) {
  if (threadIdx.x == 0) {
    int spins = 0;
    const int* ctr = p.gh > 0 ? &p.ctr[kCtrGateDone] : &p.ctr[kCtrRankDone];
    const int target = p.gh > 0 ? 1 : p.RB;
    while (load_dev(ctr) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        atomicOr(&p.ctr[kCtrError], 1);
        break;
      }
    }
  }
  __syncthreads();
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

// B fragments of the 16 rows of this wave's tile of a row band: for each
// K = 32 rank step, 8 ranks of the lane's row (zero past r).
__device__ __forceinline__ void b_fragments(const DecodeParams& p, int band,
                                            u32x4 (&bfr)[kRankSteps]) {
  const int lane = threadIdx.x & 63, wave = wave_id(), q = lane >> 4, c16 = lane & 15;
  const int nrow = band * 64 + 16 * wave + c16;
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

// Store y for this wave's tile of a finished row band.
template <int MT>
__device__ __forceinline__ void store_row(const DecodeParams& p, int band, const f32x4 (&yv)[MT]) {
  const int lane = threadIdx.x & 63, wave = wave_id(), q = lane >> 4, c16 = lane & 15;
  const int nrow = band * 64 + 16 * wave + c16;
  if (nrow < p.N)
    for (int mt = 0; mt < MT; ++mt)
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * mt + 4 * q + i;
        if (t < p.T) p.y[(size_t)t * p.N + nrow] = (uint16_t)f32_to_bf16_rne(yv[mt][i]);
      }
}

// Add a partial sum to a band (slot sidx of nparts) and report whether this
// workgroup arrived last; the last one gets the sum of all partials in slot
// order in v and clears the band's counter.
template <int MT>
__device__ __forceinline__ bool arrive(const DecodeParams& p, int band, int sidx, int nparts,
                                       int* s_last, f32x4 (&v)[MT]) {
  const int tid = threadIdx.x, col = 16 * wave_id() + (tid & 15);
  put_part<MT>(p, band, sidx, col, v);
  wait_vmem();
  __syncthreads();
  if (tid == 0) *s_last = atomicAdd(&p.ctr[kCtrBand + band], 1) == nparts - 1;
  __syncthreads();
  const bool last = *s_last;
  if (last) {
    sum_parts<MT>(p, band, nparts, col, v);
    if (tid == 0) store_dev(&p.ctr[kCtrBand + band], 0);
  }
  return last;
}

// The correction workgroups: once the rank bands are published, alpha v B^T
// of row bands wg, wg + cw, ... (kCorrBands / MT of them) goes in as each
// band's extra partial (slot nseg); whoever arrives last at a band stores it.
// All their B fragments are requested together, their partials stored
// together, and one wait covers all the stores.  The finishers of the bands
// from cw * kCorrBands / MT on add the correction themselves.
template <int MT>
__device__ void correction_partials(const DecodeParams& p, int wg, int* s_mask) {
  constexpr int kCorrBatch = kCorrBands / MT;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int col = 16 * wave + (lane & 15);
  // B does not depend on the rank bands: its fragments are requested first.
  u32x4 bfr[kCorrBatch][kRankSteps];
  for (int i = 0; i < kCorrBatch; ++i) b_fragments(p, min(wg + i * p.cw, p.NB - 1), bfr[i]);
  wait_ranks(p);
  u32x4 hi[kRankSteps][MT], lo[kRankSteps][MT];
  alpha_v_operands<MT>(p, hi, lo);
  {
    const int nb0 = wg;
    int nseg[kCorrBatch];
    bool ok[kCorrBatch];
    f32x4 v[kCorrBatch][MT];
    for (int i = 0; i < kCorrBatch; ++i) {
      const int nb = nb0 + i * p.cw, band = p.RB + nb;
      const long long bbeg = (long long)band * p.KB, bend = bbeg + p.KB;
      ok[i] = nb < p.NB;
      nseg[i] = ok[i] ? owner_of(p, bend - 1) - owner_of(p, bbeg) + 1 : 0;
      if (ok[i] && nseg[i] + 1 > p.maxseg) {  // cannot happen with a planner-sized workspace
        if (tid == 0) atomicOr(&p.ctr[kCtrError], 2);
        ok[i] = false;
      }
      for (int mt = 0; mt < MT; ++mt) v[i][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (ok[i]) add_correction<MT>(p, bfr[i], hi, lo, v[i]);
    }
    for (int i = 0; i < kCorrBatch; ++i)
      if (ok[i]) put_part<MT>(p, p.RB + nb0 + i * p.cw, nseg[i], col, v[i]);
    wait_vmem();
    __syncthreads();
    if (wave == 0) {  // lane i counts band i in; the arrivals go out together
      bool last = false;
      if (lane < kCorrBatch) {
        const int nb = nb0 + lane * p.cw, band = p.RB + nb;
        const long long bbeg = (long long)band * p.KB, bend = bbeg + p.KB;
        const int ns = nb < p.NB ? owner_of(p, bend - 1) - owner_of(p, bbeg) + 1 : 0;
        if (nb < p.NB && ns + 1 <= p.maxseg)
          last = atomicAdd(&p.ctr[kCtrBand + band], 1) == ns;
      }
      const uint64_t m = __ballot(last);
      if (lane == 0) *s_mask = (int)(m & ((1u << kCorrBatch) - 1));
    }
    __syncthreads();
    const int mask = *s_mask;
    for (int i = 0; i < kCorrBatch; ++i)
      if (mask & (1 << i)) {  // arrived last: every segment's partial is in
        const int nb = nb0 + i * p.cw, band = p.RB + nb;
        sum_parts<MT>(p, band, nseg[i] + 1, col, v[i]);
        if (tid == 0) store_dev(&p.ctr[kCtrBand + band], 0);
        store_row<MT>(p, nb, v[i]);
      }
  }
}

template <int MT, bool GROUPED>
__global__ __launch_bounds__(256, 2) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t xlds[2 * Burst<MT>::kBuf];
  __shared__ __attribute__((aligned(16))) uint8_t mlds[GROUPED ? 4 * kMetaWave : 16];
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int wg = blockIdx.x;
  const long long u0 = unit_begin(p, wg), u1 = unit_begin(p, wg + 1);
  int burst = 0;

  for (long long u = u0; u < u1;) {
    const int band = (int)(u / p.KB);
    const long long bbeg = (long long)band * p.KB, bend = bbeg + p.KB;
    const int lo = (int)(u - bbeg);
    const int hi = (int)(min(u1, bend) - bbeg);
    u = min(u1, bend);
    const int first = owner_of(p, bbeg);
    const int nseg = owner_of(p, bend - 1) - first + 1;
    const int sidx = wg - first;
    const bool rank = band < p.RB;
    // a row band whose correction a correction workgroup adds takes one more
    // partial
    const bool corr = !rank && corrected<MT>(p, band - p.RB);
    const int nparts = nseg + (corr ? 1 : 0);
    if (nparts > p.maxseg) {  // cannot happen with a workspace sized by the planner
      if (tid == 0) atomicOr(&p.ctr[kCtrError], 2);
      continue;
    }

    f32x4 v[MT];
    if (rank) rank_segment<MT>(p, band, lo, hi, xlds, burst, v);
    else row_segment<MT, GROUPED>(p, band - p.RB, lo, hi, xlds, mlds, burst, v);

    const bool fin = nparts == 1 || arrive<MT>(p, band, sidx, nparts, &s_last, v);
    if (fin) {
      if (rank) {
        finish_rank<MT>(p, band, v);
        wait_vmem();
        __syncthreads();
        if (tid == 0) s_last = atomicAdd(&p.ctr[kCtrRankDone], 1) == p.RB - 1;
        __syncthreads();
        if (p.gh > 0 && s_last) gate_mlp(p, xlds, 2 * Burst<MT>::kBuf / 4);
      } else {
        if (p.r > 0 && !corr) {
          u32x4 bfr[kRankSteps];
          b_fragments(p, band - p.RB, bfr);
          wait_ranks(p);
          u32x4 vhi[kRankSteps][MT], vlo[kRankSteps][MT];
          alpha_v_operands<MT>(p, vhi, vlo);
          add_correction<MT>(p, bfr, vhi, vlo, v);
        }
        store_row<MT>(p, band - p.RB, v);
      }
    }
  }
  if (wg < p.cw) correction_partials<MT>(p, wg, &s_last);

  if (p.RB > 0 && tid == 0) {
    wait_vmem();
    if (atomicAdd(&p.ctr[kCtrExit], 1) == p.P - 1) {
      store_dev(&p.ctr[kCtrRankDone], 0);
      store_dev(&p.ctr[kCtrGateDone], 0);
      store_dev(&p.ctr[kCtrExit], 0);
    }
  }
}

template <int MT, bool GROUPED>
hipError_t go(const DecodeParams& p, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<MT, GROUPED>), dim3(p.P), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

// Workgroups the current device keeps resident: two per compute unit.
static int resident_slots() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev] = 2 * cus;
  }
  return cached[dev];
}

hipError_t launch_decode(const Shape& s, const LayerArgs& a, const WsPtrs& w, hipStream_t st) {
  const DecodePlan pl = plan_decode(s, resident_slots());
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
  p.y = static_cast<uint16_t*>(a.y);
  p.T = s.T;
  p.K = s.K;
  p.N = s.N;
  p.r = s.r;
  p.G = s.K / s.g;
  p.ZW = (p.G + 7) / 8;
  p.KB = s.KB();
  p.RB = pl.rank_bands;
  p.NB = pl.bands;
  p.P = pl.workgroups;
  p.rank_cost = pl.rank_cost;
  p.ctot = pl.cost;
  p.maxseg = pl.maxseg;
  p.cw = pl.correction_wgs;
  if (s.T <= 16) return s.grouped ? go<1, true>(p, st) : go<1, false>(p, st);
  return s.grouped ? go<2, true>(p, st) : go<2, false>(p, st);
}

}  // namespace spear
