// Decode path (1..32 tokens): one fused, bandwidth-bound kernel.
//
// SPEAR summary, section 2.2 A (phase-aware adaptive kernel fusion): in the
// memory-bound decode phase the compensator is fused into the epilogue of the
// low-bit GEMM, so the whole compensated layer is one kernel.  One launch
// streams the packed weights once, computes the rank-r projection of every
// token once, gates it, and adds alpha * B * v before the single bf16 store.
//
// Work: a "unit" is one 128-column block of one band, where a band is either
// 64 output rows of packed codes or 16 rows of A (bf16), both 4 KB per unit.
// The rank bands come first in the unit order.  The P workgroups each take an
// equal contiguous run of units (stream-K), processed band segment by band
// segment; the four waves split a segment's blocks.  A band covered by
// several workgroups has its partial sums combined by whichever arrives last
// (in segment order, so results are deterministic); partial sums move through
// device-scope stores and loads (coherent across XCDs, no L2-wide fence).
//
// Inner loop (per wave, per block, row band):
//   * codes: 16 bytes per lane per 16-row tile (4 tiles), straight into
//     registers, NS blocks ahead; bf16 operands 128 + c by byte permutes;
//   * x: loaded with fully used cache lines (4 tokens x 256 B per load), put
//     through the wave's own LDS slot and read back in the matrix-core layout
//     (a direct fragment load would touch two half-used lines per token);
//   * group scales and zero-points: staged in LDS per segment, not reloaded
//     per block;
//   * matrix cores 16x16x32: tokens (padded to 16 or 32) x 16 rows x 32 K; a
//     ones-operand product gives the block sums of x that remove the offset.
// The band finisher adds alpha * B * v as a small K = r matrix-core product
// (v split into bf16 high and low parts) and stores y.
//
// Waiting: finishers of row bands wait for the rank bands to publish.  Rank
// units are the first units, owned by the lowest workgroup indices, which the
// dispatcher starts first, so they run before anyone waits; the wait is
// bounded and raises an error word instead of hanging.
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
  float alpha;
  float* part;             // [bands][maxseg][T][64] partial sums
  float* wv32;             // [T][r] alpha * v
  int* ctr;                // counter words
  uint16_t* y;             // [T][N] bf16
  int T, K, N, r, G, ZW, has_z;
  int KB, RB, NB, U, P, maxseg;
};

constexpr int RT = 4;                  // 16-row tiles per row band (64 rows)
constexpr int XROW = 272;              // LDS row of one token: 256 B + 16 B pad
constexpr int kMetaBlocks = 32;        // max blocks of one wave in one segment
constexpr int kMetaBytes = 64 * kMetaBlocks * 4;
constexpr int kSpinLimit = 1 << 20;    // bounded wait (about a second)

template <int MT>
struct Lds {
  static constexpr int kXBytes = MT * 16 * XROW;
  static constexpr int kWave = kXBytes + kMetaBytes;
  static constexpr int kTotal = 4 * kWave;
};

__device__ __forceinline__ int owner_of(long long u, const DecodeParams& p) {
  return (int)(((u + 1) * p.P - 1) / p.U);
}

// The blocks of `wave` inside a segment [lo, hi).
__device__ __forceinline__ void wave_range(int lo, int hi, int wave, int& b0, int& b1) {
  const int nb = hi - lo;
  b0 = lo + nb * wave / 4;
  b1 = lo + nb * (wave + 1) / 4;
}

// Runs compute(b, stage) for b in [b0, b1) with the loads of the next NS-1
// blocks in flight.  issue() runs for every slot with the block clamped into
// range, so the count of loads in flight never depends on a branch.
template <int NS, class Stage, class Issue, class Compute>
__device__ __forceinline__ void stream(int b0, int b1, Stage (&st)[NS], Issue issue,
                                       Compute compute) {
  if (b0 >= b1) return;
  const int last = b1 - 1;
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) issue(min(b0 + i, last), st[i]);
  for (int base = b0; base < b1; base += NS) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      issue(min(base + i + NS - 1, last), st[(i + NS - 1) % NS]);
      if (base + i < b1) compute(base + i, st[i]);
    }
  }
}

// x of one block: MT*16 tokens x 256 bytes, loaded as 4 tokens x 256 B per
// instruction (lane l: token 4c + l/16, 16-byte piece l%16); tokens past T
// read as zero through the buffer bound.
template <int MT>
struct XLoad {
  u32x4 g[4 * MT];
};

template <int MT>
__device__ __forceinline__ void x_issue(rsrc_t xs, uint32_t xrowB, int lane, int blk,
                                        XLoad<MT>& s) {
  const uint32_t base = (uint32_t)(lane >> 4) * xrowB + 16u * (lane & 15);
  for (int c = 0; c < 4 * MT; ++c)
    s.g[c] = bload16(xs, base + 4u * c * xrowB, (uint32_t)blk * 256);
}

// Write the block to this wave's LDS slot, read back fragment (mt, i) of lane
// (token c16 + 16 mt, K group q).  The packed-code path needs piece 4q + i
// (a lane's 16 code bytes span 32 consecutive columns); the rank path, where
// both operands are plain bf16, uses piece 4i + q so that one A load reads 64
// consecutive bytes of each row.
template <int MT, bool RANK_ORDER>
__device__ __forceinline__ void x_to_frags(uint8_t* slot, int lane, const XLoad<MT>& s,
                                           u32x4 (&f)[MT][4]) {
  const int tt = lane >> 4, pc = lane & 15;
  for (int c = 0; c < 4 * MT; ++c)
    *reinterpret_cast<u32x4*>(slot + (4 * c + tt) * XROW + 16 * pc) = s.g[c];
  const int q = lane >> 4, c16 = lane & 15;
  for (int mt = 0; mt < MT; ++mt)
    for (int i = 0; i < 4; ++i) {
      const int piece = RANK_ORDER ? 4 * i + q : 4 * q + i;
      f[mt][i] = *reinterpret_cast<const u32x4*>(slot + (16 * mt + c16) * XROW + piece * 16);
    }
}

// ------------------------------------------------------------- rank segment
// 16 rows of A (ranks 16 rb .. 16 rb + 15), blocks [lo, hi).  Every wave
// returns the workgroup sum of u in uo.
template <int MT>
__device__ void rank_segment(const DecodeParams& p, int rb, int lo, int hi, uint8_t* pool,
                             f32x4 (&uo)[MT]) {
  constexpr int NS = 3;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q = lane >> 4, c16 = lane & 15;
  uint8_t* slot = pool + wave * Lds<MT>::kWave;
  int b0, b1;
  wave_range(lo, hi, wave, b0, b1);
  const uint32_t xrowB = (uint32_t)p.K * 2;
  const rsrc_t xs = make_rsrc(p.x, (uint32_t)p.T * xrowB);
  const rsrc_t as = make_rsrc(p.A + (size_t)16 * rb * p.K, 16 * xrowB);
  const uint32_t ao = (uint32_t)c16 * xrowB + 16 * q;  // piece 4i + q of row c16

  struct Stage {
    u32x4 a[4];
    XLoad<MT> x;
  };
  Stage st[NS];
  f32x4 u[MT];
  for (int mt = 0; mt < MT; ++mt) u[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  stream<NS>(
      b0, b1, st,
      [&](int blk, Stage& s) {
        for (int i = 0; i < 4; ++i) s.a[i] = bload16(as, ao + 64 * i, (uint32_t)blk * 256);
        x_issue<MT>(xs, xrowB, lane, blk, s.x);
      },
      [&](int, const Stage& s) {
        u32x4 xf[MT][4];
        x_to_frags<MT, true>(slot, lane, s.x, xf);
        for (int mt = 0; mt < MT; ++mt)
          for (int i = 0; i < 4; ++i) u[mt] = mfma16x16x32(xf[mt][i], s.a[i], u[mt]);
      });

  __syncthreads();
  float* red = reinterpret_cast<float*>(pool);  // [4][MT][4][64]
  for (int mt = 0; mt < MT; ++mt)
    for (int v = 0; v < 4; ++v) red[((wave * MT + mt) * 4 + v) * 64 + lane] = u[mt][v];
  __syncthreads();
  for (int mt = 0; mt < MT; ++mt)
    for (int v = 0; v < 4; ++v) {
      float s = 0.f;
      for (int w = 0; w < 4; ++w) s += red[((w * MT + mt) * 4 + v) * 64 + lane];
      uo[mt][v] = s;
    }
}

// -------------------------------------------------------------- row segment
// 64 output rows n0 .. n0 + 63, blocks [lo, hi).  Returns the partial y of
// row tile `wave` in yo (scales already applied).
template <int MT, bool GROUPED>
__device__ void row_segment(const DecodeParams& p, int band, int lo, int hi, uint8_t* pool,
                            f32x4 (&yo)[MT]) {
  constexpr int NS = MT == 1 ? 3 : 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q = lane >> 4, c16 = lane & 15;
  uint8_t* slot = pool + wave * Lds<MT>::kWave;
  uint32_t* meta = reinterpret_cast<uint32_t*>(slot + Lds<MT>::kXBytes);  // [64 rows][32 blocks]
  const int n0 = band * kDecodeBandRows;
  const int rows = min(kDecodeBandRows, p.N - n0);
  int b0, b1;
  wave_range(lo, hi, wave, b0, b1);
  const int nwb = b1 - b0;

  if constexpr (GROUPED) {
    // scale (fp16 bits) and zero-point of (row, block) for this wave's blocks
    for (int e = lane; e < 64 * nwb; e += 64) {
      const int row = e / nwb, bb = e - row * nwb, blk = b0 + bb;
      const int n = n0 + min(row, rows - 1);
      const uint32_t s = p.scales[(size_t)n * p.G + blk];
      const uint32_t z =
          p.has_z ? (p.zeros[(size_t)n * p.ZW + (blk >> 3)] >> (4 * (blk & 7))) & 15u : 8u;
      meta[row * kMetaBlocks + bb] = s | (z << 16);
    }
  }

  const uint32_t wrowB = (uint32_t)p.K / 2, xrowB = (uint32_t)p.K * 2;
  const rsrc_t ws = make_rsrc(p.wq + (size_t)n0 * (p.K / 8), (uint32_t)rows * wrowB);
  const rsrc_t xs = make_rsrc(p.x, (uint32_t)p.T * xrowB);
  uint32_t wo[RT];
  for (int rt = 0; rt < RT; ++rt) wo[rt] = (uint32_t)(16 * rt + c16) * wrowB + 16 * q;

  struct Stage {
    u32x4 w[RT];
    XLoad<MT> x;
  };
  Stage st[NS];
  f32x4 acc[MT][RT], ssum[MT];
  for (int mt = 0; mt < MT; ++mt) {
    ssum[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int rt = 0; rt < RT; ++rt) acc[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const u32x4 ones = {kBf16One, kBf16One, kBf16One, kBf16One};

  stream<NS>(
      b0, b1, st,
      [&](int blk, Stage& s) {
        for (int rt = 0; rt < RT; ++rt) s.w[rt] = bload16(ws, wo[rt], (uint32_t)blk * 64);
        x_issue<MT>(xs, xrowB, lane, blk, s.x);
      },
      [&](int blk, const Stage& s) {
        u32x4 xp[MT][4];
        x_to_frags<MT, false>(slot, lane, s.x, xp);
        for (int mt = 0; mt < MT; ++mt)
          for (int i = 0; i < 4; ++i) xp[mt][i] = x_permute8(xp[mt][i]);
        f32x4 sb[MT];
        for (int mt = 0; mt < MT; ++mt) {
          if constexpr (GROUPED) {
            sb[mt] = mfma16x16x32(xp[mt][0], ones, f32x4{0.f, 0.f, 0.f, 0.f});
            for (int i = 1; i < 4; ++i) sb[mt] = mfma16x16x32(xp[mt][i], ones, sb[mt]);
          } else {
            for (int i = 0; i < 4; ++i) ssum[mt] = mfma16x16x32(xp[mt][i], ones, ssum[mt]);
          }
        }
        for (int rt = 0; rt < RT; ++rt) {
          u32x4 wb[4];
          wb[0] = codes_to_bf16_offset(s.w[rt].x);
          wb[1] = codes_to_bf16_offset(s.w[rt].y);
          wb[2] = codes_to_bf16_offset(s.w[rt].z);
          wb[3] = codes_to_bf16_offset(s.w[rt].w);
          if constexpr (GROUPED) {
            const uint32_t m = meta[(16 * rt + c16) * kMetaBlocks + (blk - b0)];
            const float sc = half_bits_to_f32((uint16_t)(m & 0xFFFFu));
            const float mz = -(float)(128u + (m >> 16));
            for (int mt = 0; mt < MT; ++mt) {
              f32x4 P = mfma16x16x32(xp[mt][0], wb[0], f32x4{0.f, 0.f, 0.f, 0.f});
              P = mfma16x16x32(xp[mt][1], wb[1], P);
              P = mfma16x16x32(xp[mt][2], wb[2], P);
              P = mfma16x16x32(xp[mt][3], wb[3], P);
              for (int v = 0; v < 4; ++v)
                acc[mt][rt][v] = fmaf(sc, fmaf(mz, sb[mt][v], P[v]), acc[mt][rt][v]);
            }
          } else {
            for (int mt = 0; mt < MT; ++mt)
              for (int i = 0; i < 4; ++i) acc[mt][rt] = mfma16x16x32(xp[mt][i], wb[i], acc[mt][rt]);
          }
        }
      });

  if constexpr (!GROUPED) {  // per-channel: one scale and one offset correction per row
    for (int rt = 0; rt < RT; ++rt) {
      const int n = n0 + min(16 * rt + c16, rows - 1);
      const float sc = half_bits_to_f32(p.scales[n]);
      const int z = p.has_z ? (int)(p.zeros[(size_t)n * p.ZW] & 15u) : 8;
      const float mz = -(float)(128 + z);
      for (int mt = 0; mt < MT; ++mt)
        for (int v = 0; v < 4; ++v) acc[mt][rt][v] = sc * fmaf(mz, ssum[mt][v], acc[mt][rt][v]);
    }
  }

  // Sum the four waves; wave w then owns row tile w.
  __syncthreads();
  float* red = reinterpret_cast<float*>(pool);  // [4][MT][RT][4][64]
  for (int mt = 0; mt < MT; ++mt)
    for (int rt = 0; rt < RT; ++rt)
      for (int v = 0; v < 4; ++v)
        red[(((wave * MT + mt) * RT + rt) * 4 + v) * 64 + lane] = acc[mt][rt][v];
  __syncthreads();
  for (int mt = 0; mt < MT; ++mt)
    for (int v = 0; v < 4; ++v) {
      float s = 0.f;
      for (int w = 0; w < 4; ++w) s += red[(((w * MT + mt) * RT + wave) * 4 + v) * 64 + lane];
      yo[mt][v] = s;
    }
}

// Partial sums of a band: [maxseg][T][64] floats per band, written and read
// at device scope.  Column c of a partial is row c of a row band, or rank
// 16 rb + c of a rank band (only columns 0..15 used).
template <int MT>
__device__ __forceinline__ void put_part(const DecodeParams& p, int band, int sidx, int col,
                                         const f32x4 (&v)[MT]) {
  const int q = (threadIdx.x & 63) >> 4;
  float* base = p.part + ((size_t)band * p.maxseg + sidx) * p.T * 64;
  for (int mt = 0; mt < MT; ++mt)
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * mt + 4 * q + i;
      if (t < p.T) store_dev(base + (size_t)t * 64 + col, v[mt][i]);
    }
}

template <int MT>
__device__ __forceinline__ void sum_parts(const DecodeParams& p, int band, int nseg, int col,
                                          f32x4 (&v)[MT]) {
  const int q = (threadIdx.x & 63) >> 4;
  for (int mt = 0; mt < MT; ++mt)
    for (int i = 0; i < 4; ++i) {
      const int t = min(16 * mt + 4 * q + i, p.T - 1);
      float s = 0.f;
#pragma unroll 4
      for (int k = 0; k < nseg; ++k)
        s += load_dev(p.part + (((size_t)band * p.maxseg + k) * p.T + t) * 64 + col);
      v[mt][i] = s;
    }
}

// Finish a rank band: gate and publish alpha * v for ranks 16 rb .. +15.
template <int MT>
__device__ void finish_rank(const DecodeParams& p, int rb, const f32x4 (&u)[MT]) {
  const int lane = threadIdx.x & 63, q = lane >> 4, c16 = lane & 15;
  const int j = 16 * rb + c16;
  const float g = p.gv[j], b = p.bv[j];
  for (int mt = 0; mt < MT; ++mt)
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * mt + 4 * q + i;
      if (t < p.T) {
        const float uu = u[mt][i];
        store_dev(&p.wv32[(size_t)t * p.r + j], p.alpha * (sigmoidf_safe(fmaf(g, uu, b)) * uu));
      }
    }
}

// Finish a row band (wave = row tile): + alpha * v B^T, then store y.
template <int MT>
__device__ void finish_row(const DecodeParams& p, int band, f32x4 (&yv)[MT]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q = lane >> 4, c16 = lane & 15;
  const int n0 = band * kDecodeBandRows;
  const int nrow = n0 + 16 * wave + c16;
  if (p.r > 0) {
    if (tid == 0) {
      int spins = 0;
      while (load_dev(&p.ctr[kCtrRankDone]) < p.RB) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > kSpinLimit) {
          atomicOr(&p.ctr[kCtrError], 1);
          break;
        }
      }
    }
    __syncthreads();
    const rsrc_t bs = make_rsrc(p.B, (uint32_t)p.N * p.r * 2);
    const uint32_t bro = (uint32_t)min(nrow, p.N - 1) * p.r * 2;
    for (int j0 = 0; j0 < p.r; j0 += 32) {
      const int jj = j0 + 8 * q;  // this lane's 8 ranks of the K = 32 step
      const bool jok = jj < p.r;
      const u32x4 bfr = jok ? bload16(bs, bro + 2 * jj, 0) : u32x4{0, 0, 0, 0};
      for (int mt = 0; mt < MT; ++mt) {
        const int t = min(16 * mt + c16, p.T - 1);
        u32x4 hi = {0, 0, 0, 0}, lo = {0, 0, 0, 0};
        if (jok) {
          const float* src = p.wv32 + (size_t)t * p.r + jj;
          uint32_t h[8], l[8];
          for (int e = 0; e < 8; ++e) {
            const float v = load_dev(src + e);
            h[e] = f32_to_bf16_rne(v);
            l[e] = f32_to_bf16_rne(v - __uint_as_float(h[e] << 16));
          }
          hi = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                     h[6] | (h[7] << 16)};
          lo = u32x4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16),
                     l[6] | (l[7] << 16)};
        }
        yv[mt] = mfma16x16x32(hi, bfr, yv[mt]);
        yv[mt] = mfma16x16x32(lo, bfr, yv[mt]);
      }
    }
  }
  if (nrow < p.N)
    for (int mt = 0; mt < MT; ++mt)
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * mt + 4 * q + i;
        if (t < p.T) p.y[(size_t)t * p.N + nrow] = (uint16_t)f32_to_bf16_rne(yv[mt][i]);
      }
}

template <int MT, bool GROUPED>
__global__ __launch_bounds__(256, 2) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t pool[Lds<MT>::kTotal];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c16 = lane & 15;
  const int wg = blockIdx.x;
  const long long u0 = (long long)p.U * wg / p.P, u1 = (long long)p.U * (wg + 1) / p.P;

  for (long long u = u0; u < u1;) {
    const int band = (int)(u / p.KB);
    const long long bend = (long long)(band + 1) * p.KB;
    const int lo = (int)(u - (long long)band * p.KB);
    const int hi = (int)(min(u1, bend) - (long long)band * p.KB);
    u = min(u1, bend);
    const int first = owner_of((long long)band * p.KB, p);
    const int nseg = owner_of(bend - 1, p) - first + 1;
    const int sidx = wg - first;
    const bool rank = band < p.RB;

    f32x4 v[MT];
    if (rank) rank_segment<MT>(p, band, lo, hi, pool, v);
    else row_segment<MT, GROUPED>(p, band - p.RB, lo, hi, pool, v);
    const int col = rank ? c16 : 16 * wave + c16;
    const bool owner = rank ? wave == 0 : true;  // rank band: one copy of the sum

    bool fin = nseg == 1;
    if (!fin) {
      if (owner) put_part<MT>(p, band, sidx, col, v);
      wait_vmem();
      __syncthreads();
      if (tid == 0) s_last = atomicAdd(&p.ctr[kCtrBand + band], 1) == nseg - 1;
      __syncthreads();
      fin = s_last;
      if (fin) {
        if (owner) sum_parts<MT>(p, band, nseg, col, v);
        if (tid == 0) store_dev(&p.ctr[kCtrBand + band], 0);
      }
    }
    if (fin) {
      if (rank) {
        if (wave == 0) finish_rank<MT>(p, band, v);
        wait_vmem();
        __syncthreads();
        if (tid == 0) atomicAdd(&p.ctr[kCtrRankDone], 1);
      } else {
        finish_row<MT>(p, band - p.RB, v);
      }
    }
    __syncthreads();  // the LDS pool is reused by the next segment
  }

  if (p.RB > 0 && tid == 0) {
    wait_vmem();
    if (atomicAdd(&p.ctr[kCtrExit], 1) == p.P - 1) {
      store_dev(&p.ctr[kCtrRankDone], 0);
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
  p.U = pl.units;
  p.P = pl.workgroups;
  p.maxseg = pl.maxseg;
  if (s.T <= 16) return s.grouped ? go<1, true>(p, st) : go<1, false>(p, st);
  return s.grouped ? go<2, true>(p, st) : go<2, false>(p, st);
}

}  // namespace spear
