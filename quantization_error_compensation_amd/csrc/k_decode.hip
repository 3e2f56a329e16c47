// Decode path (1..32 tokens): one fused, bandwidth-bound kernel.
//
// SPEAR summary, section 2.2 A (phase-aware adaptive kernel fusion): in the
// memory-bound decode phase the compensator is fused into the epilogue of the
// low-bit GEMM, so the whole compensated layer is a single kernel.  Here one
// launch streams the packed weights once, computes the rank-r projection of
// every token once, gates it, and adds alpha * B * v in fp32 before the single
// bf16 store of y.
//
// Work items (one per workgroup of 4 waves, handed out by an atomic ticket so
// that the first tickets always go to the projection items):
//   * rank items: 16 rows of A x one K split.  Partial u = A x of the split goes
//     to the workspace; the last split of a rank band sums the partials in
//     split order, applies the gate and publishes alpha * v for its 16 ranks.
//   * row items: 64 output rows x one K split.  Each wave streams a contiguous
//     run of 128-column blocks: 16 bytes (32 codes) per lane per row tile, so a
//     wave reads 64 contiguous bytes of 16 rows per block and both halves of
//     each 128-byte line in consecutive blocks.  Loads are unconditional
//     (clamped indices) and kept NS blocks ahead in a register ring.
// Codes become bf16 operands 128 + c by bit operations; the matrix cores
// (16x16x32) multiply them with the tokens (padded to 16 or 32), four row
// tiles sharing each activation fragment.  A ones-operand product gives the
// block sums of x that remove the offset; scales are applied in fp32.  After
// the K loop the waves are summed in LDS, each split adds its share of the
// rank terms (after the rank items have published), and the last split of a
// band sums the partials in split order and stores y once.
//
// Waiting: row items wait for the rank items only after their own K loop.
// Rank items took the lowest tickets, so they are running before any row item
// can wait; the wait is bounded and flags an error word instead of hanging.
// Partial sums, published projections and counters move between workgroups
// through device-scope stores and loads (no L2-wide fences, see common.hpp).
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
  float* upart;            // [splits][T][r]
  float* wv32;             // [T][r]  alpha * v
  float* ypart;            // [splits][T][N]
  int* ctr;                // counter words
  uint16_t* y;             // [T][N] bf16
  int T, K, N, r, splits, G, ZW, has_z, bands, rank_bands;
};

constexpr int RT = 4;                 // 16-row tiles per wave (64-row band)
constexpr int kSpinLimit = 1 << 20;   // bounded wait for the rank items (about a second)

__device__ __forceinline__ void split_range(int KB, int split, int splits, int wave, int& b0,
                                            int& b1) {
  const int kb0 = (int)((long long)KB * split / splits);
  const int kb1 = (int)((long long)KB * (split + 1) / splits);
  const int nb = kb1 - kb0;
  b0 = kb0 + nb * wave / 4;
  b1 = kb0 + nb * (wave + 1) / 4;
}

// Runs compute(b, stage) for b in [b0, b1) with the loads of the next NS-1
// blocks in flight.  issue() is called for every slot, with the block index
// clamped into range, so the number of loads in flight never depends on a
// branch.
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

// ---------------------------------------------------------------- rank item
template <int MT>
__device__ void rank_item(const DecodeParams& p, int rb, int split,
                          float (&red)[4][MT][RT][4][64], int& s_last) {
  constexpr int NS = 3;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q = lane >> 4, c16 = lane & 15;
  int b0, b1;
  split_range(p.K / kBlockK, split, p.splits, wave, b0, b1);
  const uint32_t rowB = (uint32_t)p.K * 2;
  const rsrc_t xs = make_rsrc(p.x, (uint32_t)p.T * rowB);           // tokens past T read 0
  const rsrc_t as = make_rsrc(p.A + (size_t)16 * rb * p.K, 16 * rowB);
  uint32_t xo[MT];
  for (int mt = 0; mt < MT; ++mt) xo[mt] = (uint32_t)(16 * mt + c16) * rowB + 64 * q;
  const uint32_t ao = (uint32_t)c16 * rowB + 64 * q;

  struct Stage {
    u32x4 x[MT][4];
    u32x4 a[4];
  };
  Stage st[NS];
  f32x4 u[MT];
  for (int mt = 0; mt < MT; ++mt) u[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  stream<NS>(b0, b1, st,
             [&](int blk, Stage& s) {
               const uint32_t so = (uint32_t)blk * 256;
               for (int i = 0; i < 4; ++i) s.a[i] = bload16(as, ao + 16 * i, so);
               for (int mt = 0; mt < MT; ++mt)
                 for (int i = 0; i < 4; ++i) s.x[mt][i] = bload16(xs, xo[mt] + 16 * i, so);
             },
             [&](int, const Stage& s) {
               for (int mt = 0; mt < MT; ++mt)
                 for (int i = 0; i < 4; ++i) u[mt] = mfma16x16x32(s.x[mt][i], s.a[i], u[mt]);
             });

  for (int mt = 0; mt < MT; ++mt)
    for (int v = 0; v < 4; ++v) red[wave][mt][0][v][lane] = u[mt][v];
  __syncthreads();
  const int j = 16 * rb + c16;
  if (wave == 0) {
    for (int mt = 0; mt < MT; ++mt)
      for (int v = 0; v < 4; ++v) {
        const int t = 16 * mt + 4 * q + v;
        const float s = red[0][mt][0][v][lane] + red[1][mt][0][v][lane] +
                        red[2][mt][0][v][lane] + red[3][mt][0][v][lane];
        if (t < p.T) store_dev(&p.upart[((size_t)split * p.T + t) * p.r + j], s);
      }
  }
  wait_vmem();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&p.ctr[kCtrRankBand + rb], 1) == p.splits - 1;
  __syncthreads();
  if (!s_last) return;
  if (wave == 0) {
    for (int mt = 0; mt < MT; ++mt)
      for (int v = 0; v < 4; ++v) {
        const int t = 16 * mt + 4 * q + v;
        if (t >= p.T) continue;
        float acc = 0.f;
#pragma unroll 8
        for (int s = 0; s < p.splits; ++s)
          acc += load_dev(&p.upart[((size_t)s * p.T + t) * p.r + j]);
        const float gate = sigmoidf_safe(fmaf(p.gv[j], acc, p.bv[j]));
        store_dev(&p.wv32[(size_t)t * p.r + j], p.alpha * (gate * acc));
      }
  }
  wait_vmem();
  __syncthreads();
  if (tid == 0) {
    store_dev(&p.ctr[kCtrRankBand + rb], 0);
    atomicAdd(&p.ctr[kCtrRankDone], 1);
  }
}

// ----------------------------------------------------------------- row item
template <int MT, bool GROUPED>
__device__ void row_item(const DecodeParams& p, int band, int split,
                         float (&red)[4][MT][RT][4][64], int& s_last) {
  constexpr int NS = MT == 1 ? 3 : 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q = lane >> 4, c16 = lane & 15;
  const int n0 = band * kDecodeBandRows;
  const int rows = min(kDecodeBandRows, p.N - n0);
  int b0, b1;
  split_range(p.K / kBlockK, split, p.splits, wave, b0, b1);

  // One resource per operand, based at this band: rows past d_out read zero.
  const uint32_t wrowB = (uint32_t)p.K / 2, xrowB = (uint32_t)p.K * 2;
  const rsrc_t ws = make_rsrc(p.wq + (size_t)n0 * (p.K / 8), (uint32_t)rows * wrowB);
  const rsrc_t xs = make_rsrc(p.x, (uint32_t)p.T * xrowB);
  const rsrc_t ss = make_rsrc(p.scales + (size_t)n0 * p.G, (uint32_t)rows * p.G * 2);
  const rsrc_t zs = make_rsrc(p.zeros + (size_t)(p.has_z ? n0 : 0) * p.ZW,
                              p.has_z ? (uint32_t)rows * p.ZW * 4 : 0u);
  uint32_t wo[RT], so[RT], zo[RT];
  for (int rt = 0; rt < RT; ++rt) {
    const uint32_t rl = 16 * rt + c16;  // row within the band
    wo[rt] = rl * wrowB + 16 * q;
    so[rt] = rl * p.G * 2;
    zo[rt] = rl * p.ZW * 4;
  }
  uint32_t xo[MT];
  for (int mt = 0; mt < MT; ++mt) xo[mt] = (uint32_t)(16 * mt + c16) * xrowB + 64 * q;

  struct Stage {
    u32x4 w[RT];
    u32x4 x[MT][4];
    uint32_t sc[RT];
    uint32_t zw[RT];
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
        const uint32_t wso = (uint32_t)blk * 64, xso = (uint32_t)blk * 256;
        for (int rt = 0; rt < RT; ++rt) s.w[rt] = bload16(ws, wo[rt], wso);
        for (int mt = 0; mt < MT; ++mt)
          for (int i = 0; i < 4; ++i) s.x[mt][i] = bload16(xs, xo[mt] + 16 * i, xso);
        if constexpr (GROUPED) {
          for (int rt = 0; rt < RT; ++rt) {
            s.sc[rt] = bload2(ss, so[rt], (uint32_t)blk * 2);
            s.zw[rt] = bload4(zs, zo[rt], (uint32_t)(blk >> 3) * 4);
          }
        }
      },
      [&](int blk, const Stage& s) {
        u32x4 xp[MT][4];
        for (int mt = 0; mt < MT; ++mt)
          for (int i = 0; i < 4; ++i) xp[mt][i] = x_permute8(s.x[mt][i]);
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
            const float sc = half_bits_to_f32((uint16_t)s.sc[rt]);
            const int z = p.has_z ? (int)((s.zw[rt] >> (4 * (blk & 7))) & 15u) : 8;
            const float mz = -(float)(128 + z);
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
      const int n = min(n0 + 16 * rt + c16, p.N - 1);
      const float sc = half_bits_to_f32(p.scales[n]);
      const int z = p.has_z ? (int)(p.zeros[(size_t)n * p.ZW] & 15u) : 8;
      const float mz = -(float)(128 + z);
      for (int mt = 0; mt < MT; ++mt)
        for (int v = 0; v < 4; ++v) acc[mt][rt][v] = sc * fmaf(mz, ssum[mt][v], acc[mt][rt][v]);
    }
  }

  // Sum the four waves; wave w then owns row tile w.
  for (int mt = 0; mt < MT; ++mt)
    for (int rt = 0; rt < RT; ++rt)
      for (int v = 0; v < 4; ++v) red[wave][mt][rt][v][lane] = acc[mt][rt][v];
  __syncthreads();
  const int rt = wave;
  const int n = n0 + 16 * rt + c16;
  const bool row_ok = 16 * rt < rows;
  f32x4 part[MT];
  for (int mt = 0; mt < MT; ++mt)
    for (int v = 0; v < 4; ++v)
      part[mt][v] = red[0][mt][rt][v][lane] + red[1][mt][rt][v][lane] + red[2][mt][rt][v][lane] +
                    red[3][mt][rt][v][lane];

  // This split's share of the rank terms, once the rank items have published.
  if (p.r > 0) {
    if (tid == 0) {
      int spins = 0;
      while (load_dev(&p.ctr[kCtrRankDone]) < p.rank_bands) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > kSpinLimit) {
          atomicOr(&p.ctr[kCtrError], 1);
          break;
        }
      }
    }
    __syncthreads();
    const int j0 = (int)((long long)p.r * split / p.splits);
    const int j1 = (int)((long long)p.r * (split + 1) / p.splits);
    const uint16_t* brow = p.B + (size_t)min(n, p.N - 1) * p.r;
    for (int j = j0; j < j1; ++j) {
      const float bj = __uint_as_float((uint32_t)brow[j] << 16);
      for (int mt = 0; mt < MT; ++mt)
        for (int v = 0; v < 4; ++v) {
          const int t = min(16 * mt + 4 * q + v, p.T - 1);
          part[mt][v] = fmaf(bj, load_dev(&p.wv32[(size_t)t * p.r + j]), part[mt][v]);
        }
    }
  }

  if (p.splits == 1) {
    if (row_ok)
      for (int mt = 0; mt < MT; ++mt)
        for (int v = 0; v < 4; ++v) {
          const int t = 16 * mt + 4 * q + v;
          if (t < p.T) p.y[(size_t)t * p.N + n] = (uint16_t)f32_to_bf16_rne(part[mt][v]);
        }
    return;
  }
  if (row_ok)
    for (int mt = 0; mt < MT; ++mt)
      for (int v = 0; v < 4; ++v) {
        const int t = 16 * mt + 4 * q + v;
        if (t < p.T) store_dev(&p.ypart[((size_t)split * p.T + t) * p.N + n], part[mt][v]);
      }
  wait_vmem();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&p.ctr[kCtrRowBand + band], 1) == p.splits - 1;
  __syncthreads();
  if (!s_last) return;
  for (int e = tid; e < p.T * rows; e += 256) {
    const int t = e / rows, nn = n0 + e % rows;
    float sum = 0.f;
#pragma unroll 8
    for (int s = 0; s < p.splits; ++s) sum += load_dev(&p.ypart[((size_t)s * p.T + t) * p.N + nn]);
    p.y[(size_t)t * p.N + nn] = (uint16_t)f32_to_bf16_rne(sum);
  }
  if (tid == 0) store_dev(&p.ctr[kCtrRowBand + band], 0);
}

template <int MT, bool GROUPED>
__global__ __launch_bounds__(256, 2) void decode_kernel(DecodeParams p) {
  __shared__ float red[4][MT][RT][4][64];
  __shared__ int s_ticket, s_last;
  const int tid = threadIdx.x;
  if (tid == 0) s_ticket = atomicAdd(&p.ctr[kCtrTicket], 1);
  __syncthreads();
  const int ticket = s_ticket;
  const int nrank = p.rank_bands * p.splits;
  const int total = nrank + p.bands * p.splits;
  if (ticket < nrank) {
    rank_item<MT>(p, ticket / p.splits, ticket % p.splits, red, s_last);
  } else if (ticket < total) {
    const int w = ticket - nrank;
    row_item<MT, GROUPED>(p, w / p.splits, w % p.splits, red, s_last);
  } else if (tid == 0) {
    atomicOr(&p.ctr[kCtrError], 2);  // counters were not zero at launch
  }
  __syncthreads();
  if (tid == 0) {
    wait_vmem();
    if (atomicAdd(&p.ctr[kCtrExit], 1) == total - 1) {
      store_dev(&p.ctr[kCtrTicket], 0);
      store_dev(&p.ctr[kCtrRankDone], 0);
      store_dev(&p.ctr[kCtrExit], 0);
    }
  }
}

template <int MT, bool GROUPED>
hipError_t go(const DecodeParams& p, int grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<MT, GROUPED>), dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const Shape& s, const LayerArgs& a, const WsPtrs& w, hipStream_t st) {
  const DecodePlan pl = plan_decode(s);
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
  p.upart = w.upart;
  p.wv32 = w.wv32;
  p.ypart = w.ypart;
  p.ctr = w.counters;
  p.y = static_cast<uint16_t*>(a.y);
  p.T = s.T;
  p.K = s.K;
  p.N = s.N;
  p.r = s.r;
  p.splits = pl.splits;
  p.G = s.K / s.g;
  p.ZW = (p.G + 7) / 8;
  p.bands = pl.bands;
  p.rank_bands = pl.rank_bands;
  const int grid = pl.workgroups();
  if (s.T <= 16) return s.grouped ? go<1, true>(p, grid, st) : go<1, false>(p, grid, st);
  return s.grouped ? go<2, true>(p, grid, st) : go<2, false>(p, grid, st);
}

}  // namespace spear
