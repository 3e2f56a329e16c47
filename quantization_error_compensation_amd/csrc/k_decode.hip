// Decode path (1..32 tokens): a bandwidth-bound fused GEMV.
//
// SPEAR summary, section 2.2 A (phase-aware adaptive kernel fusion): in the
// memory-bound decode phase the compensator is fused into the epilogue of the
// low-bit GEMM, so the correction adds no separate kernel on the critical path
// after the weights are streamed.  Here:
//
//   * Each workgroup owns a band of 64 output rows and one K split; its four
//     waves take contiguous runs of 128-column blocks.  A lane streams 16
//     bytes (32 codes) of one row per block, so a wave reads 64 contiguous
//     bytes of each of 16 rows per block and the two halves of each 128-byte
//     line in consecutive blocks.
//   * The codes become bf16 operands 128 + c with bit operations only and are
//     multiplied on the matrix cores (16x16x32) with the tokens, padded to 16
//     or 32; 16 rows x 4 row tiles share each activation fragment.
//   * Scales are applied in fp32: per 128-column group (group-wise) or once
//     per row (per-channel); the +128 offset is removed with the per-block
//     sums of x computed once per token by the projection kernel.
//   * Epilogue: the four waves' sums are added in LDS, each K split adds its
//     share of the rank terms alpha * sum_j B[n,j] v[t,j] in fp32, and the
//     last split to finish a band sums the partials in split order and stores
//     y once, rounded to bf16.
#include "common.hpp"
#include "internal.hpp"

namespace spear {
namespace {

struct DecodeParams {
  const uint16_t* x;       // [T][K] bf16
  const uint32_t* wq;      // [N][K/8]
  const uint16_t* scales;  // [N][G] fp16
  const uint32_t* zeros;   // [N][ZW] or null
  const uint16_t* B;       // [N][r] bf16
  const float* wv32;       // [T][r]  alpha * v
  const float* sblk;       // [KB][Tp]
  float* ypart;            // [splits][T][N]
  int* counters;           // one per band
  uint16_t* y;             // [T][N] bf16
  int T, K, N, r, Tp, splits, G, ZW;
};

constexpr int RT = 4;  // 16-row tiles per wave (64-row band)

template <int MT, bool GROUPED>
__global__ __launch_bounds__(256, 2) void decode_kernel(DecodeParams p) {
  __shared__ float red[4][MT][RT][4][64];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, c16 = lane & 15;
  const int band = blockIdx.x / p.splits, split = blockIdx.x % p.splits;
  const int n0 = band * kDecodeBandRows;
  const int KB = p.K / kBlockK;
  const int kb0 = (int)((long long)KB * split / p.splits);
  const int kb1 = (int)((long long)KB * (split + 1) / p.splits);
  const int nb = kb1 - kb0;
  const int wb0 = kb0 + nb * wave / 4, wb1 = kb0 + nb * (wave + 1) / 4;
  const size_t rowWords = (size_t)p.K / 8;

  bool rt_ok[RT];
  const uint32_t* wr[RT];
  for (int rt = 0; rt < RT; ++rt) {
    rt_ok[rt] = n0 + 16 * rt < p.N;  // N is a multiple of 16: whole tiles
    const int n = rt_ok[rt] ? n0 + 16 * rt + c16 : 0;
    wr[rt] = p.wq + (size_t)n * rowWords + 4 * q;
  }
  bool tok_ok[MT];
  const uint16_t* xr[MT];
  for (int mt = 0; mt < MT; ++mt) {
    const int t = 16 * mt + c16;
    tok_ok[mt] = t < p.T;
    xr[mt] = p.x + (size_t)(tok_ok[mt] ? t : 0) * p.K + 32 * q;
  }

  f32x4 acc[MT][RT];
  f32x4 ssum[MT];
  for (int mt = 0; mt < MT; ++mt) {
    ssum[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int rt = 0; rt < RT; ++rt) acc[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Raw loads of one block, issued one block ahead of their use.
  struct Stage {
    u32x4 w[RT];
    u32x4 x[MT][4];
    f32x4 s[MT];
    uint16_t sc[RT];
    uint32_t zw[RT];
  };
  auto issue = [&](int blk, Stage& st) {
    for (int rt = 0; rt < RT; ++rt)
      st.w[rt] = rt_ok[rt] ? load16(wr[rt] + (size_t)blk * 16) : u32x4{0, 0, 0, 0};
    for (int mt = 0; mt < MT; ++mt) {
      for (int i = 0; i < 4; ++i)
        st.x[mt][i] = tok_ok[mt] ? load16(xr[mt] + (size_t)blk * kBlockK + 8 * i)
                                 : u32x4{0, 0, 0, 0};
      st.s[mt] = *reinterpret_cast<const f32x4*>(p.sblk + (size_t)blk * p.Tp + 16 * mt + 4 * q);
    }
    if constexpr (GROUPED) {
      for (int rt = 0; rt < RT; ++rt) {
        const int n = rt_ok[rt] ? n0 + 16 * rt + c16 : 0;
        st.sc[rt] = p.scales[(size_t)n * p.G + blk];
        st.zw[rt] = p.zeros ? p.zeros[(size_t)n * p.ZW + blk / 8] : 0u;
      }
    }
  };

  auto compute = [&](int blk, const Stage& cur) {
    u32x4 xp[MT][4];
    for (int mt = 0; mt < MT; ++mt)
      for (int i = 0; i < 4; ++i) xp[mt][i] = x_permute8(cur.x[mt][i]);
    for (int rt = 0; rt < RT; ++rt) {
      if (!rt_ok[rt]) continue;
      u32x4 wb[4];
      wb[0] = codes_to_bf16_offset(cur.w[rt].x);
      wb[1] = codes_to_bf16_offset(cur.w[rt].y);
      wb[2] = codes_to_bf16_offset(cur.w[rt].z);
      wb[3] = codes_to_bf16_offset(cur.w[rt].w);
      if constexpr (GROUPED) {
        const float s = half_bits_to_f32(cur.sc[rt]);
        const int z = p.zeros ? (int)((cur.zw[rt] >> (4 * (blk & 7))) & 15u) : 8;
        const float mz = -(float)(128 + z);
        for (int mt = 0; mt < MT; ++mt) {
          f32x4 P = mfma16x16x32(xp[mt][0], wb[0], f32x4{0.f, 0.f, 0.f, 0.f});
          P = mfma16x16x32(xp[mt][1], wb[1], P);
          P = mfma16x16x32(xp[mt][2], wb[2], P);
          P = mfma16x16x32(xp[mt][3], wb[3], P);
          for (int v = 0; v < 4; ++v)
            acc[mt][rt][v] = fmaf(s, fmaf(mz, cur.s[mt][v], P[v]), acc[mt][rt][v]);
        }
      } else {
        for (int mt = 0; mt < MT; ++mt)
          for (int i = 0; i < 4; ++i) acc[mt][rt] = mfma16x16x32(xp[mt][i], wb[i], acc[mt][rt]);
      }
    }
    if constexpr (!GROUPED)
      for (int mt = 0; mt < MT; ++mt) ssum[mt] += cur.s[mt];
  };

  // Two register stages in ping-pong: block b+1 is in flight while b computes.
  Stage sa, sb;
  int blk = wb0;
  if (blk < wb1) issue(blk, sa);
  while (blk < wb1) {
    if (blk + 1 < wb1) issue(blk + 1, sb);
    compute(blk, sa);
    if (++blk >= wb1) break;
    if (blk + 1 < wb1) issue(blk + 1, sa);
    compute(blk, sb);
    ++blk;
  }

  if constexpr (!GROUPED) {  // per-channel: one scale and one offset correction per row
    for (int rt = 0; rt < RT; ++rt) {
      if (!rt_ok[rt]) continue;
      const int n = n0 + 16 * rt + c16;
      const float s = half_bits_to_f32(p.scales[n]);
      const int z = p.zeros ? (int)(p.zeros[(size_t)n * p.ZW] & 15u) : 8;
      const float mz = -(float)(128 + z);
      for (int mt = 0; mt < MT; ++mt)
        for (int v = 0; v < 4; ++v) acc[mt][rt][v] = s * fmaf(mz, ssum[mt][v], acc[mt][rt][v]);
    }
  }

  // Sum the four waves; wave w then owns row tile w.
  for (int mt = 0; mt < MT; ++mt)
    for (int rt = 0; rt < RT; ++rt)
      for (int v = 0; v < 4; ++v) red[wave][mt][rt][v][lane] = acc[mt][rt][v];
  __syncthreads();
  const int rt = wave;
  const bool row_ok = n0 + 16 * rt < p.N;
  const int n = n0 + 16 * rt + c16;
  f32x4 part[MT];
  for (int mt = 0; mt < MT; ++mt)
    for (int v = 0; v < 4; ++v)
      part[mt][v] = red[0][mt][rt][v][lane] + red[1][mt][rt][v][lane] +
                    red[2][mt][rt][v][lane] + red[3][mt][rt][v][lane];

  // This split's share of the rank terms: alpha * sum_j B[n,j] v[t,j].
  if (row_ok && p.r > 0) {
    const int j0 = (int)((long long)p.r * split / p.splits);
    const int j1 = (int)((long long)p.r * (split + 1) / p.splits);
    for (int j = j0; j < j1; ++j) {
      const float bj = __uint_as_float((uint32_t)p.B[(size_t)n * p.r + j] << 16);
      for (int mt = 0; mt < MT; ++mt)
        for (int v = 0; v < 4; ++v) {
          const int t = 16 * mt + 4 * q + v;
          if (t < p.T) part[mt][v] = fmaf(bj, p.wv32[(size_t)t * p.r + j], part[mt][v]);
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
        if (t < p.T) p.ypart[((size_t)split * p.T + t) * p.N + n] = part[mt][v];
      }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(&p.counters[band], 1);
    s_last = (prev == p.splits - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int e = threadIdx.x; e < p.T * kDecodeBandRows; e += 256) {
    const int t = e / kDecodeBandRows, nn = n0 + e % kDecodeBandRows;
    if (nn >= p.N) continue;
    float sum = 0.f;
    for (int s = 0; s < p.splits; ++s) sum += p.ypart[((size_t)s * p.T + t) * p.N + nn];
    p.y[(size_t)t * p.N + nn] = (uint16_t)f32_to_bf16_rne(sum);
  }
  if (threadIdx.x == 0) p.counters[band] = 0;
}

template <int MT, bool GROUPED>
hipError_t go(const DecodeParams& p, int grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<MT, GROUPED>), dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const Shape& s, const LayerArgs& a, const WsPtrs& w, hipStream_t st) {
  const DecodePlan pl = plan_decode(s);
  const ProjPlan pp = plan_projection(s);
  DecodeParams p;
  p.x = static_cast<const uint16_t*>(a.x);
  p.wq = a.wq;
  p.scales = a.scales;
  p.zeros = a.zeros;
  p.B = static_cast<const uint16_t*>(a.B);
  p.wv32 = w.wv32;
  p.sblk = w.sblk;
  p.ypart = w.ypart;
  p.counters = w.counters + kDecodeCounterBase;
  p.y = static_cast<uint16_t*>(a.y);
  p.T = s.T;
  p.K = s.K;
  p.N = s.N;
  p.r = s.r;
  p.Tp = pp.tiles * kProjTokens;
  p.splits = pl.splits;
  p.G = s.K / s.g;
  p.ZW = (p.G + 7) / 8;
  const int grid = pl.bands * pl.splits;
  if (s.T <= 16) return s.grouped ? go<1, true>(p, grid, st) : go<1, false>(p, grid, st);
  return s.grouped ? go<2, true>(p, grid, st) : go<2, false>(p, grid, st);
}

}  // namespace spear
