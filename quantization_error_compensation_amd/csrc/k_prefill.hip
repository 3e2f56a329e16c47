// Prefill path (any token count; used above 32 tokens): matrix-core GEMM on
// exact integer codes with the compensator product fused into the epilogue.
//
// SPEAR summary, section 2.2 A: in the compute-bound prefill phase the
// compensator must not slow the GEMM down.  Here the rank-r projection and
// gate are computed once per token by the projection kernel (a small GEMM,
// about r/N of the work), and the back-projection alpha * B * v is a K = r
// matrix-core product accumulated into the same registers as the main GEMM
// before the single store of y.
//
// Tile: 128 tokens x 128 output rows per workgroup of 4 waves (2 x 2), each
// wave 64 x 64 = 2 x 2 tiles of the 32x32x16 bf16 MFMA.  K advances in
// 128-column blocks (one scale group when g = 128), double-buffered in LDS:
//   x tile   128 x 128 bf16, each 8-column block stored in the operand order
//            0,4,1,5,2,6,3,7 of the integer-code operands (row stride 272 B);
//   W tile   128 rows x 64 B of packed codes (row stride 80 B).
// A lane's weight operand for K step s is word 8*(lane/32) + s of its row;
// the matching activations are 8-column block 8*(lane/32) + s of its token.
// Group-wise scales: each block's partial products restart from zero and are
// folded in with s * (P - (128 + z) * sum_x).  Per-channel: one chain over
// all of K, corrected once at the end.
#include "common.hpp"
#include "internal.hpp"

namespace spear {
namespace {

struct PrefillParams {
  const uint16_t* x;       // [T][K] bf16
  const uint32_t* wq;      // [N][K/8]
  const uint16_t* scales;  // [N][G]
  const uint32_t* zeros;   // [N][ZW] or null
  const uint16_t* B;       // [N][r] bf16
  const uint16_t* wvhi;    // [T][r] bf16
  const uint16_t* wvlo;    // [T][r] bf16
  const float* sblk;       // [KB][Tp]
  const float* stot;       // [T]
  uint16_t* y;             // [T][N]
  int T, K, N, r, Tp, G, ZW, tiles_m, tiles_n;
};

constexpr int XS = 272;   // x tile row stride in LDS (bytes)
constexpr int WS = 80;    // W tile row stride in LDS (bytes)
constexpr int XTILE = kPrefillBM * XS;
constexpr int WTILE = kPrefillBN * WS;

template <bool GROUPED>
__global__ __launch_bounds__(256, 1) void prefill_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][XTILE];
  __shared__ __attribute__((aligned(16))) uint8_t ws[2][WTILE];
  __shared__ float gs[2][kPrefillBN];   // group scale per row
  __shared__ float gz[2][kPrefillBN];   // -(128 + z) per row
  __shared__ float gx[2][kPrefillBM];   // block sum of x per token

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int i32 = lane & 31, q = lane >> 5;

  // Tiles are n-major so that a run of workgroups shares a W tile; runs are
  // placed on one XCD (workgroups are dealt to the 8 XCDs round-robin).
  const int ntiles = p.tiles_m * p.tiles_n;
  int tile = blockIdx.x;
  if ((ntiles & 7) == 0) tile = (blockIdx.x & 7) * (ntiles >> 3) + (blockIdx.x >> 3);
  const int tn = tile / p.tiles_m, tm = tile % p.tiles_m;
  const int m0 = tm * kPrefillBM, n0 = tn * kPrefillBN;
  const int KB = p.K / kBlockK;
  const size_t rowWords = (size_t)p.K / 8;

  // Cooperative global -> register -> LDS copy of one K block.
  struct Regs {
    u32x4 x[8];
    u32x4 w[2];
    float s, z, sx;
  };
  auto gload = [&](int kb, Regs& R) {
    for (int c = 0; c < 8; ++c) {
      const int chunk = tid + 256 * c, row = chunk >> 4, b8 = chunk & 15;
      const int t = m0 + row;
      R.x[c] = t < p.T ? load16(p.x + (size_t)t * p.K + (size_t)kb * kBlockK + 8 * b8)
                       : u32x4{0, 0, 0, 0};
    }
    for (int c = 0; c < 2; ++c) {
      const int chunk = tid + 256 * c, row = chunk >> 2, part = chunk & 3;
      const int n = n0 + row;
      R.w[c] = n < p.N ? load16(p.wq + (size_t)n * rowWords + (size_t)kb * 16 + 4 * part)
                       : u32x4{0, 0, 0, 0};
    }
    if constexpr (GROUPED) {
      if (tid < kPrefillBN) {
        const int n = n0 + tid;
        if (n < p.N) {
          R.s = half_bits_to_f32(p.scales[(size_t)n * p.G + kb]);
          const int z = p.zeros ? (int)((p.zeros[(size_t)n * p.ZW + kb / 8] >> (4 * (kb & 7))) & 15u) : 8;
          R.z = -(float)(128 + z);
        } else {
          R.s = 0.f;
          R.z = 0.f;
        }
      } else {
        const int t = m0 + tid - kPrefillBN;
        R.sx = t < p.T ? p.sblk[(size_t)kb * p.Tp + t] : 0.f;
      }
    }
  };
  auto sstore = [&](int stg, const Regs& R) {
    for (int c = 0; c < 8; ++c) {
      const int chunk = tid + 256 * c, row = chunk >> 4, b8 = chunk & 15;
      *reinterpret_cast<u32x4*>(&xs[stg][row * XS + b8 * 16]) = x_permute8(R.x[c]);
    }
    for (int c = 0; c < 2; ++c) {
      const int chunk = tid + 256 * c, row = chunk >> 2, part = chunk & 3;
      *reinterpret_cast<u32x4*>(&ws[stg][row * WS + part * 16]) = R.w[c];
    }
    if constexpr (GROUPED) {
      if (tid < kPrefillBN) {
        gs[stg][tid] = R.s;
        gz[stg][tid] = R.z;
      } else {
        gx[stg][tid - kPrefillBN] = R.sx;
      }
    }
  };

  f32x16 acc[2][2];
  f32x16 tot[2][2];
  for (int a = 0; a < 2; ++a)
    for (int b = 0; b < 2; ++b)
      for (int v = 0; v < 16; ++v) {
        acc[a][b][v] = 0.f;
        tot[a][b][v] = 0.f;
      }

  auto compute = [&](int stg) {
    u32x4 wd[2][2];
    for (int ns = 0; ns < 2; ++ns) {
      const int row = wn * 64 + ns * 32 + i32;
      wd[ns][0] = *reinterpret_cast<const u32x4*>(&ws[stg][row * WS + q * 32]);
      wd[ns][1] = *reinterpret_cast<const u32x4*>(&ws[stg][row * WS + q * 32 + 16]);
    }
    for (int s = 0; s < 8; ++s) {
      u32x4 xa[2], wb[2];
      for (int ms = 0; ms < 2; ++ms) {
        const int row = wm * 64 + ms * 32 + i32;
        xa[ms] = *reinterpret_cast<const u32x4*>(&xs[stg][row * XS + (8 * q + s) * 16]);
      }
      for (int ns = 0; ns < 2; ++ns) {
        const u32x4 d = wd[ns][s >> 2];
        const uint32_t word = (s & 3) == 0 ? d.x : (s & 3) == 1 ? d.y : (s & 3) == 2 ? d.z : d.w;
        wb[ns] = codes_to_bf16_offset(word);
      }
      for (int ms = 0; ms < 2; ++ms)
        for (int ns = 0; ns < 2; ++ns) {
          if (GROUPED && s == 0) {
            f32x16 zero;
            for (int v = 0; v < 16; ++v) zero[v] = 0.f;
            acc[ms][ns] = mfma32x32x16(xa[ms], wb[ns], zero);
          } else {
            acc[ms][ns] = mfma32x32x16(xa[ms], wb[ns], acc[ms][ns]);
          }
        }
    }
    if constexpr (GROUPED) {
      for (int ns = 0; ns < 2; ++ns) {
        const int nr = wn * 64 + ns * 32 + i32;
        const float sc = gs[stg][nr], mz = gz[stg][nr];
        for (int ms = 0; ms < 2; ++ms)
          for (int v = 0; v < 16; ++v) {
            const int tr = wm * 64 + ms * 32 + 8 * (v >> 2) + 4 * q + (v & 3);
            tot[ms][ns][v] = fmaf(sc, fmaf(mz, gx[stg][tr], acc[ms][ns][v]), tot[ms][ns][v]);
          }
      }
    }
  };

  // Main K loop: block kb+1 is loaded into registers while kb computes.
  {
    Regs R;
    gload(0, R);
    sstore(0, R);
  }
  __syncthreads();
  for (int kb = 0; kb < KB; ++kb) {
    const int cur = kb & 1;
    Regs R;
    const bool more = kb + 1 < KB;
    if (more) gload(kb + 1, R);
    compute(cur);
    if (more) sstore(cur ^ 1, R);
    __syncthreads();
  }

  // Epilogue: scales (per-channel), then + alpha * v B^T, then one bf16 store.
  if constexpr (!GROUPED) {
    for (int ns = 0; ns < 2; ++ns) {
      const int n = n0 + wn * 64 + ns * 32 + i32;
      float sc = 0.f, mz = 0.f;
      if (n < p.N) {
        sc = half_bits_to_f32(p.scales[n]);
        const int z = p.zeros ? (int)(p.zeros[(size_t)n * p.ZW] & 15u) : 8;
        mz = -(float)(128 + z);
      }
      for (int ms = 0; ms < 2; ++ms)
        for (int v = 0; v < 16; ++v) {
          const int t = m0 + wm * 64 + ms * 32 + 8 * (v >> 2) + 4 * q + (v & 3);
          const float st = t < p.T ? p.stot[t] : 0.f;
          tot[ms][ns][v] = sc * fmaf(mz, st, acc[ms][ns][v]);
        }
    }
  }
  if (p.r > 0) {
    for (int js = 0; js < p.r / 16; ++js) {
      u32x4 vh[2], vl[2], bm[2];
      for (int ms = 0; ms < 2; ++ms) {
        const int t = m0 + wm * 64 + ms * 32 + i32;
        const size_t off = (size_t)t * p.r + 16 * js + 8 * q;
        vh[ms] = t < p.T ? load16(p.wvhi + off) : u32x4{0, 0, 0, 0};
        vl[ms] = t < p.T ? load16(p.wvlo + off) : u32x4{0, 0, 0, 0};
      }
      for (int ns = 0; ns < 2; ++ns) {
        const int n = n0 + wn * 64 + ns * 32 + i32;
        bm[ns] = n < p.N ? load16(p.B + (size_t)n * p.r + 16 * js + 8 * q) : u32x4{0, 0, 0, 0};
      }
      for (int ms = 0; ms < 2; ++ms)
        for (int ns = 0; ns < 2; ++ns) {
          tot[ms][ns] = mfma32x32x16(vh[ms], bm[ns], tot[ms][ns]);
          tot[ms][ns] = mfma32x32x16(vl[ms], bm[ns], tot[ms][ns]);
        }
    }
  }
  for (int ms = 0; ms < 2; ++ms)
    for (int ns = 0; ns < 2; ++ns) {
      const int n = n0 + wn * 64 + ns * 32 + i32;
      if (n >= p.N) continue;
      for (int v = 0; v < 16; ++v) {
        const int t = m0 + wm * 64 + ms * 32 + 8 * (v >> 2) + 4 * q + (v & 3);
        if (t < p.T) p.y[(size_t)t * p.N + n] = (uint16_t)f32_to_bf16_rne(tot[ms][ns][v]);
      }
    }
}

}  // namespace

hipError_t launch_prefill(const Shape& s, const LayerArgs& a, const WsPtrs& w, hipStream_t st) {
  const ProjPlan pp = plan_projection(s);
  PrefillParams p;
  p.x = static_cast<const uint16_t*>(a.x);
  p.wq = a.wq;
  p.scales = a.scales;
  p.zeros = a.zeros;
  p.B = static_cast<const uint16_t*>(a.B);
  p.wvhi = w.wvhi;
  p.wvlo = w.wvlo;
  p.sblk = w.sblk;
  p.stot = w.stot;
  p.y = static_cast<uint16_t*>(a.y);
  p.T = s.T;
  p.K = s.K;
  p.N = s.N;
  p.r = s.r;
  p.Tp = pp.tiles * kProjTokens;
  p.G = s.K / s.g;
  p.ZW = (p.G + 7) / 8;
  p.tiles_m = (s.T + kPrefillBM - 1) / kPrefillBM;
  p.tiles_n = (s.N + kPrefillBN - 1) / kPrefillBN;
  const int grid = p.tiles_m * p.tiles_n;
  if (s.grouped)
    hipLaunchKernelGGL(prefill_kernel<true>, dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(prefill_kernel<false>, dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace spear
