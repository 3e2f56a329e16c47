// Rank-r projection and gate of the error compensator for the prefill path.
//
// SPEAR summary, section 2.1 A (input-adaptive error compensators): the
// compensator projects the activation x into a low-rank space with A and
// gates each token's projection.  For a prefill batch this is a small GEMM
// (r/N of the main one), computed once per token:
//     u[t,j]  = sum_k A[j,k] x[t,k]                   (matrix cores, fp32 acc)
//     wv[t,j] = alpha * sigmoid(g[j] u[t,j] + b[j]) * u[t,j]
// together with the per-128-column sums of x (as exact bf16 triples), which
// the prefill GEMM uses to remove the +128 offset of its integer-code
// operands, and whole-row sums.
//
// projection_kernel: one workgroup per (64-token tile, K split), each wave
// 16 of the tokens against every rank; the split's partial u (and row sum)
// goes to the workspace.  finish_kernel: one thread per (token, j)
// sums the split partials in split order (deterministic), applies the gate
// and writes alpha * v in fp32 and as a bf16 high/low pair.  With the
// bottleneck-MLP gate (SPEAR summary, section 2.1 A), which needs every rank
// of a token, finish_mlp_kernel does the same with one workgroup per token:
//     h[k] = relu(b1[k] + sum_i W1[k,i] u[i]),
//     wv[j] = alpha * sigmoid(b2[j] + sum_k W2[j,k] h[k]) * u[j].
#include "common.hpp"
#include "internal.hpp"

namespace spear {
namespace {

struct ProjParams {
  const uint16_t* x;   // [T][K] bf16
  const uint16_t* A;   // [r][K] bf16
  const float* gv;     // [r]
  const float* bv;     // [r]
  int gh;              // bottleneck-MLP gate width (0: elementwise gate gv, bv)
  const float* w1;     // [gh][r]
  const float* b1;     // [gh]
  const float* w2;     // [r][gh]
  const float* b2;     // [r]
  float alpha;
  float* upart;        // [splits][T][r + 1]
  uint32_t* sblk;      // [KB][Tp][2]: block sums of x as bf16 (hi | mid << 16, lo)
  float* stot;         // [T]
  float* wv32;         // [T][r]
  uint16_t* wvhi;      // [T][r]
  uint16_t* wvlo;      // [T][r]
  int T, K, r, Tp, splits, tiles;
};

// The x tile (kProjTokens tokens) and all r rows of A for one 128-column
// block go to LDS by direct buffer-to-LDS loads, 16 consecutive lanes
// reading one 256-byte row (a load whose consecutive lanes read different
// rows costs the address unit a cache-line lookup per lane group); 16-byte
// piece e of row t sits at position e ^ (t % 16), so the fragment reads (one
// lane per row) spread over the banks.  Two stages: the next block's loads
// are issued after the barrier that retires the stage, before this block is
// multiplied.  Wave w takes tokens 16 w .. + 15 of the tile against every
// rank, and their block sums (a product with a tile of ones).
template <int RTX>  // RTX = r / 16 rank tiles
__global__ __launch_bounds__(256, 1) void projection_kernel(ProjParams p) {
  warm_kernel_args<sizeof(ProjParams)>();
  static_assert(kProjTokens == 64, "four waves of 16 tokens");
  constexpr int XB = kProjTokens * 256;  // x stage bytes
  constexpr int AB = 16 * RTX * 256;     // A stage bytes
  constexpr int SB = XB + AB;
  constexpr int RA = RTX > 0 ? RTX : 1;  // array extent (rank 0 still sums x)
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * SB];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int q = lane >> 4, c16 = lane & 15;
  // Workgroup -> (tile, split), split-major: the tiles of one K split are
  // adjacent, and runs of adjacent workgroups are placed on one XCD
  // (workgroups are dealt to the 8 XCDs round-robin), so each XCD fetches
  // only its splits' columns of A into its L2 instead of all of A.
  const int total = p.tiles * p.splits;
  int idx = blockIdx.x;
  if ((total & 7) == 0) idx = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int split = idx / p.tiles, tile = idx - split * p.tiles;
  const int KB = p.K / kBlockK;
  const int kb0 = (int)((long long)KB * split / p.splits);
  const int kb1 = (int)((long long)KB * (split + 1) / p.splits);
  const int t0 = tile * kProjTokens;
  const int rows_t = min(kProjTokens, p.T - t0);
  // views: token rows past T and rank rows past r read as zero
  const u32x4 xr = sdesc(p.x + (size_t)t0 * p.K, (uint32_t)rows_t * p.K * 2);
  const u32x4 ar = sdesc(p.A, (uint32_t)p.r * p.K * 2);
  const uint32_t lds0 = lds_addr(smem);

  // Loads per wave and block: 4 of x (4 tokens x 256 B each) and RTX of A.
  auto issue = [&](int kb, int stage) {
    const uint32_t S = lds0 + stage * SB;
    for (int j = 0; j < 4; ++j) {
      const int g = 4 * wave + j, t = 4 * g + (lane >> 4);
      const uint32_t e = (uint32_t)((lane & 15) ^ (t & 15));
      dma16(xr, S + g * 1024, (uint32_t)t * p.K * 2 + e * 16 + (uint32_t)kb * 256);
    }
    for (int k = 0; k < RTX; ++k) {
      const int g = RTX * wave + k, row = 4 * g + (lane >> 4);
      const uint32_t e = (uint32_t)((lane & 15) ^ (row & 15));
      dma16(ar, S + XB + g * 1024, (uint32_t)row * p.K * 2 + e * 16 + (uint32_t)kb * 256);
    }
  };

  f32x4 u[RA];
  f32x4 ssum = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int rt = 0; rt < RTX; ++rt) u[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 ones = {kBf16One, kBf16One, kBf16One, kBf16One};
  const int tl = 16 * wave + c16;  // this lane's token row in the tile

  issue(kb0, 0);
  for (int kb = kb0; kb < kb1; ++kb) {
    const int i = kb - kb0;
    // this block's loads are done (the two block-sum stores of the previous
    // block, issued after them, may still be in flight), then every wave's
    // are, and every wave is done with the other stage
    if (i == 0) wait_vmcnt<0>();
    else wait_vmcnt<2>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kb + 1 < kb1) issue(kb + 1, (i + 1) & 1);
    const uint8_t* X = smem + (i & 1) * SB;
    const uint8_t* Am = X + XB;
    f32x4 sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {  // K step s: piece 4 s + q of each row
      const int pc = 4 * s + q;
      const u32x4 xf = *reinterpret_cast<const u32x4*>(X + tl * 256 + ((pc ^ (tl & 15)) * 16));
      sb = mfma16x16x32(xf, ones, sb);
      for (int rt = 0; rt < RTX; ++rt) {
        const int j = 16 * rt + c16;
        const u32x4 af = *reinterpret_cast<const u32x4*>(Am + j * 256 + ((pc ^ (j & 15)) * 16));
        u[rt] = mfma16x16x32(xf, af, u[rt]);
      }
    }
    ssum += sb;
    // every column of the ones-product holds the row sum; column 0 stores
    // it as three bf16 parts hi + mid + lo that add up to the fp32 sum
    // exactly (the prefill GEMM feeds them to the matrix cores).  Two
    // stores per block in every wave (lanes of other columns masked).
    {
      const int t = t0 + 16 * wave + 4 * q;
      u32x4 tw[2];
      for (int v = 0; v < 4; ++v) {
        const float sv = t + v < p.T ? sb[v] : 0.f;
        const uint32_t hi = f32_to_bf16_rne(sv);
        const float r1 = sv - __uint_as_float(hi << 16);
        const uint32_t mid = f32_to_bf16_rne(r1);
        const uint32_t lo = f32_to_bf16_rne(r1 - __uint_as_float(mid << 16));
        tw[v >> 1][2 * (v & 1)] = hi | (mid << 16);
        tw[v >> 1][2 * (v & 1) + 1] = lo;
      }
      if (c16 == 0) {
        uint32_t* dst = p.sblk + ((size_t)kb * p.Tp + t) * 2;
        *reinterpret_cast<u32x4*>(dst) = tw[0];
        *reinterpret_cast<u32x4*>(dst + 4) = tw[1];
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // This split's partial u (and row sums): lane holds tokens 4 q + v of the
  // wave's 16 against rank 16 rt + c16.
  const int R1 = p.r + 1;
  for (int v = 0; v < 4; ++v) {
    const int t = t0 + 16 * wave + 4 * q + v;
    if (t >= p.T) continue;
    float* dst = p.upart + ((size_t)split * p.T + t) * R1;
    for (int rt = 0; rt < RTX; ++rt) dst[16 * rt + c16] = u[rt][v];
    if (c16 == 0) dst[p.r] = ssum[v];
  }
}

__global__ __launch_bounds__(256) void finish_kernel(ProjParams p) {
  warm_kernel_args<sizeof(ProjParams)>();
  const int R1 = p.r + 1;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= p.T * R1) return;
  const int t = e / R1, j = e % R1;
  float acc = 0.f;
#pragma unroll 8
  for (int s = 0; s < p.splits; ++s) acc += p.upart[((size_t)s * p.T + t) * R1 + j];
  if (j == p.r) {
    p.stot[t] = acc;
    return;
  }
  const float gate = sigmoidf_safe(fmaf(p.gv[j], acc, p.bv[j]));
  const float wv = p.alpha * (gate * acc);
  p.wv32[(size_t)t * p.r + j] = wv;
  const uint32_t hi = f32_to_bf16_rne(wv);
  const uint32_t lo = f32_to_bf16_rne(wv - __uint_as_float(hi << 16));
  p.wvhi[(size_t)t * p.r + j] = (uint16_t)hi;
  p.wvlo[(size_t)t * p.r + j] = (uint16_t)lo;
}

template <int RTX>
hipError_t launch_rtx(const ProjParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL(projection_kernel<RTX>, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

// One workgroup per token (r <= 128 < 129 threads' worth of ranks).
__global__ __launch_bounds__(128) void finish_mlp_kernel(ProjParams p) {
  __shared__ float su[128], sh[128];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int R1 = p.r + 1;
  for (int j = tid; j < R1; j += 128) {
    float acc = 0.f;
    for (int s = 0; s < p.splits; ++s) acc += p.upart[((size_t)s * p.T + t) * R1 + j];
    if (j == p.r) p.stot[t] = acc;
    else su[j] = acc;
  }
  __syncthreads();
  for (int k = tid; k < p.gh; k += 128) {
    float a = p.b1[k];
    for (int i = 0; i < p.r; ++i) a = fmaf(p.w1[k * p.r + i], su[i], a);
    sh[k] = fmaxf(a, 0.f);
  }
  __syncthreads();
  for (int j = tid; j < p.r; j += 128) {
    float a = p.b2[j];
    for (int k = 0; k < p.gh; ++k) a = fmaf(p.w2[j * p.gh + k], sh[k], a);
    const float wv = p.alpha * (sigmoidf_safe(a) * su[j]);
    p.wv32[(size_t)t * p.r + j] = wv;
    const uint32_t hi = f32_to_bf16_rne(wv);
    const uint32_t lo = f32_to_bf16_rne(wv - __uint_as_float(hi << 16));
    p.wvhi[(size_t)t * p.r + j] = (uint16_t)hi;
    p.wvlo[(size_t)t * p.r + j] = (uint16_t)lo;
  }
}

}  // namespace

// SERQ's correction operand for the prefill epilogue (SERQ summary: one extra
// product with the salient activations, no intermediate quantization):
// wvhi[t][j] = x[t][s0 + j] (already bf16), wvlo = 0.
__global__ __launch_bounds__(256) void serq_operand_kernel(const uint16_t* x, int K, int s0, int T,
                                                           int r, uint16_t* wvhi, uint16_t* wvlo) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= T * r) return;
  const int t = e / r, j = e - t * r;
  wvhi[e] = x[(size_t)t * K + s0 + j];
  wvlo[e] = 0;
}

hipError_t launch_serq_operand(const Shape& s, const LayerArgs& a, const WsPtrs& w,
                               hipStream_t st) {
  const int elems = s.T * s.r;
  hipLaunchKernelGGL(serq_operand_kernel, dim3((elems + 255) / 256), dim3(256), 0, st,
                     static_cast<const uint16_t*>(a.x), s.K, a.s0, s.T, s.r, w.wvhi, w.wvlo);
  return hipGetLastError();
}

hipError_t launch_projection(const Shape& s, const LayerArgs& a, const WsPtrs& w,
                             hipStream_t st) {
  const ProjPlan pl = plan_projection(s);
  ProjParams p;
  p.x = static_cast<const uint16_t*>(a.x);
  p.A = static_cast<const uint16_t*>(a.A);
  p.gv = a.gv;
  p.bv = a.bv;
  p.gh = a.gh;
  p.w1 = a.w1;
  p.b1 = a.b1;
  p.w2 = a.w2;
  p.b2 = a.b2;
  p.alpha = a.alpha;
  p.upart = w.upart;
  p.sblk = w.sblk;
  p.stot = w.stot;
  p.wv32 = w.wv32;
  p.wvhi = w.wvhi;
  p.wvlo = w.wvlo;
  p.T = s.T;
  p.K = s.K;
  p.r = s.r;
  p.Tp = pl.tiles * kProjTokens;
  p.splits = pl.splits;
  p.tiles = pl.tiles;
  const dim3 grid(pl.tiles * pl.splits);
  hipError_t e;
  switch (s.r / 16) {
    case 0: e = launch_rtx<0>(p, grid, st); break;
    case 1: e = launch_rtx<1>(p, grid, st); break;
    case 2: e = launch_rtx<2>(p, grid, st); break;
    case 3: e = launch_rtx<3>(p, grid, st); break;
    case 4: e = launch_rtx<4>(p, grid, st); break;
    case 5: e = launch_rtx<5>(p, grid, st); break;
    case 6: e = launch_rtx<6>(p, grid, st); break;
    case 7: e = launch_rtx<7>(p, grid, st); break;
    case 8: e = launch_rtx<8>(p, grid, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if (a.gh > 0 && s.r > 0) {
    hipLaunchKernelGGL(finish_mlp_kernel, dim3(s.T), dim3(128), 0, st, p);
    return hipGetLastError();
  }
  const int elems = s.T * (s.r + 1);
  hipLaunchKernelGGL(finish_kernel, dim3((elems + 255) / 256), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace spear
