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
// Tile: 128 tokens x 256 output rows per workgroup of 8 waves (2 x 4), each
// wave 64 x 64 = 2 x 2 tiles of the 32x32x16 bf16 MFMA.  The bf16 activations
// are the expensive operand to move (256 B per token per 128-column block
// against 64 B of codes per row), so the tile is wide in rows: 48 KB of
// global->LDS traffic per 8.4 MFLOP.  K advances in 128-column blocks (one
// scale group when g = 128) through a 3-stage LDS ring filled by buffer loads
// that write LDS directly (no register staging); the loads of block kb + 2
// are in flight while block kb is multiplied, and one barrier per block both
// publishes a stage and retires the oldest one.
//   x stage  128 tokens x 256 B; 16-byte piece p of token t is stored at
//            position p ^ (t & 15), so the fragment reads of 16 consecutive
//            tokens hit 16 different bank groups;
//   W stage  256 rows x 64 B of packed codes, piece p of row n at
//            p ^ ((n >> 2) & 3) for the same reason;
//   sums     the block sums of x of each token (as three bf16 parts);
// and, outside the ring, two slots of group metadata for 8 blocks at a time
// (each row's fp16 scales and its zero-point word), loaded with the first
// block of each 8: one lane per row and block cost 64 cache lines per load
// instruction, once per block, which held the loads back.
// A lane's weight operand for K step s is word 8*(lane/32) + s of its row,
// converted to 128 + c in natural column order; the matching activations are
// 16-byte piece 8*(lane/32) + s of its token.  Group-wise scales: each
// block's partial products P = sum (128 + c) x - (128 + z) sum_x restart
// from zero (the offset term is one extra matrix-core step) and are folded
// in with s * P.  Per-channel: one chain over all of K, corrected once at
// the end.
//
// Split K: when the output tiles alone are fewer than the compute units can
// take, each tile's K range is split; every split but the last to finish
// stores its partial tile at device scope and bumps the tile's counter, and
// the last sums all partials in split order (deterministic) before the
// epilogue.
#include "common.hpp"
#include "internal.hpp"

namespace spear {
namespace {

struct PrefillParams {
  const uint16_t* x;       // [T][K] bf16
  const uint32_t* wq;      // [N][K/8]
  const uint16_t* scales;  // [N][G]
  const uint32_t* zeros;   // [N][ZW], or the scales when has_z == 0 (never used then)
  const uint16_t* B;       // [N][r] bf16
  const uint16_t* wvhi;    // [T][r] bf16
  const uint16_t* wvlo;    // [T][r] bf16
  const uint32_t* sblk;    // [KB][Tp][2] block sums of x, bf16 (hi | mid << 16, lo)
  const float* stot;       // [T]
  float* part;             // [tiles][splits][8 waves][64 values][64 lanes] split partials
  int* ctr;                // counter words
  void* y;                 // [T][N] bf16 (fp32 with out_f32)
  int T, K, N, r, Tp, G, ZW, has_z, tiles_m, tiles_n, splits, out_f32;
};

constexpr int kXStage = kPrefillBM * 256;  // 32 KB
constexpr int kWStage = kPrefillBN * 64;   // 16 KB
constexpr int kSStage = kPrefillBM * 8;    // block sums of x [128 tokens][8 B]
constexpr int kStage = kXStage + kWStage + kSStage;
constexpr int kStages = 3;
// Group metadata by chunks of 8 blocks (one zero-point word's groups), two
// chunk slots after the ring: per row the 5 dwords from the even scale at or
// below its first (rows laid end to end, 20 dword loads of 64 lanes), then
// the zero-point word of each row.
constexpr int kChunkScales = kPrefillBN * 5 * 4;  // 5 KB
constexpr int kChunk = kChunkScales + kPrefillBN * 4;
constexpr int kChunkBase = kStages * kStage;
static_assert(kChunkBase + 2 * kChunk <= 160 * 1024, "LDS exceeds 160 KB");
// Loads into LDS each wave issues per block: 4 x, 2 W and, with group
// scales, a quarter of the block sums (waves w and w + 4 load the same
// quarter, so every wave's count is the same); per chunk of 8 blocks, 3 more
// (scales or zero-point words), issued first.
template <bool GROUPED>
constexpr int kLoadsPerBlock = GROUPED ? 7 : 6;
constexpr int kChunkLoadsPerWave = 3;
static_assert(kPrefillWaves == 8 && kPrefillBN == 256 && kPrefillBM == 128, "tile shape");

template <bool GROUPED>
__global__ __launch_bounds__(512, 1) void prefill_kernel(PrefillParams p) {
  warm_kernel_args<sizeof(PrefillParams)>();
  __shared__ __attribute__((aligned(16))) uint8_t smem[kChunkBase + 2 * kChunk];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const int wm = wave >> 2, wn = wave & 3;
  const int i32 = lane & 31, q = lane >> 5;

  // Workgroup -> (tile, split).  Splits of a tile are adjacent and tiles are
  // n-major, so a run of workgroups shares a W tile; runs are placed on one
  // XCD (workgroups are dealt to the 8 XCDs round-robin).
  const int total = p.tiles_m * p.tiles_n * p.splits;
  int idx = blockIdx.x;
  if ((total & 7) == 0) idx = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int tile = idx / p.splits, split = idx - tile * p.splits;
  const int tn = tile / p.tiles_m, tm = tile - tn * p.tiles_m;
  const int m0 = tm * kPrefillBM, n0 = tn * kPrefillBN;
  const int KB = p.K / kBlockK;
  const int kb0 = (int)((long long)KB * split / p.splits);
  const int kb1 = (int)((long long)KB * (split + 1) / p.splits);
  const int rows_m = min(kPrefillBM, p.T - m0), rows_n = min(kPrefillBN, p.N - n0);

  // Buffer views of this tile; rows past T or N read as zero.
  const u32x4 xr = sdesc(p.x + (size_t)m0 * p.K, (uint32_t)rows_m * p.K * 2);
  const u32x4 wr = sdesc(p.wq + (size_t)n0 * (p.K / 8), (uint32_t)rows_n * (p.K / 2));
  // Scales of the tile (n0 G is even, so the view starts on a dword; reads
  // past the tile's rows give zeros).
  const u32x4 sr = sdesc(p.scales + (size_t)n0 * p.G, (uint32_t)rows_n * p.G * 2);
  // Without zero-points the view is empty: its loads read zero words.
  const u32x4 zr = p.has_z ? sdesc(p.zeros + (size_t)n0 * p.ZW, (uint32_t)rows_n * p.ZW * 4)
                           : sdesc(p.scales, 0u);
  const u32x4 gr = sdesc(p.sblk, (uint32_t)KB * p.Tp * 8);
  const uint32_t lds0 = lds_addr(smem);

  // The loads of block kb into a stage; with `chunk`, first the group
  // metadata of the chunk kb / 8 into its slot.
  auto issue = [&](int kb, int stage, bool chunk) {
    if constexpr (GROUPED) {
      if (chunk) {  // uniform: every wave issues 3 loads
        const uint32_t C = lds0 + kChunkBase + ((kb >> 3) & 1) * kChunk;
        for (int k = 0; k < kChunkLoadsPerWave; ++k) {
          const int i = kChunkLoadsPerWave * wave + k;  // 0 .. 23
          if (i < 20) {  // scales: dword f of rows laid end to end
            const int f = 64 * i + lane, n = f / 5, d = f - 5 * n;
            const uint32_t e0 = (uint32_t)(n * p.G + (kb & ~7)) & ~1u;
            dma4(sr, C + 256 * i, e0 * 2 + 4 * (uint32_t)d);
          } else {  // zero-point words of rows 64 (i - 20) + lane
            const int n = 64 * (i - 20) + lane;
            dma4(zr, C + kChunkScales + 256 * (i - 20), (uint32_t)(n * p.ZW + (kb >> 3)) * 4);
          }
        }
      }
    }
    const uint32_t S = lds0 + stage * kStage;
    for (int j = 0; j < 4; ++j) {  // x: tokens 16 wave + 4 j .. + 3
      const int t = 16 * wave + 4 * j + (lane >> 4);
      const uint32_t gp = (uint32_t)((lane & 15) ^ (t & 15));
      dma16(xr, S + (16 * wave + 4 * j) * 256,
            (uint32_t)t * p.K * 2 + gp * 16 + (uint32_t)kb * 256);
    }
    for (int j = 0; j < 2; ++j) {  // W: rows 32 wave + 16 j .. + 15
      const int n = 32 * wave + 16 * j + (lane >> 2);
      const uint32_t gp = (uint32_t)((lane & 3) ^ ((n >> 2) & 3));
      dma16(wr, S + kXStage + (32 * wave + 16 * j) * 64,
            (uint32_t)n * (p.K / 2) + gp * 16 + (uint32_t)kb * 64);
    }
    if constexpr (GROUPED) {  // block sums of x, a quarter per wave (w and w + 4 alike)
      const int j = wave & 3;
      dma4(gr, S + kXStage + kWStage + 256 * j, (uint32_t)(kb * p.Tp + m0) * 8 + 256 * j + 4 * lane);
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

  // Fragment reads from a stage.  A lane's code words: row n of its 32-row
  // slice, 16-byte pieces 2q and 2q + 1 (K steps 0-3 and 4-7).
  auto read_w = [&](const uint8_t* W, u32x4 (&wd)[2][2]) {
    for (int ns = 0; ns < 2; ++ns) {
      const int n = wn * 64 + ns * 32 + i32;
      const int sw = (n >> 2) & 3;
      wd[ns][0] = *reinterpret_cast<const u32x4*>(W + n * 64 + ((2 * q) ^ sw) * 16);
      wd[ns][1] = *reinterpret_cast<const u32x4*>(W + n * 64 + ((2 * q + 1) ^ sw) * 16);
    }
  };
  auto read_x = [&](const uint8_t* X, int s, u32x4 (&xa)[2]) {
    for (int ms = 0; ms < 2; ++ms) {
      const int t = wm * 64 + ms * 32 + i32;
      xa[ms] = *reinterpret_cast<const u32x4*>(X + t * 256 + ((8 * q + s) ^ (t & 15)) * 16);
    }
  };
  auto step = [&](const u32x4 (&xa)[2], uint32_t w0, uint32_t w1) {
    const u32x4 wb0 = codes_to_bf16_offset_natural(w0);
    const u32x4 wb1 = codes_to_bf16_offset_natural(w1);
    for (int ms = 0; ms < 2; ++ms) {
      acc[ms][0] = mfma32x32x16(xa[ms], wb0, acc[ms][0]);
      acc[ms][1] = mfma32x32x16(xa[ms], wb1, acc[ms][1]);
    }
  };
  auto fold = [&](const float (&sc)[2]) {
    for (int ms = 0; ms < 2; ++ms)
      for (int ns = 0; ns < 2; ++ns)
        for (int v = 0; v < 16; ++v) tot[ms][ns][v] = fmaf(sc[ns], acc[ms][ns][v], tot[ms][ns][v]);
  };

  // K loop over the 3-stage ring.  At the top of iteration kb this wave's
  // loads of blocks kb and kb + 1 are in flight (7 each with group scales,
  // 6 without, after any chunk loads issued ahead of them); waiting until at
  // most that many remain completes block kb (and the chunk loads of kb + 1),
  // and the barrier makes every wave's part of it visible.  Past the barrier
  // every wave has finished reading block kb - 1, so its stage takes the
  // loads of block kb + 2 (issued by each wave once per iteration, before or
  // after its compute, see below).  Past the last
  // block the loads repeat block kb1 - 1 into the free stage, which keeps the
  // count of loads in flight the same in every iteration.
  //
  // The pipeline is rotated by one K step: the operands of block kb - 1's
  // last step (its activations and code words) and its scales are read
  // before the barrier and carried in registers, so that its last four
  // matrix-core steps and its scale fold run after the barrier, while the
  // first reads of block kb are in flight.
  const uint32_t zxor = p.has_z ? 0u : 0x88888888u;
  // lanes of the upper half hold K = 8..15 of the offset step: zero there
  // (a mask, not a branch, so the reads stay ahead of their waits)
  const uint32_t qmask = q == 0 ? 0xFFFFFFFFu : 0u;
  issue(kb0, 0, true);
  issue(min(kb0 + 1, kb1 - 1), 1, kb0 + 1 < kb1 && ((kb0 + 1) & 7) == 0);
  u32x4 xc[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};  // carried: x of step 7
  uint32_t wc[2] = {0u, 0u};                                     // carried: code words of step 7
  float scc[2] = {0.f, 0.f};                                     // carried: scales
  for (int kb = kb0; kb < kb1; ++kb) {
    const int i = kb - kb0;
    wait_vmcnt<kLoadsPerBlock<GROUPED>>();
    // lgkmcnt(0) through the builtin (0xC07F: vmcnt and expcnt at their
    // maxima), which the compiler's own wait insertion sees: the carried
    // step-7 operands then count as arrived.
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // Loads of block kb + 2: the second half of the waves issues them here,
    // the first half after this block's compute (below).  The two waves of
    // a SIMD compute a block at the same time and the first half gets the
    // SIMD first; its loads, issued when its compute is done, wait at the
    // memory pipeline while the second half still computes, and the second
    // half's own loads meet a shorter queue here.
    if (wave >= kPrefillWaves / 2)
      issue(min(kb + 2, kb1 - 1), (i + 2) % kStages, kb + 2 < kb1 && ((kb + 2) & 7) == 0);

    const uint8_t* X = smem + (i % kStages) * kStage;
    const uint8_t* W = X + kXStage;
    const uint8_t* M = W + kWStage;  // block sums
    const uint8_t* CH = smem + kChunkBase + ((kb >> 3) & 1) * kChunk;
    u32x4 wd[2][2];
    read_w(W, wd);
    float sc[2] = {0.f, 0.f};
    u32x4 xo[2], wo[2];
    if constexpr (GROUPED) {
      // Offset step: P starts at -(128 + z) * sum_x through one extra K = 16
      // matrix-core step whose only non-zero terms are the three bf16 parts
      // of sum_x (token side) against the exact bf16 value -(128 + z) (row
      // side); then P gathers the eight code steps and is folded with s.
      const uint32_t* Ms = reinterpret_cast<const uint32_t*>(CH);
      const uint32_t* Mz = reinterpret_cast<const uint32_t*>(CH + kChunkScales);
      for (int ms = 0; ms < 2; ++ms) {
        const int t = wm * 64 + ms * 32 + i32;
        const u32x2 sx = *reinterpret_cast<const u32x2*>(M + t * 8);
        xo[ms] = u32x4{sx.x & qmask, sx.y & qmask, 0u, 0u};
      }
      for (int ns = 0; ns < 2; ++ns) {
        const int n = wn * 64 + ns * 32 + i32;
        // scale of block kb: position (kb & 7) + (n G & 1) of the row's 5 dwords
        const uint32_t pos = (uint32_t)(kb & 7) + ((uint32_t)(n * p.G) & 1u);
        const uint32_t sword = Ms[5 * n + (pos >> 1)];
        const uint32_t sbits = (pos & 1u) ? (sword >> 16) : (sword & 0xFFFFu);
        sc[ns] = half_bits_to_f32((uint16_t)sbits);
        // without zero-points the word reads as zero and z = 8 comes from
        // the xor (one path, so no branch splits the read from its wait)
        const uint32_t z = ((Mz[n] ^ zxor) >> (4 * (kb & 7))) & 15u;
        const uint32_t mzb = 0xC300u | z;  // bf16 bits of -(128 + z)
        wo[ns] = u32x4{(mzb | (mzb << 16)) & qmask, mzb & qmask, 0u, 0u};
      }
    }
    u32x4 xa[2];
    read_x(X, 0, xa);

    // Block kb - 1: its last K step and its fold.
    if (i > 0) {
      step(xc, wc[0], wc[1]);
      if constexpr (GROUPED) fold(scc);
    }

    // Block kb: the offset step, then K steps 0-6; step 7's operands are
    // read here and carried.
    if constexpr (GROUPED) {
      f32x16 zero;
      for (int v = 0; v < 16; ++v) zero[v] = 0.f;
      for (int ms = 0; ms < 2; ++ms)
        for (int ns = 0; ns < 2; ++ns) acc[ms][ns] = mfma32x32x16(xo[ms], wo[ns], zero);
    }
#pragma unroll
    for (int s = 0; s < 7; ++s) {
      u32x4 xn[2];
      read_x(X, s + 1, xn);
      step(xa, wd[0][s >> 2][s & 3], wd[1][s >> 2][s & 3]);
      xa[0] = xn[0];
      xa[1] = xn[1];
    }
    xc[0] = xa[0];
    xc[1] = xa[1];
    wc[0] = wd[0][1][3];
    wc[1] = wd[1][1][3];
    scc[0] = sc[0];
    scc[1] = sc[1];
    if (wave < kPrefillWaves / 2)
      issue(min(kb + 2, kb1 - 1), (i + 2) % kStages, kb + 2 < kb1 && ((kb + 2) & 7) == 0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // The last block's last step and fold.
  step(xc, wc[0], wc[1]);
  if constexpr (GROUPED) fold(scc);

  if constexpr (!GROUPED) {
    for (int ms = 0; ms < 2; ++ms)
      for (int ns = 0; ns < 2; ++ns) tot[ms][ns] = acc[ms][ns];
  }

  // Split K: partial tiles meet at device scope; the last split sums them in
  // split order.  Each lane owns 64 values; value e of wave w lives at
  // part[((tile * splits + split) * 8 + w) * 4096 + e * 64 + lane].
  if (p.splits > 1) {
    const uint32_t tile_floats = kPrefillWaves * 4096;
    const rsrc_t pr = make_rsrc(p.part + (size_t)tile * p.splits * tile_floats,
                                (uint32_t)p.splits * tile_floats * 4);
    const uint32_t mine = (uint32_t)(wave * 4096 + lane) * 4;
    for (int ms = 0; ms < 2; ++ms)
      for (int ns = 0; ns < 2; ++ns)
        for (int v = 0; v < 16; ++v)
          bstore_dev(pr, mine + (uint32_t)((ms * 2 + ns) * 16 + v) * 256,
                     (uint32_t)split * tile_floats * 4, tot[ms][ns][v]);
    wait_vmem();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&p.ctr[kCtrTile + tile], 1) == p.splits - 1;
    __syncthreads();
    if (!s_last) return;
    if (tid == 0) store_dev(&p.ctr[kCtrTile + tile], 0);
    f32x16 sum[2][2];
    for (int ms = 0; ms < 2; ++ms)
      for (int ns = 0; ns < 2; ++ns)
        for (int v = 0; v < 16; ++v) sum[ms][ns][v] = 0.f;
    for (int sp = 0; sp < p.splits; ++sp) {
      if (sp == split) {
        for (int ms = 0; ms < 2; ++ms)
          for (int ns = 0; ns < 2; ++ns) sum[ms][ns] += tot[ms][ns];
      } else {
        for (int ms = 0; ms < 2; ++ms)
          for (int ns = 0; ns < 2; ++ns)
            for (int v = 0; v < 16; ++v)
              sum[ms][ns][v] += bload_dev(pr, mine + (uint32_t)((ms * 2 + ns) * 16 + v) * 256,
                                          (uint32_t)sp * tile_floats * 4);
      }
    }
    for (int ms = 0; ms < 2; ++ms)
      for (int ns = 0; ns < 2; ++ns) tot[ms][ns] = sum[ms][ns];
  }

  // Epilogue: scales (per-channel), then + alpha * v B^T, then one bf16 store.
  if constexpr (!GROUPED) {
    for (int ns = 0; ns < 2; ++ns) {
      const int n = n0 + wn * 64 + ns * 32 + i32;
      float sc = 0.f, mz = 0.f;
      if (n < p.N) {
        sc = half_bits_to_f32(p.scales[n]);
        const int z = p.has_z ? (int)(p.zeros[(size_t)n * p.ZW] & 15u) : 8;
        mz = -(float)(128 + z);
      }
      for (int ms = 0; ms < 2; ++ms)
        for (int v = 0; v < 16; ++v) {
          const int t = m0 + wm * 64 + ms * 32 + 8 * (v >> 2) + 4 * q + (v & 3);
          const float st = t < p.T ? p.stot[t] : 0.f;
          tot[ms][ns][v] = sc * fmaf(mz, st, tot[ms][ns][v]);
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
        if (t >= p.T) continue;
        if (p.out_f32) static_cast<float*>(p.y)[(size_t)t * p.N + n] = tot[ms][ns][v];
        else static_cast<uint16_t*>(p.y)[(size_t)t * p.N + n] = (uint16_t)f32_to_bf16_rne(tot[ms][ns][v]);
      }
    }
}

}  // namespace

hipError_t launch_prefill(const Shape& s, const LayerArgs& a, const WsPtrs& w, hipStream_t st) {
  const ProjPlan pp = plan_projection(s);
  const PrefillPlan pl = plan_prefill(s);
  PrefillParams p;
  p.x = static_cast<const uint16_t*>(a.x);
  p.wq = a.wq;
  p.scales = a.scales;
  p.has_z = a.zeros != nullptr;
  p.zeros = a.zeros ? a.zeros : reinterpret_cast<const uint32_t*>(a.scales);
  p.B = static_cast<const uint16_t*>(a.B);
  p.wvhi = w.wvhi;
  p.wvlo = w.wvlo;
  p.sblk = w.sblk;
  p.stot = w.stot;
  p.part = w.ypart;
  p.ctr = w.counters;
  p.y = a.y;
  p.out_f32 = a.out_f32 ? 1 : 0;
  p.T = s.T;
  p.K = s.K;
  p.N = s.N;
  p.r = s.r;
  p.Tp = pp.tiles * kProjTokens;
  p.G = s.K / s.g;
  p.ZW = (p.G + 7) / 8;
  p.tiles_m = pl.tiles_m;
  p.tiles_n = pl.tiles_n;
  p.splits = pl.splits;
  const int grid = p.tiles_m * p.tiles_n * p.splits;
  if (s.grouped)
    hipLaunchKernelGGL(prefill_kernel<true>, dim3(grid), dim3(64 * kPrefillWaves), 0, st, p);
  else
    hipLaunchKernelGGL(prefill_kernel<false>, dim3(grid), dim3(64 * kPrefillWaves), 0, st, p);
  return hipGetLastError();
}

}  // namespace spear
