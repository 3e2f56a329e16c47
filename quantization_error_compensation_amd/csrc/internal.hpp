// Host-side plan of one call: work decomposition and workspace layout, shared
// by the entry points (api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "partition.hpp"

namespace spear {

constexpr int kBlockK = 128;          // K block: one scale group (g = 128) or a slice of a row
constexpr int kDecodeWaves = 8;                     // waves per decode workgroup, 16 rows each
constexpr int kDecodeBandRows = 16 * kDecodeWaves;  // output rows per decode row band
constexpr int kDecodeOccupancy = 1;                 // decode workgroups per compute unit
constexpr int kProjTokens = 64;       // tokens per projection workgroup (prefill path)
constexpr int kPrefillBM = 128;       // tokens per prefill tile
constexpr int kPrefillBN = 256;       // output rows per prefill tile
constexpr int kPrefillWaves = 8;      // waves per prefill workgroup (2 x 4 of 64 x 64)
constexpr int kPrefillTarget = 256;   // split K until a call has at least this many workgroups
constexpr int kCounterSlots = 4096;   // int32 words at the head of the workspace
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;  // the library's own scratch per device

// Decode counter words (all zero between calls).
constexpr int kCtrRankDone = 1;  // rank bands whose gated projection is published
constexpr int kCtrExit = 2;      // decode workgroups that have finished
constexpr int kCtrError = 3;     // error bits (SPEAR_EC_WS_*), read and cleared by the host
constexpr int kCtrGateDone = 4;  // MLP gate: 1 once alpha * v of every rank is published
constexpr int kCtrBand = 64;       // [64, 64 + bands): arrivals per band (rank bands first)
constexpr int kCtrTile = 64;       // [64, 64 + tiles): prefill split-K arrivals per output tile
constexpr int kMaxSlots = 256;     // bound on decode workgroups (one per compute unit of gfx950)

struct Shape {
  int K, N, r, g, T;
  bool grouped;  // g == 128 (per-group scales); otherwise g == K
  bool zeros;
  bool serq = false;  // SERQ call: r salient channels of x, no projection (no rank bands)
  int KB() const { return K / kBlockK; }
};

// Work split of the rank-r projection (prefill path) for T tokens.
struct ProjPlan {
  int tiles;   // token tiles of kProjTokens
  int splits;  // K splits
};

// Work split of the fused decode kernel (rank units spread over the first
// workgroups, stream-K over the row units; partition.hpp).
struct DecodePlan {
  int bands;         // output bands of kDecodeBandRows rows
  int rank_bands;    // 64-rank bands of A
  DecodeSplit split;
  int workgroups;    // persistent workgroups (split.P)
  int slots;         // partial-sum slots the workspace holds (for any slots <= kMaxSlots)
};

// Work split of the prefill GEMM: output tiles of kPrefillBM x kPrefillBN,
// each split over `splits` K ranges when the tiles alone would leave compute
// units idle (the last of a tile's splits to finish sums them in split order).
struct PrefillPlan {
  int tiles_m, tiles_n, splits;
  size_t partial_floats;  // workspace floats for split partials (0 if splits == 1)
};

ProjPlan plan_projection(const Shape& s);
PrefillPlan plan_prefill(const Shape& s);
// slots: workgroups the device keeps resident (one per CU); sizing uses kMaxSlots.
DecodePlan plan_decode(const Shape& s, int slots);

// Byte offsets of the workspace regions for one call.
struct Workspace {
  size_t counters, wv32, wvhi, wvlo, sblk, stot, upart, ypart, total;
};
Workspace layout(const Shape& s, bool decode);

// Pointers into a caller workspace.
struct WsPtrs {
  int* counters;
  float* wv32;     // [T][r]      alpha * gated projection
  uint16_t* wvhi;  // [T][r]      bf16 high part of alpha * v (prefill)
  uint16_t* wvlo;  // [T][r]      bf16 remainder (prefill)
  uint32_t* sblk;  // [KB][Tp][2] sum of x over each 128-column block as bf16 hi|mid, lo (prefill)
  float* stot;     // [T]         sum of x over the whole row (prefill)
  float* upart;    // projection partials: prefill [splits][T][r+1], decode [splits][T][r]
  float* ypart;    // decode: [slots][128 columns][T4] (T4: T rounded up to 4); prefill: split-K tile partials
};
WsPtrs carve(void* base, const Workspace& w);

struct LayerArgs {
  const void* x;
  const uint32_t* wq;
  const uint16_t* scales;
  const uint32_t* zeros;
  const void* A;
  const void* B;
  const float* gv;
  const float* bv;
  // bottleneck-MLP gate (gh > 0): gamma = sigmoid(W2 relu(W1 u + b1) + b2),
  // W1 [gh][r], b1 [gh], W2 [r][gh], b2 [r]; gh == 0: elementwise gv, bv
  int gh;
  const float* w1;
  const float* b1;
  const float* w2;
  const float* b2;
  float alpha;
  void* y;
  // SERQ (s0 >= 0): the correction is x[:, s0 .. s0 + r) R^T with R in B's
  // place (no A, no gate, alpha 1)
  int s0 = -1;
  // y is fp32 (the accumulation stored unrounded) instead of bf16
  bool out_f32 = false;
};

hipError_t launch_projection(const Shape& s, const LayerArgs& a, const WsPtrs& w,
                             hipStream_t st);
hipError_t launch_decode(const Shape& s, const LayerArgs& a, const WsPtrs& w, hipStream_t st);
hipError_t launch_prefill(const Shape& s, const LayerArgs& a, const WsPtrs& w, hipStream_t st);
hipError_t launch_serq_operand(const Shape& s, const LayerArgs& a, const WsPtrs& w, hipStream_t st);
// Device address of the library's static scratch on the current device
// (looked up and its counter words cleared on the device's first use).
hipError_t static_scratch(void** out, hipStream_t st);
hipError_t launch_quantize(int N, int K, int g, bool asym, bool per_tensor, const float* w,
                           uint32_t* wq, uint16_t* scales, uint32_t* zeros, hipStream_t st);
hipError_t launch_dequant(int N, int K, int g, const uint32_t* wq, const uint16_t* scales,
                          const uint32_t* zeros, float* out, hipStream_t st);

}  // namespace spear
