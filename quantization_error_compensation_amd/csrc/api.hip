// C ABI of libspear_ec: argument validation, work planning, workspace
// layout and the phase-aware dispatcher.  Every check runs before any HIP
// call; no C++ exception leaves this file.
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "spear_ec.h"
#include "internal.hpp"

namespace spear {

static thread_local char g_last_error[256] = "";

static int fail(int code, const char* msg) {
  snprintf(g_last_error, sizeof(g_last_error), "%s", msg);
  return code;
}

ProjPlan plan_projection(const Shape& s) {
  ProjPlan pl;
  pl.tiles = (s.T + kProjTokens - 1) / kProjTokens;
  const int KB = s.KB();
  const int want = (512 + pl.tiles - 1) / std::max(pl.tiles, 1);
  pl.splits = std::max(1, std::min(want, KB / 4));
  return pl;
}

DecodePlan plan_decode(const Shape& s, int slots) {
  DecodePlan pl;
  const int KB = s.KB();
  pl.bands = (s.N + kDecodeBandRows - 1) / kDecodeBandRows;
  pl.rank_bands = s.serq ? 0 : (s.r + 63) / 64;  // SERQ takes x's channels, no projection
  slots = std::min(std::max(slots, 1), kMaxSlots);
  // Rank workgroups also stream rows ("shared" mode) only with group-wise
  // scales, where the device tests run that mode (one and two rank bands);
  // per-channel layers keep them apart ("separate" mode).
  const bool shared = s.grouped;
  pl.split = make_split(KB, pl.rank_bands, pl.bands, slots, shared);
  pl.workgroups = pl.split.P;
  pl.slots = split_workspace_slots(KB, pl.rank_bands, pl.bands, kMaxSlots, shared);
  return pl;
}

static PrefillPlan prefill_plan_for(const Shape& s, int tiles_m) {
  PrefillPlan pl;
  pl.tiles_m = tiles_m;
  pl.tiles_n = (s.N + kPrefillBN - 1) / kPrefillBN;
  const int tiles = pl.tiles_m * pl.tiles_n;
  pl.splits = 1;
  if (tiles < kPrefillTarget) {
    const int want = (kPrefillTarget + tiles - 1) / tiles;
    pl.splits = std::max(1, std::min({8, want, s.KB() / 4}));
  }
  pl.partial_floats = pl.splits > 1
                          ? (size_t)tiles * pl.splits * kPrefillWaves * 64 * 64
                          : 0;
  return pl;
}

PrefillPlan plan_prefill(const Shape& s) {
  return prefill_plan_for(s, (s.T + kPrefillBM - 1) / kPrefillBM);
}

// Largest split-partial area of any token count up to T, so that a workspace
// sized for T tokens serves every smaller call too.
static size_t prefill_partials_bound(const Shape& s) {
  size_t m = 0;
  const int tm_max = (s.T + kPrefillBM - 1) / kPrefillBM;
  for (int tm = 1; tm <= tm_max; ++tm) m = std::max(m, prefill_plan_for(s, tm).partial_floats);
  return m;
}

static size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

Workspace layout(const Shape& s, bool decode) {
  const size_t T = (size_t)s.T, r = (size_t)s.r;
  Workspace w;
  size_t o = 0;
  w.counters = o; o = up256(o + sizeof(int) * kCounterSlots);
  w.wv32 = o;     o = up256(o + sizeof(float) * T * r);
  if (decode) {
    const DecodePlan dp = plan_decode(s, kMaxSlots);
    w.wvhi = w.wvlo = w.sblk = w.stot = w.upart = o;
    w.ypart = o;
    const size_t T4 = (T + 3) & ~(size_t)3;  // tokens rounded up to a multiple of 4
    o = up256(o + sizeof(float) * (size_t)dp.slots * T4 * kDecodeBandRows);
  } else {
    const ProjPlan pp = plan_projection(s);
    const size_t Tp = (size_t)pp.tiles * kProjTokens;
    w.wvhi = o;   o = up256(o + 2 * T * r);
    w.wvlo = o;   o = up256(o + 2 * T * r);
    w.sblk = o;   o = up256(o + 8 * (size_t)s.KB() * Tp);
    w.stot = o;   o = up256(o + sizeof(float) * Tp);
    // splits * T <= min(max(1, KB/4) * T, 16384 + T): a bound that grows with
    // T, so sizing for the largest token count covers every smaller one.
    const size_t kb4 = (size_t)std::max(1, s.KB() / 4);
    const size_t parts = std::min(kb4 * T, (size_t)16384 + T);
    (void)pp;
    w.upart = o;  o = up256(o + sizeof(float) * parts * (r + 1));
    w.ypart = o;  o = up256(o + sizeof(float) * prefill_partials_bound(s));
  }
  w.total = o;
  return w;
}

WsPtrs carve(void* base, const Workspace& w) {
  char* b = static_cast<char*>(base);
  WsPtrs p;
  p.counters = reinterpret_cast<int*>(b + w.counters);
  p.wv32 = reinterpret_cast<float*>(b + w.wv32);
  p.wvhi = reinterpret_cast<uint16_t*>(b + w.wvhi);
  p.wvlo = reinterpret_cast<uint16_t*>(b + w.wvlo);
  p.sblk = reinterpret_cast<uint32_t*>(b + w.sblk);
  p.stot = reinterpret_cast<float*>(b + w.stot);
  p.upart = reinterpret_cast<float*>(b + w.upart);
  p.ypart = reinterpret_cast<float*>(b + w.ypart);
  return p;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks shared by every entry point.
static int check_desc(const spear_ec_desc* d, bool need_rank) {
  if (!d) return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->d_in <= 0 || d->d_out <= 0 || d->rank < 0 || d->group_size <= 0)
    return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "desc has a non-positive size");
  if (d->flags & ~(SPEAR_EC_ZEROS | SPEAR_EC_PER_TENSOR | SPEAR_EC_OUT_F32))
    return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "unknown desc.flags bits");
  if ((d->flags & SPEAR_EC_PER_TENSOR) && ((d->flags & SPEAR_EC_ZEROS) || d->group_size != d->d_in))
    return fail(SPEAR_EC_ERR_UNSUPPORTED, "SPEAR_EC_PER_TENSOR needs group_size == d_in and no zeros");
  if (d->d_in % 128 != 0 || d->d_in > 131072)
    return fail(SPEAR_EC_ERR_UNSUPPORTED, "d_in must be a multiple of 128 and at most 131072");
  if (d->d_out % 16 != 0 || d->d_out > 131072)
    return fail(SPEAR_EC_ERR_UNSUPPORTED, "d_out must be a multiple of 16 and at most 131072");
  if (d->group_size != d->d_in && d->group_size != 128)
    return fail(SPEAR_EC_ERR_UNSUPPORTED, "group_size must be d_in (per-channel) or 128");
  if (need_rank && (d->rank % 16 != 0 || d->rank > 128))
    return fail(SPEAR_EC_ERR_UNSUPPORTED, "rank must be 0 or a multiple of 16 up to 128");
  return SPEAR_EC_OK;
}

static Shape make_shape(const spear_ec_desc* d, int T, bool serq = false) {
  Shape s;
  s.serq = serq;
  s.K = d->d_in;
  s.N = d->d_out;
  s.r = d->rank;
  s.g = d->group_size;
  s.T = T;
  s.grouped = d->group_size == 128 && d->d_in != 128;
  s.zeros = (d->flags & SPEAR_EC_ZEROS) != 0;
  return s;
}

static int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SPEAR_EC_OK;
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", what, hipGetErrorString(e));
  return SPEAR_EC_ERR_HIP;
}

enum Path { kAuto, kDecode, kPrefill };

// The bottleneck-MLP gate's arguments (hidden == 0: the elementwise gate).
struct MlpGate {
  int hidden;
  const float *w1, *b1, *w2, *b2;
};

// use_static: the call runs on the library's own scratch (workspace and
// workspace_bytes are ignored); it is looked up only after every check passed.
static int linear(Path path, const spear_ec_desc* d, int32_t tokens, const void* x,
                  const uint32_t* wq, const void* scales, const uint32_t* zeros, const void* A,
                  const void* B, const float* g, const float* b, float alpha, void* y,
                  void* workspace, size_t workspace_bytes, hipStream_t stream,
                  const MlpGate& mlp = MlpGate{0, nullptr, nullptr, nullptr, nullptr},
                  bool use_static = false) {
  g_last_error[0] = 0;
  int rc = check_desc(d, true);
  if (rc) return rc;
  if (tokens < 0) return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "tokens is negative");
  if (tokens > 65536) return fail(SPEAR_EC_ERR_UNSUPPORTED, "tokens must be at most 65536");
  if (path == kDecode && tokens > SPEAR_EC_DECODE_MAX_TOKENS)
    return fail(SPEAR_EC_ERR_UNSUPPORTED, "decode path takes at most 32 tokens");
  if (tokens == 0) return SPEAR_EC_OK;
  const bool has_z = (d->flags & SPEAR_EC_ZEROS) != 0;
  if (!x || !wq || !scales || !y) return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "x, wq, scales and y are required");
  if (has_z && !zeros) return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "zeros is required with SPEAR_EC_ZEROS");
  const bool gmlp = mlp.hidden > 0 && d->rank > 0;
  if (!gmlp && d->rank > 0 && (!A || !B || !g || !b))
    return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "A, B, g and b are required when rank > 0");
  if (gmlp && (!A || !B || !mlp.w1 || !mlp.b1 || !mlp.w2 || !mlp.b2))
    return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "A, B, w1, b1, w2 and b2 are required when rank > 0");
  if (!use_static && !workspace) return fail(SPEAR_EC_ERR_WORKSPACE, "workspace is NULL");
  const bool eg = d->rank > 0 && !gmlp;
  const void* ptrs[] = {x, wq, scales, y, use_static ? nullptr : workspace, has_z ? zeros : nullptr,
                        d->rank ? A : nullptr, d->rank ? B : nullptr, eg ? g : nullptr,
                        eg ? b : nullptr, gmlp ? mlp.w1 : nullptr, gmlp ? mlp.b1 : nullptr,
                        gmlp ? mlp.w2 : nullptr, gmlp ? mlp.b2 : nullptr};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(SPEAR_EC_ERR_MISALIGNED, "a pointer is not 16-byte aligned");
  const bool decode = path == kDecode || (path == kAuto && tokens <= SPEAR_EC_DECODE_MAX_TOKENS);
  const Shape s = make_shape(d, tokens);
  const Workspace wl = layout(s, decode);
  if (use_static) {
    if (wl.total > kStaticScratchBytes)
      return fail(SPEAR_EC_ERR_WORKSPACE, "the call needs more than the static scratch (64 MiB)");
    rc = hip_status(static_scratch(&workspace, stream), "static scratch set-up");
    if (rc) return rc;
  } else if (workspace_bytes < wl.total) {
    return fail(SPEAR_EC_ERR_WORKSPACE, "workspace is smaller than spear_ec_workspace_bytes()");
  }

  LayerArgs a;
  a.x = x;
  a.wq = wq;
  a.scales = static_cast<const uint16_t*>(scales);
  a.zeros = has_z ? zeros : nullptr;
  a.A = d->rank ? A : nullptr;
  a.B = d->rank ? B : nullptr;
  a.gv = eg ? g : nullptr;
  a.bv = eg ? b : nullptr;
  a.gh = gmlp ? mlp.hidden : 0;
  a.w1 = gmlp ? mlp.w1 : nullptr;
  a.b1 = gmlp ? mlp.b1 : nullptr;
  a.w2 = gmlp ? mlp.w2 : nullptr;
  a.b2 = gmlp ? mlp.b2 : nullptr;
  a.alpha = alpha;
  a.y = y;
  a.out_f32 = (d->flags & SPEAR_EC_OUT_F32) != 0;
  const WsPtrs wp = carve(workspace, wl);
  if (decode) return hip_status(launch_decode(s, a, wp, stream), "decode kernel launch");
  rc = hip_status(launch_projection(s, a, wp, stream), "projection kernel launch");
  if (rc) return rc;
  return hip_status(launch_prefill(s, a, wp, stream), "prefill kernel launch");
}

// SERQ single-matrix reconstruction through the same kernels: decode with no
// rank bands (each band's finisher adds x[:, S] R^T), prefill with the block
// sums of x from the projection kernel at rank 0, the salient channels copied
// as the epilogue operand, then the GEMM with R in B's place.
static int linear_serq(const spear_ec_desc* d, int32_t tokens, const void* x, const uint32_t* wq,
                       const void* scales, const uint32_t* zeros, int32_t s0, const void* R,
                       void* y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  int rc = check_desc(d, true);
  if (rc) return rc;
  if (d->rank <= 0) return fail(SPEAR_EC_ERR_UNSUPPORTED, "SERQ needs rank (salient channels) > 0");
  if (s0 < 0 || s0 % 8 != 0 || s0 > d->d_in - d->rank)
    return fail(SPEAR_EC_ERR_INVALID_ARGUMENT,
                "salient_begin must be a multiple of 8 with salient_begin + rank <= d_in");
  if (tokens < 0) return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "tokens is negative");
  if (tokens > 65536) return fail(SPEAR_EC_ERR_UNSUPPORTED, "tokens must be at most 65536");
  if (tokens == 0) return SPEAR_EC_OK;
  const bool has_z = (d->flags & SPEAR_EC_ZEROS) != 0;
  if (!x || !wq || !scales || !y || !R)
    return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "x, wq, scales, R and y are required");
  if (has_z && !zeros) return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "zeros is required with SPEAR_EC_ZEROS");
  if (!workspace) return fail(SPEAR_EC_ERR_WORKSPACE, "workspace is NULL");
  const void* ptrs[] = {x, wq, scales, y, workspace, R, has_z ? zeros : nullptr};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(SPEAR_EC_ERR_MISALIGNED, "a pointer is not 16-byte aligned");
  const bool decode = tokens <= SPEAR_EC_DECODE_MAX_TOKENS;
  const Shape s = make_shape(d, tokens, true);
  const Workspace wl = layout(s, decode);
  if (workspace_bytes < wl.total) return fail(SPEAR_EC_ERR_WORKSPACE, "workspace is smaller than spear_ec_workspace_bytes()");
  LayerArgs a;
  a.x = x;
  a.wq = wq;
  a.scales = static_cast<const uint16_t*>(scales);
  a.zeros = has_z ? zeros : nullptr;
  a.A = nullptr;
  a.B = R;
  a.gv = a.bv = nullptr;
  a.gh = 0;
  a.w1 = a.b1 = a.w2 = a.b2 = nullptr;
  a.alpha = 1.f;
  a.y = y;
  a.s0 = s0;
  a.out_f32 = (d->flags & SPEAR_EC_OUT_F32) != 0;
  const WsPtrs wp = carve(workspace, wl);
  if (decode) return hip_status(launch_decode(s, a, wp, stream), "decode kernel launch");
  Shape s_sums = s;  // the block sums of x only
  s_sums.r = 0;
  rc = hip_status(launch_projection(s_sums, a, wp, stream), "projection kernel launch");
  if (rc) return rc;
  rc = hip_status(launch_serq_operand(s, a, wp, stream), "SERQ operand launch");
  if (rc) return rc;
  return hip_status(launch_prefill(s, a, wp, stream), "prefill kernel launch");
}

}  // namespace spear

using namespace spear;

extern "C" {

size_t spear_ec_workspace_bytes(const spear_ec_desc* desc, int32_t max_tokens) {
  if (check_desc(desc, true) != SPEAR_EC_OK || max_tokens < 0 || max_tokens > 65536) return 0;
  size_t need = 0;
  const int td = std::min<int32_t>(max_tokens, SPEAR_EC_DECODE_MAX_TOKENS);
  // Region sizes grow with the token count, so the largest count of each
  // path bounds it; SERQ calls (rank > 0) have their own decode plan.
  for (int t : {td, (int)max_tokens}) {
    if (t <= 0) continue;
    for (bool serq : {false, true}) {
      if (serq && desc->rank == 0) continue;
      const Shape s = make_shape(desc, t, serq);
      need = std::max(need, layout(s, false).total);
      if (t <= SPEAR_EC_DECODE_MAX_TOKENS) need = std::max(need, layout(s, true).total);
    }
  }
  if (need == 0) need = layout(make_shape(desc, 1), false).total;
  return need;
}

int spear_ec_workspace_status(void* workspace, size_t workspace_bytes, hipStream_t stream,
                              int32_t* error_bits) {
  g_last_error[0] = 0;
  if (!workspace || !error_bits)
    return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "workspace and error_bits are required");
  if (workspace_bytes < sizeof(int32_t) * (kCtrError + 1))
    return fail(SPEAR_EC_ERR_WORKSPACE, "workspace is smaller than its counter words");
  int32_t* word = static_cast<int32_t*>(workspace) + kCtrError;
  int32_t bits = 0;
  int rc = hip_status(hipStreamSynchronize(stream), "stream synchronize");
  if (!rc) rc = hip_status(hipMemcpy(&bits, word, sizeof(bits), hipMemcpyDeviceToHost),
                           "error word read");
  if (!rc && bits) {
    const int32_t zero = 0;
    rc = hip_status(hipMemcpy(word, &zero, sizeof(zero), hipMemcpyHostToDevice), "error word clear");
  }
  if (!rc) *error_bits = bits;
  return rc;
}

int spear_ec_linear(const spear_ec_desc* desc, int32_t tokens, const void* x, const uint32_t* wq,
                    const void* scales, const uint32_t* zeros, const void* A, const void* B,
                    const float* g, const float* b, float alpha, void* y, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  return linear(kAuto, desc, tokens, x, wq, scales, zeros, A, B, g, b, alpha, y, workspace,
                workspace_bytes, stream);
}

int spear_ec_linear_static(const spear_ec_desc* desc, int32_t tokens, const void* x,
                           const uint32_t* wq, const void* scales, const uint32_t* zeros,
                           const void* A, const void* B, const float* g, const float* b,
                           float alpha, void* y, hipStream_t stream) {
  return linear(kAuto, desc, tokens, x, wq, scales, zeros, A, B, g, b, alpha, y, nullptr, 0, stream,
                MlpGate{0, nullptr, nullptr, nullptr, nullptr}, true);
}

int spear_ec_linear_decode(const spear_ec_desc* desc, int32_t tokens, const void* x,
                           const uint32_t* wq, const void* scales, const uint32_t* zeros,
                           const void* A, const void* B, const float* g, const float* b,
                           float alpha, void* y, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  return linear(kDecode, desc, tokens, x, wq, scales, zeros, A, B, g, b, alpha, y, workspace,
                workspace_bytes, stream);
}

int spear_ec_linear_prefill(const spear_ec_desc* desc, int32_t tokens, const void* x,
                            const uint32_t* wq, const void* scales, const uint32_t* zeros,
                            const void* A, const void* B, const float* g, const float* b,
                            float alpha, void* y, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  return linear(kPrefill, desc, tokens, x, wq, scales, zeros, A, B, g, b, alpha, y, workspace,
                workspace_bytes, stream);
}

int spear_ec_linear_mlp_gate(const spear_ec_desc* desc, int32_t tokens, const void* x,
                             const uint32_t* wq, const void* scales, const uint32_t* zeros,
                             const void* A, const void* B, int32_t hidden, const float* w1,
                             const float* b1, const float* w2, const float* b2, float alpha,
                             void* y, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  if (desc && desc->rank > 0 && (hidden < 1 || hidden > 128)) {
    g_last_error[0] = 0;
    return fail(SPEAR_EC_ERR_UNSUPPORTED, "the gate's hidden width must be 1 .. 128");
  }
  return linear(kAuto, desc, tokens, x, wq, scales, zeros, A, B, nullptr, nullptr, alpha, y,
                workspace, workspace_bytes, stream, MlpGate{hidden, w1, b1, w2, b2});
}

int spear_ec_linear_serq(const spear_ec_desc* desc, int32_t tokens, const void* x,
                         const uint32_t* wq, const void* scales, const uint32_t* zeros,
                         int32_t salient_begin, const void* R, void* y, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return linear_serq(desc, tokens, x, wq, scales, zeros, salient_begin, R, y, workspace,
                     workspace_bytes, stream);
}

int spear_ec_lut_measure(const spear_ec_desc* desc, const int32_t* tokens, int32_t n, int32_t reps,
                         const void* x, const uint32_t* wq, const void* scales,
                         const uint32_t* zeros, const void* A, const void* B, const float* g,
                         const float* b, float alpha, void* y, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, float* us_out) {
  g_last_error[0] = 0;
  if (!tokens || !us_out || n < 1 || reps < 1)
    return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "tokens, us_out, n >= 1 and reps >= 1 are required");
  for (int32_t i = 0; i < n; ++i)
    if (tokens[i] < 1 || (i > 0 && tokens[i] <= tokens[i - 1]))
      return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "tokens must be >= 1 and strictly ascending");
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = hip_status(hipEventCreate(&e0), "event create");
  if (!rc) rc = hip_status(hipEventCreate(&e1), "event create");
  for (int32_t i = 0; i < n && !rc; ++i) {
    rc = linear(kAuto, desc, tokens[i], x, wq, scales, zeros, A, B, g, b, alpha, y, workspace,
                workspace_bytes, stream);
    if (!rc) rc = hip_status(hipEventRecord(e0, stream), "event record");
    for (int32_t k = 0; k < reps && !rc; ++k)
      rc = linear(kAuto, desc, tokens[i], x, wq, scales, zeros, A, B, g, b, alpha, y, workspace,
                  workspace_bytes, stream);
    if (!rc) rc = hip_status(hipEventRecord(e1, stream), "event record");
    if (!rc) rc = hip_status(hipEventSynchronize(e1), "event synchronize");
    float ms = 0.f;
    if (!rc) rc = hip_status(hipEventElapsedTime(&ms, e0, e1), "event elapsed time");
    if (!rc) us_out[i] = ms * 1000.f / (float)reps;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  return rc;
}

int spear_ec_quantize_rtn(const spear_ec_desc* desc, const float* w, uint32_t* wq, void* scales,
                          uint32_t* zeros, hipStream_t stream) {
  g_last_error[0] = 0;
  int rc = check_desc(desc, false);
  if (rc) return rc;
  const bool asym = (desc->flags & SPEAR_EC_ZEROS) != 0;
  if (!w || !wq || !scales || (asym && !zeros))
    return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "w, wq, scales (and zeros when asymmetric) are required");
  if (!aligned16(w) || !aligned16(wq) || !aligned16(scales) || (asym && !aligned16(zeros)))
    return fail(SPEAR_EC_ERR_MISALIGNED, "a pointer is not 16-byte aligned");
  return hip_status(launch_quantize(desc->d_out, desc->d_in, desc->group_size, asym,
                                    (desc->flags & SPEAR_EC_PER_TENSOR) != 0, w, wq,
                                    static_cast<uint16_t*>(scales), asym ? zeros : nullptr, stream),
                    "quantize kernel launch");
}

int spear_ec_dequant_f32(const spear_ec_desc* desc, const uint32_t* wq, const void* scales,
                         const uint32_t* zeros, float* w_out, hipStream_t stream) {
  g_last_error[0] = 0;
  int rc = check_desc(desc, false);
  if (rc) return rc;
  const bool asym = (desc->flags & SPEAR_EC_ZEROS) != 0;
  if (!wq || !scales || !w_out || (asym && !zeros))
    return fail(SPEAR_EC_ERR_INVALID_ARGUMENT, "wq, scales, w_out (and zeros when asymmetric) are required");
  if (!aligned16(wq) || !aligned16(scales) || !aligned16(w_out) || (asym && !aligned16(zeros)))
    return fail(SPEAR_EC_ERR_MISALIGNED, "a pointer is not 16-byte aligned");
  return hip_status(launch_dequant(desc->d_out, desc->d_in, desc->group_size, wq,
                                   static_cast<const uint16_t*>(scales), asym ? zeros : nullptr,
                                   w_out, stream),
                    "dequant kernel launch");
}

const char* spear_ec_status_string(int status) {
  switch (status) {
    case SPEAR_EC_OK: return "ok";
    case SPEAR_EC_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SPEAR_EC_ERR_UNSUPPORTED: return "unsupported shape or format";
    case SPEAR_EC_ERR_MISALIGNED: return "misaligned pointer";
    case SPEAR_EC_ERR_WORKSPACE: return "workspace missing or too small";
    case SPEAR_EC_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* spear_ec_last_error(void) { return g_last_error; }

int spear_ec_version(void) { return SPEAR_EC_VERSION; }

}  // extern "C"
