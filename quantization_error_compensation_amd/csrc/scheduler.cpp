// EC-aware chunk selection from a latency table (host only).
//
// SPEAR summary, section 2.2 C (SLO-constrained EC-aware chunk scheduling):
// placing compensators on some modules only makes the cost of a step vary, so
// a fixed prefill chunk either breaks the inter-token latency (ITL) target or
// wastes it; the scheduler reads a precomputed table of kernel latencies and
// picks, for the current decode load and compensator placement, the largest
// prefill chunk whose step still meets the ITL target.
//
// A step runs, for every layer, one dispatcher call on the decode tokens and
// one on the prefill chunk (two calls per layer on one stream).  Layers are
// grouped into kinds (same shape and rank, e.g. with and without a
// compensator); a kind's table gives the latency of one call against its
// token count.  Between table points the latency is interpolated linearly
// over the running maximum of the table (a step never gets cheaper with more
// tokens); below the first point it is the first point's latency; above the
// last it grows in proportion to the tokens; zero tokens cost nothing.
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "spear_ec.h"

namespace {

double call_us(const spear_ec_lut_kind& k, int32_t tokens) {
  if (tokens <= 0 || k.n <= 0) return 0.0;
  double run = 0.0;  // running maximum of the table
  double prev_t = 0.0, prev_u = 0.0;
  for (int32_t i = 0; i < k.n; ++i) {
    const double t = k.tokens[i];
    const double u = std::max(run, (double)k.us[i]);
    run = u;
    if (tokens <= t) {
      if (i == 0) return u;
      return prev_u + (u - prev_u) * (tokens - prev_t) / (t - prev_t);
    }
    prev_t = t;
    prev_u = u;
  }
  return prev_u * (double)tokens / prev_t;  // past the table: proportional
}

bool valid(const spear_ec_lut_kind* kinds, int32_t n_kinds) {
  if (n_kinds < 0 || (n_kinds > 0 && !kinds)) return false;
  for (int32_t j = 0; j < n_kinds; ++j) {
    const spear_ec_lut_kind& k = kinds[j];
    if (k.n < 1 || !k.tokens || !k.us || k.count < 0) return false;
    for (int32_t i = 0; i < k.n; ++i) {
      if (k.tokens[i] < 1 || !(k.us[i] >= 0.f) || !std::isfinite(k.us[i])) return false;
      if (i > 0 && k.tokens[i] <= k.tokens[i - 1]) return false;
    }
  }
  return true;
}

double step_us(const spear_ec_lut_kind* kinds, int32_t n_kinds, int32_t decode_tokens,
               int32_t chunk_tokens, double overhead_us) {
  double s = overhead_us;
  for (int32_t j = 0; j < n_kinds; ++j)
    s += kinds[j].count * (call_us(kinds[j], decode_tokens) + call_us(kinds[j], chunk_tokens));
  return s;
}

}  // namespace

extern "C" {

float spear_ec_step_latency_us(const spear_ec_lut_kind* kinds, int32_t n_kinds,
                               int32_t decode_tokens, int32_t chunk_tokens, float overhead_us) {
  if (!valid(kinds, n_kinds) || decode_tokens < 0 || chunk_tokens < 0) return -1.f;
  return (float)step_us(kinds, n_kinds, decode_tokens, chunk_tokens, overhead_us);
}

int32_t spear_ec_pick_chunk(const spear_ec_lut_kind* kinds, int32_t n_kinds, int32_t decode_tokens,
                            float itl_us, float overhead_us, int32_t max_chunk, int32_t granule) {
  if (!valid(kinds, n_kinds) || decode_tokens < 0 || max_chunk < 0 || granule < 1 ||
      !std::isfinite(itl_us))
    return -1;
  // The step latency never decreases with the chunk, so the largest chunk
  // meeting the target is found by bisection over the multiples of granule.
  const int32_t hi_n = max_chunk / granule;
  // Compared in fp32, the precision spear_ec_step_latency_us reports: a
  // latency read back from it selects the chunk it was computed for.
  auto fits = [&](int32_t m) {
    return (float)step_us(kinds, n_kinds, decode_tokens, m * granule, overhead_us) <= itl_us;
  };
  if (!fits(0)) return 0;  // not even the decode tokens alone: no prefill this step
  int32_t lo = 0, hi = hi_n;
  while (lo < hi) {
    const int32_t mid = lo + (hi - lo + 1) / 2;
    if (fits(mid)) lo = mid;
    else hi = mid - 1;
  }
  return lo * granule;
}

}  // extern "C"
