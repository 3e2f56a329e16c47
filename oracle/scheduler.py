"""Plain reference for the EC-aware chunk selection (TEST INFRASTRUCTURE ONLY).

SPEAR summary, section 2.2 C: a latency-aware scheduler reads a precomputed
table of kernel latencies and picks, for the current compensator placement and
decode load, the largest prefill chunk whose step still meets the inter-token
latency target.  The readings (the pages give no formula):

  * a step makes, per layer, one call on the decode tokens and one on the
    prefill chunk; a kind of layer (same shape and rank) has one table and a
    count of such layers;
  * between table points the latency is linear in the tokens, over the
    running maximum of the table (more tokens never cost less); below the
    first point it is the first point's latency; above the last it is the
    last latency scaled by tokens / last tokens; zero tokens cost nothing;
  * the chosen chunk is a multiple of a granule up to a maximum; when even
    the decode tokens alone exceed the target the chunk is 0;
  * a step meets the target when its latency, rounded to fp32 (the precision
    a latency is reported in), is at most the fp32 target, so a latency read
    back from the table selects the chunk it was computed for.

Written with plain loops over every candidate chunk (no bisection), in Python
floats (double), with the one fp32 rounding of the comparison.
"""
from __future__ import annotations

import numpy as np


def call_us(tokens, us, t):
    if t <= 0:
        return 0.0
    env = []
    m = 0.0
    for v in us:
        m = max(m, float(v))
        env.append(m)
    if t <= tokens[0]:
        return env[0]
    for i in range(1, len(tokens)):
        if t <= tokens[i]:
            t0, t1 = tokens[i - 1], tokens[i]
            return env[i - 1] + (env[i] - env[i - 1]) * (t - t0) / (t1 - t0)
    return env[-1] * t / tokens[-1]


def step_us(kinds, decode_tokens, chunk_tokens, overhead_us=0.0):
    s = float(overhead_us)
    for k in kinds:
        s += k["count"] * (call_us(k["tokens"], k["us"], decode_tokens) +
                           call_us(k["tokens"], k["us"], chunk_tokens))
    return s


def pick_chunk(kinds, decode_tokens, itl_us, overhead_us=0.0, max_chunk=8192, granule=32):
    best = 0
    for m in range(0, max_chunk // granule + 1):
        c = m * granule
        if np.float32(step_us(kinds, decode_tokens, c, overhead_us)) <= np.float32(itl_us):
            best = c
    return best
