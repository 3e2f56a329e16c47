// Offline kernels: RTN int4 quantization + packing, and exact fp32 dequant.
//
// RTN follows the hard setting of the SPEAR summary (section 3.1, RTN with
// per-channel scales) and the group-wise asymmetric variant with zero-points.
// The layer itself never quantizes; these kernels prepare its inputs.
#include "common.hpp"
#include "internal.hpp"

namespace spear {
namespace {

// double -> binary16 bits, round to nearest even on the 53-bit significand,
// finite overflow saturating at 65504 (0x7BFF).
__device__ uint16_t f64_to_f16_rne_sat(double v) {
  const uint64_t bits = (uint64_t)__double_as_longlong(v);
  const uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
  const uint64_t a = bits & 0x7FFFFFFFFFFFFFFFull;
  if (a > 0x7FF0000000000000ull) return 0x7E00u;          // NaN
  if ((a >> 52) == 0) return sign;                         // zero / double subnormal
  int e = (int)(a >> 52) - 1023;
  if (e > 15) return sign | 0x7BFFu;
  const uint64_t m = (a & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  const int shift = e >= -14 ? 42 : 28 - e;                 // keep 11 bits / count 2^-24 quanta
  if (shift > 60) return sign;
  uint64_t keep = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (keep & 1))) ++keep;
  if (e >= -14) {
    if (keep == 2048) { keep = 1024; ++e; }
    if (e > 15) return sign | 0x7BFFu;
    return sign | (uint16_t)((e + 15) << 10) | (uint16_t)(keep - 1024);
  }
  return sign | (uint16_t)keep;  // 1024 quanta is the smallest normal, same bits
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
  return (double)(float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}

// One workgroup (4 waves) per output row; wave w handles groups w, w+4, ...
// mode kGroups: scale and codes of every group.  Per-tensor scales take two
// more passes: kRowScale writes each row's RN_fp16(max|W| / 7) (no codes;
// rounding is monotonic, so the largest of them is the tensor's), and after
// scale_max_kernel has set every row to that scale, kGivenScale writes the
// codes for the row's stored scale.
enum QuantMode { kGroups = 0, kRowScale = 1, kGivenScale = 2 };
__global__ __launch_bounds__(256) void quantize_rtn_kernel(const float* __restrict__ w,
                                                           uint32_t* __restrict__ wq,
                                                           uint16_t* __restrict__ scales,
                                                           uint32_t* __restrict__ zeros, int K,
                                                           int g, int asym, int mode) {
  __shared__ uint8_t zb[1024];
  const int n = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int G = K / g, words = g / 8;
  const float* row = w + (size_t)n * K;
  for (int j = wave; j < G; j += 4) {
    const float* grp = row + (size_t)j * g;
    float lo = 0.f, hi = 0.f, am = 0.f;
    for (int d = lane; d < words; d += 64) {
      const float4 p = reinterpret_cast<const float4*>(grp)[2 * d];
      const float4 q = reinterpret_cast<const float4*>(grp)[2 * d + 1];
      const float e[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
      for (int i = 0; i < 8; ++i) {
        lo = fminf(lo, e[i]);
        hi = fmaxf(hi, e[i]);
        am = fmaxf(am, fabsf(e[i]));
      }
    }
    double s;
    uint16_t sb;
    double z = 8.0;
    if (mode == kGivenScale) {
      sb = scales[(size_t)n * G + j];
    } else if (!asym) {
      sb = f64_to_f16_rne_sat((double)wave_max(am) / 7.0);
    } else {
      lo = wave_min(lo);
      hi = wave_max(hi);
      sb = f64_to_f16_rne_sat(((double)hi - (double)lo) / 15.0);
    }
    if (mode == kRowScale) {  // the raw rounded scale, 0 kept
      if (lane == 0) scales[(size_t)n * G + j] = sb;
      continue;
    }
    if ((sb & 0x7FFFu) == 0) sb = 0x3C00u;
    s = f16_bits_to_f64(sb);
    if (asym) z = fmin(15.0, fmax(0.0, rint(-(double)lo / s)));
    for (int d = lane; d < words; d += 64) {
      const float4 p = reinterpret_cast<const float4*>(grp)[2 * d];
      const float4 q = reinterpret_cast<const float4*>(grp)[2 * d + 1];
      const float e[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
      uint32_t word = 0;
      for (int i = 0; i < 8; ++i) {
        double c;
        if (!asym) c = fmin(7.0, fmax(-8.0, rint((double)e[i] / s))) + 8.0;
        else c = fmin(15.0, fmax(0.0, rint((double)e[i] / s) + z));
        word |= (uint32_t)c << (4 * i);
      }
      wq[(size_t)n * (K / 8) + (size_t)j * words + d] = word;
    }
    if (lane == 0) {
      scales[(size_t)n * G + j] = sb;
      if (asym) zb[j] = (uint8_t)z;
    }
  }
  if (asym) {
    __syncthreads();
    const int ZW = (G + 7) / 8;
    for (int wi = threadIdx.x; wi < ZW; wi += 256) {
      uint32_t word = 0;
      for (int i = 0; i < 8 && wi * 8 + i < G; ++i) word |= (uint32_t)zb[wi * 8 + i] << (4 * i);
      zeros[(size_t)n * ZW + wi] = word;
    }
  }
}

// One workgroup: the largest of the N row scales (positive fp16 bits order
// like their values), 1.0 if it is 0, written back to every row.
__global__ __launch_bounds__(256) void scale_max_kernel(uint16_t* __restrict__ scales, int N) {
  __shared__ uint32_t part[4];
  uint32_t m = 0;
  for (int n = threadIdx.x; n < N; n += 256) m = max(m, (uint32_t)scales[n]);
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  m = max(max(part[0], part[1]), max(part[2], part[3]));
  const uint16_t sb = (m & 0x7FFFu) == 0 ? (uint16_t)0x3C00u : (uint16_t)m;
  for (int n = threadIdx.x; n < N; n += 256) scales[n] = sb;
}

// One thread per packed word: eight fp32 outputs (c - z) * s, exact.
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ wq,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint32_t* __restrict__ zeros,
                                                      float* __restrict__ out, int N, int K,
                                                      int g) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t words = (size_t)N * (K / 8);
  if (idx >= words) return;
  const int n = (int)(idx / (K / 8));
  const int k0 = (int)(idx % (K / 8)) * 8;
  const int G = K / g, j = k0 / g;
  const float s = half_bits_to_f32(scales[(size_t)n * G + j]);
  const int z = zeros ? (int)((zeros[(size_t)n * ((G + 7) / 8) + j / 8] >> (4 * (j % 8))) & 15u) : 8;
  const uint32_t w = wq[idx];
  float o[8];
  for (int i = 0; i < 8; ++i) o[i] = (float)((int)((w >> (4 * i)) & 15u) - z) * s;
  float4* dst = reinterpret_cast<float4*>(out + (size_t)n * K + k0);
  dst[0] = make_float4(o[0], o[1], o[2], o[3]);
  dst[1] = make_float4(o[4], o[5], o[6], o[7]);
}

}  // namespace

hipError_t launch_quantize(int N, int K, int g, bool asym, bool per_tensor, const float* w,
                           uint32_t* wq, uint16_t* scales, uint32_t* zeros, hipStream_t st) {
  if (N == 0) return hipSuccess;
  if (!per_tensor) {
    hipLaunchKernelGGL(quantize_rtn_kernel, dim3(N), dim3(256), 0, st, w, wq, scales, zeros, K, g,
                       asym ? 1 : 0, (int)kGroups);
    return hipGetLastError();
  }
  // per-tensor: symmetric, g == K (one scale per row in the stored format)
  hipLaunchKernelGGL(quantize_rtn_kernel, dim3(N), dim3(256), 0, st, w, wq, scales, zeros, K, K,
                     0, (int)kRowScale);
  hipLaunchKernelGGL(scale_max_kernel, dim3(1), dim3(256), 0, st, scales, N);
  hipLaunchKernelGGL(quantize_rtn_kernel, dim3(N), dim3(256), 0, st, w, wq, scales, zeros, K, K,
                     0, (int)kGivenScale);
  return hipGetLastError();
}

hipError_t launch_dequant(int N, int K, int g, const uint32_t* wq, const uint16_t* scales,
                          const uint32_t* zeros, float* out, hipStream_t st) {
  const size_t words = (size_t)N * (K / 8);
  if (words == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st, wq,
                     scales, zeros, out, N, K, g);
  return hipGetLastError();
}

}  // namespace spear
