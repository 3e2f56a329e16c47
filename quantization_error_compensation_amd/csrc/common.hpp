// Device helpers shared by the libspear_ec kernels (gfx950 / CDNA4).
//
// Integer-code operands.  The matrix cores take bf16 operands.  An int4 code c
// is turned into the bf16 value 128 + c by placing its nibble under the
// exponent byte: 0x4300 is 128.0 in bf16 and the low 7 mantissa bits then
// count units.  Eight codes of a 32-bit word become four packed bf16 pairs
// with two masks, one shift and four byte permutes.  The products
// (128 + c) * x are exact in fp32, and the offset comes out in the matrix
// cores as well:
//     sum_k (c_k - z) x_k = sum_k (128 + c_k) x_k - (128 + z) * sum_k x_k,
// -(128 + z) being exact in bf16 (decode multiplies x by it in every K step;
// prefill multiplies it by the block sums of x, split into three bf16
// parts, in one extra K step per block).  The group scale s is applied in
// fp32.  Nothing is rounded to bf16 on the weight side, so the dequantized
// weight the layer sees is the exact (c - z) * s of the format.
//
// K order.  The pairs built from a word hold columns (0,2), (4,6), (1,3),
// (5,7) of its eight, so a matrix-core operand carries the columns of an
// 8-column block in the order 0,2,4,6,1,3,5,7.  A dot product does not depend
// on the order of its terms, so the activations are permuted the same way
// (x_permute8) and the packed weights keep their canonical layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spear {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kBf16Offset128 = 0x43004300u;  // bf16 pair (128.0, 128.0)
constexpr uint32_t kBf16One = 0x3F803F80u;        // bf16 pair (1.0, 1.0)

// Eight codes (nibble j = column j of the block) -> bf16 pairs of 128 + c in
// the operand order 0,2,4,6,1,3,5,7: the even and odd nibbles are split into
// bytes, and v_perm_b32 places each byte under the bf16 exponent byte 0x43.
__device__ __forceinline__ u32x4 codes_to_bf16_offset(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // bytes: c0 c2 c4 c6
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // bytes: c1 c3 c5 c7
  const uint32_t m = 0x43434343u;
  u32x4 o;
  o.x = __builtin_amdgcn_perm(lo, m, 0x01050004u);  // (c0, c2)
  o.y = __builtin_amdgcn_perm(lo, m, 0x01070006u);  // (c4, c6)
  o.z = __builtin_amdgcn_perm(hi, m, 0x01050004u);  // (c1, c3)
  o.w = __builtin_amdgcn_perm(hi, m, 0x01070006u);  // (c5, c7)
  return o;
}

// Eight codes -> bf16 pairs of 128 + c in natural column order (c0,c1),
// (c2,c3), (c4,c5), (c6,c7): the even and odd nibbles are split into bytes,
// interleaved back into column order, then placed under the exponent byte.
__device__ __forceinline__ u32x4 codes_to_bf16_offset_natural(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;                        // bytes: c0 c2 c4 c6
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;                 // bytes: c1 c3 c5 c7
  const uint32_t a = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // c0 c1 c2 c3
  const uint32_t b = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // c4 c5 c6 c7
  const uint32_t m = 0x43434343u;
  u32x4 o;
  o.x = __builtin_amdgcn_perm(a, m, 0x01050004u);  // (c0, c1)
  o.y = __builtin_amdgcn_perm(a, m, 0x01070006u);  // (c2, c3)
  o.z = __builtin_amdgcn_perm(b, m, 0x01050004u);  // (c4, c5)
  o.w = __builtin_amdgcn_perm(b, m, 0x01070006u);  // (c6, c7)
  return o;
}

// Eight consecutive bf16 activations (packed in 4 words) -> the same operand
// order 0,2,4,6,1,3,5,7 as codes_to_bf16_offset.
__device__ __forceinline__ u32x4 x_permute8(u32x4 d) {
  u32x4 o;
  o.x = __builtin_amdgcn_perm(d.y, d.x, 0x05040100u);  // (x0, x2)
  o.y = __builtin_amdgcn_perm(d.w, d.z, 0x05040100u);  // (x4, x6)
  o.z = __builtin_amdgcn_perm(d.y, d.x, 0x07060302u);  // (x1, x3)
  o.w = __builtin_amdgcn_perm(d.w, d.z, 0x07060302u);  // (x5, x7)
  return o;
}

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Logistic function in the form whose exp() argument is never positive.
__device__ __forceinline__ float sigmoidf_safe(float z) {
  if (z >= 0.f) return 1.f / (1.f + expf(-z));
  const float e = expf(z);
  return e / (1.f + e);
}

// Counters shared between workgroups: relaxed atomics at device scope.
__device__ __forceinline__ int load_dev(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed.  The
// compiler fences keep earlier stores from being moved past the wait.
__device__ __forceinline__ void wait_vmem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Raw buffer resource over [base, base + bytes): loads at offsets past the end
// return zero, which masks rows past d_out and tokens past T.  Offsets are
// 32-bit; every resource here spans at most one band of rows or one operand.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// Loads straight into LDS (no registers on the way), issued from inline
// assembly.  The compiler tracks the LDS writes of its builtin form of these
// loads and, unable to tell ring stages apart, waits for every such load
// still in flight before any LDS read; a kernel that pipelines stages through
// LDS then stalls on the stage it has just issued.  These forms are invisible
// to that tracking: the kernel orders them itself with s_waitcnt vmcnt and a
// barrier before it reads a stage.  They count in vmcnt like every vector
// memory load.  M0 (the LDS base of the load) is saved and restored.
//
// Buffer descriptor as four scalar words: base, stride 0, byte count (loads
// at offsets past it return zero), raw dword format.
__device__ __forceinline__ u32x4 sdesc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 d;
  d.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
  d.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  d.z = __builtin_amdgcn_readfirstlane(bytes);
  d.w = 0x00020000u;
  return d;
}
// Byte address in the workgroup's LDS of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  uint32_t a = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
  asm("" : "+s"(a));  // held in a register: a folded constant is no valid operand below
  return a;
}
// Lane i's 16 (or 4) bytes at desc + off land at LDS address lds + 16 i (or
// 4 i); lds must be wave-uniform (it is read from the first lane).  The
// whole offset is the per-lane one, so every byte is checked against the
// descriptor's range (past it: zero).  The global address of a lane's load
// is aligned to its size (16 or 4 bytes).
__device__ __forceinline__ void dma16(u32x4 desc, uint32_t lds, uint32_t off) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(desc)
      : "memory");
}
__device__ __forceinline__ void dma4(u32x4 desc, uint32_t lds, uint32_t off) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(desc)
      : "memory");
}
// Wait until at most N of this wave's vector memory loads are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t bload2(rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

// Bring the whole kernel-argument block of the running kernel (Bytes long)
// into the scalar cache with one memory round trip: one 4-byte scalar load
// per 64-byte line, all issued before a single wait in the same asm block (so
// no load is left in flight past it).  Without it the compiler fetches the
// argument fields where it first needs them, one line after another, each
// a cache miss waited for before the next (some 2 us at a kernel's start).
template <int Bytes>
__device__ __forceinline__ void warm_kernel_args() {
  static_assert(Bytes >= 4 && Bytes <= 384, "argument block size");
  const auto kp = __builtin_amdgcn_kernarg_segment_ptr();
  uint32_t a, b, c, d, e, f, g;
  asm volatile(
      "s_load_dword %0, %7, 0x0\n\t"
      "s_load_dword %1, %7, %8\n\t"
      "s_load_dword %2, %7, %9\n\t"
      "s_load_dword %3, %7, %10\n\t"
      "s_load_dword %4, %7, %11\n\t"
      "s_load_dword %5, %7, %12\n\t"
      "s_load_dword %6, %7, %13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=s"(a), "=s"(b), "=s"(c), "=s"(d), "=s"(e), "=s"(f), "=s"(g)
      : "s"(kp), "n"(Bytes > 0x40 ? 0x40 : 0), "n"(Bytes > 0x80 ? 0x80 : 0),
        "n"(Bytes > 0xC0 ? 0xC0 : 0), "n"(Bytes > 0x100 ? 0x100 : 0),
        "n"(Bytes > 0x140 ? 0x140 : 0), "n"((Bytes - 4) & ~3)
      : "memory");
}

// Index of the calling wave in its workgroup as a wave-uniform value, so that
// offsets derived from it stay in scalar registers (a buffer load whose scalar
// offset the compiler cannot prove uniform is wrapped in a per-lane loop).
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Data handed from one workgroup to another without cache-wide fences.  A
// release fence writes the whole XCD L2 back and an acquire invalidates it;
// done by every workgroup they stall the streaming ones.  Instead such data is
// stored and loaded with the device-scope cache policy (sc1: coherent across
// XCDs, no L2-wide maintenance), and the writer waits for its stores to
// complete (wait_vmem) before it bumps the arrival counter.  These are plain
// memory operations to the compiler, so many can be in flight at once; a
// relaxed atomic of the same scope compiles to the same instruction but is
// never reordered with other atomics, which serializes a run of them on the
// memory latency.
constexpr int kDeviceScope = 16;  // buffer cache-policy bits: sc1
__device__ __forceinline__ float bload_dev(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kDeviceScope));
}
__device__ __forceinline__ u32x4 bload16_dev(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kDeviceScope));
}
__device__ __forceinline__ void bstore_dev(rsrc_t r, uint32_t voff, uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, kDeviceScope);
}
__device__ __forceinline__ void bstore16_dev(rsrc_t r, uint32_t voff, uint32_t soff, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff, kDeviceScope);
}

// Plain global loads from a wave-uniform base plus a 32-bit byte offset (the
// scalar-base addressing form: no per-load 64-bit address arithmetic and no
// buffer descriptor held in scalar registers).
__device__ __forceinline__ u32x4 gload16(const void* base, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(static_cast<const char*>(base) + off);
}
__device__ __forceinline__ uint32_t gload4(const void* base, uint32_t off) {
  return *reinterpret_cast<const uint32_t*>(static_cast<const char*>(base) + off);
}
__device__ __forceinline__ uint32_t gload2(const void* base, uint32_t off) {
  return *reinterpret_cast<const uint16_t*>(static_cast<const char*>(base) + off);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace spear
