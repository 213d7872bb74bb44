// Device-side helpers shared by the routing and GEMM kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kGroup = 64;        // weights per quantisation group along K
constexpr int kBlockRows = 128;   // rows per GEMM tile
constexpr int kRouteTokens = 16;  // tokens per routing block (top-k, histogram, scatter)
constexpr int kWave = 64;
// Head of a layer workspace that must be zero before a call and that every
// call leaves zero: the one-launch routing's completion counter (256 bytes)
// and its 64-bit logit slots for up to kHandoffTokens tokens x 256 experts.
constexpr int kHandoffTokens = 8;
constexpr int kHandoffBytes = 256 + kHandoffTokens * 256 * 8;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16, round to nearest, ties to even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Order-preserving map of a float onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_from_order_key(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = __shfl_xor(uint32_t(v), mask, kWave);
  uint32_t hi = __shfl_xor(uint32_t(v >> 32), mask, kWave);
  return (uint64_t(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Within each 8-element (16-byte) chunk of bf16 values, the GEMM kernels keep
// activations in the order [0,4,1,5,2,6,3,7]: the order in which one 32-bit
// word of eight 4-bit codes unpacks into four bf16 pairs (see gemm_q4.hip).
// in: natural chunk as 4 words (x1:x0, x3:x2, x5:x4, x7:x6); out: permuted.
__device__ __forceinline__ u32x4 permute_chunk(u32x4 v) {
  u32x4 o;
  o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);  // (x4 : x0)
  o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);  // (x5 : x1)
  o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);  // (x6 : x2)
  o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);  // (x7 : x3)
  return o;
}
// Inverse of permute_chunk.
__device__ __forceinline__ u32x4 unpermute_chunk(u32x4 v) {
  u32x4 o;
  o.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);  // (x1 : x0)
  o.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);  // (x3 : x2)
  o.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);  // (x5 : x4)
  o.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);  // (x7 : x6)
  return o;
}

// Sum of the 8 bf16 values of a chunk (order irrelevant), in fp32.
__device__ __forceinline__ float chunk_sum(u32x4 v) {
  float a = bf16_lo_to_f32(v.x) + bf16_hi_to_f32(v.x);
  float b = bf16_lo_to_f32(v.y) + bf16_hi_to_f32(v.y);
  float c = bf16_lo_to_f32(v.z) + bf16_hi_to_f32(v.z);
  float d = bf16_lo_to_f32(v.w) + bf16_hi_to_f32(v.w);
  return (a + b) + (c + d);
}

// Same sum in fp64 (exact for the 8 values: bf16 products of a sum stay far
// inside fp64's 53-bit significand).
__device__ __forceinline__ double chunk_sum_f64(u32x4 v) {
  double a = double(bf16_lo_to_f32(v.x)) + double(bf16_hi_to_f32(v.x));
  double b = double(bf16_lo_to_f32(v.y)) + double(bf16_hi_to_f32(v.y));
  double c = double(bf16_lo_to_f32(v.z)) + double(bf16_hi_to_f32(v.z));
  double d = double(bf16_lo_to_f32(v.w)) + double(bf16_hi_to_f32(v.w));
  return (a + b) + (c + d);
}

// Split a float into three bf16 values whose exact sum is the float
// (each step's remainder is exact in fp32).
__device__ __forceinline__ void split3_bf16(float v, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  const uint32_t h = f32_to_bf16_rne(v);
  const float r1 = v - __uint_as_float(h << 16);
  const uint32_t m = f32_to_bf16_rne(r1);
  const float r2 = r1 - __uint_as_float(m << 16);
  hi = uint16_t(h);
  mid = uint16_t(m);
  lo = uint16_t(f32_to_bf16_rne(r2));
}

// Shared-expert gate of one token, g = sigmoid(x . w) in fp32, computed by a
// whole workgroup (blockDim.x a multiple of 64, at most 1024 threads): thread i
// takes the 8-element chunks i, i + blockDim.x, ... of H; the partial sums are
// added in a fixed tree (lane exchanges, then the waves in order). Every
// thread of the workgroup must call it; every thread gets g.
// c + a.lo * b.lo + a.hi * b.hi for two packed bf16 pairs (fp32). The pairs
// are passed as plain 32-bit values: bit-casting a vector element expression
// in place reads element 0 with this compiler.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float token_gate(const uint16_t* xt, const uint16_t* w, int H, float* red) {
  float d = 0.0f;
  for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
    const u32x4 xv = *reinterpret_cast<const u32x4*>(xt + c);
    const u32x4 wv = *reinterpret_cast<const u32x4*>(w + c);
    d = dot2_bf16(xv.x, wv.x, d);
    d = dot2_bf16(xv.y, wv.y, d);
    d = dot2_bf16(xv.z, wv.z, d);
    d = dot2_bf16(xv.w, wv.w, d);
  }
  d = wave_sum_f32(d);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = d;
  __syncthreads();
  float z = 0.0f;
  for (int i = 0; i < int(blockDim.x >> 6); ++i) z += red[i];
  return 1.0f / (1.0f + expf(-z));
}

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Per activation row the GEMM needs each 64-wide group's sum X_g, split
// exactly into three bf16 parts (hi, mid, lo). The side table stores 8 bf16 per
// group, [hi, mid, lo, hi, mid, hi, 0, 0], so that one 8-element MFMA operand
// slice covers exactly one group: the bias correction pairs it with the parts
// (h, m, l) of the group's coefficient as (h, h, h, m, m, l, 0, 0), which
// gives X_g times the coefficient up to terms of 2^-24 relative.
// xpart_cols(K) = 8 * K/64.
__host__ __device__ constexpr int xpart_cols(int K) { return 8 * (K / kGroup); }

}  // namespace moe
