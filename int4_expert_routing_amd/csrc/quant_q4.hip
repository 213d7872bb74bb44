// 4-bit groupwise-affine quantiser for gfx950: bf16 weights -> the layout the
// grouped GEMM and the decode kernels read (codes packed 8 per uint32 word,
// nibble i = element 8w+i; bf16 scale and bias per 64 consecutive elements
// along K).
//
// Pages: "Perplexity Open Sources Lily ..." Technical Details, prefill bullet
// (groupwise affine 4-bit weights, 64 per group) and its Chinese 技术解析 (a
// bf16 scale per 64 weights). The pages do not say how weights are quantised;
// this is the min-max affine quantiser, every step in fp32 so that the codes
// are reproducible:
//   lo = min, hi = max of the group (-0 -> +0);  s = bf16(fp32(hi - lo) / 15);
//   b = lo;  q = 0 if s == 0, else min(15, max(0, rint((w - b) / s))).
//
// Work split: 8 lanes per group, each lane loads 8 consecutive bf16 (16 bytes),
// so one wave load covers 8 groups = 1 KB of contiguous weights (four such
// loads per lane, see the kernel); min and max meet
// through three lane exchanges inside the 8-lane team; each lane writes its 8
// codes as one word (8 lanes = 32 contiguous bytes) and the team's first lane
// writes the scale and bias.
#include "moe_internal.h"

namespace moe {

// One group's codes, scale and bias from its 8 lanes' weights v (lane sub
// holds elements 8*sub .. 8*sub+7). Every lane of the wave calls this (the
// min/max exchange is wave-wide); lanes with ok == false store nothing.
__device__ __forceinline__ void quantize_team(u32x4 v, bool ok, long team, int sub, uint32_t* __restrict__ q,
                                              uint16_t* __restrict__ s, uint16_t* __restrict__ b) {
  const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(wd[i] << 16);
    x[2 * i + 1] = __uint_as_float(wd[i] & 0xFFFF0000u);
  }
  float lo = x[0], hi = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    lo = fminf(lo, x[i]);
    hi = fmaxf(hi, x[i]);
  }
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) {
    lo = fminf(lo, __shfl_xor(lo, m, kWave));
    hi = fmaxf(hi, __shfl_xor(hi, m, kWave));
  }
  lo = lo + 0.0f;   // -0 -> +0
  const uint32_t s_bits = f32_to_bf16_rne((hi - lo) / 15.0f);
  const float sv = __uint_as_float(s_bits << 16);
  uint32_t word = 0;
  if (sv != 0.0f) {
    // q = rint(fl((w - lo) / s)) without a full division per weight: t = (w - lo)
    // * rcp(s) is within 2^-18 of the correctly rounded quotient (rcp 1 ulp, one
    // rounding each; quotients are below 16), so rint(t) is the same integer
    // unless t lies within 2^-16 of a half-integer. A lane with such a weight,
    // or a scale outside [2^-100, 2^100] (reciprocal kept normal), takes the
    // IEEE division for all 8 of its weights (for the others it gives the same
    // integer, by the same bound).
    // Fast path: t + 2^23 rounds t to the nearest integer, ties to even, so
    // the low mantissa bits of the sum are rint(t); and rint(t) is in 0..15
    // without a clamp there: d >= 0, and d <= hi - lo while s is at least
    // (hi - lo)/15 less one bf16 rounding, so t < 15.1.
    const bool fast = sv >= 0x1p-100f && sv <= 0x1p100f;
    const float rs = __builtin_amdgcn_rcpf(sv);
    float d[8];
    uint32_t fw = 0;
    bool near_half = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      d[i] = x[i] - lo;
      const float t = d[i] * rs;
      const float a = t + 0x1p23f;
      near_half |= __builtin_fabsf(t - (a - 0x1p23f)) > 0.5f - 0x1p-16f;
      fw |= (__float_as_uint(a) & 0xFu) << (4 * i);
    }
    if (fast && !near_half) {
      word = fw;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float r = fminf(fmaxf(__builtin_rintf(d[i] / sv), 0.0f), 15.0f);
        word |= uint32_t(r) << (4 * i);
      }
    }
  }
  if (!ok) return;
  q[team * 8 + sub] = word;
  if (sub == 0) {
    s[team] = uint16_t(s_bits);
    b[team] = uint16_t(__float_as_uint(lo) >> 16);
  }
}

// A workgroup takes kQuantPer x 32 consecutive groups: load j of a wave reads
// 8 consecutive groups (1 KB), and all kQuantPer loads of a lane are issued
// before the first is used, so four times the bytes are in flight per lane.
constexpr int kQuantPer = 4;

__global__ __launch_bounds__(256) void quantize_q4_kernel(const uint16_t* __restrict__ w, long groups,
                                                          uint32_t* __restrict__ q, uint16_t* __restrict__ s,
                                                          uint16_t* __restrict__ b) {
  const long team0 = long(blockIdx.x) * (kQuantPer * 32) + (threadIdx.x >> 3);
  const int sub = int(threadIdx.x & 7);
  u32x4 v[kQuantPer];
#pragma unroll
  for (int j = 0; j < kQuantPer; ++j) {
    const long team = team0 + j * 32;
    v[j] = team < groups ? *reinterpret_cast<const u32x4*>(w + team * kGroup + sub * 8) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < kQuantPer; ++j) {
    const long team = team0 + j * 32;
    quantize_team(v[j], team < groups, team, sub, q, s, b);
  }
}

hipError_t launch_quantize(const uint16_t* w, long rows, int K, uint32_t* q, uint16_t* s, uint16_t* b,
                           hipStream_t stream) {
  const long groups = rows * long(K / kGroup);
  if (groups == 0) return hipSuccess;
  const long blocks = (groups + kQuantPer * 32 - 1) / (kQuantPer * 32);
  hipLaunchKernelGGL(quantize_q4_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, w, groups, q, s, b);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Prepack: the canonical stack reordered into the packed layout (see QStack):
// codes [n][N][G][8] -> [n][G][N][8], and the scale and bias arrays
// [n][N][G] -> pairs of consecutive groups [n][G/2][N]. One thread per 16-byte
// half of a (row, group) code block or per pair word, indexed in output order
// so that the writes are contiguous.
__global__ __launch_bounds__(256) void prepack_codes_kernel(const uint32_t* __restrict__ q, uint32_t* __restrict__ out,
                                                            long total, int N, int G) {
  const long i = long(blockIdx.x) * blockDim.x + threadIdx.x;   // (e, g, r, half)
  if (i >= total) return;
  const int half = int(i & 1);
  const long rr = i >> 1;
  const int r = int(rr % N);
  const long t = rr / N;
  const int g = int(t % G);
  const long e = t / G;
  *reinterpret_cast<u32x4*>(out + i * 4) =
      *reinterpret_cast<const u32x4*>(q + ((e * N + r) * G + g) * 8 + half * 4);
}

__global__ __launch_bounds__(256) void prepack_pairs_kernel(const uint16_t* __restrict__ s,
                                                            const uint16_t* __restrict__ b, uint32_t* __restrict__ sp,
                                                            uint32_t* __restrict__ bp, long total, int N, int G) {
  const long i = long(blockIdx.x) * blockDim.x + threadIdx.x;   // (e, p, r)
  if (i >= total) return;
  const int r = int(i % N);
  const long t = i / N;
  const int p = int(t % (G / 2));
  const long e = t / (G / 2);
  const long src = ((e * N + r) * G) / 2 + p;   // the pair's word in the canonical arrays (G even)
  sp[i] = reinterpret_cast<const uint32_t*>(s)[src];
  bp[i] = reinterpret_cast<const uint32_t*>(b)[src];
}

hipError_t launch_prepack(const QStack& src, int n, int N, int K, uint32_t* q, uint32_t* sp, uint32_t* bp,
                          hipStream_t stream) {
  const int G = K / kGroup;
  const long codes = long(n) * G * N * 2;
  const long pairs = long(n) * (G / 2) * N;
  if (codes > 0) {
    hipLaunchKernelGGL(prepack_codes_kernel, dim3(unsigned((codes + 255) / 256)), dim3(256), 0, stream, src.q, q,
                       codes, N, G);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (pairs > 0)
    hipLaunchKernelGGL(prepack_pairs_kernel, dim3(unsigned((pairs + 255) / 256)), dim3(256), 0, stream, src.s, src.b,
                       sp, bp, pairs, N, G);
  return hipGetLastError();
}

}  // namespace moe
