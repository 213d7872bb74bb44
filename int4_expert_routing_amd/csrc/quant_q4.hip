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
// so a wave covers 8 groups = 1 KB of contiguous weights; min and max meet
// through three lane exchanges inside the 8-lane team; each lane writes its 8
// codes as one word (8 lanes = 32 contiguous bytes) and the team's first lane
// writes the scale and bias.
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void quantize_q4_kernel(const uint16_t* __restrict__ w, long groups,
                                                          uint32_t* __restrict__ q, uint16_t* __restrict__ s,
                                                          uint16_t* __restrict__ b) {
  const long gid = long(blockIdx.x) * blockDim.x + threadIdx.x;
  const long team = gid >> 3;
  const int sub = int(gid & 7);
  const bool ok = team < groups;
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  if (ok) v = *reinterpret_cast<const u32x4*>(w + team * kGroup + sub * 8);
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
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float r = fminf(fmaxf(__builtin_rintf((x[i] - lo) / sv), 0.0f), 15.0f);
      word |= uint32_t(r) << (4 * i);
    }
  }
  if (!ok) return;
  q[team * 8 + sub] = word;
  if (sub == 0) {
    s[team] = uint16_t(s_bits);
    b[team] = uint16_t(__float_as_uint(lo) >> 16);
  }
}

hipError_t launch_quantize(const uint16_t* w, long rows, int K, uint32_t* q, uint16_t* s, uint16_t* b,
                           hipStream_t stream) {
  const long groups = rows * long(K / kGroup);
  if (groups == 0) return hipSuccess;
  const long threads = groups * 8;
  hipLaunchKernelGGL(quantize_q4_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, stream, w, groups, q,
                     s, b);
  return hipGetLastError();
}

}  // namespace moe
