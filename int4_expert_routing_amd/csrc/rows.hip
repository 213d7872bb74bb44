// Row kernels around the grouped GEMMs: activation preparation (operand chunk
// order and the exact group-sum table) and the weighted combine of the experts'
// output rows.
#include "moe_internal.h"
#include "prep_rows.h"

namespace moe {

// ---------------------------------------------------------------------------
// Activation preparation (prep_rows.h) as a launch of its own.
__global__ __launch_bounds__(kPrepThreads) void prep_rows_kernel(PrepArgs p) { prep_rows_block(p, blockIdx.x); }

hipError_t launch_prep_rows(const uint16_t* A, int rows, int K, uint16_t* a_perm, uint16_t* a_part,
                            hipStream_t stream) {
  const long blocks = prep_rows_blocks(rows, K);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(prep_rows_kernel, dim3(unsigned(blocks)), dim3(kPrepThreads), 0, stream,
                     PrepArgs{A, rows, K, a_perm, a_part});
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weighted combine: y[t] = bf16(g[t] S[t] + sum_j w[t][j] * Y[row_of_pair[t*k+j]]),
// summed in that order (shared row first, then j ascending) with fp32 FMAs;
// g[t] = 1, or the shared-expert gate of the token when a gate vector is given.
// One workgroup per token; a thread owns 4 consecutive columns in each of the
// H/1024 column chunks; Y is read once, with non-temporal loads. KK > 0 fixes k
// at compile time, so that every row
// load of the token (both column chunks at H = 2048) is issued before the
// first FMA; KK = 0 is the generic loop.
template <int KK>
__global__ __launch_bounds__(256) void combine_kernel(const float* Y, const float* w, const int32_t* row_of_pair,
                                                      int T, int k_rt, int H, int shared_row0, uint16_t* y,
                                                      const uint16_t* x, const uint16_t* shared_gate) {
  constexpr int kChunks = 2;   // column chunks of 1024 handled together
  const int t = blockIdx.x;
  __shared__ float gred[256 / kWave];
  const float g = shared_gate ? token_gate(x + size_t(t) * H, shared_gate, H, gred) : 1.0f;   // uniform branch
  const int k = KK > 0 ? KK : k_rt;
  int rows[KK > 0 ? KK : 1];
  float ws[KK > 0 ? KK : 1];
#pragma unroll
  for (int j = 0; j < KK; ++j) {
    rows[j] = row_of_pair[size_t(t) * k + j];
    ws[j] = w[size_t(t) * k + j];
  }
  for (int c0 = threadIdx.x * 4; c0 < H; c0 += kChunks * 1024) {
    f32x4 acc[kChunks];
    bool in[kChunks];
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      const int c = c0 + u * 1024;
      in[u] = c < H;
      acc[u] = in[u] ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Y + size_t(shared_row0 + t) * H + c)) : f32x4{};
      if (shared_gate) acc[u] *= g;
    }
    if constexpr (KK > 0) {
      f32x4 v[KK][kChunks];
#pragma unroll
      for (int j = 0; j < KK; ++j)
#pragma unroll
        for (int u = 0; u < kChunks; ++u)
          v[j][u] = in[u] ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Y + size_t(rows[j]) * H + c0 + u * 1024)) : f32x4{};
#pragma unroll
      for (int j = 0; j < KK; ++j)
#pragma unroll
        for (int u = 0; u < kChunks; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[u][e] = __builtin_fmaf(ws[j], v[j][u][e], acc[u][e]);
    } else {
      for (int j = 0; j < k; ++j) {
        const int row = row_of_pair[size_t(t) * k + j];
        const float wj = w[size_t(t) * k + j];
#pragma unroll
        for (int u = 0; u < kChunks; ++u) {
          if (!in[u]) continue;
          const f32x4 v = *reinterpret_cast<const f32x4*>(Y + size_t(row) * H + c0 + u * 1024);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[u][e] = __builtin_fmaf(wj, v[e], acc[u][e]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      if (!in[u]) continue;
      const uint32_t lo = f32_to_bf16_rne(acc[u][0]) | (f32_to_bf16_rne(acc[u][1]) << 16);
      const uint32_t hi = f32_to_bf16_rne(acc[u][2]) | (f32_to_bf16_rne(acc[u][3]) << 16);
      *reinterpret_cast<uint2*>(y + size_t(t) * H + c0 + u * 1024) = make_uint2(lo, hi);
    }
  }
}

hipError_t launch_combine(const float* Y, const float* w, const int32_t* row_of_pair, int T, int k, int H,
                          int shared_row0, uint16_t* y, const uint16_t* x, const uint16_t* shared_gate,
                          hipStream_t stream) {
  if (T == 0) return hipSuccess;
  switch (k) {
    case 8:
      hipLaunchKernelGGL(combine_kernel<8>, dim3(T), dim3(256), 0, stream, Y, w, row_of_pair, T, k, H, shared_row0, y,
                         x, shared_gate);
      break;
    case 2:
      hipLaunchKernelGGL(combine_kernel<2>, dim3(T), dim3(256), 0, stream, Y, w, row_of_pair, T, k, H, shared_row0, y,
                         x, shared_gate);
      break;
    default:
      hipLaunchKernelGGL(combine_kernel<0>, dim3(T), dim3(256), 0, stream, Y, w, row_of_pair, T, k, H, shared_row0, y,
                         x, shared_gate);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
