// Activation preparation for the grouped GEMM: each row's 16-byte chunks in
// the operand order, plus the exact group-sum side table. A workgroup body, so
// that it can run as its own launch or as extra workgroups of another one.
#pragma once

#include "moe_common.h"

namespace moe {

struct PrepArgs {
  const uint16_t* A;   // bf16 [rows][K]
  int rows, K;
  uint16_t* a_perm;    // bf16 [rows][K], chunks in the order [0,4,1,5,2,6,3,7]
  uint16_t* a_part;    // bf16 [rows][xpart_cols(K)], three-part splits of the group sums
};

constexpr int kPrepThreads = 256;

inline long prep_rows_blocks(int rows, int K) {
  const long threads = long(rows) * (K / kGroup) * 8;
  return (threads + kPrepThreads - 1) / kPrepThreads;
}

// Workgroup `block` of kPrepThreads threads: 8 lanes per 64-wide group, one
// 16-byte chunk each; the group sum in fp64, rounded once.
__device__ __forceinline__ void prep_rows_block(const PrepArgs& p, long block) {
  const int G = p.K / kGroup;
  const int KPx = xpart_cols(p.K);
  const long gid = block * kPrepThreads + threadIdx.x;
  const long team = gid >> 3;
  const int sub = int(gid & 7);
  const long total = long(p.rows) * G;
  const bool ok = team < total;
  const int row = ok ? int(team / G) : 0;
  const int g = ok ? int(team % G) : 0;
  u32x4 v = u32x4{0, 0, 0, 0};
  if (ok) v = *reinterpret_cast<const u32x4*>(p.A + size_t(row) * p.K + g * kGroup + 8 * sub);
  double s = chunk_sum_f64(v);
  s += __shfl_xor(s, 1, kWave);
  s += __shfl_xor(s, 2, kWave);
  s += __shfl_xor(s, 4, kWave);
  if (!ok) return;
  *reinterpret_cast<u32x4*>(p.a_perm + size_t(row) * p.K + g * kGroup + 8 * sub) = permute_chunk(v);
  uint16_t* xp = p.a_part + size_t(row) * KPx;
  if (sub == 0) {
    uint16_t h, m, l;
    split3_bf16(float(s), h, m, l);
    const u32x4 e = {uint32_t(h) | (uint32_t(m) << 16), uint32_t(l) | (uint32_t(h) << 16),
                     uint32_t(m) | (uint32_t(h) << 16), 0u};
    *reinterpret_cast<u32x4*>(xp + 8 * g) = e;
  }
}

}  // namespace moe
