// Device helpers shared by the grouped GEMM and the decode kernels: the tile
// list (shared-expert tiles first, then the routed tiles of the block map), the
// activation-row gather, and the exact 4-bit operand unpack.
#pragma once

#include "gemm_args.h"

namespace moe {

// Exact MFMA/dot operand of a 4-bit code q: the bf16 value 1 + q/16, whose bit
// pattern is 0x3F80 | (q << 3). kMagic is two bf16 1.0; kNib keeps a code moved
// to mantissa bits 3..6 of each 16-bit half.
constexpr uint32_t kMagic = 0x3F803F80u;
constexpr uint32_t kNib = 0x00780078u;

struct TileInfo {
  int e, r0, r1;
};

__device__ __forceinline__ bool tile_info(const GemmArgs& a, int tile, TileInfo& ti) {
  if (tile < a.n_shared_tiles) {
    ti.e = a.E;
    ti.r0 = a.routed_rows + tile * a.sh_bm;
    ti.r1 = min(ti.r0 + a.sh_bm, a.routed_rows + a.shared_rows);
    return true;
  }
  const int i = tile - a.n_shared_tiles;
  if (!a.routed_tiles || i >= *a.num_tiles) return false;
  ti.e = a.tile_map[2 * i];
  ti.r0 = a.tile_map[2 * i + 1];
  const int end = a.offsets[ti.e + 1];
  ti.r1 = min(ti.r0 + a.bm, end);
  if (a.merge_tail) {
    // an expert's rows beyond its full tiles, at most 32 of them, join the
    // last full tile (up to 160 rows), whose tile then covers them, and
    // their own tile has nothing to do
    if (ti.r1 == end && end - ti.r0 <= 32 && ti.r0 - a.offsets[ti.e] >= kBlockRows) return false;
    if (end - ti.r0 > kBlockRows && end - ti.r0 <= kBlockRows + 32) ti.r1 = end;
  }
  return true;
}

__device__ __forceinline__ int src_row(const GemmArgs& a, int r) {
  if (r >= a.routed_rows) return r - a.shared_src_base;
  return a.sorted_rows ? a.sorted_rows[r] / a.row_div : r;
}

// (a & m) | c in one VALU op. The VOP3 encoding takes no literal constants, so
// the mask and the magic value are passed in registers.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(m), "v"(c));
  return d;
}

// Word w holds codes k..k+7 (nibble i = code k+i). Register pair i gets codes
// (k+i, k+i+4), which sit at bits 4i and 4i+16; each is moved to mantissa bits
// 3..6 of its half (shift by 3 - 4i) and ORed into bf16 1.0.
__device__ __forceinline__ bf16x8 unpack_word(uint32_t w, uint32_t nib, uint32_t magic) {
  u32x4 r;
  r.x = and_or(w << 3, nib, magic);
  r.y = and_or(w >> 1, nib, magic);
  r.z = and_or(w >> 5, nib, magic);
  r.w = and_or(w >> 9, nib, magic);
  return __builtin_bit_cast(bf16x8, r);
}

}  // namespace moe
