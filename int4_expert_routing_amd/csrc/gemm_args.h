// Arguments of the grouped 4-bit GEMM kernel (internal, not part of the C ABI).
#pragma once

#include "moe_common.h"

namespace moe {

// One stack of n 4-bit matrices of shape [N][K] (G = K/64 groups).
//   packed == 0 (canonical): q [n][N][K/8] u32, s and b [n][N][G] bf16;
//   packed == 1: q [n][G][N][8] u32 (one group of consecutive rows is
//     contiguous), s and b [n][G/2][N] u32 holding the bf16 values of groups
//     2p (low half) and 2p+1 (high half).
struct QStack {
  const uint32_t* q;
  const uint16_t* s;
  const uint16_t* b;
  int packed;
};

enum GemmEpilogue { kEpiF32 = 0, kEpiSwigluNatural = 1, kEpiSwigluInternal = 2 };

struct GemmArgs {
  const uint16_t* A;        // activations in the permuted chunk order [a_rows][K]
  const uint16_t* Apart;    // group sums split in three bf16 parts [a_rows][xpart_cols(K)]
  const int32_t* sorted_rows;  // gather for routed rows: src = sorted_rows[r] / row_div; null = identity
  int row_div;
  int routed_rows;          // rows [0, routed_rows) belong to routed tiles
  int shared_src_base;      // a shared-expert row r reads activation row r - shared_src_base
  QStack w0[2];             // [0] routed experts, [1] shared expert (gate, or the only matrix)
  QStack w1[2];             // up projection (SwiGLU epilogues only)
  int E;                    // a tile whose expert is E uses the shared stack
  const int32_t* offsets;
  const int32_t* tile_map;  // (expert, first row) of each routed tile of at most bm rows
  const int32_t* num_tiles;
  int bm;                   // rows per routed tile (32, 64 or kBlockRows)
  int n_shared_tiles;       // the first n_shared_tiles tiles cover the shared rows, sh_bm each
  int sh_bm;                // rows per shared tile (kBlockRows, or 32 in one-column-block launches)
  int routed_tiles;         // 1: the routed tiles of the block map follow them; 0: shared tiles only
  int merge_tail;           // 1 (bm == kBlockRows, a complete block map in expert order): an expert's last
                            // tile of at most 32 rows is computed by the full tile before it
  int shared_rows;
  int N, K, NT;             // NT = column tiles per row tile
  void* out;                // f32 [rows][N], or bf16 [rows][N]
  uint16_t* out_part;       // group-sum table of the bf16 output (internal SwiGLU only)
};

// one_block: the one-column-block kernel (every tile of the launch holds at
// most 32 rows: routed tiles of 32 rows, sh_bm == 32; NT = N / 64 for the
// SwiGLU epilogues, N / 128 for STORE_F32)
hipError_t launch_gemm(const GemmArgs& ga, int epilogue, int max_row_tiles, hipStream_t stream,
                       bool one_block = false);

}  // namespace moe
