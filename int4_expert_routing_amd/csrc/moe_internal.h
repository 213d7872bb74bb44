// Internal kernel argument structs and launchers (not part of the C ABI).
#pragma once

#include "moe_common.h"
#include "../../include/moe_q4.h"

namespace moe {

constexpr int kMaxExperts = MOE_MAX_EXPERTS;
constexpr int kMaxTopk = MOE_MAX_TOPK;
constexpr int kMaxK = 2048;  // largest reduction size of the grouped GEMM (LDS budget)

struct RouteArgs {
  const uint16_t* x;        // bf16 [T][H] (router GEMM input) or null
  const uint16_t* wr;       // bf16 [E][H]
  const float* logits_in;   // float [T][E] when logits are given, or [n_parts][T][E] partial sums
  int n_parts;              // number of partial-sum planes in logits_in (1 = plain logits)
  float* logit_parts;       // workspace for the router's K-range partials [kRouterSplits][T][E]
  const float* bias;        // float [E] or null
  float* logits_out;        // float [T][E]: router GEMM output (layer path)
  int32_t* topk_ids;        // [T][k]
  float* topk_w;            // [T][k]
  int32_t* block_counts;    // [nblk][E]
  int32_t* rank_in_block;   // [T*k]
  int T, H, E, k;
  // a single routing block (T <= kRouteTokens) also finishes the tables
  // itself: counts, offsets, block map and scatter (no scan/scatter launches)
  int finish;
  int block_rows;
  int32_t* counts;          // [E]
  int32_t* offsets;         // [E+1]
  int32_t* tile_map;        // [max_tiles][2]
  int32_t* num_tiles;       // [1]
  int32_t* sorted_rows;     // [T*k]
  int32_t* row_of_pair;     // [T*k]
};

struct ScanArgs {
  const int32_t* block_counts;
  int32_t* block_base;      // [nblk][E]
  int32_t* counts;          // [E]
  int32_t* offsets;         // [E+1]
  int32_t* tile_map;        // [max_tiles][2]
  int32_t* num_tiles;       // [1]
  int nblk, E, block_rows;
};

struct ScatterArgs {
  const int32_t* topk_ids;
  const int32_t* block_base;
  const int32_t* rank_in_block;
  int32_t* sorted_rows;
  int32_t* row_of_pair;
  int T, E, k;
};

// Few-token layer calls split the router GEMM's K range in kRouterSplits.
constexpr int kRouterSplits = 8;
constexpr int kRouterSplitMaxT = 256;
int router_splits(int T, int H);

hipError_t launch_route(const RouteArgs& ra, const ScanArgs& sa, const ScatterArgs& ca, bool from_x,
                        hipStream_t stream);

// One stack of 4-bit matrices [n][N][K/8] with bf16 scale/bias [n][N][K/64].
struct QStack {
  const uint32_t* q;
  const uint16_t* s;
  const uint16_t* b;
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
  const int32_t* tile_map;
  const int32_t* num_tiles;
  int n_shared_tiles;       // the first n_shared_tiles tiles cover the shared rows
  int shared_rows;
  int N, K, NT;             // NT = column tiles per row tile
  void* out;                // f32 [rows][N], or bf16 [rows][N]
  uint16_t* out_part;       // group-sum table of the bf16 output (internal SwiGLU only)
};

hipError_t launch_gemm(const GemmArgs& ga, int epilogue, int max_row_tiles, hipStream_t stream);

// Decode-shaped kernels: row tiles of at most kDecodeMaxRows rows (every tile
// of a layer call with T <= kDecodeMaxRows tokens).
constexpr int kDecodeMaxRows = 8;
bool decode_supported(int N, int K, int epilogue);
// ga.NT = N/16 column blocks (SwiGLU, internal epilogue: h in the operand chunk
// order, no group-sum table) or N/32 (STORE_F32). natural_rows: ga.A holds rows
// in natural element order (the kernel reorders them while staging).
hipError_t launch_decode(const GemmArgs& ga, int epilogue, bool natural_rows, int max_row_tiles,
                         hipStream_t stream);

hipError_t launch_prep_rows(const uint16_t* A, int rows, int K, uint16_t* a_perm, uint16_t* a_part,
                            hipStream_t stream);

hipError_t launch_combine(const float* Y, const float* w, const int32_t* row_of_pair, int T, int k, int H,
                          int shared_row0, uint16_t* y, hipStream_t stream);

}  // namespace moe
