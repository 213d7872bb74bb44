// Internal kernel argument structs and launchers (not part of the C ABI).
#pragma once

#include "gemm_args.h"
#include "../../include/moe_q4.h"

namespace moe {

constexpr int kMaxExperts = MOE_MAX_EXPERTS;
constexpr int kMaxTopk = MOE_MAX_TOPK;

struct RouteArgs {
  const uint16_t* x;        // bf16 [T][H] (router GEMM input) or null
  const uint16_t* wr;       // bf16 [E][H]
  const float* logits_in;   // float [T][E] when logits are given, or [n_parts][T][E] partial sums
  int n_parts;              // number of partial-sum planes in logits_in (1 = plain logits)
  int coherent;             // read logits_in with device-coherent loads (written by other workgroups)
  float* logit_parts;       // workspace for the router's K-range partials [router_splits][T][E]
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
  // optional (finish only): per tile {expert, first row, rows, token ids of
  // its rows at 4 bits each}, for tiles of at most 8 rows
  u32x4* tile_desc;
  // optional: a zeroed device counter and zeroed logit slots
  // [kHandoffTokens][kMaxExperts]; with them, routing from x for at most
  // kHandoffTokens tokens runs as one launch (and leaves both zero)
  int32_t* done;
  uint64_t* slots;
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

// Number of K ranges the router GEMM splits into at T tokens (8, 4, 2 or 1),
// and the token count above which the 64 x 128 tile router kernel runs.
constexpr int kRouterTileMinT = 1024;
int router_splits(int T, int H, int E);

// prep (optional): the grouped GEMM's activation preparation, run as extra
// workgroups of the scan launch when there is one (*prep_done says whether it
// ran; otherwise the caller launches it itself).
struct PrepArgs;
hipError_t launch_route(const RouteArgs& ra, const ScanArgs& sa, const ScatterArgs& ca, bool from_x,
                        hipStream_t stream, const PrepArgs* prep = nullptr, bool* prep_done = nullptr);

// Decode-shaped kernels: row tiles of at most kDecodeMaxRows rows (every tile
// of a layer call with T <= kDecodeMaxRows tokens).
constexpr int kDecodeMaxRows = 8;
// Gate/up projection with SwiGLU: K in {256, 512, 1024, 2048}, N % 16 == 0,
// ga.NT = N/16 column blocks, ga.A = the call's T rows in natural element
// order; h is written in the operand chunk order with no group-sum table. The
// shared expert's T rows form one tile (n_shared_tiles = 1, shared_rows = T);
// routed tiles are described by the routing's tile_desc. max_rows (>= T)
// bounds every tile's row count (1..kDecodeMaxRows).
bool decode_supported(int N, int K);
hipError_t launch_decode(const GemmArgs& ga, const u32x4* tile_desc, int max_row_tiles, int max_rows,
                         hipStream_t stream);

// Down projection fused with the weighted combine, for the same few-token
// calls: y[t] = bf16(sum_j w[t][j] * (h[row_of_pair[t*k+j]] . Wd[e_tj]) +
// h[shared_row0 + t] . Wd_shared), one workgroup per (token, 16 columns).
struct DownCombineArgs {
  const uint16_t* h;          // bf16 [routed rows + T][K], operand chunk order
  QStack down;                // routed experts [E][N][K/8]
  QStack down_shared;         // shared expert [1][N][K/8]
  const int32_t* topk_ids;    // [T][k]
  const float* topk_w;        // [T][k]
  const int32_t* row_of_pair; // [T][k]
  int T, k, N, K, shared_row0;
  uint16_t* y;                // bf16 [T][N]
  const uint16_t* x;          // bf16 [T][N] layer input (for the shared-expert gate)
  const uint16_t* shared_gate;  // bf16 [N] gate vector, or null (ungated shared expert)
};
bool decode_down_combine_supported(int N, int K);
hipError_t launch_decode_down_combine(const DownCombineArgs& da, hipStream_t stream);

// The whole few-token layer as one persistent launch (H = 2048, I = 256 or
// 512, T <= kDecodeMaxRows, T * k <= 64): routing, gate/up and down + combine
// as work items handed over through tagged words in `fz`, the workspace head
// after the one-launch routing's part. hipErrorInvalidConfiguration: the
// device cannot hold a resident grid (use the three-launch path).
struct FusedLaunch {
  GemmArgs g;            // gate/up arguments of the decode path (A = x, NT = I / 16, shared_rows = T)
  DownCombineArgs d;     // down + combine arguments (h, topk and row tables unused)
  const uint16_t* wr;    // router weights [E][H]
  const float* bias;     // logit bias [E] or null
  float* logits_out;     // [T][E] or null
  int32_t* ids_out;      // [T][k] or null
  float* w_out;          // [T][k] or null
  uint8_t* fz;
};
bool decode_fused_supported(int T, int k, int H, int I);
hipError_t launch_decode_fused(const FusedLaunch& fl, hipStream_t stream);

// Min-max affine 4-bit quantiser: bf16 [rows][K] -> codes [rows][K/8],
// bf16 scale and bias [rows][K/64].
hipError_t launch_quantize(const uint16_t* w, long rows, int K, uint32_t* q, uint16_t* s, uint16_t* b,
                           hipStream_t stream);

// Canonical stack -> packed layout (codes, scale pairs, bias pairs); K % 128 == 0.
hipError_t launch_prepack(const QStack& src, int n, int N, int K, uint32_t* q, uint32_t* sp, uint32_t* bp,
                          hipStream_t stream);

hipError_t launch_prep_rows(const uint16_t* A, int rows, int K, uint16_t* a_perm, uint16_t* a_part,
                            hipStream_t stream);

// x: bf16 [T][H] activations and shared_gate: bf16 [H] gate vector, or null
// (ungated shared expert)
hipError_t launch_combine(const float* Y, const float* w, const int32_t* row_of_pair, int T, int k, int H,
                          int shared_row0, uint16_t* y, const uint16_t* x, const uint16_t* shared_gate,
                          hipStream_t stream);

}  // namespace moe
