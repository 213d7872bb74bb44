// extern "C" entry points of the library: argument validation, workspace
// layout, and the launch sequence of each call (all on the caller's stream,
// no host synchronisation).
#include <mutex>

#include "moe_internal.h"
#include "prep_rows.h"

// Workspace of moe_layer_forward_noalloc: one array per GPU, held until the
// process ends. Host code never uses this name as an address (in host code it
// is a stand-in for the device symbol): the device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moe {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

// Workspace of one layer call. Offsets in bytes from the workspace base.
struct LayerLayout {
  size_t done, logits, logit_parts, ids, w, block_counts, block_base, rank, counts, offsets, sorted_rows, row_of_pair,
      tile_map, tile_desc, num_tiles, x_perm, x_part, h, h_part, Y, total;
};

int64_t max_tiles_of(int64_t T, int64_t E, int64_t k, int64_t bm) {
  const int64_t pairs = T * k;
  return pairs / bm + (E < pairs ? E : pairs);
}

// Routed tile height of a layer call: the caller's, else 128 rows, or 32 rows
// when the experts average at most 48 rows (prefill calls of up to 1536 tokens
// at E = 256, k = 8). With 32-row tiles every tile of the grouped GEMMs holds
// at most 32 rows and they run as one-column-block launches (finer work items,
// five workgroups per CU). Measured at H = 2048, I = 512, E = 256, k = 8
// (layer µs, 32-row / 128-row tiles): T = 256 149 / 192, 512 156 / 201,
// 768 169 / 211, 1024 206 / 242, 1280 247 / 260, 1536 262 / 271,
// 2048 316 / 295, 3072 436 / 353.
int layer_bm(const moe_dims& d) {
  if (d.block_rows > 0) return d.block_rows;
  if (d.T > kDecodeMaxRows && int64_t(d.T) * d.k <= int64_t(48) * d.E) return 32;
  return kBlockRows;
}

LayerLayout layer_layout(const moe_dims& d) {
  const size_t T = size_t(d.T), E = size_t(d.E), k = size_t(d.k), H = size_t(d.H), I = size_t(d.I);
  const size_t nblk = size_t(ceil_div(d.T, kRouteTokens));
  const size_t rows = T * k + T;
  const int bm = layer_bm(d);
  Carve c;
  LayerLayout L;
  // completion counter of the one-launch routing (few tokens): kept at
  // offset 0 for every T, zero before a call and after it
  L.done = c.take(T > 0 ? size_t(MOE_WORKSPACE_HEAD_BYTES) : 0);
  L.logits = c.take(T * E * 4);
  const int ks = router_splits(d.T, d.H, d.E);
  L.logit_parts = c.take(size_t(ks > 1 ? ks : 0) * T * E * 4);
  L.ids = c.take(T * k * 4);
  L.w = c.take(T * k * 4);
  L.block_counts = c.take(nblk * E * 4);
  L.block_base = c.take(nblk * E * 4);
  L.rank = c.take(T * k * 4);
  L.counts = c.take(E * 4);
  L.offsets = c.take((E + 1) * 4);
  L.sorted_rows = c.take(T * k * 4);
  L.row_of_pair = c.take(T * k * 4);
  L.tile_map = c.take(size_t(max_tiles_of(d.T, d.E, d.k, bm)) * 8);
  L.tile_desc = c.take(d.T <= kDecodeMaxRows ? size_t(max_tiles_of(d.T, d.E, d.k, bm)) * 16 : 0);
  L.num_tiles = c.take(4);
  L.x_perm = c.take(T * H * 2);
  L.x_part = c.take(T * size_t(xpart_cols(d.H)) * 2);
  L.h = c.take(rows * I * 2);
  L.h_part = c.take(rows * size_t(xpart_cols(d.I)) * 2);
  L.Y = c.take(rows * H * 4);
  L.total = c.off;
  return L;
}

int check_route_dims(const moe_dims* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->T < 0 || d->E < 1 || d->E > kMaxExperts || d->k < 1 || d->k > d->E || d->k > kMaxTopk)
    return MOE_ERR_SHAPE;
  if (d->block_rows < 0) return MOE_ERR_SHAPE;
  // T*k*(rows) must stay within int32 indexing.
  if (int64_t(d->T) * (d->k + 1) > (int64_t(1) << 30)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// The GEMM and router kernels address their activation operands through
// buffer descriptors with 32-bit byte offsets: every such operand must stay
// below 2 GiB.
constexpr int64_t kMaxOperandBytes = int64_t(1) << 31;

int check_layer_dims(const moe_dims* d) {
  const int st = check_route_dims(d);
  if (st != MOE_OK) return st;
  if (d->H < 64 || d->I < 64 || d->H % 64 != 0 || d->I % 64 != 0) return MOE_ERR_SHAPE;
  // the grouped GEMM loads scale/bias words and group-sum entries two groups
  // at a time: the reduction sizes need an even number of 64-wide groups
  if (d->H % 128 != 0 || d->I % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (d->block_rows != 0 && d->block_rows != 32 && d->block_rows != 64 && d->block_rows != kBlockRows)
    return MOE_ERR_UNSUPPORTED;
  if (int64_t(d->T) * (d->k + 1) * d->H > (int64_t(1) << 40)) return MOE_ERR_SHAPE;
  // x (router, activation prep), h (down GEMM) and W_r within 32-bit offsets
  const int64_t rows = int64_t(d->T) * (d->k + 1);
  if (int64_t(d->T) * d->H * 2 >= kMaxOperandBytes || rows * d->I * 2 >= kMaxOperandBytes ||
      int64_t(d->E) * d->H * 2 >= kMaxOperandBytes)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_weights(const moe_q4_weights* w, int n, int N, int K) {
  if (!w) return MOE_ERR_NULL;
  if (!w->q || !w->s || !w->b) return MOE_ERR_NULL;
  if (w->n_experts != n || w->N != N || w->K != K) return MOE_ERR_SHAPE;
  if (w->layout != MOE_Q4_CANONICAL && w->layout != MOE_Q4_PREPACKED) return MOE_ERR_SHAPE;
  if (w->layout == MOE_Q4_PREPACKED && K % (2 * kGroup) != 0) return MOE_ERR_SHAPE;
  if (!aligned16(w->q)) return MOE_ERR_ALIGN;
  if (!aligned16(w->s) || !aligned16(w->b)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

QStack stack_of(const moe_q4_weights* w) { return QStack{w->q, w->s, w->b, w->layout == MOE_Q4_PREPACKED ? 1 : 0}; }

// byte offsets of the scale and bias pair planes inside a prepacked buffer
struct PackLayout {
  size_t s, b, total;
};
PackLayout pack_layout(int64_t n, int64_t N, int64_t K) {
  const int64_t G = K / kGroup;
  Carve c;
  c.take(size_t(n * N * K / 2));
  PackLayout p;
  p.s = c.take(size_t(n * (G / 2) * N * 4));
  p.b = c.take(size_t(n * (G / 2) * N * 4));
  p.total = c.off;
  return p;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(base) + off);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: inconsistent or out-of-range sizes";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a pointer is not suitably aligned";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: not implemented for these sizes";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown moe_status";
  }
}

int moe_check_dims(const moe_dims* dims) { return check_layer_dims(dims); }

int32_t moe_max_tiles(const moe_dims* d) {
  if (check_route_dims(d) != MOE_OK) return 0;
  const int bm = d->block_rows > 0 ? d->block_rows : kBlockRows;
  return int32_t(max_tiles_of(d->T, d->E, d->k, bm));
}

size_t moe_workspace_bytes(const moe_dims* d) {
  if (check_route_dims(d) != MOE_OK || d->T == 0) return 0;
  moe_dims dd = *d;
  if (dd.H < 0 || dd.I < 0) return 0;
  return layer_layout(dd).total;
}

int moe_route(const float* logits, const float* logit_bias, const moe_dims* dims, int32_t* topk_ids,
              float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_rows, int32_t* row_of_pair,
              int32_t* tile_map, int32_t* num_tiles, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_route_dims(dims);
  if (st != MOE_OK) return st;
  if (dims->block_rows < 1) return MOE_ERR_SHAPE;
  if (dims->T == 0) return MOE_OK;   // nothing to do; other arguments are not examined
  if (!logits || !topk_ids || !topk_w || !counts || !offsets || !sorted_rows || !row_of_pair || !tile_map ||
      !num_tiles)
    return MOE_ERR_NULL;
  if (!aligned4(logits) || !aligned4(topk_ids) || !aligned4(topk_w) || !aligned4(counts) || !aligned4(offsets) ||
      !aligned4(sorted_rows) || !aligned4(row_of_pair) || !aligned4(tile_map) || !aligned4(num_tiles) ||
      (logit_bias && !aligned4(logit_bias)))
    return MOE_ERR_ALIGN;
  if (dims->T == 0) return MOE_OK;
  moe_dims d = *dims;
  d.H = 0;
  d.I = 0;
  const LayerLayout L = layer_layout(d);
  if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  const int nblk = ceil_div(d.T, kRouteTokens);
  RouteArgs ra{};
  ra.logits_in = logits;
  ra.bias = logit_bias;
  ra.topk_ids = topk_ids;
  ra.topk_w = topk_w;
  ra.block_counts = at<int32_t>(workspace, L.block_counts);
  ra.rank_in_block = at<int32_t>(workspace, L.rank);
  ra.T = d.T;
  ra.E = d.E;
  ra.k = d.k;
  ScanArgs sa{ra.block_counts, at<int32_t>(workspace, L.block_base), counts, offsets, tile_map, num_tiles,
              nblk, d.E, d.block_rows};
  ScatterArgs ca{topk_ids, sa.block_base, ra.rank_in_block, sorted_rows, row_of_pair, d.T, d.E, d.k};
  const hipError_t err = launch_route(ra, sa, ca, false, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

size_t moe_gemm_workspace_bytes(int32_t a_rows, int32_t K) {
  if (a_rows < 0 || K <= 0 || K % kGroup) return 0;
  Carve c;
  c.take(size_t(a_rows) * K * 2);
  c.take(size_t(a_rows) * xpart_cols(K) * 2);
  return c.off;
}

int moe_grouped_gemm_q4(const uint16_t* A, int32_t a_rows, const int32_t* sorted_rows, int32_t row_div,
                        const moe_q4_weights* W0, const moe_q4_weights* W1, const int32_t* offsets,
                        const int32_t* tile_map, const int32_t* num_tiles, int32_t max_tiles, int32_t epilogue,
                        void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!A || !W0 || !offsets || !tile_map || !num_tiles || !out) return MOE_ERR_NULL;
  if (epilogue != MOE_EPI_STORE_F32 && epilogue != MOE_EPI_SWIGLU_BF16) return MOE_ERR_SHAPE;
  if (a_rows < 0 || max_tiles < 0) return MOE_ERR_SHAPE;
  if (sorted_rows && row_div < 1) return MOE_ERR_SHAPE;
  const int n = W0->n_experts, N = W0->N, K = W0->K;
  if (n < 1 || N < 1 || K < kGroup || K % kGroup) return MOE_ERR_SHAPE;
  if (K % (2 * kGroup)) return MOE_ERR_UNSUPPORTED;   // an even number of 64-wide groups
  if (int64_t(a_rows) * K * 2 >= kMaxOperandBytes) return MOE_ERR_UNSUPPORTED;
  int st = check_weights(W0, n, N, K);
  if (st != MOE_OK) return st;
  if (epilogue == MOE_EPI_SWIGLU_BF16) {
    st = check_weights(W1, n, N, K);
    if (st != MOE_OK) return st;
    if (W1->layout != W0->layout) return MOE_ERR_SHAPE;
    if (N % 64) return MOE_ERR_UNSUPPORTED;
  } else if (N % 128) {
    return MOE_ERR_UNSUPPORTED;
  }
  if (!aligned16(A) || !aligned16(out)) return MOE_ERR_ALIGN;
  if (a_rows == 0 || max_tiles == 0) return MOE_OK;
  const size_t need = moe_gemm_workspace_bytes(a_rows, K);
  if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  Carve c;
  uint16_t* a_perm = at<uint16_t>(workspace, c.take(size_t(a_rows) * K * 2));
  uint16_t* a_part = at<uint16_t>(workspace, c.take(size_t(a_rows) * xpart_cols(K) * 2));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_prep_rows(A, a_rows, K, a_perm, a_part, s) != hipSuccess) return MOE_ERR_HIP;
  GemmArgs ga{};
  ga.A = a_perm;
  ga.Apart = a_part;
  ga.sorted_rows = sorted_rows;
  ga.row_div = sorted_rows ? row_div : 1;
  ga.routed_rows = 0x7FFFFFFF;   // every tile is a routed tile
  ga.shared_src_base = 0;
  ga.w0[0] = ga.w0[1] = stack_of(W0);
  ga.w1[0] = ga.w1[1] = epilogue == MOE_EPI_SWIGLU_BF16 ? stack_of(W1) : stack_of(W0);
  ga.E = -1;                     // no shared-expert tiles
  ga.offsets = offsets;
  ga.tile_map = tile_map;
  ga.num_tiles = num_tiles;
  ga.bm = kBlockRows;
  ga.n_shared_tiles = 0;
  ga.sh_bm = kBlockRows;
  ga.routed_tiles = 1;
  ga.shared_rows = 0;
  ga.N = N;
  ga.K = K;
  ga.out = out;
  int epi;
  if (epilogue == MOE_EPI_STORE_F32) {
    ga.NT = ceil_div(N, 256);
    epi = kEpiF32;
  } else {
    ga.NT = ceil_div(N, 128);
    epi = kEpiSwigluNatural;
  }
  return launch_gemm(ga, epi, max_tiles, s) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

static int layer_forward_impl(const uint16_t* x, const uint16_t* router_w, const float* logit_bias,
                              const moe_q4_weights* gate, const moe_q4_weights* up, const moe_q4_weights* down,
                              const moe_q4_weights* sh_gate, const moe_q4_weights* sh_up,
                              const moe_q4_weights* sh_down, const moe_dims* dims, uint16_t* y, float* logits_out,
                              int32_t* topk_ids_out, float* topk_w_out, void* workspace, size_t workspace_bytes,
                              void* stream, void* const* events, int n_events, const moe_layer_options* opts) {
  int st = check_layer_dims(dims);
  if (st != MOE_OK) return st;
  const moe_dims d = *dims;
  if (d.T == 0) return MOE_OK;   // nothing to do; other arguments are not examined
  if (!x || !router_w || !y) return MOE_ERR_NULL;
  if ((st = check_weights(gate, d.E, d.I, d.H)) != MOE_OK) return st;
  if ((st = check_weights(up, d.E, d.I, d.H)) != MOE_OK) return st;
  if ((st = check_weights(down, d.E, d.H, d.I)) != MOE_OK) return st;
  if ((st = check_weights(sh_gate, 1, d.I, d.H)) != MOE_OK) return st;
  if ((st = check_weights(sh_up, 1, d.I, d.H)) != MOE_OK) return st;
  if ((st = check_weights(sh_down, 1, d.H, d.I)) != MOE_OK) return st;
  // the gate/up kernels read a stack slot's two matrices with one layout
  if (gate->layout != up->layout || sh_gate->layout != sh_up->layout) return MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(router_w) || !aligned16(y)) return MOE_ERR_ALIGN;
  if ((logit_bias && !aligned4(logit_bias)) || (logits_out && !aligned4(logits_out)) ||
      (topk_ids_out && !aligned4(topk_ids_out)) || (topk_w_out && !aligned4(topk_w_out)))
    return MOE_ERR_ALIGN;
  if (n_events < 0 || (n_events > 0 && !events)) return MOE_ERR_NULL;
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return MOE_ERR_NULL;
  const uint16_t* shared_gate = opts ? opts->shared_gate : nullptr;
  hipStream_t s2 = opts ? static_cast<hipStream_t>(opts->side_stream) : nullptr;
  if (shared_gate && !aligned16(shared_gate)) return MOE_ERR_ALIGN;
  if (s2 && (!opts->fork_event || !opts->join_event)) return MOE_ERR_NULL;
  const LayerLayout L = layer_layout(d);
  if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = workspace;
  // stage boundary i records events[i] when the caller asked for timing
  auto mark = [&](int i) -> bool {
    return i >= n_events || hipEventRecord(static_cast<hipEvent_t>(events[i]), s) == hipSuccess;
  };
  // the side stream waits for everything enqueued on the main stream so far
  auto fork = [&]() -> bool {
    return hipEventRecord(static_cast<hipEvent_t>(opts->fork_event), s) == hipSuccess &&
           hipStreamWaitEvent(s2, static_cast<hipEvent_t>(opts->fork_event), 0) == hipSuccess;
  };
  // the main stream waits for everything enqueued on the side stream
  auto join = [&]() -> bool {
    return hipEventRecord(static_cast<hipEvent_t>(opts->join_event), s2) == hipSuccess &&
           hipStreamWaitEvent(s, static_cast<hipEvent_t>(opts->join_event), 0) == hipSuccess;
  };
  if (!mark(0)) return MOE_ERR_HIP;
  const int T = d.T, E = d.E, k = d.k, H = d.H, I = d.I;
  const int nblk = ceil_div(T, kRouteTokens);
  const int bm = layer_bm(d);   // routed tile height

  // few tokens: every tile has at most kDecodeMaxRows rows, and the weight
  // stream, not the MFMA, bounds the layer (decode-shaped kernels, which read x
  // in natural order and need no group-sum tables)
  const bool decode = T <= kDecodeMaxRows && decode_supported(I, H) &&
                      decode_down_combine_supported(H, I);

  // 1. activations: permuted chunk order + group sums. With several routing
  // blocks (and no side stream, which forks after this step) they run as
  // extra workgroups of the routing's scan launch, which leaves most of the
  // GPU idle otherwise; else as a launch of their own here.
  uint16_t* x_perm = at<uint16_t>(ws, L.x_perm);
  uint16_t* x_part = at<uint16_t>(ws, L.x_part);
  const PrepArgs prep{x, T, H, x_perm, x_part};
  const bool fold_prep = !decode && !s2 && nblk > 1;
  if ((!decode && !fold_prep && launch_prep_rows(x, T, H, x_perm, x_part, s) != hipSuccess) || !mark(1))
    return MOE_ERR_HIP;

  // gate/up arguments: routed tiles + shared-expert tiles
  const int routed_rows = T * k;
  // 32-row routed tiles (prefill): one-column-block GEMM launches, whose
  // shared-expert tiles are 32 rows as well
  const bool one_block = !decode && bm == 32;
  const int sh_bm = one_block ? 32 : kBlockRows;
  const int n_sh = ceil_div(T, sh_bm);   // the shared expert's rows in tiles of sh_bm rows
  const int max_routed = int(max_tiles_of(T, E, k, bm));
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* tile_map = at<int32_t>(ws, L.tile_map);
  int32_t* num_tiles = at<int32_t>(ws, L.num_tiles);
  int32_t* sorted_rows = at<int32_t>(ws, L.sorted_rows);
  int32_t* row_of_pair = at<int32_t>(ws, L.row_of_pair);
  u32x4* tile_desc = at<u32x4>(ws, L.tile_desc);
  uint16_t* h = at<uint16_t>(ws, L.h);
  uint16_t* h_part = at<uint16_t>(ws, L.h_part);
  GemmArgs g1{};
  g1.A = decode ? x : x_perm;
  g1.Apart = x_part;
  g1.sorted_rows = sorted_rows;
  g1.row_div = k;
  g1.routed_rows = routed_rows;
  g1.shared_src_base = routed_rows;
  g1.w0[0] = stack_of(gate);
  g1.w0[1] = stack_of(sh_gate);
  g1.w1[0] = stack_of(up);
  g1.w1[1] = stack_of(sh_up);
  g1.E = E;
  g1.offsets = offsets;
  g1.tile_map = tile_map;
  g1.num_tiles = num_tiles;
  g1.bm = bm;
  g1.n_shared_tiles = decode ? 1 : n_sh;   // decode: the shared expert's T rows form one tile
  g1.sh_bm = sh_bm;
  g1.routed_tiles = 1;
  g1.merge_tail = bm == kBlockRows ? 1 : 0;   // the routing's block map is complete and in expert order
  g1.shared_rows = T;
  g1.N = I;
  g1.K = H;
  g1.NT = decode ? I / 16 : one_block ? I / 64 : I / 128;
  g1.out = h;
  g1.out_part = h_part;
  // down arguments (prefill): fp32 rows of every routed and shared row
  float* Y = at<float>(ws, L.Y);
  GemmArgs g2 = g1;
  g2.A = h;
  g2.Apart = h_part;
  g2.sorted_rows = nullptr;
  g2.row_div = 1;
  g2.shared_src_base = 0;
  g2.w0[0] = stack_of(down);
  g2.w0[1] = stack_of(sh_down);
  g2.w1[0] = g2.w0[0];
  g2.w1[1] = g2.w0[1];
  g2.N = H;
  g2.K = I;
  g2.NT = one_block ? ceil_div(H, 128) : ceil_div(H, 256);
  g2.out = Y;
  g2.out_part = nullptr;

  // Side stream: the shared expert needs no routing, so its tiles run there
  // while the main stream routes (after the activation prep, which both read);
  // the main stream then runs only the routed tiles and joins before the
  // combine.
  if (s2) {
    if (!fork()) return MOE_ERR_HIP;
    GemmArgs s1 = g1;
    s1.routed_tiles = 0;
    if (decode) {
      if (launch_decode(s1, tile_desc, 1, T, s2) != hipSuccess) return MOE_ERR_HIP;
    } else {
      GemmArgs s2a = g2;
      s2a.routed_tiles = 0;
      if (launch_gemm(s1, kEpiSwigluInternal, n_sh, s2, one_block) != hipSuccess ||
          launch_gemm(s2a, kEpiF32, n_sh, s2, one_block) != hipSuccess)
        return MOE_ERR_HIP;
    }
    g1.n_shared_tiles = 0;
    g2.n_shared_tiles = 0;
    g1.shared_rows = 0;
  }

  // 2-4. router GEMM, top-k, histogram, scan, scatter, block map
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, L.ids);
  float* wts = topk_w_out ? topk_w_out : at<float>(ws, L.w);

  // few tokens at the full hidden size: the whole layer as one persistent launch
  if (decode && !s2 && opts && opts->persistent_decode && decode_fused_supported(T, k, H, I)) {
    const DownCombineArgs da{h, stack_of(down), stack_of(sh_down), ids, wts, row_of_pair, T, k, H, I,
                             routed_rows, y, x, shared_gate};
    const FusedLaunch fl{g1, da, router_w, logit_bias, logits_out, topk_ids_out, topk_w_out,
                         at<uint8_t>(ws, L.done + kHandoffBytes)};
    const hipError_t ef = launch_decode_fused(fl, s);
    if (ef == hipSuccess) return (mark(2) && mark(3) && mark(4) && mark(5)) ? MOE_OK : MOE_ERR_HIP;
    if (ef != hipErrorInvalidConfiguration) return MOE_ERR_HIP;
    // no resident grid possible on this device: the three-launch path below
  }
  RouteArgs ra{};
  ra.x = x;
  ra.wr = router_w;
  ra.bias = logit_bias;
  ra.logits_out = logits_out ? logits_out : at<float>(ws, L.logits);
  ra.logit_parts = at<float>(ws, L.logit_parts);
  ra.topk_ids = ids;
  ra.topk_w = wts;
  ra.block_counts = at<int32_t>(ws, L.block_counts);
  ra.rank_in_block = at<int32_t>(ws, L.rank);
  ra.T = T;
  ra.H = H;
  ra.E = E;
  ra.k = k;
  ScanArgs sa{ra.block_counts, at<int32_t>(ws, L.block_base), at<int32_t>(ws, L.counts), offsets, tile_map,
              num_tiles, nblk, E, bm};
  ScatterArgs ca{ids, sa.block_base, ra.rank_in_block, sorted_rows, row_of_pair, T, E, k};
  ra.tile_desc = decode ? tile_desc : nullptr;
  ra.done = at<int32_t>(ws, L.done);   // the workspace base: the routing finds the status word from it
  static_assert(MOE_WORKSPACE_STATUS_OFFSET + 4 <= MOE_WORKSPACE_HEAD_BYTES, "status word inside the head");
  ra.slots = at<uint64_t>(ws, L.done + 256);
  bool prep_done = false;
  if (launch_route(ra, sa, ca, true, s, fold_prep ? &prep : nullptr, &prep_done) != hipSuccess) return MOE_ERR_HIP;
  if (fold_prep && !prep_done && launch_prep_rows(x, T, H, x_perm, x_part, s) != hipSuccess) return MOE_ERR_HIP;
  if (!mark(2)) return MOE_ERR_HIP;

  // 5. gate/up grouped GEMM with SwiGLU
  const int n_tiles1 = (decode ? g1.n_shared_tiles : (s2 ? 0 : n_sh)) + max_routed;
  const hipError_t e1 = decode ? launch_decode(g1, tile_desc, n_tiles1, T, s)
                               : launch_gemm(g1, kEpiSwigluInternal, n_tiles1, s, one_block);
  if (e1 != hipSuccess || !mark(3)) return MOE_ERR_HIP;

  // 6-7 (few tokens). down projection fused with the weighted combine
  if (decode) {
    if (s2 && !join()) return MOE_ERR_HIP;
    const DownCombineArgs da{h, stack_of(down), stack_of(sh_down), ids, wts, row_of_pair, T, k, H, I,
                             routed_rows, y, x, shared_gate};
    if (launch_decode_down_combine(da, s) != hipSuccess || !mark(4) || !mark(5)) return MOE_ERR_HIP;
    return MOE_OK;
  }

  // 6. down grouped GEMM (fp32 rows)
  const hipError_t e2 = launch_gemm(g2, kEpiF32, (s2 ? 0 : n_sh) + max_routed, s, one_block);
  if (e2 != hipSuccess || !mark(4)) return MOE_ERR_HIP;

  // 7. weighted combine + (gated) shared expert, bf16 output
  if (s2 && !join()) return MOE_ERR_HIP;
  if (launch_combine(Y, wts, row_of_pair, T, k, H, routed_rows, y, x, shared_gate, s) != hipSuccess || !mark(5))
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_layer_forward(const uint16_t* x, const uint16_t* router_w, const float* logit_bias,
                      const moe_q4_weights* gate, const moe_q4_weights* up, const moe_q4_weights* down,
                      const moe_q4_weights* sh_gate, const moe_q4_weights* sh_up, const moe_q4_weights* sh_down,
                      const moe_dims* dims, uint16_t* y, float* logits_out, int32_t* topk_ids_out,
                      float* topk_w_out, void* workspace, size_t workspace_bytes, void* stream) {
  return layer_forward_impl(x, router_w, logit_bias, gate, up, down, sh_gate, sh_up, sh_down, dims, y, logits_out,
                            topk_ids_out, topk_w_out, workspace, workspace_bytes, stream, nullptr, 0, nullptr);
}

int moe_layer_forward_ex(const uint16_t* x, const uint16_t* router_w, const float* logit_bias,
                         const moe_q4_weights* gate, const moe_q4_weights* up, const moe_q4_weights* down,
                         const moe_q4_weights* sh_gate, const moe_q4_weights* sh_up, const moe_q4_weights* sh_down,
                         const moe_dims* dims, uint16_t* y, float* logits_out, int32_t* topk_ids_out,
                         float* topk_w_out, void* workspace, size_t workspace_bytes, void* stream,
                         const moe_layer_options* opts) {
  return layer_forward_impl(x, router_w, logit_bias, gate, up, down, sh_gate, sh_up, sh_down, dims, y, logits_out,
                            topk_ids_out, topk_w_out, workspace, workspace_bytes, stream, nullptr, 0, opts);
}

int moe_layer_forward_timed(const uint16_t* x, const uint16_t* router_w, const float* logit_bias,
                            const moe_q4_weights* gate, const moe_q4_weights* up, const moe_q4_weights* down,
                            const moe_q4_weights* sh_gate, const moe_q4_weights* sh_up,
                            const moe_q4_weights* sh_down, const moe_dims* dims, uint16_t* y, float* logits_out,
                            int32_t* topk_ids_out, float* topk_w_out, void* workspace, size_t workspace_bytes,
                            void* stream, void* const* events, int32_t n_events) {
  return layer_forward_impl(x, router_w, logit_bias, gate, up, down, sh_gate, sh_up, sh_down, dims, y, logits_out,
                            topk_ids_out, topk_w_out, workspace, workspace_bytes, stream, events, n_events, nullptr);
}

}  // extern "C"

namespace moe {
namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];   // device address of `scratch` on each device, once resolved

// Zeroes the first n 32-bit words of p (a kernel, not a memset, so that the
// call can be captured in a graph).
__global__ void zero_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace
}  // namespace moe

extern "C" {

int moe_layer_forward_noalloc(const uint16_t* x, const uint16_t* router_w, const float* logit_bias,
                              const moe_q4_weights* gate, const moe_q4_weights* up, const moe_q4_weights* down,
                              const moe_q4_weights* sh_gate, const moe_q4_weights* sh_up,
                              const moe_q4_weights* sh_down, const moe_dims* dims, uint16_t* y, float* logits_out,
                              int32_t* topk_ids_out, float* topk_w_out, void* stream) {
  int st = check_layer_dims(dims);
  if (st != MOE_OK) return st;
  if (dims->T == 0) return MOE_OK;
  if (layer_layout(*dims).total > size_t(MOE_NOALLOC_SCRATCH_BYTES)) return MOE_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return MOE_ERR_HIP;
  void* ptr = nullptr;
  bool first = false;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
      g_scratch_ptr[dev] = p;
      first = true;
    }
    ptr = g_scratch_ptr[dev];
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (first) {
    // the workspace head must be zero before the first layer call; every call
    // leaves it zero
    const int words = MOE_WORKSPACE_HEAD_BYTES / 4;
    hipLaunchKernelGGL(zero_words_kernel, dim3(ceil_div(words, 256)), dim3(256), 0, s,
                       static_cast<uint32_t*>(ptr), words);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  }
  return layer_forward_impl(x, router_w, logit_bias, gate, up, down, sh_gate, sh_up, sh_down, dims, y, logits_out,
                            topk_ids_out, topk_w_out, ptr, size_t(MOE_NOALLOC_SCRATCH_BYTES), stream, nullptr, 0,
                            nullptr);
}

size_t moe_prepack_q4_bytes(int32_t n_experts, int32_t N, int32_t K) {
  if (n_experts < 1 || N < 1 || K < 2 * kGroup || K % (2 * kGroup)) return 0;
  return pack_layout(n_experts, N, K).total;
}

int moe_prepack_q4(const moe_q4_weights* src, void* dst, size_t dst_bytes, moe_q4_weights* packed, void* stream) {
  if (!src || !packed) return MOE_ERR_NULL;
  const int n = src->n_experts, N = src->N, K = src->K;
  if (n < 1 || N < 1 || K < kGroup || K % kGroup) return MOE_ERR_SHAPE;
  if (src->layout != MOE_Q4_CANONICAL) return MOE_ERR_SHAPE;
  if (K % (2 * kGroup)) return MOE_ERR_UNSUPPORTED;   // pairs of groups
  if (int64_t(n) * N * K > (int64_t(1) << 40)) return MOE_ERR_SHAPE;
  int st = check_weights(src, n, N, K);
  if (st != MOE_OK) return st;
  if (!dst) return MOE_ERR_NULL;
  if (!aligned16(dst)) return MOE_ERR_ALIGN;
  const PackLayout p = pack_layout(n, N, K);
  if (dst_bytes < p.total) return MOE_ERR_WORKSPACE;
  uint8_t* base = static_cast<uint8_t*>(dst);
  uint32_t* q = reinterpret_cast<uint32_t*>(base);
  uint32_t* sp = reinterpret_cast<uint32_t*>(base + p.s);
  uint32_t* bp = reinterpret_cast<uint32_t*>(base + p.b);
  if (launch_prepack(stack_of(src), n, N, K, q, sp, bp, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  *packed = *src;
  packed->q = q;
  packed->s = reinterpret_cast<const uint16_t*>(sp);
  packed->b = reinterpret_cast<const uint16_t*>(bp);
  packed->layout = MOE_Q4_PREPACKED;
  return MOE_OK;
}

int moe_quantize_q4(const uint16_t* w, int64_t rows, int32_t K, uint32_t* q, uint16_t* s, uint16_t* b,
                    void* stream) {
  if (rows < 0 || K <= 0 || K % kGroup != 0) return MOE_ERR_SHAPE;
  // thread indexes (rows * K/64 groups x 8 lanes) stay within a 32-bit grid of 256-thread blocks
  if (rows > (int64_t(1) << 40) / K) return MOE_ERR_SHAPE;
  if (rows == 0) return MOE_OK;
  if (!w || !q || !s || !b) return MOE_ERR_NULL;
  if (!aligned16(w) || !aligned16(q) || (reinterpret_cast<uintptr_t>(s) & 1u) || (reinterpret_cast<uintptr_t>(b) & 1u))
    return MOE_ERR_ALIGN;
  return launch_quantize(w, long(rows), K, q, s, b, static_cast<hipStream_t>(stream)) == hipSuccess ? MOE_OK
                                                                                                   : MOE_ERR_HIP;
}

}  // extern "C"
