// GPU-resident MoE routing for gfx950: router GEMM + top-k + softmax, per-block
// histogram, prefix scan, stable scatter and block map, with no host
// synchronisation between the steps (page "Perplexity Open Sources Lily ..."
// Technical Details, Model bullet: the router picks 8 of 256 experts; prefill
// bullet: routing histogram, prefix scan, scatter and block map stay on the GPU).
//
// Launches on one stream:
//   0. router_logits_kernel (layer path only) - logits = x W_r^T (+ bias) with
//      bf16 MFMA and fp32 accumulation, 32 tokens x 64 experts (x a K range
//      for few tokens) per single-wave workgroup.
//   1. route_topk_kernel  - one workgroup per 16 tokens, one wave per token:
//      top-k by the key (logit desc, expert asc) through a ballot radix
//      select, softmax over the chosen k, the block's expert histogram and
//      each pair's rank among the block's pairs of the same expert.
//   2. route_scan_kernel  - 16 experts per workgroup: per-expert scan over the
//      routing blocks (block bases) and expert totals.
//   3. route_scatter_kernel - one workgroup per 16 tokens: exclusive scan of the
//      totals (offsets; workgroup 0 also writes them and the block map), and
//      the final row of each pair = offset + block base + in-block rank.
//   Up to 256 routing blocks (4096 tokens), 2 and 3 run as one launch
//   (route_scan_scatter_kernel).
// Ranks count only earlier pairs, so the sort is stable and the result does not
// depend on thread timing: repeated runs give identical tables.
#include "prep_rows.h"
#include "route_block.h"

namespace moe {

constexpr int kRouteThreads = 256;
constexpr int kRouterRows = 32;                          // tokens per router-GEMM workgroup (one MFMA block)
constexpr int kTopkThreads = kRouteTokens * kWave;       // top-k: one wave per token

// Router GEMM: logits[t][e] = fp32(sum_h x[t][h] W_r[e][h]) + bias[e].
// One wave per workgroup computes a 32-token x 64-expert tile over one K
// range (blockIdx.z of KS; KS > 1 writes fp32 partial sums that the top-k
// kernel adds in a fixed order, so few-token calls still spread over many
// CUs). Both operands stream through a 4-slot LDS ring of 64-wide K chunks
// filled by buffer loads that write LDS (three chunks in flight, 12 loads per
// chunk); 16-byte chunks of each row sit XOR-swizzled so that the MFMA
// fragment reads are bank-conflict free.
constexpr int kRouterRing = 4;
constexpr int kRouterSlotX = 4096;                       // 32 rows x 128 B
constexpr int kRouterSlot = kRouterSlotX + 8192;         // + 64 expert rows x 128 B
constexpr uint32_t kRouterRsrcWord3 = 0x00020000u;       // raw buffer descriptor flags (gfx9 family)

__device__ __forceinline__ int rswz(int m) { return (m & 7) ^ ((m >> 3) & 1); }
__device__ __forceinline__ int rchunk_off(int m, int c) { return (m * 8 + (c ^ rswz(m))) * 16; }

__global__ __launch_bounds__(kWave) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ wr,
                                                             const float* __restrict__ bias, int T, int H, int E,
                                                             float* __restrict__ out) {
  extern __shared__ __align__(16) uint8_t rsm[];
  typedef __attribute__((address_space(3))) void* lptr;
  const int lane = threadIdx.x;
  const int l32 = lane & 31, half = lane >> 5;
  const int t0 = blockIdx.x * kRouterRows;
  const int e0 = blockIdx.y * 64;
  const int KS = gridDim.z;
  const int KC = H / KS;
  const int k0 = blockIdx.z * KC;
  const int nch = KC / 64;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, 0x7FFFFFFF,
                                                                     kRouterRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wr), 0, 0x7FFFFFFF,
                                                                     kRouterRsrcWord3);
  // load i fills chunk positions i*64 + lane: row i*8 + lane/8, slot lane%8,
  // which holds logical chunk (lane%8) ^ swz(row); rows past T or E re-read
  // the last valid row
  uint32_t vx[4], vw[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = i * 8 + (lane >> 3);
    const int t = min(t0 + m, T - 1);
    vx[i] = uint32_t(t) * uint32_t(H * 2) + uint32_t(((lane & 7) ^ rswz(m)) * 16);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int n = i * 8 + (lane >> 3);
    const int e = min(e0 + n, E - 1);
    vw[i] = uint32_t(e) * uint32_t(H * 2) + uint32_t(((lane & 7) ^ rswz(n)) * 16);
  }
  auto issue = [&](int c) {
    uint8_t* slot = rsm + (c % kRouterRing) * kRouterSlot;
    const int soff = (k0 + 64 * c) * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lptr)(slot + i * 1024), 16, vx[i], soff, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lptr)(slot + kRouterSlotX + i * 1024), 16, vw[i], soff, 0, 0);
  };
  issue(0);
  if (nch > 1) issue(1);
  if (nch > 2) issue(2);
  f32x16 acc0 = f32x16{}, acc1 = f32x16{};
  for (int c = 0; c < nch; ++c) {
    // chunk c has landed once at most the (12-load) chunks c+1, c+2 are outstanding
    // (s_waitcnt: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
    if (c + 2 < nch)
      __builtin_amdgcn_s_waitcnt(0x4F78);   // vmcnt(24)
    else if (c + 1 < nch)
      __builtin_amdgcn_s_waitcnt(0x0F7C);   // vmcnt(12)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    if (c + 3 < nch) issue(c + 3);   // refills the slot of chunk c-1, read in the previous iteration
    const uint8_t* slot = rsm + (c % kRouterRing) * kRouterSlot;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = 2 * kk + half;
      const bf16x8 av = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(slot + rchunk_off(l32, ch)));
      const bf16x8 b0 = __builtin_bit_cast(bf16x8,
                                           *reinterpret_cast<const u32x4*>(slot + kRouterSlotX + rchunk_off(l32, ch)));
      const bf16x8 b1 = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(slot + kRouterSlotX + rchunk_off(32 + l32, ch)));
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b1, acc1, 0, 0, 0);
    }
  }
  // output element (eb, r, lane): token 8(r/4) + 4*half + r%4, expert e0 + 32 eb + lane%32
  float* dst = out + size_t(blockIdx.z) * size_t(T) * E;
#pragma unroll
  for (int eb = 0; eb < 2; ++eb) {
    const int n = e0 + 32 * eb + l32;
    if (n >= E) continue;
    const float bv = (KS == 1 && bias) ? bias[n] : 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r >> 2) + 4 * half + (r & 3);
      if (t0 + m < T) dst[size_t(t0 + m) * E + n] = ((eb ? acc1[r] : acc0[r]) + bv) + 0.0f;
    }
  }
}

// Router GEMM for calls above a thousand tokens: a workgroup of 4 waves
// computes a 64-token x 128-expert tile over one K range (blockIdx.z of KS).
// Wave w takes tokens 32 (w & 1) .. +31 and experts 64 (w >> 1) .. +63 of the
// tile (two 32 x 32 MFMA blocks, as in the single-wave kernel), so every
// activation and router-weight row that lands in LDS serves two waves, and
// each operand row is fetched from L2 by half as many workgroups as with
// 32 x 64 tiles (the single-wave kernel's L2 re-reads bound it at T = 4096).
// The operands stream through a 3-slot LDS ring of 64-wide K chunks, two
// chunks ahead; each wave issues 6 of a chunk's 24 buffer loads that write LDS.
constexpr int kRtTok = 64, kRtExp = 128;
constexpr int kRtRing = 3;
constexpr int kRtSlotX = kRtTok * 128;                   // 64 token rows x 128 B
constexpr int kRtSlot = kRtSlotX + kRtExp * 128;         // + 128 expert rows x 128 B
constexpr int kRtThreads = 4 * kWave;

__global__ __launch_bounds__(kRtThreads, 2) void router_tile_kernel(const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ wr,
                                                                   const float* __restrict__ bias, int T, int H,
                                                                   int E, float* __restrict__ out) {
  extern __shared__ __align__(16) uint8_t rsm[];
  typedef __attribute__((address_space(3))) void* lptr;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int tb = wave & 1, ebk = wave >> 1;
  const int t0 = blockIdx.x * kRtTok;
  const int e0 = blockIdx.y * kRtExp;
  const int KS = gridDim.z;
  const int KC = H / KS;
  const int k0 = blockIdx.z * KC;
  const int nch = KC / 64;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, 0x7FFFFFFF,
                                                                     kRouterRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wr), 0, 0x7FFFFFFF,
                                                                     kRouterRsrcWord3);
  // load i of wave w fills 8 rows: token rows (2w + i)*8 + lane/8 (i < 2) and
  // expert rows (4w + i)*8 + lane/8 (i < 4); slot lane%8 holds logical chunk
  // (lane%8) ^ swz(row). Rows past T or E re-read the last valid row.
  uint32_t vx[2], vw[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = (wave * 2 + i) * 8 + (lane >> 3);
    const int t = min(t0 + m, T - 1);
    vx[i] = uint32_t(t) * uint32_t(H * 2) + uint32_t(((lane & 7) ^ rswz(m)) * 16);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = (wave * 4 + i) * 8 + (lane >> 3);
    const int e = min(e0 + n, E - 1);
    vw[i] = uint32_t(e) * uint32_t(H * 2) + uint32_t(((lane & 7) ^ rswz(n)) * 16);
  }
  auto issue = [&](int c) {
    uint8_t* slot = rsm + (c % kRtRing) * kRtSlot;
    const int soff = (k0 + 64 * c) * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lptr)(slot + (wave * 2 + i) * 1024), 16, vx[i], soff, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lptr)(slot + kRtSlotX + (wave * 4 + i) * 1024), 16, vw[i], soff,
                                               0, 0);
  };
  issue(0);
  if (nch > 1) issue(1);
  f32x16 acc0 = f32x16{}, acc1 = f32x16{};
  for (int c = 0; c < nch; ++c) {
    // this wave's loads of chunk c have landed once at most chunk c+1's 6 are
    // outstanding; the barrier makes it so for every wave and orders every
    // wave's reads of chunk c-1's slot before it is refilled with chunk c+2
    if (c + 1 < nch)
      __builtin_amdgcn_s_waitcnt(0x0F76);   // vmcnt(6)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    if (c + 2 < nch) issue(c + 2);
    const uint8_t* slot = rsm + (c % kRtRing) * kRtSlot;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = 2 * kk + half;
      const bf16x8 av =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(slot + rchunk_off(tb * 32 + l32, ch)));
      const bf16x8 b0 = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(slot + kRtSlotX + rchunk_off(ebk * 64 + l32, ch)));
      const bf16x8 b1 = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(slot + kRtSlotX + rchunk_off(ebk * 64 + 32 + l32, ch)));
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b1, acc1, 0, 0, 0);
    }
  }
  // output element (eb, r, lane): token t0 + 32 tb + 8(r/4) + 4*half + r%4,
  // expert e0 + 64 ebk + 32 eb + lane%32
  float* dst = out + size_t(blockIdx.z) * size_t(T) * E;
#pragma unroll
  for (int eb = 0; eb < 2; ++eb) {
    const int n = e0 + ebk * 64 + 32 * eb + l32;
    if (n >= E) continue;
    const float bv = (KS == 1 && bias) ? bias[n] : 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = tb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (t0 + m < T) dst[size_t(t0 + m) * E + n] = ((eb ? acc1[r] : acc0[r]) + bv) + 0.0f;
    }
  }
}

__global__ __launch_bounds__(kTopkThreads) void route_topk_kernel(RouteArgs a) { topk_block(a, blockIdx.x); }

// Few-token routing in one launch (T <= kSmallRouteMaxT, from x). Workgroup e
// (256 threads) computes the logits of expert e for every token: thread i takes
// the 8-element chunks i, i + 256, ... of H, adds x_t . W_r[e] over them with
// v_dot2 (fp32), and the partial sums are reduced in a fixed tree (lane
// exchanges, then the four waves in order). With E workgroups of one expert
// each, every workgroup has all of its loads in flight at once.
//
// Hand-off without cache-wide fences. Each logit goes to its own 64-bit slot
// in the workspace as (1 << 32 | float bits), written with one agent-scope
// atomic store; each workgroup then counts itself on an agent-scope counter.
// The workgroup that counts last reads every slot with agent-scope atomic
// loads and re-reads a slot until its marker bit is set, so it can only ever
// use the value this call wrote: no ordering between the slot stores and the
// counter is needed for correctness (AMDGPU memory model: atomics at agent
// scope are coherent for every workgroup; a store becomes visible to the
// loads in finite time), so a workgroup counts itself without waiting for its
// slot stores to complete. The reader
// then zeroes the slots and the counter (agent-scope atomic stores; the next
// call's workgroups start after this kernel ends), writes the logits to
// logits_out, and runs the top-k, softmax and tables as a single routing
// block with its threads (one wave per token). A release/acquire pair on
// the counter instead costs a write-back of the L2 per workgroup: 12.3 us
// against 9.9 us for this kernel at T = 1. Up to 4 tokens a workgroup has 256
// threads and 4 experts; at 5..8 tokens, 512 threads (8 waves for the top-k)
// and 8 experts, one wave each.
constexpr int kSmallThreads = 256;
constexpr int kSmallRouteMaxT = 8;                       // tokens of the one-launch routing
constexpr uint64_t kSlotPollTicks = 20000000;            // 200 ms of the 100 MHz counter: bound on one slot's wait
constexpr int kSmallEpw = 4;                             // experts per workgroup (up to 4 tokens)
static_assert(kSmallRouteMaxT == kHandoffTokens && kMaxExperts <= 256, "slot layout of the workspace head");
__host__ __device__ constexpr int small_threads(int tb) { return tb <= 4 ? kSmallThreads : 64 * tb; }
constexpr int kSmallStageMaxH = 2048;                    // rows staged in LDS at 3..8 tokens: up to 32 KB

// c + a.lo * b.lo + a.hi * b.hi for two packed bf16 pairs (fp32). The pairs are
// taken as plain 32-bit values: bit-casting a vector element expression in
// place reads element 0 with this compiler.
__device__ __forceinline__ float bf16_dot2(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// EPW experts per workgroup: 256 / EPW threads per expert, each taking every
// (256 / EPW)-th 8-element chunk of H; up to kSmallChunks chunks per thread
// are loaded before the first product.
constexpr int kSmallChunks = 8;

template <int TB, int EPW>   // token bucket: TB >= T tokens are computed, rows past T repeat row T-1 and are not stored
__global__ __launch_bounds__(small_threads(TB)) void route_small_kernel(RouteArgs a, int32_t* done, uint64_t* slots) {
  constexpr int NT = small_threads(TB);
  constexpr int TPE = NT / EPW;                            // threads per expert
  constexpr bool STAGE = TB >= 4;                          // rows staged in LDS
  constexpr int CHUNKS = STAGE ? 4 : kSmallChunks;         // weight chunk loads in flight per thread
  static_assert(EPW == 1 || (TPE <= kWave && kWave % TPE == 0), "an expert's threads: the workgroup or part of one wave");
  static_assert(TB <= NT / kWave && TB <= kSmallRouteMaxT, "one wave per token in the top-k");
  __shared__ float red[NT / kWave][TB];
  __shared__ float lg[TB * kMaxExperts];
  __shared__ int last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ej = tid / TPE, q = tid % TPE;
  const int e = blockIdx.x * EPW + ej;
  const int T = a.T, H = a.H, E = a.E;
  const int nch = H / 8;
  float acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = 0.0f;
  if constexpr (STAGE) {
    // 3..8 tokens: the rows (rows past T repeat row T-1) are staged once in
    // LDS (dynamic, TB * H bf16) and read there by every expert's wave; the
    // first weight chunks' loads are issued before the staging. (With the
    // rows in registers as below, the compiler interleaves their loads with
    // the products at 4 and more tokens: several round trips instead of one.)
    extern __shared__ __align__(16) u32x4 xsm[];   // [TB][nch]
    const uint16_t* wr = a.wr + size_t(min(e, E - 1)) * H;
    u32x4 wv[CHUNKS];
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) wv[i] = *reinterpret_cast<const u32x4*>(wr + min(q + i * TPE, nch - 1) * 8);
    // at most XPT chunks per thread (H <= kSmallStageMaxH), all loaded before
    // the first store: a fixed count, so no loop-carried wait on the loads
    constexpr int XPT = TB * (kSmallStageMaxH / 8) / NT;
    const int nx = TB * nch;
    u32x4 v[XPT];
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int ic = min(j * NT + tid, nx - 1);
      const int r = ic / nch, ch = ic - r * nch;
      v[j] = *reinterpret_cast<const u32x4*>(a.x + size_t(min(r, T - 1)) * H + ch * 8);
    }
#pragma unroll
    for (int j = 0; j < XPT; ++j)
      if (j * NT + tid < nx) xsm[j * NT + tid] = v[j];
    __syncthreads();
    for (int c0 = q; c0 < nch; c0 += CHUNKS * TPE) {
      if (c0 != q) {
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) wv[i] = *reinterpret_cast<const u32x4*>(wr + min(c0 + i * TPE, nch - 1) * 8);
      }
#pragma unroll
      for (int i = 0; i < CHUNKS; ++i) {
        if (c0 + i * TPE >= nch) wv[i] = u32x4{0u, 0u, 0u, 0u};
        const int ch = min(c0 + i * TPE, nch - 1);
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          const u32x4 xv = xsm[t * nch + ch];
          acc[t] = bf16_dot2(wv[i].x, xv.x, acc[t]);
          acc[t] = bf16_dot2(wv[i].y, xv.y, acc[t]);
          acc[t] = bf16_dot2(wv[i].z, xv.z, acc[t]);
          acc[t] = bf16_dot2(wv[i].w, xv.w, acc[t]);
        }
      }
    }
  } else if (e < E) {
    const uint16_t* wr = a.wr + size_t(e) * H;
    for (int c0 = q; c0 < nch; c0 += CHUNKS * TPE) {
      // every load of up to CHUNKS chunks is issued before the first product
      u32x4 wv[CHUNKS], xv[CHUNKS][TB];
#pragma unroll
      for (int i = 0; i < CHUNKS; ++i) {
        const int ch = min(c0 + i * TPE, nch - 1);
        wv[i] = *reinterpret_cast<const u32x4*>(wr + ch * 8);
#pragma unroll
        for (int t = 0; t < TB; ++t)
          xv[i][t] = *reinterpret_cast<const u32x4*>(a.x + size_t(min(t, T - 1)) * H + ch * 8);
      }
      // chunks past the end (their loads re-read the last chunk) enter with
      // zero weights: no branch, so the compiler keeps every load ahead of
      // the first product instead of one round trip per chunk
#pragma unroll
      for (int i = 0; i < CHUNKS; ++i) {
        if (c0 + i * TPE >= nch) wv[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          acc[t] = bf16_dot2(wv[i].x, xv[i][t].x, acc[t]);
          acc[t] = bf16_dot2(wv[i].y, xv[i][t].y, acc[t]);
          acc[t] = bf16_dot2(wv[i].z, xv[i][t].z, acc[t]);
          acc[t] = bf16_dot2(wv[i].w, xv[i][t].w, acc[t]);
        }
      }
    }
  }
  // fixed reduction tree: lane exchanges within the expert's threads, then (one
  // expert per workgroup) the four waves in order
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    float v = acc[t];
#pragma unroll
    for (int m = (TPE < kWave ? TPE : kWave) / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    acc[t] = v;
    if (EPW == 1 && lane == 0) red[wave][t] = v;
  }
  if (EPW == 1) __syncthreads();
  if (q < T && e < E) {   // thread q of expert e stores token q's logit
    float v;
    if (EPW == 1) {
      static_assert(EPW > 1 || NT == 4 * kWave, "one expert per workgroup: four waves");
      v = (red[0][q] + red[1][q]) + (red[2][q] + red[3][q]);
    } else {
      v = acc[0];
#pragma unroll
      for (int t = 1; t < TB; ++t) v = q == t ? acc[t] : v;
    }
    if (a.bias) v = v + a.bias[e];
    v = v + 0.0f;   // turns -0 into +0
    __hip_atomic_store(slots + q * E + e, (uint64_t(1) << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (tid == 0)
    last = __hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == int(gridDim.x) - 1;
  __syncthreads();
  if (!last) return;   // uniform
  // collect the logits (waiting for any slot not yet visible) into LDS and
  // logits_out, and zero the slots. The wait for a slot is bounded by the
  // real-time counter; one that runs out sets the workspace's status word
  // (`done` is the workspace base) and the call's results are invalid.
  for (int i = tid; i < T * E; i += NT) {
    uint64_t v = __hip_atomic_load(slots + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((v >> 32) == 0) {
      const uint64_t t0 = wall_clock64();
      do {
        for (int n = 0; n < 64 && (v >> 32) == 0; ++n)
          v = __hip_atomic_load(slots + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } while ((v >> 32) == 0 && wall_clock64() - t0 <= kSlotPollTicks);
      if ((v >> 32) == 0)
        __hip_atomic_store(reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(done) + MOE_WORKSPACE_STATUS_OFFSET),
                           1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __hip_atomic_store(slots + i, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float f = __uint_as_float(uint32_t(v));
    a.logits_out[i] = f;
    lg[i] = f;
  }
  if (tid == 0) __hip_atomic_store(done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  RouteArgs b = a;
  b.logits_in = lg;   // the top-k reads the logits from LDS (generic pointer)
  b.coherent = 0;
  b.n_parts = 1;
  b.bias = nullptr;
  b.logits_out = nullptr;
  b.finish = 1;
  topk_block(b, 0);
}

// Per-expert scan over the routing blocks, 16 experts per workgroup:
// block_base[b][e] = sum of block_counts[b'][e] over b' < b, and
// counts[e] = the sum over all blocks. Thread (e, p) sums a contiguous range
// of blocks, the 16 ranges of an expert are scanned in LDS, and each thread
// writes the bases of its range.
constexpr int kScanExperts = 16;
constexpr int kScanParts = kRouteThreads / kScanExperts;

// Workgroups past the scan's run the activation preparation of the grouped
// GEMM (prep_rows.h), which needs nothing from the routing: it fills the GPU
// while the few scan workgroups and the scatter that follows run.
static_assert(kPrepThreads == kRouteThreads, "one block size for the scan and the preparation");
__global__ __launch_bounds__(kRouteThreads) void route_scan_kernel(ScanArgs a, PrepArgs prep) {
  __shared__ int32_t part[kScanParts][kScanExperts];
  const int nscan = ceil_div(a.E, kScanExperts);
  if (int(blockIdx.x) >= nscan) {   // uniform
    prep_rows_block(prep, long(blockIdx.x) - nscan);
    return;
  }
  const int tid = threadIdx.x;
  const int el = tid % kScanExperts, p = tid / kScanExperts;
  const int e = blockIdx.x * kScanExperts + el;
  const bool ok = e < a.E;
  const int chunk = ceil_div(a.nblk, kScanParts);
  const int b0 = min(a.nblk, p * chunk), b1 = min(a.nblk, b0 + chunk);
  int32_t s = 0;
  if (ok) {
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      int32_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = a.block_counts[size_t(b + i) * a.E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[i];
    }
    for (; b < b1; ++b) s += a.block_counts[size_t(b) * a.E + e];
  }
  part[p][el] = s;
  __syncthreads();
  if (tid < kScanExperts) {
    int32_t run = 0;
    for (int q = 0; q < kScanParts; ++q) {
      const int32_t v = part[q][tid];
      part[q][tid] = run;
      run += v;
    }
    if (blockIdx.x * kScanExperts + tid < a.E) a.counts[blockIdx.x * kScanExperts + tid] = run;
  }
  __syncthreads();
  if (ok) {
    int32_t run = part[p][el];
    for (int b = b0; b < b1; ++b) {
      a.block_base[size_t(b) * a.E + e] = run;
      run += a.block_counts[size_t(b) * a.E + e];
    }
  }
}

// Final row of each pair: its expert's offset (exclusive scan of counts,
// recomputed by every workgroup) + its block's base + its rank in the block.
// Workgroup 0 also writes offsets and the block map.
__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(ScatterArgs a, ScanArgs sa) {
  __shared__ int32_t off_s[kMaxExperts];
  __shared__ int32_t scan_tot[2 * (kRouteThreads / kWave)];
  const int tid = threadIdx.x;
  const int E = a.E;
  const int c = tid < E ? sa.counts[tid] : 0;
  const int ntl = ceil_div(c, sa.block_rows);
  int32_t oc = c, tc = ntl;   // inclusive scans of counts and tile counts
  block_scan2(oc, tc, scan_tot);
  if (tid < E) off_s[tid] = oc - c;   // exclusive: the expert's first row
  if (blockIdx.x == 0 && tid < E) {
    const int o = oc - c;
    sa.offsets[tid] = o;
    const int first = tc - ntl;
    for (int i = 0; i < ntl; ++i) {
      sa.tile_map[2 * (first + i)] = tid;
      sa.tile_map[2 * (first + i) + 1] = o + i * sa.block_rows;
    }
    if (tid == E - 1) {
      sa.offsets[E] = oc;
      *sa.num_tiles = tc;
    }
  }
  __syncthreads();
  const int blk = blockIdx.x;
  const int t0 = blk * kRouteTokens;
  const int nt = min(kRouteTokens, a.T - t0);
  const int npairs = nt * a.k;
  for (int p = tid; p < npairs; p += kRouteThreads) {
    const size_t f = size_t(t0) * a.k + p;
    const int e = a.topk_ids[f];
    const int pos = off_s[e] + a.block_base[size_t(blk) * E + e] + a.rank_in_block[f];
    a.sorted_rows[pos] = int32_t(f);
    a.row_of_pair[f] = pos;
  }
}

// Scan and scatter in one launch, for calls of at most kFusedScanBlocks
// routing blocks: workgroup b < nblk sums every block's count of expert
// e = thread (all blocks: the expert's total; blocks before b: the base of
// block b) from the block counts, scans the totals as route_scatter_kernel
// does, and places its block's pairs; workgroup 0 also writes counts,
// offsets and the block map. Every workgroup reads the whole count matrix
// (nblk x E words, from L2), which replaces the scan launch and its block
// bases. Workgroups past nblk run the activation preparation. (At 256 blocks,
// T = 4096, each thread's 256 count loads go out 32 at a time; the fused
// launch measured ~4 us faster than the scan and scatter launches there.)
constexpr int kFusedScanBlocks = 256;
__global__ __launch_bounds__(kRouteThreads) void route_scan_scatter_kernel(ScatterArgs a, ScanArgs sa,
                                                                           PrepArgs prep) {
  __shared__ int32_t off_s[kMaxExperts];
  __shared__ int32_t base_s[kMaxExperts];
  __shared__ int32_t scan_tot[2 * (kRouteThreads / kWave)];
  const int blk = blockIdx.x;
  if (blk >= sa.nblk) {   // uniform
    prep_rows_block(prep, long(blk) - sa.nblk);
    return;
  }
  const int tid = threadIdx.x;
  const int E = a.E;
  int c = 0, base = 0;
  if (tid < E) {
    // block order, so the block base is the running sum when block blk is reached
    int b = 0;
    for (; b + 32 <= sa.nblk; b += 32) {
      int32_t v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = sa.block_counts[size_t(b + i) * E + tid];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        base += (b + i < blk) ? v[i] : 0;
        c += v[i];
      }
    }
    for (; b < sa.nblk; ++b) {
      const int32_t v = sa.block_counts[size_t(b) * E + tid];
      base += b < blk ? v : 0;
      c += v;
    }
  }
  const int ntl = ceil_div(c, sa.block_rows);
  int32_t oc = c, tc = ntl;   // inclusive scans of counts and tile counts
  block_scan2(oc, tc, scan_tot);
  if (tid < E) {
    off_s[tid] = oc - c;
    base_s[tid] = base;
  }
  if (blk == 0 && tid < E) {
    const int o = oc - c;
    sa.counts[tid] = c;
    sa.offsets[tid] = o;
    const int first = tc - ntl;
    for (int i = 0; i < ntl; ++i) {
      sa.tile_map[2 * (first + i)] = tid;
      sa.tile_map[2 * (first + i) + 1] = o + i * sa.block_rows;
    }
    if (tid == E - 1) {
      sa.offsets[E] = oc;
      *sa.num_tiles = tc;
    }
  }
  __syncthreads();
  const int t0 = blk * kRouteTokens;
  const int nt = min(kRouteTokens, a.T - t0);
  const int npairs = nt * a.k;
  for (int p = tid; p < npairs; p += kRouteThreads) {
    const size_t f = size_t(t0) * a.k + p;
    const int e = a.topk_ids[f];
    const int pos = off_s[e] + base_s[e] + a.rank_in_block[f];
    a.sorted_rows[pos] = int32_t(f);
    a.row_of_pair[f] = pos;
  }
}

int router_splits(int T, int H, int E) {
  // Up to about a thousand tokens the single-wave 32 x 64 tiles are few (16 x 4
  // = 64 workgroups at T = 512), so K is split 8 ways. Above that the 64 x 128
  // tile kernel runs, with K split so that about 512 workgroups (two per CU)
  // stream the operands. The top-k kernel adds the partials in plane order.
  int ks;
  if (T <= kRouterTileMinT) {
    ks = 8;
  } else {
    const int tiles = ceil_div(T, kRtTok) * ceil_div(E, kRtExp);
    ks = 1;
    while (ks < 8 && tiles * ks * 2 <= 512) ks <<= 1;
  }
  while (ks > 1 && H % (64 * ks) != 0) ks >>= 1;
  return ks;
}

hipError_t launch_route(const RouteArgs& ra, const ScanArgs& sa, const ScatterArgs& ca, bool from_x,
                        hipStream_t stream, const PrepArgs* prep, bool* prep_done) {
  if (prep_done) *prep_done = false;
  const int nblk = ceil_div(ra.T, kRouteTokens);
  const int nrb = ceil_div(ra.T, kRouterRows);
  RouteArgs rb = ra;
  // one routing block: the top-k kernel also builds the tables
  rb.finish = nblk == 1 ? 1 : 0;
  rb.block_rows = sa.block_rows;
  rb.counts = sa.counts;
  rb.offsets = sa.offsets;
  rb.tile_map = sa.tile_map;
  rb.num_tiles = sa.num_tiles;
  rb.sorted_rows = ca.sorted_rows;
  rb.row_of_pair = ca.row_of_pair;
  if (from_x && ra.T <= kSmallRouteMaxT && ra.done && ra.slots && ra.logits_out && ra.H % 8 == 0 &&
      (ra.T <= 2 || ra.H <= kSmallStageMaxH)) {
    // one launch: complete logits per expert slice, top-k by the last workgroup
    // (measured faster than the MFMA router + top-k launches up to 8 tokens;
    // its per-token cost is higher, so larger calls keep the two launches)
    constexpr int EPW = kSmallEpw;
    const dim3 grid(ceil_div(ra.E, EPW)), block(kSmallThreads);
    if (ra.T <= 1)
      hipLaunchKernelGGL((route_small_kernel<1, EPW>), grid, block, 0, stream, rb, ra.done, ra.slots);
    else if (ra.T <= 2)
      hipLaunchKernelGGL((route_small_kernel<2, EPW>), grid, block, 0, stream, rb, ra.done, ra.slots);
    else if (ra.T <= 4)
      hipLaunchKernelGGL((route_small_kernel<4, EPW>), grid, block, size_t(4) * ra.H * 2, stream, rb, ra.done,
                         ra.slots);
    else
      hipLaunchKernelGGL((route_small_kernel<kSmallRouteMaxT, 8>), dim3(ceil_div(ra.E, 8)),
                         dim3(small_threads(kSmallRouteMaxT)), size_t(kSmallRouteMaxT) * ra.H * 2, stream, rb,
                         ra.done, ra.slots);
    return hipGetLastError();
  }
  if (from_x) {
    // logits (biased) into logits_out, or K-range partials into logit_parts
    // that the top-k kernel sums (adding the bias, writing logits_out)
    const int ks = router_splits(ra.T, ra.H, ra.E);
    float* dst = ks > 1 ? ra.logit_parts : ra.logits_out;
    if (ra.T <= kRouterTileMinT)
      hipLaunchKernelGGL(router_logits_kernel, dim3(nrb, ceil_div(ra.E, 64), ks), dim3(kWave),
                         kRouterRing * kRouterSlot, stream, ra.x, ra.wr, ra.bias, ra.T, ra.H, ra.E, dst);
    else
      hipLaunchKernelGGL(router_tile_kernel, dim3(ceil_div(ra.T, kRtTok), ceil_div(ra.E, kRtExp), ks),
                         dim3(kRtThreads), kRtRing * kRtSlot, stream, ra.x, ra.wr, ra.bias, ra.T, ra.H, ra.E, dst);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (ks > 1) {
      rb.logits_in = ra.logit_parts;
      rb.n_parts = ks;
    } else {
      rb.logits_in = ra.logits_out;
      rb.n_parts = 1;
      rb.bias = nullptr;
      rb.logits_out = nullptr;
    }
  } else {
    rb.n_parts = 1;
    rb.logits_out = nullptr;
  }
  hipLaunchKernelGGL(route_topk_kernel, dim3(nblk), dim3(kTopkThreads), 0, stream, rb);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || rb.finish) return err;
  const long nprep = prep ? prep_rows_blocks(prep->rows, prep->K) : 0;
  if (prep_done) *prep_done = prep != nullptr;
  if (nblk <= kFusedScanBlocks) {
    hipLaunchKernelGGL(route_scan_scatter_kernel, dim3(unsigned(nblk + nprep)), dim3(kRouteThreads), 0, stream, ca,
                       sa, prep ? *prep : PrepArgs{});
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_scan_kernel, dim3(unsigned(ceil_div(ra.E, kScanExperts) + nprep)), dim3(kRouteThreads), 0,
                     stream, sa, prep ? *prep : PrepArgs{});
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nblk), dim3(kRouteThreads), 0, stream, ca, sa);
  return hipGetLastError();
}

}  // namespace moe
