// GPU-resident MoE routing for gfx950: router GEMM + top-k + softmax, per-block
// histogram, prefix scan, stable scatter and block map, with no host
// synchronisation between the steps (page "Perplexity Open Sources Lily ..."
// Technical Details, Model bullet: the router picks 8 of 256 experts; prefill
// bullet: routing histogram, prefix scan, scatter and block map stay on the GPU).
//
// Launches on one stream:
//   0. router_logits_kernel (layer path only) - logits = x W_r^T (+ bias) with
//      bf16 MFMA and fp32 accumulation, 32 tokens x 64 experts per workgroup.
//   1. route_topk_kernel  - one workgroup per 16 tokens, one wave per token:
//      top-k by the key (logit desc, expert asc) through a ballot radix
//      select, softmax over the chosen k, the block's expert histogram and
//      each pair's rank among the block's pairs of the same expert.
//   2. route_scan_kernel  - one workgroup: per-expert scan over blocks, exclusive
//      scan over experts (offsets), and the tile list of the block map.
//   3. route_scatter_kernel - one workgroup per 16 tokens: final row of each
//      pair = block base of its expert + its in-block rank.
// Ranks count only earlier pairs, so the sort is stable and the result does not
// depend on thread timing: repeated runs give identical tables.
#include "moe_internal.h"

namespace moe {

constexpr int kRouteThreads = 256;
constexpr int kRouterRows = 32;                          // tokens per router-GEMM workgroup (one MFMA block)
constexpr int kTopkThreads = kRouteTokens * kWave;       // top-k: one wave per token
constexpr int kMaxKeysPerLane = kMaxExperts / kWave;

// Router GEMM: logits[t][e] = fp32(sum_h x[t][h] W_r[e][h]) + bias[e] for a
// 32-token x 64-expert tile per workgroup. The four waves split K in 64-wide
// chunks (wave w takes chunks w, w+4, ...), accumulate two 32x32 blocks each
// with bf16 MFMA, prefetch the next chunk while multiplying the current one,
// and reduce their partial sums through LDS.
__global__ __launch_bounds__(kRouteThreads) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                                     const uint16_t* __restrict__ wr,
                                                                     const float* __restrict__ bias, int T, int H,
                                                                     int E, float* __restrict__ logits) {
  __shared__ float red[4][2][16][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int t0 = blockIdx.x * kRouterRows;
  const int e0 = blockIdx.y * 64;
  const int nt = min(kRouterRows, T - t0);
  const bool row_ok = l32 < nt;
  const int n0 = e0 + l32, n1 = e0 + 32 + l32;
  const bool ok0 = n0 < E, ok1 = n1 < E;
  const uint16_t* xr = x + size_t(t0 + (row_ok ? l32 : 0)) * H + 32 * half;
  const uint16_t* w0 = wr + size_t(ok0 ? n0 : 0) * H + 32 * half;
  const uint16_t* w1 = wr + size_t(ok1 ? n1 : 0) * H + 32 * half;
  const int nchunks = H / 64;
  f32x16 acc0 = f32x16{}, acc1 = f32x16{};
  u32x4 ca[4], cb0[4], cb1[4];
  auto load = [&](int c, u32x4 (&A)[4], u32x4 (&B0)[4], u32x4 (&B1)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      A[j] = row_ok ? *reinterpret_cast<const u32x4*>(xr + c * 64 + 8 * j) : u32x4{0, 0, 0, 0};
      B0[j] = ok0 ? *reinterpret_cast<const u32x4*>(w0 + c * 64 + 8 * j) : u32x4{0, 0, 0, 0};
      B1[j] = ok1 ? *reinterpret_cast<const u32x4*>(w1 + c * 64 + 8 * j) : u32x4{0, 0, 0, 0};
    }
  };
  int c = wave;
  if (c < nchunks) load(c, ca, cb0, cb1);
  while (c < nchunks) {
    u32x4 na[4], nb0[4], nb1[4];
    const int cn = c + 4;
    if (cn < nchunks) load(cn, na, nb0, nb1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, ca[j]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, cb0[j]), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, cb1[j]), acc1, 0, 0, 0);
    }
    if (cn < nchunks) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ca[j] = na[j];
        cb0[j] = nb0[j];
        cb1[j] = nb1[j];
      }
    }
    c = cn;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    red[wave][0][r][lane] = acc0[r];
    red[wave][1][r][lane] = acc1[r];
  }
  __syncthreads();
  // output element (eb, r, lane): token 8(r/4) + 4*half + r%4, expert e0 + 32 eb + lane%32
  for (int i = tid; i < 2 * 16 * 64; i += kRouteThreads) {
    const int ln = i & 63, r = (i >> 6) & 15, eb = i >> 10;
    const float v = red[0][eb][r][ln] + red[1][eb][r][ln] + red[2][eb][r][ln] + red[3][eb][r][ln];
    const int m = 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
    const int n = e0 + 32 * eb + (ln & 31);
    if (m < nt && n < E) logits[size_t(t0 + m) * E + n] = (v + (bias ? bias[n] : 0.0f)) + 0.0f;
  }
}

// Top-k of one token held by one wave: lane l holds the order keys of experts
// l, l+64, l+128, l+192 (0 for experts >= E, below every finite logit's key).
// The k-th largest key tau is found by a most-significant-bit-first radix
// select whose counts are wave ballots; the chosen set is every key > tau plus
// the lowest-index experts with key == tau, which is the set the key
// (logit desc, expert asc) orders first.
__device__ __forceinline__ uint32_t kth_largest(const uint32_t (&u)[kMaxKeysPerLane], int k) {
  uint32_t tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < kMaxKeysPerLane; ++i) cnt += __popcll(__ballot(u[i] >= cand));
    tau = cnt >= k ? cand : tau;
  }
  return tau;
}

__global__ __launch_bounds__(kTopkThreads) void route_topk_kernel(RouteArgs a) {
  __shared__ uint32_t sel_key[kRouteTokens][kMaxTopk];
  __shared__ int32_t sel_e[kRouteTokens][kMaxTopk];
  __shared__ int32_t ids_s[kRouteTokens * kMaxTopk];
  __shared__ int32_t hist[kMaxExperts];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int blk = blockIdx.x;
  const int t0 = blk * kRouteTokens;
  const int nt = min(kRouteTokens, a.T - t0);
  const int E = a.E, k = a.k;
  const uint64_t below = (1ull << lane) - 1ull;

  for (int e = tid; e < E; e += kTopkThreads) hist[e] = 0;

  const int m = wave;                                            // this wave's token
  if (m < nt) {
    uint32_t u[kMaxKeysPerLane];
#pragma unroll
    for (int i = 0; i < kMaxKeysPerLane; ++i) {
      const int e = lane + 64 * i;
      uint32_t key = 0u;
      if (e < E) {
        float v = a.logits_in[size_t(t0 + m) * E + e];
        if (a.bias) v = v + a.bias[e];
        key = float_order_key(v + 0.0f);                         // + 0.0f turns -0 into +0
      }
      u[i] = key;
    }
    const uint32_t tau = kth_largest(u, k);
    int n_gt = 0;
    uint64_t tie[kMaxKeysPerLane];
#pragma unroll
    for (int i = 0; i < kMaxKeysPerLane; ++i) {
      n_gt += __popcll(__ballot(u[i] > tau));
      tie[i] = __ballot(u[i] == tau);
    }
    // ties at tau are taken in expert order: expert lane + 64 i ranks after
    // every tie of a lower i and after the lower lanes' ties of the same i
    const int need = k - n_gt;
    int ties_before = 0;
    int slot_base = 0;
#pragma unroll
    for (int i = 0; i < kMaxKeysPerLane; ++i) {
      const bool is_tie = (tie[i] >> lane) & 1ull;
      const int tie_rank = ties_before + __popcll(tie[i] & below);
      const bool chosen = u[i] > tau || (is_tie && tie_rank < need);
      const uint64_t cm = __ballot(chosen);
      if (chosen) {
        const int slot = slot_base + __popcll(cm & below);
        sel_key[m][slot] = u[i];
        sel_e[m][slot] = lane + 64 * i;
      }
      ties_before += __popcll(tie[i]);
      slot_base += __popcll(cm);
    }
    __builtin_amdgcn_wave_barrier();
    // lane j < k: its chosen element's position in (logit desc, expert asc) order
    int pos = 0;
    uint32_t my_key = 0;
    int my_e = 0;
    if (lane < k) {
      my_key = sel_key[m][lane];
      my_e = sel_e[m][lane];
      for (int q = 0; q < k; ++q) {
        const uint32_t kq = sel_key[m][q];
        const int eq = sel_e[m][q];
        pos += (kq > my_key || (kq == my_key && eq < my_e)) ? 1 : 0;
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < k) {
      sel_key[m][pos] = my_key;
      sel_e[m][pos] = my_e;
    }
    __builtin_amdgcn_wave_barrier();
    float my_l = 0.0f;
    if (lane < k) {
      my_e = sel_e[m][lane];
      my_l = float_from_order_key(sel_key[m][lane]);
    }
    const float l0 = float_from_order_key(sel_key[m][0]);
    const float ex = lane < k ? expf(my_l - l0) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) sum += __shfl_xor(sum, msk, kWave);
    if (lane < k) {
      const size_t f = size_t(t0 + m) * k + lane;
      a.topk_ids[f] = my_e;
      a.topk_w[f] = ex / sum;
      ids_s[m * k + lane] = my_e;
    }
  }
  __syncthreads();

  // Histogram of the block's pairs and each pair's rank among the earlier pairs
  // of the same expert (pair order f = t*k + j), which makes the scatter
  // stable. Wave 0 walks the pairs 64 at a time; lanes with the same expert
  // find each other through one ballot per expert-index bit.
  if (wave == 0) {
    const int npairs = nt * k;
    for (int c0 = 0; c0 < npairs; c0 += kWave) {
      const int p = c0 + lane;
      const int e = p < npairs ? ids_s[p] : kMaxExperts;   // past the end: a value no expert has
      uint64_t same = ~0ull;
#pragma unroll
      for (int bit = 0; bit < 9; ++bit) {
        const uint64_t bb = __ballot((e >> bit) & 1);
        same &= ((e >> bit) & 1) ? bb : ~bb;
      }
      if (p < npairs) {
        const int base = hist[e];
        const int before = __popcll(same & below);
        a.rank_in_block[size_t(t0) * k + p] = base + before;
        if (before == 0) hist[e] = base + __popcll(same);   // every lane of the group has read hist[e]
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kTopkThreads) a.block_counts[size_t(blk) * E + e] = hist[e];
}

// Inclusive scan of v over n <= 1024 entries held in LDS (one per thread).
__device__ void block_inclusive_scan(int32_t* v, int32_t* tmp, int n) {
  const int tid = threadIdx.x;
  for (int d = 1; d < n; d <<= 1) {
    int32_t x = 0;
    if (tid < n) x = v[tid] + (tid >= d ? v[tid - d] : 0);
    __syncthreads();
    if (tid < n) v[tid] = x;
    __syncthreads();
  }
  (void)tmp;
}

__global__ __launch_bounds__(1024) void route_scan_kernel(ScanArgs a) {
  __shared__ int32_t psum[1024];
  __shared__ int32_t cnt[kMaxExperts];
  __shared__ int32_t off[kMaxExperts];
  __shared__ int32_t ntl[kMaxExperts];
  const int tid = threadIdx.x;
  const int E = a.E;
  const int parts = 1024 / E;
  const int chunk = ceil_div(a.nblk, parts);
  const int e = tid % E;
  const int part = tid / E;
  const bool active = part < parts;
  const int b0 = part * chunk;
  const int b1 = min(a.nblk, b0 + chunk);

  if (active) {
    int32_t s = 0;
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      int32_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = a.block_counts[size_t(b + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[i];
    }
    for (; b < b1; ++b) s += a.block_counts[size_t(b) * E + e];
    psum[part * E + e] = s;
  }
  __syncthreads();
  if (tid < E) {
    int32_t run = 0;
    for (int p = 0; p < parts; ++p) {
      const int32_t v = psum[p * E + tid];
      psum[p * E + tid] = run;
      run += v;
    }
    cnt[tid] = run;
    off[tid] = run;
    ntl[tid] = ceil_div(run, a.block_rows);
  }
  __syncthreads();
  block_inclusive_scan(off, nullptr, E);   // inclusive scan of counts
  block_inclusive_scan(ntl, nullptr, E);   // inclusive scan of tiles per expert
  if (active) {
    int32_t run = off[e] - cnt[e] + psum[part * E + e];
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      int32_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = a.block_counts[size_t(b + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a.block_base[size_t(b + i) * E + e] = run;
        run += v[i];
      }
    }
    for (; b < b1; ++b) {
      a.block_base[size_t(b) * E + e] = run;
      run += a.block_counts[size_t(b) * E + e];
    }
  }
  if (tid < E) {
    const int32_t c = cnt[tid];
    const int32_t o = off[tid] - c;
    a.counts[tid] = c;
    a.offsets[tid] = o;
    const int nt_e = ceil_div(c, a.block_rows);
    const int t_first = ntl[tid] - nt_e;
    for (int i = 0; i < nt_e; ++i) {
      a.tile_map[2 * (t_first + i)] = tid;
      a.tile_map[2 * (t_first + i) + 1] = o + i * a.block_rows;
    }
    if (tid == E - 1) {
      a.offsets[E] = off[tid];
      *a.num_tiles = ntl[tid];
    }
  }
}

__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(ScatterArgs a) {
  const int blk = blockIdx.x;
  const int t0 = blk * kRouteTokens;
  const int nt = min(kRouteTokens, a.T - t0);
  const int npairs = nt * a.k;
  for (int p = threadIdx.x; p < npairs; p += kRouteThreads) {
    const size_t f = size_t(t0) * a.k + p;
    const int e = a.topk_ids[f];
    const int pos = a.block_base[size_t(blk) * a.E + e] + a.rank_in_block[f];
    a.sorted_rows[pos] = int32_t(f);
    a.row_of_pair[f] = pos;
  }
}

hipError_t launch_route(const RouteArgs& ra, const ScanArgs& sa, const ScatterArgs& ca, bool from_x,
                        hipStream_t stream) {
  const int nblk = ceil_div(ra.T, kRouteTokens);
  const int nrb = ceil_div(ra.T, kRouterRows);
  if (from_x) {
    // logits (biased) into logits_out, then top-k from them without the bias
    hipLaunchKernelGGL(router_logits_kernel, dim3(nrb, ceil_div(ra.E, 64)), dim3(kRouteThreads), 0, stream, ra.x,
                       ra.wr, ra.bias, ra.T, ra.H, ra.E, ra.logits_out);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    RouteArgs rb = ra;
    rb.logits_in = ra.logits_out;
    rb.bias = nullptr;
    rb.logits_out = nullptr;
    hipLaunchKernelGGL(route_topk_kernel, dim3(nblk), dim3(kTopkThreads), 0, stream, rb);
  } else {
    hipLaunchKernelGGL(route_topk_kernel, dim3(nblk), dim3(kTopkThreads), 0, stream, ra);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, sa);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nblk), dim3(kRouteThreads), 0, stream, ca);
  return hipGetLastError();
}

}  // namespace moe
