// GPU-resident MoE routing for gfx950: router GEMM + top-k + softmax, per-block
// histogram, prefix scan, stable scatter and block map, with no host
// synchronisation between the steps (page "Perplexity Open Sources Lily ..."
// Technical Details, Model bullet: the router picks 8 of 256 experts; prefill
// bullet: routing histogram, prefix scan, scatter and block map stay on the GPU).
//
// Launches on one stream:
//   0. router_logits_kernel (layer path only) - logits = x W_r^T (+ bias) with
//      bf16 MFMA and fp32 accumulation, 32 tokens x 64 experts per workgroup.
//   1. route_topk_kernel  - one workgroup per 32 tokens: top-k by the key
//      (logit desc, expert asc), softmax over the chosen k, the block's expert
//      histogram and each pair's rank among the block's pairs of the same expert.
//   2. route_scan_kernel  - one workgroup: per-expert scan over blocks, exclusive
//      scan over experts (offsets), and the tile list of the block map.
//   3. route_scatter_kernel - one workgroup per 32 tokens: final row of each
//      pair = block base of its expert + its in-block rank.
// Ranks count only earlier pairs, so the sort is stable and the result does not
// depend on thread timing: repeated runs give identical tables.
#include "moe_internal.h"

namespace moe {

constexpr int kRouteThreads = 256;
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
  const int t0 = blockIdx.x * kRouteTokens;
  const int e0 = blockIdx.y * 64;
  const int nt = min(kRouteTokens, T - t0);
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

__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(RouteArgs a) {
  extern __shared__ float lds_f[];
  float* lg = lds_f;                                          // [32][E]
  int32_t* ids_s = reinterpret_cast<int32_t*>(lg + kRouteTokens * a.E);  // [32*k]
  int32_t* hist = ids_s + kRouteTokens * a.k;                 // [E]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int blk = blockIdx.x;
  const int t0 = blk * kRouteTokens;
  const int nt = min(kRouteTokens, a.T - t0);
  const int E = a.E, k = a.k;

  for (int e = tid; e < E; e += kRouteThreads) hist[e] = 0;

  for (int i = tid; i < nt * E; i += kRouteThreads) {
    const int n = i % E;
    float v = a.logits_in[size_t(t0) * E + i];
    if (a.bias) v = v + a.bias[n];
    lg[i] = v + 0.0f;   // + 0.0f turns -0 into +0
  }
  __syncthreads();

  // Top-k: each wave selects for 8 tokens at once (lane holds experts lane +
  // 64 i of every token), so the 8 tokens' cross-lane max reductions are
  // independent and their shuffle latencies overlap.
  {
    constexpr int TPW = kRouteTokens / (kRouteThreads / kWave);   // tokens per wave
    const int mbase = wave * TPW;
    uint64_t key[TPW][kMaxKeysPerLane];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
      for (int i = 0; i < kMaxKeysPerLane; ++i) {
        const int e = lane + 64 * i;
        const int m = mbase + tt;
        key[tt][i] = (e < E && m < nt) ? (uint64_t(float_order_key(lg[m * E + e])) << 32) | uint32_t(0xFFFFFFFFu - e)
                                       : 0ull;
      }
    int my_e[TPW];
    float my_l[TPW];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      my_e[tt] = 0;
      my_l[tt] = 0.0f;
    }
    for (int j = 0; j < k; ++j) {
      uint64_t best[TPW];
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        best[tt] = key[tt][0];
#pragma unroll
        for (int i = 1; i < kMaxKeysPerLane; ++i) best[tt] = key[tt][i] > best[tt] ? key[tt][i] : best[tt];
      }
#pragma unroll
      for (int msk = 32; msk >= 1; msk >>= 1)
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
          const uint64_t o = shfl_xor_u64(best[tt], msk);
          best[tt] = o > best[tt] ? o : best[tt];
        }
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        const int ej = int(0xFFFFFFFFu - uint32_t(best[tt]));
#pragma unroll
        for (int i = 0; i < kMaxKeysPerLane; ++i)
          if (lane + 64 * i == ej) key[tt][i] = 0ull;
        if (lane == j) {
          my_e[tt] = ej;
          my_l[tt] = float_from_order_key(uint32_t(best[tt] >> 32));
        }
      }
    }
    float ex[TPW];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const float l0 = __shfl(my_l[tt], 0, kWave);
      ex[tt] = lane < k ? expf(my_l[tt] - l0) : 0.0f;
    }
    float sum[TPW];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) sum[tt] = ex[tt];
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1)
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) sum[tt] += __shfl_xor(sum[tt], msk, kWave);
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int m = mbase + tt;
      if (lane < k && m < nt) {
        const size_t f = size_t(t0 + m) * k + lane;
        a.topk_ids[f] = my_e[tt];
        a.topk_w[f] = ex[tt] / sum[tt];
        ids_s[m * k + lane] = my_e[tt];
      }
    }
  }
  __syncthreads();

  const int npairs = nt * k;
  for (int p = tid; p < npairs; p += kRouteThreads) atomicAdd(&hist[ids_s[p]], 1);
  // Rank of each pair among the earlier pairs of this block with the same
  // expert (pair order f = t*k + j), which makes the scatter stable.
  for (int p = tid; p < npairs; p += kRouteThreads) {
    const int e = ids_s[p];
    int r = 0;
    for (int q = 0; q < p; ++q) r += ids_s[q] == e;
    a.rank_in_block[size_t(t0) * k + p] = r;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) a.block_counts[size_t(blk) * E + e] = hist[e];
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
  const size_t lds = sizeof(float) * kRouteTokens * ra.E + sizeof(int32_t) * (kRouteTokens * ra.k + ra.E);
  if (from_x) {
    // logits (biased) into logits_out, then top-k from them without the bias
    hipLaunchKernelGGL(router_logits_kernel, dim3(nblk, ceil_div(ra.E, 64)), dim3(kRouteThreads), 0, stream, ra.x,
                       ra.wr, ra.bias, ra.T, ra.H, ra.E, ra.logits_out);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    RouteArgs rb = ra;
    rb.logits_in = ra.logits_out;
    rb.bias = nullptr;
    rb.logits_out = nullptr;
    hipLaunchKernelGGL(route_topk_kernel, dim3(nblk), dim3(kRouteThreads), lds, stream, rb);
  } else {
    hipLaunchKernelGGL(route_topk_kernel, dim3(nblk), dim3(kRouteThreads), lds, stream, ra);
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
