// Top-k selection, softmax and routing tables of one routing block of up to
// kRouteTokens tokens, run by one workgroup (shared by the routing kernels and
// the persistent decode kernel). Page "Perplexity Open Sources Lily ..."
// Technical Details (the router picks 8 of 256 experts; histogram, prefix
// scan, scatter and block map on the GPU).
#pragma once

#include "moe_internal.h"

namespace moe {

constexpr int kMaxKeysPerLane = kMaxExperts / kWave;
constexpr int kMaxCand = 64;   // candidates of the fast top-k path (token_topk)

// A token's logits from NP K-range partial planes (plane stride `plane`):
// every load is issued before the first add, and the planes are added in
// order, so the result does not depend on when the loads return.
template <int NP>
__device__ __forceinline__ void sum_parts(const float* parts, size_t plane, const size_t (&f)[kMaxKeysPerLane],
                                          float (&v)[kMaxKeysPerLane]) {
  float pv[kMaxKeysPerLane][NP];
#pragma unroll
  for (int i = 0; i < kMaxKeysPerLane; ++i)
#pragma unroll
    for (int p = 0; p < NP; ++p) pv[i][p] = parts[size_t(p) * plane + f[i]];
#pragma unroll
  for (int i = 0; i < kMaxKeysPerLane; ++i) {
    v[i] = pv[i][0];
#pragma unroll
    for (int p = 1; p < NP; ++p) v[i] += pv[i][p];
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

// Inclusive scan of one int over the 64 lanes of a wave with DPP: shifts by
// 1, 2, 4 and 8 inside each row of 16 lanes, then the last lane of row 0
// (and of row 2) into rows 1 (and 3), and lane 31 into rows 2 and 3. Lanes
// with no source add 0. Only VALU operations, no LDS round trip.
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2, 3
  return v;
}

// Inclusive scans of two per-thread values over the whole workgroup (thread
// order), one value pair per thread: a DPP scan inside each wave, then each
// wave adds the totals of the waves before it. tot holds 2 x (waves) ints of
// LDS; every thread of the workgroup must call this.
__device__ __forceinline__ void block_scan2(int32_t& a, int32_t& b, int32_t* tot) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nw = blockDim.x >> 6;
  a = wave_scan_incl(a);
  b = wave_scan_incl(b);
  if (lane == kWave - 1) {
    tot[w] = a;
    tot[nw + w] = b;
  }
  __syncthreads();
  int32_t pa = 0, pb = 0;
  for (int i = 0; i < w; ++i) {
    pa += tot[i];
    pb += tot[nw + i];
  }
  a += pa;
  b += pb;
}

// Top-k of one token held by one wave (keys as in kth_largest): leaves the k
// chosen keys and experts in (logit desc, expert asc) order in sel_key[0..k-1]
// and sel_e[0..k-1]; cand is kMaxCand entries of scratch. All three are the
// wave's own LDS rows.
__device__ __forceinline__ void token_topk(const uint32_t (&u)[kMaxKeysPerLane], int k, uint64_t* cand,
                                           uint32_t* sel_key, int32_t* sel_e) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  // Fast path. Let mk be the k-th largest of the 64 lanes' largest keys: at
  // least k keys are >= mk, so the k-th largest key is >= mk and every chosen
  // key is among the candidates {keys >= mk}; every other key is strictly
  // smaller than all chosen ones. The threshold used is mk with its low 16
  // bits cleared (<= mk, so the candidates still hold every chosen key; a
  // 16-pass radix on the lane maxima' top halves finds it). The candidates
  // (usually about k) are gathered in LDS as key << 32 | ~expert, which orders
  // them as (logit desc, expert asc) does, and lane j counts the candidates
  // above its own: that count is its position, and positions 0..k-1 are the
  // chosen experts, in order. Exact ties that leave more than kMaxCand
  // candidates take the general path.
  uint32_t mx = u[0];
#pragma unroll
  for (int i = 1; i < kMaxKeysPerLane; ++i) mx = u[i] > mx ? u[i] : mx;
  const uint32_t mxh = mx >> 16;
  uint32_t ph = 0;
  for (int b = 15; b >= 0; --b) {
    const uint32_t cand = ph | (1u << b);
    ph = __popcll(__ballot(mxh >= cand)) >= k ? cand : ph;
  }
  const uint32_t thr = ph << 16;
  uint64_t cmask[kMaxKeysPerLane];
  int n_cand = 0;
#pragma unroll
  for (int i = 0; i < kMaxKeysPerLane; ++i) {
    cmask[i] = __ballot(u[i] >= thr);
    n_cand += __popcll(cmask[i]);
  }
  if (n_cand <= kMaxCand) {   // uniform
    int base = 0;
#pragma unroll
    for (int i = 0; i < kMaxKeysPerLane; ++i) {
      if ((cmask[i] >> lane) & 1ull)
        cand[base + __popcll(cmask[i] & below)] = (uint64_t(u[i]) << 32) | uint32_t(~uint32_t(lane + 64 * i));
      base += __popcll(cmask[i]);
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < n_cand) {
      const uint64_t mine = cand[lane];
      int pos = 0;
      for (int q0 = 0; q0 < n_cand; q0 += 8) {
        uint64_t cq[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) cq[q] = cand[min(q0 + q, n_cand - 1)];
#pragma unroll
        for (int q = 0; q < 8; ++q) pos += int(q0 + q < n_cand) & int(cq[q] > mine);
      }
      if (pos < k) {
        sel_key[pos] = uint32_t(mine >> 32);
        sel_e[pos] = int(~uint32_t(mine));
      }
    }
    __builtin_amdgcn_wave_barrier();
  } else {
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
        sel_key[slot] = u[i];
        sel_e[slot] = lane + 64 * i;
      }
      ties_before += __popcll(tie[i]);
      slot_base += __popcll(cm);
    }
    __builtin_amdgcn_wave_barrier();
    // lane j < k: its chosen element's position in (logit desc, expert asc)
    // order, counted without branches over all k chosen elements (read in
    // groups of eight, each group's loads issued together)
    int pos = 0;
    uint32_t my_key = 0;
    int my_e = 0;
    if (lane < k) {
      my_key = sel_key[lane];
      my_e = sel_e[lane];
      for (int q0 = 0; q0 < k; q0 += 8) {
        uint32_t kq[8];
        int eq[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          kq[q] = sel_key[min(q0 + q, k - 1)];
          eq[q] = sel_e[min(q0 + q, k - 1)];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
          pos += int(q0 + q < k) & (int(kq[q] > my_key) | (int(kq[q] == my_key) & int(eq[q] < my_e)));
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < k) {
      sel_key[pos] = my_key;
      sel_e[pos] = my_e;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Softmax over a token's chosen logits (sel_key in rank order): lane j < k gets
// its expert and weight; the k terms are added in rank order.
__device__ __forceinline__ void token_softmax(const uint32_t* sel_key, const int32_t* sel_e, int k, int& my_e,
                                              float& wgt) {
  const int lane = threadIdx.x & 63;
  float my_l = 0.0f;
  my_e = 0;
  if (lane < k) {
    my_e = sel_e[lane];
    my_l = float_from_order_key(sel_key[lane]);
  }
  const float l0 = float_from_order_key(sel_key[0]);
  const float ex = lane < k ? expf(my_l - l0) : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
  wgt = ex / sum;
}

// The tables of a single routing block of at most 64 pairs (the few-token
// case), built by one wave: the same results as the general path of
// topk_block below (stable ranks, offsets, block map, scatter, descriptors).
// Lane p holds pair p; lane l holds experts l, l + 64, l + 128, l + 192 for
// the counts. Every count and tile count is at most 64, so an expert's count
// and tile count and those of the expert 64 above it share one 32-bit word (8
// bits each) and two DPP scans give every offset and first tile. Each pair
// then finds its row and tile from its expert's offset and its rank; the
// first pair of a tile writes the block map entry and the descriptor, whose
// token nibbles the tile's pairs have OR-ed into LDS. hist: E zeros in LDS.
__device__ __forceinline__ void small_tables(const RouteArgs& a, const int32_t* ids_s, int32_t* hist, int np) {
  __shared__ int32_t off_w[kMaxExperts];
  __shared__ int32_t tf_w[kMaxExperts];
  __shared__ uint32_t tok_w[kWave];
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  const int E = a.E, k = a.k, bm = a.block_rows;
  const bool live = lane < np;
  const int e = live ? ids_s[lane] : kMaxExperts;   // past the end: a value no expert has
  uint64_t same = ~0ull;
#pragma unroll
  for (int bit = 0; bit < 9; ++bit) {
    const uint64_t bb = __ballot((e >> bit) & 1);
    same &= ((e >> bit) & 1) ? bb : ~bb;
  }
  const int rank = __popcll(same & below);
  const int cnt = __popcll(same);
  if (live && rank == 0) hist[e] = cnt;
  tok_w[lane] = 0u;
  __builtin_amdgcn_wave_barrier();
  static_assert(kMaxKeysPerLane == 4 && kWave <= 255, "two experts per word, 8-bit fields");
  int c[kMaxKeysPerLane], ntl[kMaxKeysPerLane];
#pragma unroll
  for (int i = 0; i < kMaxKeysPerLane; ++i) {
    const int ee = lane + 64 * i;
    c[i] = ee < E ? hist[ee] : 0;
    ntl[i] = ceil_div(c[i], bm);
  }
  const uint32_t p0 = uint32_t(c[0]) | uint32_t(ntl[0]) << 8 | uint32_t(c[1]) << 16 | uint32_t(ntl[1]) << 24;
  const uint32_t p1 = uint32_t(c[2]) | uint32_t(ntl[2]) << 8 | uint32_t(c[3]) << 16 | uint32_t(ntl[3]) << 24;
  const uint32_t s0 = uint32_t(wave_scan_incl(int(p0))), s1 = uint32_t(wave_scan_incl(int(p1)));
  const uint32_t x0 = s0 - p0, x1 = s1 - p1;   // exclusive, field by field (no borrow: s >= p per field)
  const uint32_t t0 = uint32_t(__builtin_amdgcn_readlane(int(s0), kWave - 1));
  const uint32_t t1 = uint32_t(__builtin_amdgcn_readlane(int(s1), kWave - 1));
  auto fld = [](uint32_t v, int f) { return int((v >> (8 * f)) & 0xFFu); };
  int o[kMaxKeysPerLane], tf[kMaxKeysPerLane];
  int base = 0, tbase = 0;
  o[0] = fld(x0, 0);
  tf[0] = fld(x0, 1);
  base += fld(t0, 0);
  tbase += fld(t0, 1);
  o[1] = base + fld(x0, 2);
  tf[1] = tbase + fld(x0, 3);
  base += fld(t0, 2);
  tbase += fld(t0, 3);
  o[2] = base + fld(x1, 0);
  tf[2] = tbase + fld(x1, 1);
  base += fld(t1, 0);
  tbase += fld(t1, 1);
  o[3] = base + fld(x1, 2);
  tf[3] = tbase + fld(x1, 3);
  base += fld(t1, 2);
  tbase += fld(t1, 3);
#pragma unroll
  for (int i = 0; i < kMaxKeysPerLane; ++i) {
    const int ee = lane + 64 * i;
    if (ee < E) {
      a.counts[ee] = c[i];
      a.offsets[ee] = o[i];
      off_w[ee] = o[i];
      tf_w[ee] = tf[i];
    }
  }
  if (lane == 0) {
    a.offsets[E] = base;
    *a.num_tiles = tbase;
  }
  __builtin_amdgcn_wave_barrier();
  int pos = 0, tile = 0, rr = 0;
  if (live) {
    pos = off_w[e] + rank;
    tile = tf_w[e] + rank / bm;
    rr = rank % bm;
    a.sorted_rows[pos] = lane;
    a.row_of_pair[lane] = pos;
    if (rr == 0) {
      a.tile_map[2 * tile] = e;
      a.tile_map[2 * tile + 1] = pos;
    }
    if (a.tile_desc && rr < 8) atomicOr(&tok_w[tile], uint32_t(lane / k) << (4 * rr));
  }
  if (!a.tile_desc) return;
  __builtin_amdgcn_wave_barrier();
  if (live && rr == 0) a.tile_desc[tile] = u32x4{uint32_t(e), uint32_t(pos), uint32_t(min(bm, cnt - rank)), tok_w[tile]};
}

// The tables of a routing block of one token: its k experts are distinct, so
// every count is 0 or 1, an expert's offset is the number of chosen experts
// below it (four ballots), and a pair's row (its tile, its rank in the
// sorted rows) is the number of the token's other experts below its own. The
// same results as small_tables, with no scan and no LDS round trip beyond the
// count flags. Run by one wave; hist: E zeros in LDS.
__device__ __forceinline__ void one_token_tables(const RouteArgs& a, const int32_t* ids_s, int32_t* hist) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  const int E = a.E, k = a.k;
  const bool live = lane < k;
  const int e = live ? ids_s[lane] : 0;
  if (live) hist[e] = 1;
  int rank = 0;
  for (int q = 0; q < k; ++q) rank += int(__builtin_amdgcn_readlane(e, q) < e);
  __builtin_amdgcn_wave_barrier();
  int c[kMaxKeysPerLane];
#pragma unroll
  for (int i = 0; i < kMaxKeysPerLane; ++i) c[i] = lane + 64 * i < E ? hist[lane + 64 * i] : 0;
  int base = 0;
#pragma unroll
  for (int i = 0; i < kMaxKeysPerLane; ++i) {
    const int ee = lane + 64 * i;
    const uint64_t m = __ballot(c[i] != 0);
    if (ee < E) {
      a.counts[ee] = c[i];
      a.offsets[ee] = base + __popcll(m & below);
    }
    base += __popcll(m);
  }
  if (lane == 0) {
    a.offsets[E] = k;
    *a.num_tiles = k;
  }
  if (live) {
    a.row_of_pair[lane] = rank;
    a.sorted_rows[rank] = lane;
    a.tile_map[2 * rank] = e;
    a.tile_map[2 * rank + 1] = rank;
    if (a.tile_desc) a.tile_desc[rank] = u32x4{uint32_t(e), uint32_t(rank), 1u, 0u};
  }
}

// Top-k, softmax, histogram and ranks of routing block blk (and, for a single
// block, the tables), run by one 1024-thread workgroup.
__device__ __forceinline__ void topk_block(const RouteArgs& a, int blk) {
  __shared__ uint32_t sel_key[kRouteTokens][kMaxTopk];
  __shared__ int32_t sel_e[kRouteTokens][kMaxTopk];
  __shared__ int32_t ids_s[kRouteTokens * kMaxTopk];
  __shared__ int32_t rank_s[kRouteTokens * kMaxTopk];
  __shared__ int32_t hist[kMaxExperts];
  __shared__ uint64_t cand[kRouteTokens][kMaxCand];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blk * kRouteTokens;
  const int nt = min(kRouteTokens, a.T - t0);
  const int E = a.E, k = a.k;
  const uint64_t below = (1ull << lane) - 1ull;

  const int nthr = blockDim.x;   // at least E and one wave per token of the block
  for (int e = tid; e < E; e += nthr) hist[e] = 0;

  const int m = wave;                                            // this wave's token
  if (m < nt) {
    // every load of the token's logits (or of their K-range partials) is
    // issued before the first use, so the wave waits for one round trip;
    // experts past E read the last expert's entry and get key 0
    float v[kMaxKeysPerLane];
    size_t f[kMaxKeysPerLane];
#pragma unroll
    for (int i = 0; i < kMaxKeysPerLane; ++i) f[i] = size_t(t0 + m) * E + min(lane + 64 * i, E - 1);
    if (a.n_parts == 8) {
      sum_parts<8>(a.logits_in, size_t(a.T) * E, f, v);
    } else if (a.n_parts == 4) {
      sum_parts<4>(a.logits_in, size_t(a.T) * E, f, v);
    } else if (a.n_parts == 2) {
      sum_parts<2>(a.logits_in, size_t(a.T) * E, f, v);
    } else if (a.coherent) {
#pragma unroll
      for (int i = 0; i < kMaxKeysPerLane; ++i)
        v[i] = __hip_atomic_load(a.logits_in + f[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
#pragma unroll
      for (int i = 0; i < kMaxKeysPerLane; ++i) {
        v[i] = a.logits_in[f[i]];
        for (int p = 1; p < a.n_parts; ++p) v[i] += a.logits_in[size_t(p) * a.T * E + f[i]];
      }
    }
    uint32_t u[kMaxKeysPerLane];
#pragma unroll
    for (int i = 0; i < kMaxKeysPerLane; ++i) {
      const int e = lane + 64 * i;
      uint32_t key = 0u;
      if (e < E) {
        float x = v[i];
        if (a.bias) x = x + a.bias[e];
        x = x + 0.0f;                                            // turns -0 into +0
        if (a.logits_out) a.logits_out[f[i]] = x;
        key = float_order_key(x);
      }
      u[i] = key;
    }
    token_topk(u, k, cand[m], sel_key[m], sel_e[m]);
    int my_e;
    float wgt;
    token_softmax(sel_key[m], sel_e[m], k, my_e, wgt);
    if (lane < k) {
      const size_t f = size_t(t0 + m) * k + lane;
      a.topk_ids[f] = my_e;
      a.topk_w[f] = wgt;
      ids_s[m * k + lane] = my_e;
    }
  }
  __syncthreads();

  const int npairs_all = nt * k;
  if (a.finish && nt == 1) {   // uniform
    if (wave == 0) one_token_tables(a, ids_s, hist);
    return;
  }
  if (a.finish && npairs_all <= kWave) {   // uniform
    if (wave == 0) small_tables(a, ids_s, hist, npairs_all);
    return;
  }

  // Histogram of the block's pairs and each pair's rank among the earlier pairs
  // of the same expert (pair order f = t*k + j), which makes the scatter
  // stable. Wave 0 walks the pairs 64 at a time; lanes with the same expert
  // find each other through one ballot per expert-index bit.
  if (wave == 0) {
    const int npairs = npairs_all;
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
        if (!a.finish) a.rank_in_block[size_t(t0) * k + p] = base + before;
        rank_s[p] = base + before;
        if (before == 0) hist[e] = base + __popcll(same);   // every lane of the group has read hist[e]
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  if (!a.finish) {   // uniform: the scan and scatter kernels follow
    for (int e = tid; e < E; e += nthr) a.block_counts[size_t(blk) * E + e] = hist[e];
    return;
  }

  // One block holds every pair: offsets are the exclusive scan of the
  // histogram, the block map lists ceil(count / block_rows) tiles per expert
  // in expert order, and each pair's row is its expert's offset plus its rank.
  __shared__ int32_t off_s[kMaxExperts];
  __shared__ int32_t scan_tot[2 * kRouteTokens];
  __shared__ int32_t sorted_s[kRouteTokens * kMaxTopk];
  const int c = tid < E ? hist[tid] : 0;
  const int ntl = ceil_div(c, a.block_rows);
  int32_t oc = c, tc = ntl;   // inclusive scans of counts and tile counts
  block_scan2(oc, tc, scan_tot);
  if (tid < E) {
    const int o = oc - c;
    off_s[tid] = o;
    a.counts[tid] = c;
    a.offsets[tid] = o;
    const int first = tc - ntl;
    for (int i = 0; i < ntl; ++i) {
      a.tile_map[2 * (first + i)] = tid;
      a.tile_map[2 * (first + i) + 1] = o + i * a.block_rows;
    }
    if (tid == E - 1) {
      a.offsets[E] = oc;
      *a.num_tiles = tc;
    }
  }
  __syncthreads();
  for (int p = tid; p < npairs_all; p += nthr) {
    const int pos = off_s[ids_s[p]] + rank_s[p];
    a.sorted_rows[pos] = p;
    a.row_of_pair[p] = pos;
    sorted_s[pos] = p;
  }
  if (!a.tile_desc) return;   // uniform
  __syncthreads();
  if (tid < E && c > 0) {
    const int o = off_s[tid];
    const int first = tc - ntl;
    for (int i = 0; i < ntl; ++i) {
      const int r0 = o + i * a.block_rows;
      const int n = min(a.block_rows, c - i * a.block_rows);
      uint32_t tok = 0;
      for (int j = 0; j < n && j < 8; ++j) tok |= uint32_t(sorted_s[r0 + j] / k) << (4 * j);
      a.tile_desc[first + i] = u32x4{uint32_t(tid), uint32_t(r0), uint32_t(n), tok};
    }
  }
}

}  // namespace moe
