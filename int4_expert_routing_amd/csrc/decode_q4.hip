// Decode-shaped expert GEMVs for gfx950: the same per-expert products as the
// grouped GEMM (gemm_q4.hip), laid out for the few-token case where each expert
// sees at most 8 rows and the layer is bound by streaming the chosen experts'
// 4-bit weights from HBM (page "Perplexity Open Sources Lily ..." Technical
// Details, decode bullet: decode reads the active experts' weights once per
// token; itinai.com post: expansion of the 4-bit weights on chip only).
//
// Arithmetic (exact operand, fp32 accumulation, as in the grouped GEMM): each
// code becomes the bf16 value 1 + q/16, a v_dot2 with the row's activations
// accumulates P_g = sum_{k in g} x_k (1 + q_k/16) per 64-wide group, and the
// group folds as acc += 16 s_g P_g + (b_g - 16 s_g) X_g, where X_g is the
// row's group sum, computed in fp32 from the staged row.
#include "gemm_tiles.h"
#include "route_block.h"

namespace moe {

constexpr uint32_t kDecRsrcWord3 = 0x00020000u;   // raw buffer descriptor flags (gfx9 family)

typedef __attribute__((address_space(3))) void* dec_lds_t;

// LDS row layout for lanes that read `parts` equal consecutive slices of K (4
// per wave: one per lane quarter): slice i starts 16*i bytes later than an
// unpadded layout would put it, so the four quarters of a wave read four
// distinct bank ranges.
__host__ __device__ constexpr int dec_row_bytes(int K, int parts = 4) { return 2 * K + 16 * parts; }
__device__ __forceinline__ int dec_off(int K, int r, int k, int parts = 4) {
  return r * dec_row_bytes(K, parts) + 2 * k + (k / (K / parts)) * 16;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// GQ consecutive bf16 values in one load: the scale and bias arrays are
// 16-byte aligned and a lane's GQ values start at a multiple of 2*GQ bytes.
template <int GQ>
__device__ __forceinline__ void load_groups(const uint16_t* p, uint16_t (&v)[GQ]) {
  if constexpr (GQ == 8) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = uint16_t(ws[i]);
      v[2 * i + 1] = uint16_t(ws[i] >> 16);
    }
  } else if constexpr (GQ == 4) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    v[0] = uint16_t(w.x);
    v[1] = uint16_t(w.x >> 16);
    v[2] = uint16_t(w.y);
    v[3] = uint16_t(w.y >> 16);
  } else if constexpr (GQ == 2) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    v[0] = uint16_t(w);
    v[1] = uint16_t(w >> 16);
  } else {
    v[0] = p[0];
  }
}

// Scale or bias values of GQ consecutive groups g0.. of one column from a
// packed stack's pair plane [n][G/2][N] u32 (GQ >= 2 implies g0 even).
template <int GQ>
__device__ __forceinline__ void load_group_pairs(const uint16_t* plane, int el, int G, int N, int col, int g0,
                                                 uint16_t (&v)[GQ]) {
  const uint32_t* pl = reinterpret_cast<const uint32_t*>(plane) + (size_t(el) * (G / 2) + g0 / 2) * N + col;
  if constexpr (GQ == 1) {
    const uint32_t w = pl[0];
    v[0] = uint16_t((g0 & 1) ? (w >> 16) : w);
  } else {
    uint32_t w[GQ / 2];
#pragma unroll
    for (int i = 0; i < GQ / 2; ++i) w[i] = pl[size_t(i) * N];
#pragma unroll
    for (int i = 0; i < GQ / 2; ++i) {
      v[2 * i] = uint16_t(w[i]);
      v[2 * i + 1] = uint16_t(w[i] >> 16);
    }
  }
}

// The codes a lane streams: STEPS 16-byte steps covering GQ = STEPS/2 groups
// g0.. of one column (step st = half st%2 of group g0 + st/2), from either
// layout.
template <int STEPS>
__device__ __forceinline__ void load_code_steps(const QStack& m, int el, int N, int K, int col, int g0,
                                                u32x4 (&w)[STEPS]) {
  const int G = K / kGroup;
  if (m.packed) {
#pragma unroll
    for (int st = 0; st < STEPS; ++st)
      w[st] = *reinterpret_cast<const u32x4*>(m.q + ((size_t(el) * G + g0 + st / 2) * N + col) * 8 + (st & 1) * 4);
  } else {
    const u32x4* qp = reinterpret_cast<const u32x4*>(m.q + (size_t(el) * N + col) * (K / 8) + g0 * 8);
#pragma unroll
    for (int st = 0; st < STEPS; ++st) w[st] = qp[st];
  }
}

template <int GQ>
__device__ __forceinline__ void load_scale_bias(const QStack& m, int el, int N, int K, int col, int g0,
                                                uint16_t (&sv)[GQ], uint16_t (&bv)[GQ]) {
  const int G = K / kGroup;
  if (m.packed) {
    load_group_pairs<GQ>(m.s, el, G, N, col, g0, sv);
    load_group_pairs<GQ>(m.b, el, G, N, col, g0, bv);
  } else {
    const size_t wrow = size_t(el) * N + col;
    load_groups<GQ>(m.s + wrow * G + g0, sv);
    load_groups<GQ>(m.b + wrow * G + g0, bv);
  }
}

// ---------------------------------------------------------------------------
// Gate/up projection with SwiGLU (few-token calls).
//
// Workgroup = (row tile, 16 columns of h), 2*KS waves: wave w computes the gate
// (w even) or up (w odd) matrix's 16 columns over slice w/2 of KS equal slices
// of K. Its 64 lanes are 16 columns x 4 quarters of the slice, so a lane
// streams STEPS*16 contiguous code bytes of one column into registers; every
// code, scale and bias load is issued at once, so the weight stream is in
// flight while the activation rows are staged in LDS (put into the operand
// order [0,4,1,5,2,6,3,7] per 8-element chunk on the way). A tile's expert,
// rows and their tokens come from one 16-byte descriptor written by the
// routing, so a workgroup waits on one dependent load before its weight
// stream starts. Quarters are summed with two lane exchanges, slices in LDS in
// a fixed order, and h = silu(gate) * up is written in bf16 in the operand
// order the down projection reads.
template <int STEPS, int KS>
struct DecShape {
  static constexpr int K = STEPS * 128 * KS;
  static constexpr int G = K / kGroup;
  static constexpr int GQ = STEPS / 2;     // groups per lane
  static constexpr int W = 2 * KS;         // waves
  static constexpr int PARTS = 4 * KS;     // lane slices of K
};

// LDS of one workgroup whose tiles have at most nr rows: activation rows
// [nr][row bytes] and their group sums [nr][K/64] f32; the epilogue reuses the
// row area (at least as large as its [W][nr][16] f32 + [nr][16] bf16).
__host__ __device__ constexpr int dec_xt_off(int steps, int ks, int nr) {
  return nr * dec_row_bytes(steps * 128 * ks, 4 * ks);
}
__host__ __device__ constexpr int dec_lds_bytes(int steps, int ks, int nr) {
  return dec_xt_off(steps, ks, nr) + nr * (steps * 128 * ks / kGroup) * 4;
}

struct DecTile {
  int e, r0, n;
  uint32_t tok;   // token of row j at bits 4j..4j+3
};

// h_tag: null (h stored as bf16 into a.out), or the persistent kernel's tagged
// h rows [rows][N/2] (each u64: tag << 32 | two bf16 of h in operand order)
template <int NR, int STEPS, int KS>
__device__ __forceinline__ void swiglu_tile(const GemmArgs& a, const DecTile& ti, int cb, uint8_t* smem, int nrmax,
                                            uint64_t* h_tag = nullptr, uint32_t tag = 0) {
  using S = DecShape<STEPS, KS>;
  constexpr int K = S::K, G = S::G, GQ = S::GQ, PARTS = S::PARTS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, kq = lane >> 4;
  const int up = wave & 1, ks = wave >> 1;
  const int slice = ks * 4 + kq;            // the lane's slice of K
  uint8_t* xs = smem;
  float* Xt = reinterpret_cast<float*>(smem + dec_xt_off(STEPS, KS, nrmax));

  // ---- this lane's codes, scales and biases into registers -----------------
  const int stack = ti.e == a.E ? 1 : 0;
  const int el = stack ? 0 : ti.e;
  const QStack& mat = up ? a.w1[stack] : a.w0[stack];
  u32x4 w[STEPS];
  load_code_steps<STEPS>(mat, el, a.N, K, cb * 16 + c, slice * GQ, w);
  uint16_t sv[GQ], bv[GQ];
  load_scale_bias<GQ>(mat, el, a.N, K, cb * 16 + c, slice * GQ, sv, bv);

  // ---- activation rows (operand order) and their group sums into LDS -------
  // every chunk load of the rows is issued before the first store
  constexpr int kChunks = NR * (K / 8), kPer = (kChunks + S::W * 64 - 1) / (S::W * 64);
  u32x4 xv[kPer];
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int i = min(tid + it * S::W * 64, kChunks - 1);
    const int r = i / (K / 8), ch = i % (K / 8);
    const int src = int((ti.tok >> (4 * r)) & 15u);
    xv[it] = *reinterpret_cast<const u32x4*>(a.A + size_t(src) * K + ch * 8);
  }
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int i = tid + it * S::W * 64;
    if (i < kChunks) {
      const int r = i / (K / 8), ch = i % (K / 8);
      *reinterpret_cast<u32x4*>(xs + dec_off(K, r, ch * 8, PARTS)) = permute_chunk(xv[it]);
    }
  }
  __syncthreads();
  for (int i = tid; i < NR * G; i += S::W * 64) {
    const int r = i / G, g = i % G;
    float sum = 0.0f;
#pragma unroll
    for (int ch = 0; ch < 8; ++ch)
      sum += chunk_sum(*reinterpret_cast<const u32x4*>(xs + dec_off(K, r, g * kGroup + ch * 8, PARTS)));
    Xt[r * G + g] = sum;
  }
  __syncthreads();

  // ---- dot products over the lane's slice -----------------------------------
  float acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.0f;
  const uint32_t nib = kNib, magic = kMagic;
#pragma unroll
  for (int gl = 0; gl < GQ; ++gl) {
    float P[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) P[r] = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int st = 2 * gl + h;
      const uint32_t wd[4] = {w[st].x, w[st].y, w[st].z, w[st].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 p = __builtin_bit_cast(u32x4, unpack_word(wd[j], nib, magic));
        const int k0 = slice * (K / PARTS) + 32 * st + 8 * j;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const u32x4 xv = *reinterpret_cast<const u32x4*>(xs + dec_off(K, r, k0, PARTS));
          P[r] = dot2(p.x, xv.x, P[r]);
          P[r] = dot2(p.y, xv.y, P[r]);
          P[r] = dot2(p.z, xv.z, P[r]);
          P[r] = dot2(p.w, xv.w, P[r]);
        }
      }
    }
    const float s16 = 16.0f * __uint_as_float(uint32_t(sv[gl]) << 16);
    const float off = __uint_as_float(uint32_t(bv[gl]) << 16) - s16;
    const int g = slice * GQ + gl;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      acc[r] = __builtin_fmaf(s16, P[r], acc[r]);
      acc[r] = __builtin_fmaf(off, Xt[r * G + g], acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    acc[r] += __shfl_xor(acc[r], 16, kWave);
    acc[r] += __shfl_xor(acc[r], 32, kWave);
  }

  // ---- slices summed in order, SwiGLU, bf16 h in operand order -------------
  __syncthreads();   // every wave is done with the rows (the epilogue reuses them)
  float* part = reinterpret_cast<float*>(smem);                               // [W][NR][16]
  uint16_t* hs = reinterpret_cast<uint16_t*>(part + S::W * NR * 16);          // [NR][16]
  if (lane < 16) {
#pragma unroll
    for (int r = 0; r < NR; ++r) part[(wave * NR + r) * 16 + c] = acc[r];
  }
  __syncthreads();
  if (tid < NR * 16) {
    const int r = tid >> 4, cc = tid & 15;
    float gv = 0.0f, uv = 0.0f;
#pragma unroll
    for (int k2 = 0; k2 < KS; ++k2) {
      gv += part[((2 * k2) * NR + r) * 16 + cc];
      uv += part[((2 * k2 + 1) * NR + r) * 16 + cc];
    }
    const float hv = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
    hs[r * 16 + cc] = uint16_t(f32_to_bf16_rne(hv));
  }
  __syncthreads();
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  if (tid < NR * 2) {
    // row tid/2, chunk tid%2 of this column block, stored in the operand order
    const int r = tid >> 1, ch = tid & 1;
    const u32x4 v = permute_chunk(*reinterpret_cast<const u32x4*>(hs + r * 16 + ch * 8));
    if (h_tag) {
      uint64_t* dst = h_tag + size_t(ti.r0 + r) * (a.N / 2) + (cb * 16 + ch * 8) / 2;
      const uint64_t hi = uint64_t(tag) << 32;
      __hip_atomic_store(dst + 0, hi | v.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(dst + 1, hi | v.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(dst + 2, hi | v.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(dst + 3, hi | v.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      *reinterpret_cast<u32x4*>(out + size_t(ti.r0 + r) * a.N + cb * 16 + ch * 8) = v;
    }
  }
}

// Tiles: the shared expert's (one tile of all T rows), then the routed
// tiles' descriptors. Register budget: 64 VGPRs, so that 8 waves fit per SIMD
// (four 8-wave workgroups per CU at K = 2048) and more of the weight stream is
// in flight; the compiler keeps the few values past that budget in scratch
// (T=8 layer 45.9 -> 44.2 us; 67 VGPRs before).
template <int STEPS, int KS>
__global__ __launch_bounds__(2 * KS * 64) __attribute__((amdgpu_waves_per_eu(8)))
void decode_swiglu_kernel(GemmArgs a, const u32x4* tile_desc, int nrmax) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tile = blockIdx.x / a.NT;
  const int cb = blockIdx.x % a.NT;
  DecTile ti;
  if (tile < a.n_shared_tiles) {
    // the shared expert: one tile of every token's row (row routed_rows + t
    // is token t), so its weights stream once per call
    ti.e = a.E;
    ti.r0 = a.routed_rows;
    ti.n = a.shared_rows;
    ti.tok = 0u;
    for (int j = 0; j < a.shared_rows; ++j) ti.tok |= uint32_t(j) << (4 * j);
  } else {
    const int i = tile - a.n_shared_tiles;
    if (!a.routed_tiles) return;
    const int nt = *a.num_tiles;
    const u32x4 d = tile_desc[i];   // in bounds for every launched tile; used only if i < nt
    if (i >= nt) return;
    ti.e = int(d.x);
    ti.r0 = int(d.y);
    ti.n = int(d.z);
    ti.tok = d.w;
  }
  switch (ti.n) {
    case 1: swiglu_tile<1, STEPS, KS>(a, ti, cb, smem, nrmax); break;
    case 2: swiglu_tile<2, STEPS, KS>(a, ti, cb, smem, nrmax); break;
    case 3: swiglu_tile<3, STEPS, KS>(a, ti, cb, smem, nrmax); break;
    case 4: swiglu_tile<4, STEPS, KS>(a, ti, cb, smem, nrmax); break;
    case 5: swiglu_tile<5, STEPS, KS>(a, ti, cb, smem, nrmax); break;
    case 6: swiglu_tile<6, STEPS, KS>(a, ti, cb, smem, nrmax); break;
    case 7: swiglu_tile<7, STEPS, KS>(a, ti, cb, smem, nrmax); break;
    case 8: swiglu_tile<8, STEPS, KS>(a, ti, cb, smem, nrmax); break;
    default: break;   // callers guarantee 1..nrmax rows per tile, nrmax <= kDecodeMaxRows
  }
}

// ---------------------------------------------------------------------------
// Down projection fused with the weighted combine (few-token calls).
//
// Workgroup = (token t, 16 output columns), W = min(k + 1, 16) waves. The
// token's pairs are j = 0..k-1 (routed expert topk_ids[t][j], h row
// row_of_pair[t*k+j], weight topk_w[t][j]) and j = k (the shared expert, h row
// shared_row0 + t, weight 1). Wave w takes pairs w, w + W, ...: it stages the
// pair's h row and its group sums in its own LDS area, streams the 16 columns'
// codes of that expert straight into registers (lane = column c x quarter kq
// of K, as in the kernel above) and accumulates w_j * (h . Wd column) in pair
// order. The waves' sums are then added in wave order, so the result does not
// depend on timing, and y[t] is rounded to bf16 once.
__host__ __device__ constexpr int dc_wave_bytes(int K) { return dec_row_bytes(K) + (K / kGroup) * 4; }
constexpr int kDcMaxWaves = 16;

// One (token t, 16 output columns) unit of the down projection and combine,
// run by the W waves of a workgroup (LDS: W * dc_wave_bytes(K) + W * 33 floats).
// pair(j) gives (expert, h row, weight) of the token's routed pair j < k;
// stage_row(row, xs) writes that h row (K bf16 in operand order) into the
// wave's LDS row xs with the wave's 64 lanes.
struct DcPair {
  int el, row;
  float w;
};

template <int STEPS, class PairFn, class RowFn>
__device__ __forceinline__ void down_combine_unit(const DownCombineArgs& a, int t, int col0, int W, uint8_t* smem,
                                                  PairFn pair, RowFn stage_row) {
  constexpr int K = STEPS * 128;
  constexpr int G = K / kGroup;
  constexpr int GQ = STEPS / 2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, kq = lane >> 4;
  uint8_t* wl = smem + wave * dc_wave_bytes(K);
  uint8_t* xs = wl;                                                     // the pair's h row
  float* Xt = reinterpret_cast<float*>(wl + dec_row_bytes(K));          // its group sums
  float* red = reinterpret_cast<float*>(smem + W * dc_wave_bytes(K));   // [W][16]
  float* sred = red + W * 16;                                           // [W][16] gated shared pair
  float* gpart = sred + W * 16;                                         // [W] gate partial sums
  const uint32_t nib = kNib, magic = kMagic;
  const bool gated = a.shared_gate != nullptr;

  // gated shared expert: this thread's part of x_t . w_sg (added in a fixed
  // order after the pairs); the shared pair then enters with weight g
  if (gated) {
    float d = 0.0f;
    for (int cc = tid * 8; cc < a.N; cc += W * 64 * 8) {
      const u32x4 xv = *reinterpret_cast<const u32x4*>(a.x + size_t(t) * a.N + cc);
      const u32x4 wv = *reinterpret_cast<const u32x4*>(a.shared_gate + cc);
      d = dot2(xv.x, wv.x, d);
      d = dot2(xv.y, wv.y, d);
      d = dot2(xv.z, wv.z, d);
      d = dot2(xv.w, wv.w, d);
    }
    d = wave_sum_f32(d);
    if (lane == 0) gpart[wave] = d;
  }

  float tot = 0.0f, sacc = 0.0f;
  for (int j = wave; j <= a.k; j += W) {
    const bool routed = j < a.k;
    DcPair pj{0, a.shared_row0 + t, 1.0f};
    if (routed) pj = pair(j);
    const QStack& mat = routed ? a.down : a.down_shared;
    // the lane's codes: quarter kq of its column's K (GQ groups)
    u32x4 w[STEPS];
    load_code_steps<STEPS>(mat, pj.el, a.N, K, col0 + c, kq * GQ, w);
    uint16_t sv[GQ], bv[GQ];
    load_scale_bias<GQ>(mat, pj.el, a.N, K, col0 + c, kq * GQ, sv, bv);
    // stage the h row (already in operand order) and its fp32 group sums
    __builtin_amdgcn_wave_barrier();   // the previous pair's reads of xs and Xt are done
    stage_row(pj.row, xs);
    __builtin_amdgcn_wave_barrier();
    if (lane < G) {
      float sum = 0.0f;
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) sum += chunk_sum(*reinterpret_cast<const u32x4*>(xs + dec_off(K, 0, lane * kGroup + ch * 8)));
      Xt[lane] = sum;
    }
    __builtin_amdgcn_wave_barrier();
    float acc = 0.0f;
#pragma unroll
    for (int gl = 0; gl < GQ; ++gl) {
      float P = 0.0f;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int s = 2 * gl + hh;
        const uint32_t wd[4] = {w[s].x, w[s].y, w[s].z, w[s].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 pv = __builtin_bit_cast(u32x4, unpack_word(wd[q], nib, magic));
          const u32x4 xv = *reinterpret_cast<const u32x4*>(xs + dec_off(K, 0, kq * (K / 4) + 32 * s + 8 * q));
          P = dot2(pv.x, xv.x, P);
          P = dot2(pv.y, xv.y, P);
          P = dot2(pv.z, xv.z, P);
          P = dot2(pv.w, xv.w, P);
        }
      }
      const float s16 = 16.0f * __uint_as_float(uint32_t(sv[gl]) << 16);
      const float off = __uint_as_float(uint32_t(bv[gl]) << 16) - s16;
      acc = __builtin_fmaf(s16, P, acc);
      acc = __builtin_fmaf(off, Xt[kq * GQ + gl], acc);
    }
    acc += __shfl_xor(acc, 16, kWave);
    acc += __shfl_xor(acc, 32, kWave);
    if (routed || !gated)
      tot = __builtin_fmaf(pj.w, acc, tot);
    else
      sacc = acc;
  }
  if (lane < 16) {
    red[wave * 16 + lane] = tot;
    sred[wave * 16 + lane] = sacc;
  }
  __syncthreads();
  if (tid < 16) {
    float sum = 0.0f;
    for (int i = 0; i < W; ++i) sum += red[i * 16 + tid];
    if (gated) {
      float z = 0.0f, sv = 0.0f;
      for (int i = 0; i < W; ++i) {
        z += gpart[i];
        sv += sred[i * 16 + tid];
      }
      sum = __builtin_fmaf(1.0f / (1.0f + expf(-z)), sv, sum);
    }
    a.y[size_t(t) * a.N + col0 + tid] = uint16_t(f32_to_bf16_rne(sum));
  }
}

template <int STEPS>
__global__ __launch_bounds__(kDcMaxWaves * 64) void decode_down_combine_kernel(DownCombineArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int K = STEPS * 128;
  const int ncb = a.N / 16;
  const int t = blockIdx.x / ncb;
  const int col0 = (blockIdx.x % ncb) * 16;
  const int lane = threadIdx.x & 63;
  auto pair = [&](int j) {
    const size_t f = size_t(t) * a.k + j;
    return DcPair{a.topk_ids[f], a.row_of_pair[f], a.topk_w[f]};
  };
  auto stage_row = [&](int row, uint8_t* xs) {
    const uint16_t* hr = a.h + size_t(row) * K;
    for (int ch = lane; ch < K / 8; ch += 64)
      *reinterpret_cast<u32x4*>(xs + dec_off(K, 0, ch * 8)) = *reinterpret_cast<const u32x4*>(hr + ch * 8);
  };
  down_combine_unit<STEPS>(a, t, col0, int(blockDim.x >> 6), smem, pair, stage_row);
}

bool decode_down_combine_supported(int N, int K) {
  const int steps = K / 128;
  return K % 128 == 0 && (steps == 2 || steps == 4 || steps == 8 || steps == 16) && N % 16 == 0;
}

hipError_t launch_decode_down_combine(const DownCombineArgs& da, hipStream_t stream) {
  if (!decode_down_combine_supported(da.N, da.K)) return hipErrorInvalidValue;
  if (da.T == 0) return hipSuccess;
  const int W = da.k + 1 < kDcMaxWaves ? da.k + 1 : kDcMaxWaves;
  const dim3 grid(unsigned(da.T) * unsigned(da.N / 16)), block(unsigned(W) * 64u);
  const size_t lds = size_t(W) * dc_wave_bytes(da.K) + size_t(W) * (2 * 16 + 1) * 4;
  switch (da.K / 128) {
    case 2: hipLaunchKernelGGL(decode_down_combine_kernel<2>, grid, block, lds, stream, da); break;
    case 4: hipLaunchKernelGGL(decode_down_combine_kernel<4>, grid, block, lds, stream, da); break;
    case 8: hipLaunchKernelGGL(decode_down_combine_kernel<8>, grid, block, lds, stream, da); break;
    default: hipLaunchKernelGGL(decode_down_combine_kernel<16>, grid, block, lds, stream, da); break;
  }
  return hipGetLastError();
}

bool decode_supported(int N, int K) {
  return (K == 256 || K == 512 || K == 1024 || K == 2048) && N % 16 == 0;
}

hipError_t launch_decode(const GemmArgs& ga, const u32x4* tile_desc, int max_row_tiles, int max_rows,
                         hipStream_t stream) {
  if (!decode_supported(ga.N, ga.K) || ga.NT != ga.N / 16 || max_rows < 1 || max_rows > kDecodeMaxRows ||
      ga.n_shared_tiles != (ga.shared_rows > 0 ? 1 : 0) || ga.shared_rows > max_rows || !tile_desc)
    return hipErrorInvalidValue;
  const dim3 grid(unsigned(max_row_tiles) * unsigned(ga.NT));
  if (grid.x == 0) return hipSuccess;
  // K slices per column set: K/512 (at least 1, at most 4), so a lane streams
  // 64 or 128 codes and a workgroup has 2, 4 or 8 waves
  switch (ga.K) {
    case 256:
      hipLaunchKernelGGL((decode_swiglu_kernel<2, 1>), grid, dim3(128), dec_lds_bytes(2, 1, max_rows), stream, ga,
                         tile_desc, max_rows);
      break;
    case 512:
      hipLaunchKernelGGL((decode_swiglu_kernel<4, 1>), grid, dim3(128), dec_lds_bytes(4, 1, max_rows), stream, ga,
                         tile_desc, max_rows);
      break;
    case 1024:
      hipLaunchKernelGGL((decode_swiglu_kernel<4, 2>), grid, dim3(256), dec_lds_bytes(4, 2, max_rows), stream, ga,
                         tile_desc, max_rows);
      break;
    default:
      hipLaunchKernelGGL((decode_swiglu_kernel<4, 4>), grid, dim3(512), dec_lds_bytes(4, 4, max_rows), stream, ga,
                         tile_desc, max_rows);
      break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Persistent decode kernel: the whole few-token layer in one launch.
//
// The three launches above leave a chain of dependent memory round trips with
// a kernel boundary between each pair of stages; the weight stream itself is a
// small part of a decode call. Here one grid of workgroups takes work items in
// phase order (item index = phase order):
//   routing items (one wave per expert: the logits of every token),
//   gate/up items (one (row tile, 16 columns of h) each; tile 0 is the shared
//     expert, which needs no routing; tile i > 0 is the i-th chosen expert in
//     ascending order, with its rows),
//   down items (one (token, 16 output columns) each, the down projection fused
//     with the weighted combine).
// There is no routing hand-off item: the first gate/up or down item of a
// routed tile that a workgroup takes reads every token's logits, runs the same
// top-k and softmax as the routing kernels and builds the few-token tables
// (rows sorted by expert, then by pair) in its own LDS, which serve the
// workgroup's later items too. So a routed item waits for one global round
// trip after the router (the logits), not three (logits, top-k, descriptors).
// Workgroup b takes items b, b + gridDim.x, ... in increasing order, and every
// workgroup is resident at once (the host sizes the grid from the occupancy),
// so an item only ever waits for items of earlier phases, which their
// workgroups reach before any later item: no wait can block the grid. The
// kernel is instantiated per token bucket (1, 2, 4, 8), which keeps it within
// 128 VGPRs, two workgroups per CU: at T = 1 every item is resident at once.
//
// Hand-off without fences: every value one item passes to another (a logit, a
// pair of bf16 of h) is written as one 64-bit agent-scope atomic store
// tag << 32 | value, and read with agent-scope atomic loads until the tag
// matches (AMDGPU memory model: agent-scope atomics are coherent for every
// workgroup and become visible in finite time). The tag is the call's epoch
// + 1: every workgroup reads the epoch word when it starts, and the last
// workgroup to finish advances it (and returns the exit counter to zero), so a
// later call can never take a stale word for a fresh one. Every wait is
// bounded by the 100 MHz real-time counter; a wait that gives up writes 1 to
// the status word (the call's results are then invalid) instead of hanging
// the GPU.
// Waiting is cheap for the producers: a consumer first watches one counter of
// finished producer items with one lane and a back-off, and only then reads
// the tagged words it needs (which normally carry the tag by then; the tags,
// not the counters, make the values safe to use, so the counters need no
// fences either). Every polled word would otherwise draw a request from every
// lane of every waiting workgroup, and that traffic on a few cache lines
// delays the very stores it waits for. Adds to one word are serialised
// (~11 ns each, measured), so no counter has many producers: the routing items
// count into eight copies (a consumer watches the copy of its workgroup index
// mod 8), and each gate/up tile has its own counter, which its NT column items
// count into and the down items of its rows watch. Each counter has its own
// cache line.
constexpr int kFzThreads = 512;
constexpr int kFzWaves = kFzThreads / kWave;
constexpr int kFzMaxT = kDecodeMaxRows;
constexpr int kFzMaxPairs = 64;                              // T * k
constexpr int kFzMaxRows = kFzMaxPairs + kFzMaxT;            // routed + shared h rows
constexpr int kFzMaxHalfI = 256;                             // I <= 512
constexpr int kFzH = 2048;                                   // hidden size of the kernel
constexpr uint64_t kFzPollTicks = 20000000;                  // 200 ms of the 100 MHz counter
static_assert(kFzWaves >= kFzMaxT, "one wave per token in the local routing");
// byte offsets inside the region (the workspace head after the one-launch
// routing's part)
constexpr size_t kFzEpoch = 0, kFzExit = 64, kFzStatus = 128;
constexpr int kFzMaxTiles = 1 + kFzMaxPairs;                 // the shared tile + one per chosen expert
constexpr int kFzCntCopies = 8;                              // copies of the routing counter
constexpr size_t kFzLine = 128;                              // one counter per cache line
constexpr size_t kFzRouteCnt = 256;                                                 // [kFzCntCopies] lines
constexpr size_t kFzTileCnt = kFzRouteCnt + kFzCntCopies * kFzLine;                 // [kFzMaxTiles] lines
constexpr size_t kFzSlots = kFzTileCnt + kFzMaxTiles * kFzLine;                     // [kFzMaxT][kMaxExperts]
constexpr size_t kFzHrows = kFzSlots + size_t(kFzMaxT) * kMaxExperts * 8;          // [kFzMaxRows][kFzMaxHalfI]
constexpr size_t kFzBytes = kFzHrows + size_t(kFzMaxRows) * kFzMaxHalfI * 8;
static_assert(kHandoffBytes + kFzBytes == MOE_WORKSPACE_HEAD_BYTES, "workspace head size in the header");
static_assert(kFzCntCopies + kFzMaxTiles <= kFzThreads, "one thread per counter when the counters are reset");

__device__ __forceinline__ uint64_t fz_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fz_store(uint64_t* p, uint32_t tag, uint32_t v) {
  __hip_atomic_store(p, (uint64_t(tag) << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The values of N words once each carries the tag (need[i] == false: the lane
// waits for nothing there). Every lane of the wave calls this: all N loads go
// out together, and only words not yet tagged are read again; bounded as
// described above.
template <int N>
__device__ __forceinline__ void fz_wait_n(const uint64_t* const (&p)[N], const bool (&need)[N], uint32_t tag,
                                          uint32_t* status, uint32_t (&out)[N]) {
  uint64_t v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = need[i] ? fz_load(p[i]) : (uint64_t(tag) << 32);
  auto ready = [&]() {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok = ok && (v[i] >> 32) == tag;
    return ok;
  };
  if (!__all(ready())) {
    const uint64_t t0 = wall_clock64();
    while (true) {
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int i = 0; i < N; ++i)
        if ((v[i] >> 32) != tag) v[i] = fz_load(p[i]);
      if (__all(ready())) break;
      if (wall_clock64() - t0 > kFzPollTicks) {
        if (!ready()) __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = uint32_t(v[i]);
}

// Lane 0 of the calling wave watches the counter until it reaches n (bounded as
// above); returns to every lane once it does.
__device__ __forceinline__ void fz_wait_count(const uint32_t* cnt, uint32_t n, uint32_t* status) {
  uint32_t v = 0;
  if ((threadIdx.x & 63) == 0) {
    v = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v < n) {
      const uint64_t t0 = wall_clock64();
      while (true) {
        __builtin_amdgcn_s_sleep(4);
        v = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (v >= n) break;
        if (wall_clock64() - t0 > kFzPollTicks) {
          __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// This workgroup's item is done: its stores are complete (waited for by every
// wave), then thread i < copies counts the item in counter copy i (copies
// kFzLine bytes apart).
__device__ __forceinline__ void fz_count_done(uint8_t* cnt, int copies) {
  __builtin_amdgcn_s_waitcnt(0);   // this wave's stores have completed
  __syncthreads();
  if (int(threadIdx.x) < copies)
    __hip_atomic_fetch_add(reinterpret_cast<uint32_t*>(cnt + threadIdx.x * kFzLine), 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

struct FusedArgs {
  GemmArgs g;            // gate/up: A = x (natural order), E, N = I, K = H, NT = I / 16, shared_rows = T
  DownCombineArgs d;     // down + combine (its table pointers are unused: the kernel's own tables)
  const uint16_t* wr;    // router [E][H]
  const float* bias;     // [E] or null
  float* logits_out;     // [T][E] or null
  int32_t* ids_out;      // [T][k] or null
  float* w_out;          // [T][k] or null
  uint8_t* fz;           // the region described above
  int n_route, n_gu, n_dn;
};

// The few-token routing tables of one workgroup (LDS).
struct FzRoute {
  uint64_t cand[kFzMaxT][kMaxCand];
  uint32_t sel_key[kFzMaxT][kMaxTopk];
  int32_t sel_e[kFzMaxT][kMaxTopk];
  int32_t ids[kFzMaxPairs];       // pair t*k + j: expert
  float w[kFzMaxPairs];           //   weight
  int32_t row[kFzMaxPairs];       //   h row (expert-sorted order)
  int32_t first[kFzMaxPairs];     //   1 if no earlier pair has its expert
  int32_t row_tile[kFzMaxPairs];  // routed h row: its tile (1 + the index below)
  int32_t tile_e[kFzMaxPairs];    // routed tile i (the i-th chosen expert, ascending): expert
  int32_t tile_r0[kFzMaxPairs];   //   first h row
  int32_t tile_n[kFzMaxPairs];    //   rows
  uint32_t tile_tok[kFzMaxPairs]; //   token of row j at bits 4j..4j+3
  int32_t n_tiles;
};

// Routing item: wave w computes expert (item * kFzWaves + w)'s logit of every
// token. Lane l takes 8-element chunks l, l + 64, l + 128, l + 192 of H (added
// in that order) and the lanes meet in a fixed tree, as in the one-launch
// routing kernel, so both give the same bits. Every load is issued at once;
// from 3 tokens on, x is staged in LDS by the whole workgroup.
template <int TM>
__device__ __forceinline__ void fz_route_item(const FusedArgs& f, int item, uint32_t tag, uint8_t* smem) {
  constexpr int H = kFzH, NCH = H / 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = f.g.shared_rows, E = f.g.E;
  const int e = item * kFzWaves + wave;
  const uint16_t* wr = f.wr + size_t(min(e, E - 1)) * H;
  const uint16_t* x = f.g.A;
  u32x4 wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wv[i] = *reinterpret_cast<const u32x4*>(wr + (lane + 64 * i) * 8);
  float acc[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) acc[t] = 0.0f;
  if constexpr (TM <= 2) {
    u32x4 xv[TM][4];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xv[t][i] = *reinterpret_cast<const u32x4*>(x + size_t(min(t, T - 1)) * H + (lane + 64 * i) * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        acc[t] = dot2(wv[i].x, xv[t][i].x, acc[t]);
        acc[t] = dot2(wv[i].y, xv[t][i].y, acc[t]);
        acc[t] = dot2(wv[i].z, xv[t][i].z, acc[t]);
        acc[t] = dot2(wv[i].w, xv[t][i].w, acc[t]);
      }
  } else {
    // x [T][H] into LDS: chunk c of token t at (t * NCH + c) * 16
    constexpr int PER = TM * NCH / kFzThreads;
    u32x4 xs[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * kFzThreads;
      xs[i] = *reinterpret_cast<const u32x4*>(x + size_t(min(c, T * NCH - 1)) * 8);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * kFzThreads;
      if (c < T * NCH) *reinterpret_cast<u32x4*>(smem + c * 16) = xs[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        if (t < T) {
          const u32x4 xv = *reinterpret_cast<const u32x4*>(smem + (t * NCH + lane + 64 * i) * 16);
          acc[t] = dot2(wv[i].x, xv.x, acc[t]);
          acc[t] = dot2(wv[i].y, xv.y, acc[t]);
          acc[t] = dot2(wv[i].z, xv.z, acc[t]);
          acc[t] = dot2(wv[i].w, xv.w, acc[t]);
        }
      }
  }
  float mine = 0.0f;
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const float v = wave_sum_f32(acc[t]);
    mine = lane == t ? v : mine;
  }
  if (e < E && lane < T) {
    float v = mine;
    if (f.bias) v = v + f.bias[e];
    v = v + 0.0f;   // turns -0 into +0
    fz_store(reinterpret_cast<uint64_t*>(f.fz + kFzSlots) + lane * E + e, tag, __float_as_uint(v));
  }
}

// The workgroup's routing: wave m < T waits for token m's logits, selects its
// top-k and softmax weights (the same functions as the routing kernels, so
// the same results); wave 0 then orders the T*k pairs by (expert, pair) into h
// rows and lists the chosen experts in ascending order as tiles. emit: also
// write logits, ids and weights to the caller's buffers.
__device__ __forceinline__ void fz_local_route(const FusedArgs& f, uint32_t tag, FzRoute& rt, bool emit) {
  const int tid = threadIdx.x, lane = tid & 63, m = tid >> 6;
  const int T = f.g.shared_rows, E = f.g.E, k = f.d.k;
  uint32_t* status = reinterpret_cast<uint32_t*>(f.fz + kFzStatus);
  const uint64_t* slots = reinterpret_cast<const uint64_t*>(f.fz + kFzSlots);
  if (m == 0)
    fz_wait_count(reinterpret_cast<const uint32_t*>(f.fz + kFzRouteCnt + (blockIdx.x % kFzCntCopies) * kFzLine),
                  uint32_t(f.n_route), status);
  __syncthreads();
  if (m < T) {
    const uint64_t* p[kMaxKeysPerLane];
    bool need[kMaxKeysPerLane];
#pragma unroll
    for (int i = 0; i < kMaxKeysPerLane; ++i) {
      const int e = lane + 64 * i;
      p[i] = slots + m * E + min(e, E - 1);
      need[i] = e < E;
    }
    uint32_t bits[kMaxKeysPerLane];
    fz_wait_n<kMaxKeysPerLane>(p, need, tag, status, bits);
    uint32_t u[kMaxKeysPerLane];
#pragma unroll
    for (int i = 0; i < kMaxKeysPerLane; ++i) {
      const int e = lane + 64 * i;
      u[i] = e < E ? float_order_key(__uint_as_float(bits[i])) : 0u;
      if (emit && e < E && f.logits_out) f.logits_out[m * E + e] = __uint_as_float(bits[i]);
    }
    token_topk(u, k, rt.cand[m], rt.sel_key[m], rt.sel_e[m]);
    int my_e;
    float wgt;
    token_softmax(rt.sel_key[m], rt.sel_e[m], k, my_e, wgt);
    if (lane < k) {
      rt.ids[m * k + lane] = my_e;
      rt.w[m * k + lane] = wgt;
      if (emit && f.ids_out) f.ids_out[m * k + lane] = my_e;
      if (emit && f.w_out) f.w_out[m * k + lane] = wgt;
    }
  }
  __syncthreads();
  if (m == 0) {
    // lane p: pair p (T * k <= 64)
    // (every loop reads its entries in groups of eight, each group's loads
    // issued together)
    const int np = T * k, p = lane;
    const int ep = p < np ? rt.ids[p] : 0x7FFFFFFF;
    int less = 0, before = 0, cnt = 0;
    for (int q0 = 0; q0 < np; q0 += 8) {
      int eq[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) eq[q] = rt.ids[min(q0 + q, np - 1)];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int in = int(q0 + q < np);
        less += in & int(eq[q] < ep);
        before += in & int(eq[q] == ep) & int(q0 + q < p);
        cnt += in & int(eq[q] == ep);
      }
    }
    const bool first = p < np && before == 0;
    rt.first[p] = int(first);
    __builtin_amdgcn_wave_barrier();
    int tix = 0;
    for (int q0 = 0; q0 < np; q0 += 8) {
      int eq[8], fq[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        eq[q] = rt.ids[min(q0 + q, np - 1)];
        fq[q] = rt.first[min(q0 + q, np - 1)];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) tix += int(q0 + q < np) & fq[q] & int(eq[q] < ep);
    }
    if (first) {
      rt.tile_e[tix] = ep;
      rt.tile_r0[tix] = less;
      rt.tile_n[tix] = cnt;
      rt.tile_tok[tix] = 0u;
    }
    const uint64_t fm = __ballot(first);
    if (lane == 0) rt.n_tiles = int(__popcll(fm));
    __builtin_amdgcn_wave_barrier();
    if (p < np) {
      rt.row[p] = less + before;
      rt.row_tile[less + before] = 1 + tix;
      // a tile has at most T <= 8 rows: its row j's token fits in 4 bits
      atomicOr(&rt.tile_tok[tix], uint32_t(p / k) << (4 * before));
    }
  }
  __syncthreads();
}

template <int TM>
__device__ __forceinline__ void fz_swiglu(const GemmArgs& g, const DecTile& ti, int cb, uint8_t* smem, uint64_t* h,
                                          uint32_t tag) {
  switch (ti.n) {
    case 1: swiglu_tile<1, 4, 4>(g, ti, cb, smem, TM, h, tag); break;
    case 2: if constexpr (TM >= 2) swiglu_tile<2, 4, 4>(g, ti, cb, smem, TM, h, tag); break;
    case 3: if constexpr (TM >= 4) swiglu_tile<3, 4, 4>(g, ti, cb, smem, TM, h, tag); break;
    case 4: if constexpr (TM >= 4) swiglu_tile<4, 4, 4>(g, ti, cb, smem, TM, h, tag); break;
    case 5: if constexpr (TM >= 8) swiglu_tile<5, 4, 4>(g, ti, cb, smem, TM, h, tag); break;
    case 6: if constexpr (TM >= 8) swiglu_tile<6, 4, 4>(g, ti, cb, smem, TM, h, tag); break;
    case 7: if constexpr (TM >= 8) swiglu_tile<7, 4, 4>(g, ti, cb, smem, TM, h, tag); break;
    case 8: if constexpr (TM >= 8) swiglu_tile<8, 4, 4>(g, ti, cb, smem, TM, h, tag); break;
    default: break;   // 1..T rows per tile
  }
}

// Down item: one (token, 16 output columns); the pairs come from the
// workgroup's tables and the h rows from tagged words.
template <int DSTEPS>
__device__ __forceinline__ void fz_dn_item(const FusedArgs& f, int di, uint32_t tag, uint8_t* smem,
                                           const FzRoute& rt) {
  constexpr int K = DSTEPS * 128;
  const DownCombineArgs& a = f.d;
  const int ncb = a.N / 16;
  const int t = di / ncb, col0 = (di % ncb) * 16;
  const int lane = threadIdx.x & 63;
  uint32_t* status = reinterpret_cast<uint32_t*>(f.fz + kFzStatus);
  const uint64_t* h = reinterpret_cast<const uint64_t*>(f.fz + kFzHrows);
  auto pair = [&](int j) {
    const int p = t * a.k + j;
    return DcPair{rt.ids[p], rt.row[p], rt.w[p]};
  };
  auto stage_row = [&](int row, uint8_t* xs) {
    // every column item of the row's tile is done (shared rows: tile 0)
    const int tile = row < f.g.routed_rows ? rt.row_tile[row] : 0;
    fz_wait_count(reinterpret_cast<const uint32_t*>(f.fz + kFzTileCnt + tile * kFzLine), uint32_t(f.g.NT), status);
    const uint64_t* hr = h + size_t(row) * (K / 2);   // row < T * k + T <= kFzMaxRows
    constexpr int N = K / 2 / kWave;
    const uint64_t* p[N];
    bool need[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      p[i] = hr + i * kWave + lane;
      need[i] = true;
    }
    uint32_t v[N];
    fz_wait_n<N>(p, need, tag, status, v);
#pragma unroll
    for (int i = 0; i < N; ++i) *reinterpret_cast<uint32_t*>(xs + dec_off(K, 0, 2 * (i * kWave + lane))) = v[i];
  };
  down_combine_unit<DSTEPS>(a, t, col0, kFzWaves, smem, pair, stage_row);
}

template <int TM, int DSTEPS>
__global__ __launch_bounds__(kFzThreads) __attribute__((amdgpu_waves_per_eu(TM <= 2 ? 4 : 2)))
void decode_fused_kernel(FusedArgs f) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ FzRoute rt;
  __shared__ uint32_t tag_s;
  uint32_t* epoch = reinterpret_cast<uint32_t*>(f.fz + kFzEpoch);
  if (threadIdx.x == 0) tag_s = __hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  __syncthreads();
  const uint32_t tag = tag_s;
  const GemmArgs& g = f.g;
  const int T = g.shared_rows;
  uint64_t* h = reinterpret_cast<uint64_t*>(f.fz + kFzHrows);
  const int n0 = f.n_route, n1 = n0 + f.n_gu, n2 = n1 + f.n_dn;
  bool have_rt = false;   // uniform: this workgroup's tables are built
  for (int item = blockIdx.x; item < n2; item += gridDim.x) {
    if (item < n0) {
      fz_route_item<TM>(f, item, tag, smem);
      fz_count_done(f.fz + kFzRouteCnt, kFzCntCopies);
    } else if (item < n1) {
      const int gi = item - n0, tile = gi / g.NT, cb = gi % g.NT;
      if (tile == 0) {
        // the shared expert: one tile of every token's row (row routed_rows + t
        // is token t)
        DecTile ti{g.E, g.routed_rows, T, 0u};
        for (int j = 0; j < T; ++j) ti.tok |= uint32_t(j) << (4 * j);
        fz_swiglu<TM>(g, ti, cb, smem, h, tag);
        fz_count_done(f.fz + kFzTileCnt, 1);
      } else {
        if (!have_rt) {
          fz_local_route(f, tag, rt, item == n0 + g.NT);   // the first routed item writes the routing outputs
          have_rt = true;
        }
        const int i = tile - 1;
        if (i < rt.n_tiles) {   // uniform
          const DecTile ti{rt.tile_e[i], rt.tile_r0[i], rt.tile_n[i], rt.tile_tok[i]};
          fz_swiglu<TM>(g, ti, cb, smem, h, tag);
          fz_count_done(f.fz + kFzTileCnt + tile * kFzLine, 1);
        }
      }
    } else {
      if (!have_rt) {
        fz_local_route(f, tag, rt, false);
        have_rt = true;
      }
      fz_dn_item<DSTEPS>(f, item - n1, tag, smem, rt);
    }
    __syncthreads();   // LDS is reused by the next item
  }
  __shared__ int last_s;
  if (threadIdx.x == 0) {
    uint32_t* ex = reinterpret_cast<uint32_t*>(f.fz + kFzExit);
    last_s = __hip_atomic_fetch_add(ex, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  }
  __syncthreads();
  if (last_s) {   // uniform
    // every workgroup has read the epoch and finished: the counters back at
    // zero, and the next call's tag
    const int tid = threadIdx.x;
    if (tid < kFzCntCopies + kFzMaxTiles)
      __hip_atomic_store(reinterpret_cast<uint32_t*>(f.fz + kFzRouteCnt + tid * kFzLine), 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) {
      __hip_atomic_store(reinterpret_cast<uint32_t*>(f.fz + kFzExit), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

bool decode_fused_supported(int T, int k, int H, int I) {
  return T >= 1 && T <= kFzMaxT && T * k <= kFzMaxPairs && H == kFzH && (I == 256 || I == 512);
}

static_assert(kHandoffBytes + kFzStatus == MOE_WORKSPACE_STATUS_OFFSET, "status word offset in the header");

namespace {
constexpr int kFzMaxDevices = 64;
constexpr int kFzVariants = 8;   // token bucket (1, 2, 4, 8) x I (256, 512)
int g_fz_grid[kFzMaxDevices][kFzVariants];   // resident workgroups per device and variant (0: not queried)

template <int TM, int DSTEPS>
hipError_t fz_launch(const FusedArgs& f, int dev, int slot, size_t lds, hipStream_t stream) {
  if (g_fz_grid[dev][slot] == 0) {
    // every workgroup of the grid must be resident at once (the items wait on
    // one another): the grid is at most the resident capacity of the device
    int per_cu = 0, cus = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_fused_kernel<TM, DSTEPS>,
                                                                kFzThreads, lds);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (per_cu < 1 || cus < 1) return hipErrorInvalidConfiguration;
    g_fz_grid[dev][slot] = per_cu * cus;
  }
  const int items = f.n_route + f.n_gu + f.n_dn;
  const int grid = min(items, g_fz_grid[dev][slot]);
  hipLaunchKernelGGL((decode_fused_kernel<TM, DSTEPS>), dim3(grid), dim3(kFzThreads), lds, stream, f);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_fused(const FusedLaunch& fl, hipStream_t stream) {
  const int T = fl.g.shared_rows, I = fl.g.N, E = fl.g.E, k = fl.d.k;
  if (!decode_fused_supported(T, k, fl.g.K, I) || fl.d.N != kFzH || fl.d.K != I || fl.g.NT != I / 16 ||
      fl.g.routed_rows != T * k || E < k || E > kMaxExperts)
    return hipErrorInvalidValue;
  FusedArgs f{fl.g, fl.d, fl.wr, fl.bias, fl.logits_out, fl.ids_out, fl.w_out, fl.fz, 0, 0, 0};
  f.n_route = ceil_div(E, kFzWaves);
  f.n_gu = (1 + min(E, T * k)) * fl.g.NT;   // the shared tile, then one tile per chosen expert
  f.n_dn = T * (kFzH / 16);
  const int tm = T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8;
  const size_t lds_gu = size_t(dec_lds_bytes(4, 4, tm));
  const size_t lds_dn = size_t(kFzWaves) * dc_wave_bytes(I) + size_t(kFzWaves) * 33 * 4;
  const size_t lds_rt = size_t(tm) * kFzH * 2;   // the routing items' staged x (tm >= 4)
  size_t lds = lds_gu > lds_dn ? lds_gu : lds_dn;
  lds = lds > lds_rt ? lds : lds_rt;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kFzMaxDevices) return hipErrorInvalidDevice;
  const int slot = (tm == 1 ? 0 : tm == 2 ? 1 : tm == 4 ? 2 : 3) * 2 + (I == 256 ? 0 : 1);
  switch (slot) {
    case 0: return fz_launch<1, 2>(f, dev, slot, lds, stream);
    case 1: return fz_launch<1, 4>(f, dev, slot, lds, stream);
    case 2: return fz_launch<2, 2>(f, dev, slot, lds, stream);
    case 3: return fz_launch<2, 4>(f, dev, slot, lds, stream);
    case 4: return fz_launch<4, 2>(f, dev, slot, lds, stream);
    case 5: return fz_launch<4, 4>(f, dev, slot, lds, stream);
    case 6: return fz_launch<8, 2>(f, dev, slot, lds, stream);
    default: return fz_launch<8, 4>(f, dev, slot, lds, stream);
  }
}

}  // namespace moe
