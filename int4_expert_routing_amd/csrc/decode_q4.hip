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
#include "moe_internal.h"

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

template <int NR, int STEPS, int KS>
__device__ __forceinline__ void swiglu_tile(const GemmArgs& a, const DecTile& ti, int cb, uint8_t* smem, int nrmax) {
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
    const u32x4 v = *reinterpret_cast<const u32x4*>(hs + r * 16 + ch * 8);
    *reinterpret_cast<u32x4*>(out + size_t(ti.r0 + r) * a.N + cb * 16 + ch * 8) = permute_chunk(v);
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

template <int STEPS>
__global__ __launch_bounds__(kDcMaxWaves * 64) void decode_down_combine_kernel(DownCombineArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int K = STEPS * 128;
  constexpr int G = K / kGroup;
  constexpr int GQ = STEPS / 2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = blockDim.x >> 6;
  const int c = lane & 15, kq = lane >> 4;
  const int ncb = a.N / 16;
  const int t = blockIdx.x / ncb;
  const int col0 = (blockIdx.x % ncb) * 16;
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
    for (int c = tid * 8; c < a.N; c += W * 64 * 8) {
      const u32x4 xv = *reinterpret_cast<const u32x4*>(a.x + size_t(t) * a.N + c);
      const u32x4 wv = *reinterpret_cast<const u32x4*>(a.shared_gate + c);
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
    const size_t f = size_t(t) * a.k + (routed ? j : 0);
    const int el = routed ? a.topk_ids[f] : 0;
    const int row = routed ? a.row_of_pair[f] : a.shared_row0 + t;
    const float wj = routed ? a.topk_w[f] : 1.0f;
    const QStack& mat = routed ? a.down : a.down_shared;
    // the lane's codes: quarter kq of its column's K (GQ groups)
    u32x4 w[STEPS];
    load_code_steps<STEPS>(mat, el, a.N, K, col0 + c, kq * GQ, w);
    uint16_t sv[GQ], bv[GQ];
    load_scale_bias<GQ>(mat, el, a.N, K, col0 + c, kq * GQ, sv, bv);
    // stage the h row (already in operand order) and its fp32 group sums
    __builtin_amdgcn_wave_barrier();   // the previous pair's reads of xs and Xt are done
    const uint16_t* hr = a.h + size_t(row) * K;
    for (int ch = lane; ch < K / 8; ch += 64)
      *reinterpret_cast<u32x4*>(xs + dec_off(K, 0, ch * 8)) = *reinterpret_cast<const u32x4*>(hr + ch * 8);
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
      tot = __builtin_fmaf(wj, acc, tot);
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

}  // namespace moe
