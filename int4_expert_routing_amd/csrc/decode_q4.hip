// Decode-shaped expert GEMV for gfx950: the same per-expert products as the
// grouped GEMM (gemm_q4.hip), laid out for the few-token case where each expert
// sees at most 8 rows and the layer is bound by streaming the chosen experts'
// 4-bit weights from HBM (page "Perplexity Open Sources Lily ..." Technical
// Details, decode bullet: decode reads the active experts' weights once per
// token; itinai.com post: expansion of the 4-bit weights on chip only).
//
// Work split: one workgroup = 8 wave64s per (row tile, column block). A wave
// owns 16 output columns; its 64 lanes are 16 columns x 4 quarters of the
// reduction dimension K, so every lane streams K/8 contiguous bytes of one
// column's codes (16-byte loads, all issued before any arithmetic) and the
// quarters are summed with two lane exchanges at the end.
//   SwiGLU: waves 0-3 gate, 4-7 up, for the same 64 columns (one 64-wide group
//           of h, so the workgroup also writes h's group-sum table);
//   STORE_F32: waves 0-7, 128 columns.
//
// Arithmetic (exact operand, fp32 accumulation, as in the grouped GEMM): each
// code becomes the bf16 value 1 + q/16, a v_dot2 with the row's activations
// accumulates P_g = sum_{k in g} x_k (1 + q_k/16) per 64-wide group, and the
// group folds as acc += 16 s_g P_g + (b_g - 16 s_g) X_g, where X_g is the
// row's group sum from the side table (three bf16 parts summed in fp32).
#include "gemm_tiles.h"

namespace moe {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;

// LDS row layout: quarter kq of a row starts 16 bytes later than an unpadded
// layout would put it, so the four quarter groups of a wave read four distinct
// bank ranges.
__host__ __device__ constexpr int dec_row_bytes(int K) { return 2 * K + 64; }
__device__ __forceinline__ int dec_off(int K, int r, int k) { return r * dec_row_bytes(K) + 2 * k + (k / (K / 4)) * 16; }

size_t decode_lds_bytes(int K) {
  return size_t(kDecodeMaxRows) * dec_row_bytes(K) + size_t(kDecodeMaxRows) * (K / kGroup) * 4 +
         size_t(kDecodeMaxRows) * 64 * 4 + size_t(kDecodeMaxRows) * 64 * 2;
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

// STEPS = K/128: 16-byte code loads per lane (32 codes each, two per group).
template <int NR, int STEPS, int EPI>
__device__ __forceinline__ void decode_tile(const GemmArgs& a, const TileInfo& ti, int cb, uint8_t* smem) {
  constexpr int K = STEPS * 128;
  constexpr int G = K / kGroup;
  constexpr int GQ = STEPS / 2;          // groups per lane quarter
  const int nrows = ti.r1 - ti.r0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, kq = lane >> 4;
  uint8_t* xs = smem;
  float* Xt = reinterpret_cast<float*>(smem + kDecodeMaxRows * dec_row_bytes(K));   // [NR][G]

  // ---- this lane's column and its code / scale / bias streams --------------
  const int stack = ti.e == a.E ? 1 : 0;
  const int el = stack ? 0 : ti.e;
  int col;
  const QStack* mat;
  if constexpr (EPI == kEpiF32) {
    col = cb * 128 + wave * 16 + c;
    mat = &a.w0[stack];
  } else {
    col = cb * 64 + (wave & 3) * 16 + c;
    mat = (wave >> 2) ? &a.w1[stack] : &a.w0[stack];
  }
  const size_t wrow = size_t(el) * a.N + col;
  const u32x4* qp = reinterpret_cast<const u32x4*>(mat->q + wrow * (K / 8) + kq * (K / 32));
  u32x4 codes[STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) codes[s] = __builtin_nontemporal_load(qp + s);
  uint16_t sv[GQ], bv[GQ];
  load_groups<GQ>(mat->s + wrow * G + kq * GQ, sv);
  load_groups<GQ>(mat->b + wrow * G + kq * GQ, bv);

  // ---- activation rows and their group sums into LDS ------------------------
  for (int i = tid; i < nrows * (K / 8); i += kDecThreads) {
    const int r = i / (K / 8), ch = i % (K / 8);
    const int src = src_row(a, ti.r0 + r);
    const u32x4 v = *reinterpret_cast<const u32x4*>(a.A + size_t(src) * K + ch * 8);
    *reinterpret_cast<u32x4*>(xs + dec_off(K, r, ch * 8)) = v;
  }
  for (int i = tid; i < nrows * G; i += kDecThreads) {
    const int r = i / G, g = i % G;
    const int src = src_row(a, ti.r0 + r);
    const uint16_t* e = a.Apart + size_t(src) * xpart_cols(K) + 8 * g;
    Xt[r * G + g] = bf16_to_f32(e[0]) + (bf16_to_f32(e[1]) + bf16_to_f32(e[2]));
  }
  __syncthreads();

  // ---- dot products over the lane's quarter of K ----------------------------
  float acc[NR], P[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = P[r] = 0.0f;
  const uint32_t nib = kNib, magic = kMagic;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const uint32_t wd[4] = {codes[s].x, codes[s].y, codes[s].z, codes[s].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 p = __builtin_bit_cast(u32x4, unpack_word(wd[j], nib, magic));
      const int k0 = kq * (K / 4) + 32 * s + 8 * j;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(xs + dec_off(K, r, k0));
        P[r] = dot2(p.x, xv.x, P[r]);
        P[r] = dot2(p.y, xv.y, P[r]);
        P[r] = dot2(p.z, xv.z, P[r]);
        P[r] = dot2(p.w, xv.w, P[r]);
      }
    }
    if (s & 1) {
      const int gl = s >> 1;
      const float s16 = 16.0f * bf16_to_f32(sv[gl]);
      const float off = bf16_to_f32(bv[gl]) - s16;
      const int g = kq * GQ + gl;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        acc[r] = __builtin_fmaf(s16, P[r], acc[r]);
        acc[r] = __builtin_fmaf(off, Xt[r * G + g], acc[r]);
        P[r] = 0.0f;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    acc[r] += __shfl_xor(acc[r], 16, kWave);
    acc[r] += __shfl_xor(acc[r], 32, kWave);
  }

  // ---- epilogues -------------------------------------------------------------
  if constexpr (EPI == kEpiF32) {
    float* out = reinterpret_cast<float*>(a.out);
    if (kq == 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r)
        if (r < nrows) out[size_t(ti.r0 + r) * a.N + col] = acc[r];
    }
  } else {
    __syncthreads();   // every wave is done reading xs (the tiles below reuse it)
    float* gs = reinterpret_cast<float*>(smem);                                   // [NR][64]
    uint16_t* hs = reinterpret_cast<uint16_t*>(smem + kDecodeMaxRows * 64 * 4);  // [NR][64]
    const int hc = (wave & 3) * 16 + c;
    if (wave < 4 && kq == 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r) gs[r * 64 + hc] = acc[r];
    }
    __syncthreads();
    if (wave >= 4 && kq == 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float gv = gs[r * 64 + hc];
        const float hv = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * acc[r];
        hs[r * 64 + hc] = uint16_t(f32_to_bf16_rne(hv));
      }
    }
    __syncthreads();
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
    if (tid < nrows * 8) {
      // row tid/8, chunk tid%8 of this column block, stored in the permuted order
      const int r = tid >> 3, ch = tid & 7;
      const u32x4 v = *reinterpret_cast<const u32x4*>(hs + r * 64 + ch * 8);
      *reinterpret_cast<u32x4*>(out + size_t(ti.r0 + r) * a.N + cb * 64 + ch * 8) = permute_chunk(v);
    }
    if (tid < nrows) {
      // the block's 64 columns are one group of h: its sum in fp64, split exactly
      double sum = 0.0;
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) sum += chunk_sum_f64(*reinterpret_cast<const u32x4*>(hs + tid * 64 + ch * 8));
      uint16_t h, m, l;
      split3_bf16(float(sum), h, m, l);
      const u32x4 e = {uint32_t(h) | (uint32_t(m) << 16), uint32_t(l) | (uint32_t(h) << 16),
                       uint32_t(m) | (uint32_t(l) << 16), 0u};
      *reinterpret_cast<u32x4*>(a.out_part + size_t(ti.r0 + tid) * xpart_cols(a.N) + 8 * cb) = e;
    }
  }
}

template <int STEPS, int EPI>
__global__ __launch_bounds__(kDecThreads) void decode_q4_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tile = blockIdx.x / a.NT;
  const int cb = blockIdx.x % a.NT;
  if (tile >= a.n_shared_tiles + *a.num_tiles) return;
  TileInfo ti;
  if (!tile_info(a, tile, ti)) return;
  switch (ti.r1 - ti.r0) {
    case 1: decode_tile<1, STEPS, EPI>(a, ti, cb, smem); break;
    case 2: decode_tile<2, STEPS, EPI>(a, ti, cb, smem); break;
    case 3: decode_tile<3, STEPS, EPI>(a, ti, cb, smem); break;
    case 4: decode_tile<4, STEPS, EPI>(a, ti, cb, smem); break;
    case 5: decode_tile<5, STEPS, EPI>(a, ti, cb, smem); break;
    case 6: decode_tile<6, STEPS, EPI>(a, ti, cb, smem); break;
    case 7: decode_tile<7, STEPS, EPI>(a, ti, cb, smem); break;
    case 8: decode_tile<8, STEPS, EPI>(a, ti, cb, smem); break;
    default: break;   // callers guarantee at most kDecodeMaxRows rows per tile
  }
}

bool decode_supported(int N, int K, int epilogue) {
  const int steps = K / 128;
  if (K % 128 != 0 || (steps != 2 && steps != 4 && steps != 8 && steps != 16)) return false;
  return epilogue == kEpiF32 ? N % 128 == 0 : (epilogue == kEpiSwigluInternal && N % 64 == 0);
}

template <int EPI>
static hipError_t launch_decode_epi(const GemmArgs& ga, dim3 grid, size_t lds, hipStream_t stream) {
  switch (ga.K / 128) {
    case 2: hipLaunchKernelGGL((decode_q4_kernel<2, EPI>), grid, dim3(kDecThreads), lds, stream, ga); break;
    case 4: hipLaunchKernelGGL((decode_q4_kernel<4, EPI>), grid, dim3(kDecThreads), lds, stream, ga); break;
    case 8: hipLaunchKernelGGL((decode_q4_kernel<8, EPI>), grid, dim3(kDecThreads), lds, stream, ga); break;
    default: hipLaunchKernelGGL((decode_q4_kernel<16, EPI>), grid, dim3(kDecThreads), lds, stream, ga); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const GemmArgs& ga, int epilogue, int max_row_tiles, hipStream_t stream) {
  if (!decode_supported(ga.N, ga.K, epilogue)) return hipErrorInvalidValue;
  const dim3 grid(unsigned(max_row_tiles) * unsigned(ga.NT));
  if (grid.x == 0) return hipSuccess;
  const size_t lds = decode_lds_bytes(ga.K);
  return epilogue == kEpiF32 ? launch_decode_epi<kEpiF32>(ga, grid, lds, stream)
                             : launch_decode_epi<kEpiSwigluInternal>(ga, grid, lds, stream);
}

}  // namespace moe
