// Decode-shaped expert GEMV for gfx950: the same per-expert products as the
// grouped GEMM (gemm_q4.hip), laid out for the few-token case where each expert
// sees at most 8 rows and the layer is bound by streaming the chosen experts'
// 4-bit weights from HBM (page "Perplexity Open Sources Lily ..." Technical
// Details, decode bullet: decode reads the active experts' weights once per
// token; itinai.com post: expansion of the 4-bit weights on chip only).
//
// Work split: one workgroup = 2 wave64s per (row tile, column block). A wave
// owns 16 output columns; its 64 lanes are 16 columns x 4 quarters of the
// reduction dimension K, so every lane streams K/8 contiguous bytes of one
// column's codes and the quarters are summed with two lane exchanges at the
// end. All code loads are issued at once, straight into LDS (buffer loads that
// write LDS), so the weight stream is in flight while the activation rows are
// staged; the K loop then runs as a short rolled loop over 64-wide groups.
//   SwiGLU: wave 0 gate, wave 1 up, for the same 16 columns of h;
//   STORE_F32: waves 0, 1 for 32 columns.
//
// Arithmetic (exact operand, fp32 accumulation, as in the grouped GEMM): each
// code becomes the bf16 value 1 + q/16, a v_dot2 with the row's activations
// accumulates P_g = sum_{k in g} x_k (1 + q_k/16) per 64-wide group, and the
// group folds as acc += 16 s_g P_g + (b_g - 16 s_g) X_g, where X_g is the
// row's group sum, computed in fp32 from the staged row.
#include "gemm_tiles.h"

namespace moe {

constexpr int kDecWaves = 2;
constexpr int kDecThreads = kDecWaves * 64;
constexpr uint32_t kDecRsrcWord3 = 0x00020000u;   // raw buffer descriptor flags (gfx9 family)

typedef __attribute__((address_space(3))) void* dec_lds_t;

// LDS row layout: quarter kq of a row starts 16 bytes later than an unpadded
// layout would put it, so the four quarter groups of a wave read four distinct
// bank ranges.
__host__ __device__ constexpr int dec_row_bytes(int K) { return 2 * K + 64; }
__device__ __forceinline__ int dec_off(int K, int r, int k) { return r * dec_row_bytes(K) + 2 * k + (k / (K / 4)) * 16; }

// LDS of one workgroup: codes [2 waves][K/128 loads][64 lanes][16 B], scale and
// bias pairs [2][K/256][64] u32, activation rows [8][row bytes], group sums
// [8][K/64] f32, source rows [8].
struct DecLds {
  int codes, sb, xs, xt, src, total;
};
__host__ __device__ constexpr DecLds dec_lds(int K) {
  const int codes = 0;
  const int sb = codes + kDecWaves * (K / 128) * 1024;
  const int xs = sb + kDecWaves * (K / 256) * 64 * 4;
  const int xt = xs + kDecodeMaxRows * dec_row_bytes(K);
  const int src = xt + kDecodeMaxRows * (K / kGroup) * 4;
  return DecLds{codes, sb, xs, xt, src, src + kDecodeMaxRows * 4};
}

size_t decode_lds_bytes(int K) { return size_t(dec_lds(K).total); }

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
// PERMUTE: the activation rows arrive in natural order and are put into the
// operand order [0,4,1,5,2,6,3,7] per 8-element chunk while staged.
template <int NR, int STEPS, int EPI, bool PERMUTE>
__device__ __forceinline__ void decode_tile(const GemmArgs& a, const TileInfo& ti, int cb, uint8_t* smem) {
  constexpr int K = STEPS * 128;
  constexpr int G = K / kGroup;
  constexpr int GQ = STEPS / 2;          // groups per lane quarter
  constexpr DecLds L = dec_lds(K);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, kq = lane >> 4;
  uint8_t* codes = smem + L.codes + wave * STEPS * 1024;
  uint32_t* sb = reinterpret_cast<uint32_t*>(smem + L.sb) + wave * GQ * 64;
  uint8_t* xs = smem + L.xs;
  float* Xt = reinterpret_cast<float*>(smem + L.xt);
  int* srcs = reinterpret_cast<int*>(smem + L.src);

  // ---- this wave's 16 columns: code stream into LDS, scales and biases -----
  const int stack = ti.e == a.E ? 1 : 0;
  const int el = stack ? 0 : ti.e;
  int col0;
  const QStack* mat;
  if constexpr (EPI == kEpiF32) {
    col0 = cb * 32 + wave * 16;
    mat = &a.w0[stack];
  } else {
    col0 = cb * 16;
    mat = wave ? &a.w1[stack] : &a.w0[stack];
  }
  const size_t wrow0 = size_t(el) * a.N + col0;
  {
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(mat->q + wrow0 * (K / 8)), 0, 0x7FFFFFFF, kDecRsrcWord3);
    const uint32_t voff = uint32_t((c * (K / 8) + kq * (K / 32)) * 4);
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (dec_lds_t)(codes + s * 1024), 16, voff, s * 16, 0, 0);
  }
  {
    uint16_t sv[GQ], bv[GQ];
    load_groups<GQ>(mat->s + (wrow0 + c) * G + kq * GQ, sv);
    load_groups<GQ>(mat->b + (wrow0 + c) * G + kq * GQ, bv);
#pragma unroll
    for (int i = 0; i < GQ; ++i) sb[i * 64 + lane] = uint32_t(sv[i]) | (uint32_t(bv[i]) << 16);
  }

  // ---- activation rows and their group sums into LDS ------------------------
  if (tid < NR) srcs[tid] = src_row(a, ti.r0 + tid);
  __syncthreads();
  for (int i = tid; i < NR * (K / 8); i += kDecThreads) {
    const int r = i / (K / 8), ch = i % (K / 8);
    u32x4 v = *reinterpret_cast<const u32x4*>(a.A + size_t(srcs[r]) * K + ch * 8);
    if (PERMUTE) v = permute_chunk(v);
    *reinterpret_cast<u32x4*>(xs + dec_off(K, r, ch * 8)) = v;
  }
  __syncthreads();
  for (int i = tid; i < NR * G; i += kDecThreads) {
    const int r = i / G, g = i % G;
    float sum = 0.0f;
#pragma unroll
    for (int ch = 0; ch < 8; ++ch)
      sum += chunk_sum(*reinterpret_cast<const u32x4*>(xs + dec_off(K, r, g * kGroup + ch * 8)));
    Xt[r * G + g] = sum;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's code loads have landed
  __syncthreads();

  // ---- dot products over the lane's quarter of K, one group per iteration ---
  float acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.0f;
  const uint32_t nib = kNib, magic = kMagic;
#pragma unroll 1
  for (int gl = 0; gl < GQ; ++gl) {
    float P[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) P[r] = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int s = 2 * gl + h;
      const u32x4 w = *reinterpret_cast<const u32x4*>(codes + s * 1024 + lane * 16);
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
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
    }
    const uint32_t sbv = sb[gl * 64 + lane];
    const float s16 = 16.0f * __uint_as_float(sbv << 16);
    const float off = __uint_as_float(sbv & 0xFFFF0000u) - s16;
    const int g = kq * GQ + gl;
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

  // ---- epilogues -------------------------------------------------------------
  if constexpr (EPI == kEpiF32) {
    float* out = reinterpret_cast<float*>(a.out);
    if (kq == 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r) out[size_t(ti.r0 + r) * a.N + col0 + c] = acc[r];
    }
  } else {
    __syncthreads();   // every wave is done reading xs (the tiles below reuse it)
    float* gs = reinterpret_cast<float*>(xs);                           // [NR][16]
    uint16_t* hs = reinterpret_cast<uint16_t*>(xs + kDecodeMaxRows * 16 * 4);  // [NR][16]
    if (wave == 0 && kq == 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r) gs[r * 16 + c] = acc[r];
    }
    __syncthreads();
    if (wave == 1 && kq == 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float gv = gs[r * 16 + c];
        const float hv = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * acc[r];
        hs[r * 16 + c] = uint16_t(f32_to_bf16_rne(hv));
      }
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
}

template <int STEPS, int EPI, bool PERMUTE>
__global__ __launch_bounds__(kDecThreads) void decode_q4_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tile = blockIdx.x / a.NT;
  const int cb = blockIdx.x % a.NT;
  if (tile >= a.n_shared_tiles + *a.num_tiles) return;
  TileInfo ti;
  if (!tile_info(a, tile, ti)) return;
  switch (ti.r1 - ti.r0) {
    case 1: decode_tile<1, STEPS, EPI, PERMUTE>(a, ti, cb, smem); break;
    case 2: decode_tile<2, STEPS, EPI, PERMUTE>(a, ti, cb, smem); break;
    case 3: decode_tile<3, STEPS, EPI, PERMUTE>(a, ti, cb, smem); break;
    case 4: decode_tile<4, STEPS, EPI, PERMUTE>(a, ti, cb, smem); break;
    case 5: decode_tile<5, STEPS, EPI, PERMUTE>(a, ti, cb, smem); break;
    case 6: decode_tile<6, STEPS, EPI, PERMUTE>(a, ti, cb, smem); break;
    case 7: decode_tile<7, STEPS, EPI, PERMUTE>(a, ti, cb, smem); break;
    case 8: decode_tile<8, STEPS, EPI, PERMUTE>(a, ti, cb, smem); break;
    default: break;   // callers guarantee at most kDecodeMaxRows rows per tile
  }
}

bool decode_supported(int N, int K, int epilogue) {
  const int steps = K / 128;
  if (K % 128 != 0 || (steps != 2 && steps != 4 && steps != 8 && steps != 16)) return false;
  return epilogue == kEpiF32 ? N % 32 == 0 : (epilogue == kEpiSwigluInternal && N % 16 == 0);
}

template <int EPI, bool PERMUTE>
static hipError_t launch_decode_epi(const GemmArgs& ga, dim3 grid, size_t lds, hipStream_t stream) {
  switch (ga.K / 128) {
    case 2: hipLaunchKernelGGL((decode_q4_kernel<2, EPI, PERMUTE>), grid, dim3(kDecThreads), lds, stream, ga); break;
    case 4: hipLaunchKernelGGL((decode_q4_kernel<4, EPI, PERMUTE>), grid, dim3(kDecThreads), lds, stream, ga); break;
    case 8: hipLaunchKernelGGL((decode_q4_kernel<8, EPI, PERMUTE>), grid, dim3(kDecThreads), lds, stream, ga); break;
    default: hipLaunchKernelGGL((decode_q4_kernel<16, EPI, PERMUTE>), grid, dim3(kDecThreads), lds, stream, ga); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const GemmArgs& ga, int epilogue, bool natural_rows, int max_row_tiles, hipStream_t stream) {
  if (!decode_supported(ga.N, ga.K, epilogue)) return hipErrorInvalidValue;
  const dim3 grid(unsigned(max_row_tiles) * unsigned(ga.NT));
  if (grid.x == 0) return hipSuccess;
  const size_t lds = decode_lds_bytes(ga.K);
  if (epilogue == kEpiF32)
    return natural_rows ? launch_decode_epi<kEpiF32, true>(ga, grid, lds, stream)
                        : launch_decode_epi<kEpiF32, false>(ga, grid, lds, stream);
  return natural_rows ? launch_decode_epi<kEpiSwigluInternal, true>(ga, grid, lds, stream)
                      : launch_decode_epi<kEpiSwigluInternal, false>(ga, grid, lds, stream);
}

}  // namespace moe
