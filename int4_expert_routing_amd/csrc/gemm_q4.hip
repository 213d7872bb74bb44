// Grouped GEMM over expert-sorted row tiles with 4-bit groupwise-affine weights
// dequantised inside the kernel, bf16 MFMA and FP32 accumulation, for gfx950.
//
// Pages: "Perplexity Open Sources Lily ..." Technical Details (prefill bullet:
// groupwise affine 4-bit, 64 weights per group, dequantisation fused into the
// grouped GEMM with FP32 accumulation; 32-row tiles on four simdgroups) and its
// Chinese 技术解析 (a bf16 scale per 64 weights); the itinai.com post (weights
// expanded only on chip, never as a full bf16 copy in memory).
//
// Exactness. A weight is W = s*q + b with q in 0..15 and s, b bf16. Rounding
// s*q+b to bf16 before a bf16 MFMA would add ~2^-9 relative error per weight.
// Instead the MFMA operand is the exact value 128+q, whose bf16 bit pattern is
// 0x4300 | q, so one AND/OR turns two packed codes into two operands. For each
// 64-wide group g of K the MFMA accumulates the exact-product partial
//     P_g = sum_{k in g} x_k (128 + q_k)            (fp32)
// and the kernel folds it as acc += s_g * P_g (one FMA per output per group).
// What is left, sum_g (b_g - 128 s_g) X_g with X_g = sum_{k in g} x_k, is a
// contraction over groups; it runs on the MFMA too, as 3 extra K columns per
// group: activations (X_hi, X_lo, X_hi) against weights (b'_hi, b'_hi, b'_lo),
// where hi/lo split a float into two bf16 values (b' = b - 128 s). X_g is
// computed once per activation row (prep kernel, or the SwiGLU epilogue that
// writes h) and stored in a side table.
//
// Operand order. One 32-bit word holds codes k..k+7 (nibble i = code k+i); the
// AND/OR unpack yields the bf16 pairs (k, k+4), (k+1, k+5), (k+2, k+6),
// (k+3, k+7). Activations are therefore stored with every 8-element chunk in
// the order [0,4,1,5,2,6,3,7] (prep kernel / SwiGLU epilogue), so both MFMA
// operands list the same K indices in the same slots.
//
// Tiling (one workgroup = 2 wave64s = 128 threads):
//   rows: 64 per tile (two 32-row MFMA blocks per wave);
//   cols: SwiGLU: 64 gate + 64 up columns (wave w: gate and up columns
//         32w..32w+31, so the SwiGLU pairs sit in the same lane and register);
//         STORE_F32: 128 columns (wave w: 64w..64w+63).
//   MFMA v_mfma_f32_32x32x16_bf16; per 64-wide group each wave issues 16 MFMAs.
//   A tiles go global -> registers -> LDS (double buffered, XOR-swizzled 16-byte
//   chunks); weight codes go global -> registers directly (each wave reads only
//   its own columns), 4 groups in flight.
// Work mapping: blockIdx.x = tile * NT + column_tile; column tiles are the fast
// index so the 8 column tiles of a row tile land on the 8 XCDs and every XCD
// keeps its own 1/8 of each expert's weights in its L2.
#include "moe_internal.h"

namespace moe {

constexpr int kGemmThreads = 128;
constexpr int kRing = 4;            // groups of weight codes in flight per wave
constexpr uint32_t kMagic = 0x43004300u;  // two bf16 128.0
constexpr uint32_t kNib = 0x000F000Fu;

struct TileInfo {
  int e, r0, r1;
};

__device__ __forceinline__ bool tile_info(const GemmArgs& a, int tile, TileInfo& ti) {
  if (tile < a.n_shared_tiles) {
    ti.e = a.E;
    ti.r0 = a.routed_rows + tile * kBlockRows;
    ti.r1 = min(ti.r0 + kBlockRows, a.routed_rows + a.shared_rows);
    return true;
  }
  const int i = tile - a.n_shared_tiles;
  if (i >= *a.num_tiles) return false;
  ti.e = a.tile_map[2 * i];
  ti.r0 = a.tile_map[2 * i + 1];
  ti.r1 = min(ti.r0 + kBlockRows, a.offsets[ti.e + 1]);
  return true;
}

__device__ __forceinline__ int src_row(const GemmArgs& a, int r) {
  if (r >= a.routed_rows) return r - a.shared_src_base;
  return a.sorted_rows ? a.sorted_rows[r] / a.row_div : r;
}

__device__ __forceinline__ bf16x8 unpack_word(uint32_t w) {
  u32x4 r;
  r.x = (w & kNib) | kMagic;
  r.y = ((w >> 4) & kNib) | kMagic;
  r.z = ((w >> 8) & kNib) | kMagic;
  r.w = ((w >> 12) & kNib) | kMagic;
  return __builtin_bit_cast(bf16x8, r);
}

// LDS byte offset of 16-byte chunk c (0..7) of row m in one A buffer.
__device__ __forceinline__ int a_chunk_off(int m, int c) { return (m * 8 + (c ^ (m & 7))) * 16; }

__device__ __forceinline__ uint32_t split_hi(float v) { return f32_to_bf16_rne(v); }
__device__ __forceinline__ uint32_t split_lo(float v) {
  const uint32_t h = f32_to_bf16_rne(v);
  return f32_to_bf16_rne(v - __uint_as_float(h << 16));
}

template <int EPI>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_q4_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int K = a.K;
  const int G = K / kGroup;
  const int KPa = aux_cols(K);
  uint8_t* abuf = smem;                                        // 2 x 8 KiB
  uint16_t* aux_s = reinterpret_cast<uint16_t*>(smem + 2 * 8192);  // [64][KPa]
  uint16_t* s_st = aux_s + kBlockRows * KPa;                  // [G][128]

  const int nt = blockIdx.x % a.NT;
  const int tile = blockIdx.x / a.NT;
  TileInfo ti;
  if (!tile_info(a, tile, ti)) return;
  const int stack = ti.e == a.E ? 1 : 0;
  const int el = stack ? 0 : ti.e;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // ---- weight rows owned by this wave: cb = 0, 1 --------------------------
  const size_t qrow = size_t(K / 8);
  const uint32_t* qp[2];
  const QStack& m0 = a.w0[stack];
  const QStack& m1 = (EPI == kEpiF32) ? a.w0[stack] : a.w1[stack];
  int ncol[2];
  if constexpr (EPI == kEpiF32) {
    ncol[0] = nt * 128 + wave * 64 + l32;
    ncol[1] = ncol[0] + 32;
  } else {
    ncol[0] = nt * 64 + wave * 32 + l32;
    ncol[1] = ncol[0];
  }
  qp[0] = m0.q + (size_t(el) * a.N + ncol[0]) * qrow + 4 * half;
  qp[1] = m1.q + (size_t(el) * a.N + ncol[1]) * qrow + 4 * half;

  // ---- prologue: stage scales of the workgroup's 128 weight rows ----------
  {
    // thread t <-> weight row (wave t/64, cb (t/32)%2, lane t%32)
    const int w_ = tid >> 6, cb_ = (tid >> 5) & 1, j_ = tid & 31;
    int n_;
    const QStack* st;
    if constexpr (EPI == kEpiF32) {
      n_ = nt * 128 + w_ * 64 + cb_ * 32 + j_;
      st = &a.w0[stack];
    } else {
      n_ = nt * 64 + w_ * 32 + j_;
      st = cb_ ? &a.w1[stack] : &a.w0[stack];
    }
    const uint16_t* sp = st->s + (size_t(el) * a.N + n_) * G;
    for (int g = 0; g < G; ++g) s_st[g * 128 + tid] = sp[g];
  }

  // ---- prologue: A side table and first A tile ----------------------------
  const int srow = tid >> 1;          // staging row 0..63
  const int shalf = tid & 1;          // which 32-element half of a group
  const int sr = ti.r0 + srow;
  const bool svalid = sr < ti.r1;
  const uint16_t* arow = a.A + size_t(svalid ? src_row(a, sr) : 0) * K + shalf * 32;
  {
    const uint16_t* auxrow = a.Aaux + size_t(svalid ? src_row(a, sr) : 0) * KPa;
    for (int c = shalf; c < KPa / 8; c += 2) {
      u32x4 v = svalid ? *reinterpret_cast<const u32x4*>(auxrow + 8 * c) : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(aux_s + srow * KPa + 8 * c) = v;
    }
  }
  u32x4 stage[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    stage[i] = svalid ? *reinterpret_cast<const u32x4*>(arow + 8 * i) : u32x4{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<u32x4*>(abuf + a_chunk_off(srow, shalf * 4 + i)) = stage[i];

  // weight-code ring: slot u holds group g with g % kRing == u
  u32x4 ring[kRing][2];
#pragma unroll
  for (int u = 0; u < kRing; ++u) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      ring[u][cb] = u < G ? *reinterpret_cast<const u32x4*>(qp[cb] + u * 8) : u32x4{0, 0, 0, 0};
  }
  __syncthreads();

  f32x16 acc[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = f32x16{};

  const int scol0 = (wave * 2 + 0) * 32 + l32;
  const int scol1 = (wave * 2 + 1) * 32 + l32;

  for (int g0 = 0; g0 < G; g0 += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int g = g0 + u;
      if (g < G) {
        const uint8_t* cur = abuf + (g & 1) * 8192;
        // next A tile into registers
        const bool more = g + 1 < G;
        if (more) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            stage[i] = svalid ? *reinterpret_cast<const u32x4*>(arow + (g + 1) * kGroup + 8 * i)
                              : u32x4{0, 0, 0, 0};
        }
        // A fragments of this group
        bf16x8 af[2][4];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int m = rb * 32 + l32;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            af[rb][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(cur + a_chunk_off(m, 4 * half + j)));
        }
        const float s0 = bf16_to_f32(s_st[g * 128 + scol0]);
        const float s1 = bf16_to_f32(s_st[g * 128 + scol1]);
        const u32x4 w0 = ring[u][0];
        const u32x4 w1 = ring[u][1];
        // refill this ring slot with group g + kRing
        if (g + kRing < G) {
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
            ring[u][cb] = *reinterpret_cast<const u32x4*>(qp[cb] + (g + kRing) * 8);
        }
        bf16x8 bf0[4], bf1[4];
        bf0[0] = unpack_word(w0.x); bf0[1] = unpack_word(w0.y); bf0[2] = unpack_word(w0.z); bf0[3] = unpack_word(w0.w);
        bf1[0] = unpack_word(w1.x); bf1[1] = unpack_word(w1.y); bf1[2] = unpack_word(w1.z); bf1[3] = unpack_word(w1.w);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          f32x16 p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[rb][0], bf0[0], f32x16{}, 0, 0, 0);
          f32x16 p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[rb][0], bf1[0], f32x16{}, 0, 0, 0);
#pragma unroll
          for (int j = 1; j < 4; ++j) {
            p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[rb][j], bf0[j], p0, 0, 0, 0);
            p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[rb][j], bf1[j], p1, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            acc[rb][0][r] = __builtin_fmaf(s0, p0[r], acc[rb][0][r]);
            acc[rb][1][r] = __builtin_fmaf(s1, p1[r], acc[rb][1][r]);
          }
        }
        if (more) {
          uint8_t* nxt = abuf + ((g + 1) & 1) * 8192;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4*>(nxt + a_chunk_off(srow, shalf * 4 + i)) = stage[i];
        }
        __syncthreads();
      }
    }
  }

  // ---- bias and offset correction: 3 extra K columns per group ------------
  // Stage the biases of the 128 weight rows into the (now free) A buffers.
  uint16_t* b_st = reinterpret_cast<uint16_t*>(abuf);   // [G][128], G*256 B <= 16 KiB
  {
    const int w_ = tid >> 6, cb_ = (tid >> 5) & 1, j_ = tid & 31;
    int n_;
    const QStack* st;
    if constexpr (EPI == kEpiF32) {
      n_ = nt * 128 + w_ * 64 + cb_ * 32 + j_;
      st = &a.w0[stack];
    } else {
      n_ = nt * 64 + w_ * 32 + j_;
      st = cb_ ? &a.w1[stack] : &a.w0[stack];
    }
    const uint16_t* bp = st->b + (size_t(el) * a.N + n_) * G;
    for (int g = 0; g < G; ++g) b_st[g * 128 + tid] = bp[g];
  }
  __syncthreads();
  for (int st = 0; st < KPa / 16; ++st) {
    bf16x8 a2[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      a2[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(aux_s + (rb * 32 + l32) * KPa + 16 * st + 8 * half));
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int scol = cb ? scol1 : scol0;
      uint32_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kk = 16 * st + 8 * half + i;
        const int g = kk / 3;
        const int t = kk - 3 * g;
        uint32_t bits = 0;
        if (g < G) {
          const float s = bf16_to_f32(s_st[g * 128 + scol]);
          const float b = bf16_to_f32(b_st[g * 128 + scol]);
          const float bp = b - 128.0f * s;
          bits = t == 2 ? split_lo(bp) : split_hi(bp);
        }
        v[i] = bits;
      }
      u32x4 pk;
      pk.x = v[0] | (v[1] << 16);
      pk.y = v[2] | (v[3] << 16);
      pk.z = v[4] | (v[5] << 16);
      pk.w = v[6] | (v[7] << 16);
      const bf16x8 b2 = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2[rb], b2, acc[rb][cb], 0, 0, 0);
    }
  }

  // ---- epilogues ------------------------------------------------------------
  if constexpr (EPI == kEpiF32) {
    float* out = reinterpret_cast<float*>(a.out);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = rb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const int row = ti.r0 + m;
        if (row < ti.r1) {
          out[size_t(row) * a.N + ncol[0]] = acc[rb][0][r];
          out[size_t(row) * a.N + ncol[1]] = acc[rb][1][r];
        }
      }
  } else {
    __syncthreads();   // everyone is done with b_st / abuf
    uint16_t* hs = reinterpret_cast<uint16_t*>(abuf);   // [64][64] bf16, natural order
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = rb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const float gv = acc[rb][0][r];
        const float uv = acc[rb][1][r];
        const float hv = gv / (1.0f + __expf(-gv)) * uv;
        hs[m * 64 + wave * 32 + l32] = uint16_t(f32_to_bf16_rne(hv));
      }
    __syncthreads();
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
    const int row = ti.r0 + srow;
    u32x4 ch[4];
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ch[i] = *reinterpret_cast<const u32x4*>(hs + srow * 64 + shalf * 32 + 8 * i);
      part += chunk_sum(ch[i]);
    }
    if constexpr (EPI == kEpiSwigluInternal) {
      const float X = part + __shfl_xor(part, 1, kWave);
      if (row < ti.r1) {
        uint16_t* dst = out + size_t(row) * a.N + nt * 64 + shalf * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(dst + 8 * i) = permute_chunk(ch[i]);
        const int KPo = aux_cols(a.N);
        uint16_t* ax = a.out_aux + size_t(row) * KPo;
        if (shalf == 0) {
          const uint16_t hi = uint16_t(split_hi(X));
          ax[3 * nt + 0] = hi;
          ax[3 * nt + 1] = uint16_t(split_lo(X));
          ax[3 * nt + 2] = hi;
        } else if (nt == 0) {
          for (int c = 3 * (a.N / kGroup); c < KPo; ++c) ax[c] = 0;
        }
      }
    } else {
      if (row < ti.r1) {
        uint16_t* dst = out + size_t(row) * a.N + nt * 64 + shalf * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(dst + 8 * i) = ch[i];
      }
    }
  }
}

size_t gemm_lds_bytes(int K) {
  const int G = K / kGroup;
  return 2 * 8192 + size_t(kBlockRows) * aux_cols(K) * 2 + size_t(G) * 128 * 2;
}

hipError_t launch_gemm(const GemmArgs& ga, int epilogue, int max_row_tiles, hipStream_t stream) {
  const dim3 grid(unsigned(max_row_tiles) * unsigned(ga.NT));
  if (grid.x == 0) return hipSuccess;
  const size_t lds = gemm_lds_bytes(ga.K);
  switch (epilogue) {
    case kEpiF32:
      hipLaunchKernelGGL(gemm_q4_kernel<kEpiF32>, grid, dim3(kGemmThreads), lds, stream, ga);
      break;
    case kEpiSwigluNatural:
      hipLaunchKernelGGL(gemm_q4_kernel<kEpiSwigluNatural>, grid, dim3(kGemmThreads), lds, stream, ga);
      break;
    default:
      hipLaunchKernelGGL(gemm_q4_kernel<kEpiSwigluInternal>, grid, dim3(kGemmThreads), lds, stream, ga);
      break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Activation preparation: permuted chunk order plus the group-sum side table
// (hi, lo, hi of each 64-wide group's fp32 sum; zero padding).
// 8 lanes per group, one 16-byte chunk each.
__global__ __launch_bounds__(256) void prep_rows_kernel(const uint16_t* A, int rows, int K, uint16_t* a_perm,
                                                        uint16_t* a_aux) {
  const int G = K / kGroup;
  const int KP = aux_cols(K);
  const long gid = long(blockIdx.x) * blockDim.x + threadIdx.x;
  const long team = gid >> 3;
  const int sub = int(gid & 7);
  const long total = long(rows) * G;
  const bool ok = team < total;
  const int row = ok ? int(team / G) : 0;
  const int g = ok ? int(team % G) : 0;
  u32x4 v = u32x4{0, 0, 0, 0};
  if (ok) v = *reinterpret_cast<const u32x4*>(A + size_t(row) * K + g * kGroup + 8 * sub);
  float s = chunk_sum(v);
  s += __shfl_xor(s, 1, kWave);
  s += __shfl_xor(s, 2, kWave);
  s += __shfl_xor(s, 4, kWave);
  if (!ok) return;
  *reinterpret_cast<u32x4*>(a_perm + size_t(row) * K + g * kGroup + 8 * sub) = permute_chunk(v);
  uint16_t* ax = a_aux + size_t(row) * KP;
  if (sub == 0) {
    const uint16_t hi = uint16_t(split_hi(s));
    ax[3 * g] = hi;
    ax[3 * g + 1] = uint16_t(split_lo(s));
    ax[3 * g + 2] = hi;
  }
  if (g == G - 1 && sub == 1)
    for (int c = 3 * G; c < KP; ++c) ax[c] = 0;
}

hipError_t launch_prep_rows(const uint16_t* A, int rows, int K, uint16_t* a_perm, uint16_t* a_aux,
                            hipStream_t stream) {
  const long threads = long(rows) * (K / kGroup) * 8;
  if (threads == 0) return hipSuccess;
  const unsigned blocks = unsigned((threads + 255) / 256);
  hipLaunchKernelGGL(prep_rows_kernel, dim3(blocks), dim3(256), 0, stream, A, rows, K, a_perm, a_aux);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weighted combine: y[t] = bf16(S[t] + sum_j w[t][j] * Y[row_of_pair[t*k+j]]).
__global__ __launch_bounds__(256) void combine_kernel(const float* Y, const float* w, const int32_t* row_of_pair,
                                                      int T, int k, int H, int shared_row0, uint16_t* y) {
  const int t = blockIdx.x;
  __shared__ int32_t rows[kMaxTopk];
  __shared__ float ws[kMaxTopk];
  if (threadIdx.x < k) {
    rows[threadIdx.x] = row_of_pair[size_t(t) * k + threadIdx.x];
    ws[threadIdx.x] = w[size_t(t) * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 4; c < H; c += 256 * 4) {
    f32x4 acc = *reinterpret_cast<const f32x4*>(Y + size_t(shared_row0 + t) * H + c);
    for (int j = 0; j < k; ++j) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(Y + size_t(rows[j]) * H + c);
      const float wj = ws[j];
      acc[0] = __builtin_fmaf(wj, v[0], acc[0]);
      acc[1] = __builtin_fmaf(wj, v[1], acc[1]);
      acc[2] = __builtin_fmaf(wj, v[2], acc[2]);
      acc[3] = __builtin_fmaf(wj, v[3], acc[3]);
    }
    uint32_t lo = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
    uint32_t hi = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
    *reinterpret_cast<uint2*>(y + size_t(t) * H + c) = make_uint2(lo, hi);
  }
}

hipError_t launch_combine(const float* Y, const float* w, const int32_t* row_of_pair, int T, int k, int H,
                          int shared_row0, uint16_t* y, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(256), 0, stream, Y, w, row_of_pair, T, k, H, shared_row0, y);
  return hipGetLastError();
}

}  // namespace moe
