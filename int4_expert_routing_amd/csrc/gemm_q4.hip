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
// 64-wide group g of K, with X_g = sum_{k in g} x_k, the MFMA chain of the group
// starts from the accumulator value -128*X_g (exact fp32, from a side table)
// and adds sum x_k (128 + q_k), leaving
//     P_g = sum_{k in g} x_k q_k                      (fp32, no cancellation)
// which the kernel folds as acc += s_g * P_g (one FMA per output per group).
// The bias term sum_g b_g X_g runs on the MFMA as 3 extra K columns per group:
// activations (X_hi, X_mid, X_lo), an exact three-part bf16 split of X_g,
// against (b_g, b_g, b_g).
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
constexpr int kAbufBytes = 8192;    // one A buffer: 64 rows x 64 bf16

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

// Starting accumulator of a group's chain for row block rb: lane holds rows
// rb*32 + 8j + 4*half + i (j, i = 0..3), the 32x32 MFMA output layout.
__device__ __forceinline__ f32x16 chain_init(const float* xneg_g, int rb, int half) {
  const f32x4* p = reinterpret_cast<const f32x4*>(xneg_g + rb * 32 + 4 * half);
  const f32x4 a = p[0], b = p[2], c = p[4], d = p[6];
  return f32x16{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3], c[0], c[1], c[2], c[3], d[0], d[1], d[2], d[3]};
}

size_t gemm_lds_bytes(int K) {
  const int G = K / kGroup;
  return 2 * kAbufBytes                           // A double buffer
         + size_t(G) * kBlockRows * 4              // -128 X_g  [G][64]
         + size_t(kBlockRows) * xpart_cols(K) * 2  // X_g parts [64][xpart_cols]
         + size_t(G) * 128 * 2;                    // scales    [G][128]
}

template <int EPI>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_q4_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int K = a.K;
  const int G = K / kGroup;
  const int KPx = xpart_cols(K);
  const int KNx = xneg_cols(K);
  uint8_t* abuf = smem;
  float* xneg_s = reinterpret_cast<float*>(smem + 2 * kAbufBytes);        // [G][64]
  uint16_t* xpart_s = reinterpret_cast<uint16_t*>(xneg_s + G * kBlockRows);  // [64][KPx]
  uint16_t* s_st = xpart_s + kBlockRows * KPx;                             // [G][128]

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
  const uint32_t* qp[2];
  qp[0] = m0.q + (size_t(el) * a.N + ncol[0]) * qrow + 4 * half;
  qp[1] = m1.q + (size_t(el) * a.N + ncol[1]) * qrow + 4 * half;

  // thread t <-> weight row (wave t/64, cb (t/32)%2, lane t%32) of the workgroup
  const QStack* st_row;
  int n_row;
  {
    const int w_ = tid >> 6, cb_ = (tid >> 5) & 1, j_ = tid & 31;
    if constexpr (EPI == kEpiF32) {
      n_row = nt * 128 + w_ * 64 + cb_ * 32 + j_;
      st_row = &a.w0[stack];
    } else {
      n_row = nt * 64 + w_ * 32 + j_;
      st_row = cb_ ? &a.w1[stack] : &a.w0[stack];
    }
  }
  {
    const uint16_t* sp = st_row->s + (size_t(el) * a.N + n_row) * G;
    for (int g = 0; g < G; ++g) s_st[g * 128 + tid] = sp[g];
  }

  // ---- prologue: side tables and the first A tile -------------------------
  const int srow = tid >> 1;          // staging row 0..63
  const int shalf = tid & 1;          // which 32-element half of a group
  const int sr = ti.r0 + srow;
  const bool svalid = sr < ti.r1;
  const int src = svalid ? src_row(a, sr) : 0;
  const uint16_t* arow = a.A + size_t(src) * K + shalf * 32;
  {
    const float* xn = a.Axneg + size_t(src) * KNx;
    for (int g = shalf; g < G; g += 2) xneg_s[g * kBlockRows + srow] = svalid ? xn[g] : 0.0f;
    const uint16_t* xp = a.Apart + size_t(src) * KPx;
    for (int c = shalf; c < KPx / 8; c += 2) {
      u32x4 v = svalid ? *reinterpret_cast<const u32x4*>(xp + 8 * c) : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(xpart_s + srow * KPx + 8 * c) = v;
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
        const uint8_t* cur = abuf + (g & 1) * kAbufBytes;
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
        const float* xg = xneg_s + g * kBlockRows;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          f32x16 p0 = chain_init(xg, rb, half);
          f32x16 p1 = chain_init(xg, rb, half);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
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
          uint8_t* nxt = abuf + ((g + 1) & 1) * kAbufBytes;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4*>(nxt + a_chunk_off(srow, shalf * 4 + i)) = stage[i];
        }
        __syncthreads();
      }
    }
  }

  // ---- bias term: 3 extra K columns per group ------------------------------
  // Stage the biases of the 128 weight rows into the (now free) A buffers.
  uint16_t* b_st = reinterpret_cast<uint16_t*>(abuf);   // [G][128], G*256 B <= 16 KiB
  {
    const uint16_t* bp = st_row->b + (size_t(el) * a.N + n_row) * G;
    for (int g = 0; g < G; ++g) b_st[g * 128 + tid] = bp[g];
  }
  __syncthreads();
  for (int st = 0; st < KPx / 16; ++st) {
    bf16x8 a2[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      a2[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xpart_s + (rb * 32 + l32) * KPx + 16 * st + 8 * half));
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int scol = cb ? scol1 : scol0;
      uint32_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int g = (16 * st + 8 * half + i) / 3;
        v[i] = g < G ? uint32_t(b_st[g * 128 + scol]) : 0u;
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
#pragma unroll
    for (int i = 0; i < 4; ++i) ch[i] = *reinterpret_cast<const u32x4*>(hs + srow * 64 + shalf * 32 + 8 * i);
    if constexpr (EPI == kEpiSwigluInternal) {
      double part = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i) part += chunk_sum_f64(ch[i]);
      const float X = float(part + __shfl_xor(part, 1, kWave));
      if (row < ti.r1) {
        uint16_t* dst = out + size_t(row) * a.N + nt * 64 + shalf * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(dst + 8 * i) = permute_chunk(ch[i]);
        const int Go = a.N / kGroup;
        const int KPo = xpart_cols(a.N);
        uint16_t* xp = a.out_part + size_t(row) * KPo;
        float* xn = a.out_xneg + size_t(row) * xneg_cols(a.N);
        if (shalf == 0) {
          uint16_t h, m, l;
          split3_bf16(X, h, m, l);
          xp[3 * nt + 0] = h;
          xp[3 * nt + 1] = m;
          xp[3 * nt + 2] = l;
          xn[nt] = -128.0f * X;
        } else if (nt == 0) {
          for (int c = 3 * Go; c < KPo; ++c) xp[c] = 0;
          for (int c = Go; c < xneg_cols(a.N); ++c) xn[c] = 0.0f;
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
// Activation preparation: permuted chunk order plus the group-sum tables.
// 8 lanes per group, one 16-byte chunk each; group sums in fp64, rounded once.
__global__ __launch_bounds__(256) void prep_rows_kernel(const uint16_t* A, int rows, int K, uint16_t* a_perm,
                                                        float* a_xneg, uint16_t* a_part) {
  const int G = K / kGroup;
  const int KPx = xpart_cols(K);
  const int KNx = xneg_cols(K);
  const long gid = long(blockIdx.x) * blockDim.x + threadIdx.x;
  const long team = gid >> 3;
  const int sub = int(gid & 7);
  const long total = long(rows) * G;
  const bool ok = team < total;
  const int row = ok ? int(team / G) : 0;
  const int g = ok ? int(team % G) : 0;
  u32x4 v = u32x4{0, 0, 0, 0};
  if (ok) v = *reinterpret_cast<const u32x4*>(A + size_t(row) * K + g * kGroup + 8 * sub);
  double s = chunk_sum_f64(v);
  s += __shfl_xor(s, 1, kWave);
  s += __shfl_xor(s, 2, kWave);
  s += __shfl_xor(s, 4, kWave);
  if (!ok) return;
  *reinterpret_cast<u32x4*>(a_perm + size_t(row) * K + g * kGroup + 8 * sub) = permute_chunk(v);
  uint16_t* xp = a_part + size_t(row) * KPx;
  float* xn = a_xneg + size_t(row) * KNx;
  if (sub == 0) {
    const float X = float(s);
    uint16_t h, m, l;
    split3_bf16(X, h, m, l);
    xp[3 * g] = h;
    xp[3 * g + 1] = m;
    xp[3 * g + 2] = l;
    xn[g] = -128.0f * X;
  }
  if (g == G - 1 && sub == 1) {
    for (int c = 3 * G; c < KPx; ++c) xp[c] = 0;
    for (int c = G; c < KNx; ++c) xn[c] = 0.0f;
  }
}

hipError_t launch_prep_rows(const uint16_t* A, int rows, int K, uint16_t* a_perm, float* a_xneg,
                            uint16_t* a_part, hipStream_t stream) {
  const long threads = long(rows) * (K / kGroup) * 8;
  if (threads == 0) return hipSuccess;
  const unsigned blocks = unsigned((threads + 255) / 256);
  hipLaunchKernelGGL(prep_rows_kernel, dim3(blocks), dim3(256), 0, stream, A, rows, K, a_perm, a_xneg, a_part);
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
