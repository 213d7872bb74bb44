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
// Instead the MFMA operand is the exact value 1 + q/16, whose bf16 bit pattern
// is 0x3F80 | (q << 3), so a shift and one AND/OR turn two packed codes into
// two operands. With W = 16s * (1 + q/16) + (b - 16s), for each 64-wide group g
// of K the MFMA chain of the group accumulates
//     P_g = sum_{k in g} x_k (1 + q_k/16)             (fp32)
// which the kernel folds as acc += 16 s_g * P_g (one FMA per output per group;
// 16 s_g is exact). The remaining sum_g (b_g - 16 s_g) X_g, X_g = sum_{k in g}
// x_k, runs on the MFMA as 8 extra K columns per group: an exact three-part
// bf16 split of X_g (from a side table) against b_g, again against -16 s_g,
// and two zero columns, so that each 8-wide operand slice is one group; every
// second group one such MFMA per row block covers the last two groups.
//
// Operand order. One 32-bit word holds codes k..k+7 (nibble i = code k+i); the
// AND/OR unpack yields the bf16 pairs (k, k+4), (k+1, k+5), (k+2, k+6),
// (k+3, k+7). Activations are therefore stored with every 8-element chunk in
// the order [0,4,1,5,2,6,3,7] (prep kernel / SwiGLU epilogue), so both MFMA
// operands list the same K indices in the same slots.
//
// Tiling (one workgroup = 8 wave64s = 512 threads, tile = up to 128 rows):
//   each wave owns 32 output columns of one weight matrix and all rows of the
//   tile, as up to four 32-row MFMA blocks; only blocks that hold real rows are
//   computed (the kernel is instantiated per live-block count), so MFMA work
//   follows the real row count at 32-row granularity.
//   SwiGLU: waves 0-3 = gate columns 0-127, waves 4-7 = up columns 0-127 of
//           the workgroup's 128 (gate and up meet in LDS at the end);
//   STORE_F32: waves 0-7 = columns 0-255.
//   MFMA v_mfma_f32_32x32x16_bf16: per 64-wide group a wave issues one chain
//   of 4 MFMAs per row block; one group's weight codes are unpacked once and
//   reused by every row block.
// Streaming: per group, the activation tile (128 rows x 64 bf16, 16-byte chunks
//   XOR-swizzled by row), the 256 columns' weight codes and the rows'
//   side-table entries land in a 3-slot LDS ring through buffer loads that
//   write LDS directly (no registers, one scalar offset per group), issued two
//   groups ahead; one s_waitcnt + s_barrier per group. Scales and biases of the
//   256 columns are staged once per tile. Every vector-memory instruction moves
//   16 bytes per lane: the per-CU load path, not the MFMA, limits this kernel
//   when instructions move less.
// Work mapping: each XCD takes a contiguous chunk of the tile list and runs
// all column slices of its tiles (see the kernel), so activation rows and
// expert weights are fetched into one XCD's L2 rather than into all eight.
#include "gemm_tiles.h"

namespace moe {

constexpr int kGemmWaves = 8;
constexpr int kGemmThreads = kGemmWaves * 64;
constexpr int kRing = 4;                 // LDS ring slots: group g lives in slot g % 4
constexpr int kSlotA = 0;                // 128 rows x 128 B of activations
constexpr int kSlotB = 16384;            // 8 waves x 64 lanes x 16 B of weight codes
constexpr int kSlotXP = 24576;           // odd groups: 128 rows x 32 B, side-table entries of groups g-1, g
constexpr int kSlotBytes = 28672;
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer descriptor flags (gfx9 family)
// s_waitcnt immediates (gfx9: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8]); only vmcnt waits.
constexpr int kWaitVm0 = 0x0F70;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Row m of an activation tile holds its 8 16-byte chunks permuted by
// c -> c ^ swz(m). Within any 16 consecutive rows, (m & 1, chunk slot) never
// repeats for a fixed c, and within any 8 consecutive rows the slots are all
// distinct, so a 16-lane (64-bank) or 8-lane (32-bank) group of one fragment
// read touches every bank once.
__device__ __forceinline__ int swz(int m) { return (m & 7) ^ ((m >> 3) & 1); }
__device__ __forceinline__ int a_chunk_off(int m, int c) { return (m * 8 + (c ^ swz(m))) * 16; }

__device__ __forceinline__ lds_ptr_t lds(void* p) { return (lds_ptr_t)p; }

// Scales and biases of a wave's 32 columns, staged at tile start as
// [pair j][column][2 groups] (4 bytes per column and group pair), so that the
// 32 lanes of one column read hit 32 consecutive LDS words.
__host__ __device__ constexpr int staged_words(int G) { return 32 * (G / 2); }

// LDS of one workgroup: the ring plus the staged scales and biases of the 256
// columns during the K loop; afterwards, for SwiGLU, the gate tile (128 x 128
// fp32) and the h tile (128 x 128 bf16).
size_t gemm_lds_bytes(int K) {
  const int G = K / kGroup;
  const size_t loop = size_t(kRing) * kSlotBytes + size_t(2) * kGemmWaves * staged_words(G) * 4;
  const size_t swiglu = size_t(kBlockRows) * 128 * 4 + size_t(kBlockRows) * 128 * 2;
  return loop > swiglu ? loop : swiglu;
}

// Per-wave streaming state: buffer descriptors, per-lane byte offsets.
struct Stream {
  __amdgpu_buffer_rsrc_t ra, rb, rxp;
  uint32_t va[2];    // activation chunk offsets (2 instructions)
  uint32_t vb;       // weight-code offset
  uint32_t vxp;      // side-table offset of (row, half) (waves 0..3, odd groups)
};

// Loads of group g into its slot: 2 activation + 1 weight-code instruction per
// wave; for odd g, waves 0..3 also load the side-table entries of groups g-1
// and g (32 contiguous bytes per row).
template <int ODD>
__device__ __forceinline__ void issue_group(const Stream& st, uint8_t* slot, int g, int wave) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(st.ra, lds(slot + kSlotA + wave * 2048 + i * 1024), 16, st.va[i],
                                             g * (kGroup * 2), 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(st.rb, lds(slot + kSlotB + wave * 1024), 16, st.vb, g * 32, 0, 0);
  if (ODD && wave < 4)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(st.rxp, lds(slot + kSlotXP + wave * 1024), 16, st.vxp, (g - 1) * 16, 0,
                                             0);
}

// Wait until at most N of this wave's buffer loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(kWaitVm0 | N);
}

__device__ __forceinline__ void fold(const f32x16& p, float sc, f32x16& acc) {
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = __builtin_fmaf(sc, p[r], acc[r]);
}

// Step g of the K loop (S = g % 4, a compile-time slot). Group g is in slot S;
// groups g+1, g+2 may still be landing; group g+3 is issued into slot
// (S+3)%4, which held group g-1.
//
// Per live row block rb: a chain of 4 MFMAs over the group's 64 K values
// gives P_g. The NRB chains are issued level by level (level l = the l-th
// 16-wide slice of the group), so consecutive MFMAs never depend on each
// other. Chain rb's P_g is folded as acc += 16 s_g P_g just before the
// chain's first MFMA of the next step, when the matrix pipe has long
// finished it. For odd g one more MFMA per block adds the bias term of groups
// g-1 and g (lanes 0..31: group g-1, 32..63: group g) from the rows' 8
// side-table entries per group against (b, b, b, -16 s, -16 s, -16 s, 0, 0)
// of the lane's column.
template <int NRB, int S>
__device__ __forceinline__ void loop_step(const Stream& st, uint8_t* ring, const uint32_t* s_pairs,
                                          const uint32_t* b_pairs, int g, int G, int wave, int lane, uint32_t& s_pair,
                                          uint32_t& b_pair, float& sc_prev, f32x16 (&q)[4], f32x16 (&acc)[4]) {
  constexpr int ODD = S & 1;
  const int l32 = lane & 31, half = lane >> 5;
  // this wave's loads of group g have landed once at most those of g+1 and
  // g+2 are outstanding; the barrier makes it so for every wave, and orders
  // every wave's reads of slot (S+3)%4 (previous step) before its refill
  // (a wave issues 3 loads per group, waves 0..3 one more for odd groups)
  if (g + 2 < G) {
    if (wave < 4)
      wait_vm<7>();
    else
      wait_vm<6>();
  } else if (g + 1 < G) {
    if (!ODD && wave < 4)
      wait_vm<4>();
    else
      wait_vm<3>();
  } else {
    wait_vm<0>();
  }
  __builtin_amdgcn_s_barrier();
  if (g + 3 < G) issue_group<!ODD>(st, ring + ((S + 3) % kRing) * kSlotBytes, g + 3, wave);
  const uint8_t* slot = ring + S * kSlotBytes;

  const u32x4 w = *reinterpret_cast<const u32x4*>(slot + kSlotB + wave * 1024 + lane * 16);
  if (!ODD) {
    s_pair = s_pairs[(g >> 1) * 32];
    b_pair = b_pairs[(g >> 1) * 32];
  }
  bf16x8 fa[2][4];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
    fa[0][rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(slot + a_chunk_off(rb * 32 + l32, 4 * half)));
  const uint32_t nib = kNib, magic = kMagic;
#pragma unroll
  for (int l = 0; l < 4; ++l) {
    if (l + 1 < 4) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        fa[(l + 1) & 1][rb] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(slot + a_chunk_off(rb * 32 + l32, 4 * half + l + 1)));
    }
    const bf16x8 bq = unpack_word(w[l], nib, magic);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      if (l == 0) {
        fold(q[rb], sc_prev, acc[rb]);
        q[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0][rb], bq, f32x16{}, 0, 0, 0);
      } else {
        q[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[l & 1][rb], bq, q[rb], 0, 0, 0);
      }
    }
  }
  sc_prev = 16.0f * __uint_as_float(ODD ? (s_pair & 0xFFFF0000u) : (s_pair << 16));
  if (ODD) {
    const int sh = half << 4;
    const uint32_t sb = (s_pair >> sh) & 0xFFFFu, bb = (b_pair >> sh) & 0xFFFFu;
    // -16 s is exact in bf16 (a power-of-two multiple), so truncating the
    // fp32 product is the rounding
    const uint32_t ns = __float_as_uint(-16.0f * __uint_as_float(sb << 16)) >> 16;
    const u32x4 pk = {bb | (bb << 16), bb | (ns << 16), ns | (ns << 16), 0u};
    const bf16x8 bv = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const bf16x8 xa =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(slot + kSlotXP + (rb * 32 + l32) * 32 + half * 16));
      acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, bv, acc[rb], 0, 0, 0);
    }
  }
}

// G is even (K is a multiple of 128).
template <int NRB>
__device__ __forceinline__ void main_loop(const Stream& st, uint8_t* ring, const uint32_t* s_pairs,
                                          const uint32_t* b_pairs, int G, int wave, int lane, f32x16 (&acc)[4]) {
  uint32_t s_pair = 0, b_pair = 0;
  float sc_prev = 0.0f;
  f32x16 q[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) q[rb] = f32x16{};
  // unrolled by the ring size so every slot offset and group parity is a constant
  for (int g = 0; g < G; g += kRing) {
    loop_step<NRB, 0>(st, ring, s_pairs, b_pairs, g, G, wave, lane, s_pair, b_pair, sc_prev, q, acc);
    loop_step<NRB, 1>(st, ring, s_pairs, b_pairs, g + 1, G, wave, lane, s_pair, b_pair, sc_prev, q, acc);
    if (g + 2 < G) {
      loop_step<NRB, 2>(st, ring, s_pairs, b_pairs, g + 2, G, wave, lane, s_pair, b_pair, sc_prev, q, acc);
      loop_step<NRB, 3>(st, ring, s_pairs, b_pairs, g + 3, G, wave, lane, s_pair, b_pair, sc_prev, q, acc);
    }
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) fold(q[rb], sc_prev, acc[rb]);
}

template <int EPI>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_q4_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int K = a.K;
  const int G = K / kGroup;
  const int KPx = xpart_cols(K);
  uint8_t* ring = smem;
  const int SW = staged_words(G);
  uint32_t* s_st = reinterpret_cast<uint32_t*>(smem + kRing * kSlotBytes);   // [8 waves][SW]
  uint32_t* b_st = s_st + kGemmWaves * SW;                                    // [8 waves][SW]

  // XCD-aware work mapping: workgroups are dispatched round-robin over the 8
  // XCDs (blockIdx % 8). The tile list (shared tiles, then routed tiles in
  // expert order) is cut into 8 contiguous chunks, chunk x runs on XCD x, and
  // within a chunk the column slices of a tile are consecutive. So every
  // column slice of a row tile reads the activation rows from the same L2, and
  // consecutive tiles of one expert share its weights in that L2.
  const int ntot = a.n_shared_tiles + *a.num_tiles;
  const int chunk = (ntot + 7) >> 3;
  const int xcd = blockIdx.x & 7;
  const int j = blockIdx.x >> 3;
  const int nt = j % a.NT;
  const int tile = xcd * chunk + j / a.NT;
  if (j / a.NT >= chunk || tile >= ntot) return;
  TileInfo ti;
  if (!tile_info(a, tile, ti)) return;
  const int stack = ti.e == a.E ? 1 : 0;
  const int el = stack ? 0 : ti.e;
  const int nrows = ti.r1 - ti.r0;
  const int nrb = (nrows + 31) >> 5;     // 32-row blocks holding real rows

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // ---- this wave's weight matrix and its 32 columns ------------------------
  // A wave past the last column (N not a multiple of the workgroup's width)
  // streams the last 32 columns again and stores nothing.
  int col0;
  const QStack* mat;
  if constexpr (EPI == kEpiF32) {
    col0 = nt * 256 + wave * 32;
    mat = &a.w0[stack];
  } else {
    col0 = nt * 128 + (wave & 3) * 32;
    mat = (wave >> 2) ? &a.w1[stack] : &a.w0[stack];
  }
  const bool live = col0 < a.N;
  col0 = live ? col0 : a.N - 32;
  const size_t wrow0 = size_t(el) * a.N + col0;
  const uint32_t* q_wave = mat->q + wrow0 * size_t(K / 8);
  const uint16_t* s_glob = mat->s + wrow0 * size_t(G);     // 32 contiguous rows of G scales
  const uint16_t* b_glob = mat->b + wrow0 * size_t(G);
  const int ncol = col0 + l32;

  // ---- streaming descriptors and per-lane offsets -------------------------
  Stream st;
  st.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.A), 0, 0x7FFFFFFF, kRsrcWord3);
  st.rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(q_wave), 0, 0x7FFFFFFF, kRsrcWord3);
  st.rxp = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.Apart), 0, 0x7FFFFFFF, kRsrcWord3);
  {
    // activation load i of wave w fills chunk positions w*128 + i*64 + lane:
    // row m = w*16 + i*8 + lane/8 and chunk slot lane%8, which holds logical
    // chunk (lane%8) ^ swz(m)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = wave * 16 + i * 8 + (lane >> 3);
      const int cidx = (lane & 7) ^ swz(m);
      const int r = ti.r0 + min(m, nrows - 1);     // padding rows re-read the last real row
      st.va[i] = uint32_t(src_row(a, r)) * uint32_t(K * 2) + uint32_t(cidx * 16);
    }
    st.vb = uint32_t((l32 * (K / 8) + 4 * half) * 4);
    // side-table load of wave w (0..3): row w*32 + lane/2, 16-byte half lane%2
    const int mx = (wave & 3) * 32 + (lane >> 1);
    st.vxp = uint32_t(src_row(a, ti.r0 + min(mx, nrows - 1))) * uint32_t(KPx * 2) + uint32_t((lane & 1) * 16);
  }

  // ---- prologue: scales and biases of the wave's 32 columns, groups 0..2 ----
  {
    // word p = j*32 + c of the wave's staging area holds column c's values of
    // groups 2j, 2j+1, i.e. 4 bytes at (c*G + 2j)*2 of the column block
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(s_glob), 0, 0x7FFFFFFF, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rbias =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(b_glob), 0, 0x7FFFFFFF, kRsrcWord3);
    for (int p0 = 0; p0 < SW; p0 += 64) {
      const int p = p0 + lane;
      if (p < SW) {
        const uint32_t off = uint32_t(((p & 31) * G + 2 * (p >> 5)) * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds(s_st + wave * SW + p0), 4, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rbias, lds(b_st + wave * SW + p0), 4, off, 0, 0, 0);
      }
    }
  }
  issue_group<0>(st, ring, 0, wave);
  issue_group<1>(st, ring + kSlotBytes, 1, wave);
  if (G > 2) issue_group<0>(st, ring + 2 * kSlotBytes, 2, wave);

  f32x16 acc[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x16{};
  const uint32_t* s_pairs = s_st + wave * SW + l32;
  const uint32_t* b_pairs = b_st + wave * SW + l32;
  switch (nrb) {
    case 1: main_loop<1>(st, ring, s_pairs, b_pairs, G, wave, lane, acc); break;
    case 2: main_loop<2>(st, ring, s_pairs, b_pairs, G, wave, lane, acc); break;
    case 3: main_loop<3>(st, ring, s_pairs, b_pairs, G, wave, lane, acc); break;
    default: main_loop<4>(st, ring, s_pairs, b_pairs, G, wave, lane, acc); break;
  }
  __syncthreads();   // every wave is done with the ring

  // ---- epilogues ------------------------------------------------------------
  if constexpr (EPI == kEpiF32) {
    float* out = reinterpret_cast<float*>(a.out);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = rb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (live && m < nrows) out[size_t(ti.r0 + m) * a.N + ncol] = acc[rb][r];
      }
  } else {
    float* gate_s = reinterpret_cast<float*>(ring);                           // [128][128] fp32
    uint16_t* hs = reinterpret_cast<uint16_t*>(ring + kBlockRows * 128 * 4);  // [128][128] bf16
    const int col = (wave & 3) * 32 + l32;
    if (wave < 4) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = rb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          gate_s[m * 128 + col] = acc[rb][r];
        }
    }
    __syncthreads();
    if (wave >= 4) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = rb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const float gv = gate_s[m * 128 + col];
          const float uv = acc[rb][r];
          const float hv = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
          hs[m * 128 + col] = uint16_t(f32_to_bf16_rne(hv));
        }
    }
    __syncthreads();
    // thread t: row t/4, quarter t%4 = 32 columns; quarters (0,1) and (2,3)
    // are the two 64-wide groups of h this workgroup produced
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
    const int srow = tid >> 2, sq = tid & 3;
    const int row = ti.r0 + srow;
    u32x4 ch[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ch[i] = *reinterpret_cast<const u32x4*>(hs + srow * 128 + sq * 32 + 8 * i);
    if constexpr (EPI == kEpiSwigluInternal) {
      double part = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i) part += chunk_sum_f64(ch[i]);
      const float X = float(part + __shfl_xor(part, 1, kWave));
      if (srow < nrows) {
        uint16_t* dst = out + size_t(row) * a.N + nt * 128 + sq * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(dst + 8 * i) = permute_chunk(ch[i]);
        if ((sq & 1) == 0) {
          const int go = 2 * nt + (sq >> 1);   // group of h this pair of quarters covers
          uint16_t h, m, l;
          split3_bf16(X, h, m, l);
          const u32x4 e = {uint32_t(h) | (uint32_t(m) << 16), uint32_t(l) | (uint32_t(h) << 16),
                           uint32_t(m) | (uint32_t(l) << 16), 0u};
          *reinterpret_cast<u32x4*>(a.out_part + size_t(row) * xpart_cols(a.N) + 8 * go) = e;
        }
      }
    } else {
      if (srow < nrows && nt * 128 + sq * 32 < a.N) {
        uint16_t* dst = out + size_t(row) * a.N + nt * 128 + sq * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(dst + 8 * i) = ch[i];
      }
    }
  }
}

hipError_t launch_gemm(const GemmArgs& ga, int epilogue, int max_row_tiles, hipStream_t stream) {
  // 8 chunks of at most ceil(max_row_tiles / 8) tiles, NT column slices each
  const dim3 grid(8u * unsigned(ceil_div(max_row_tiles, 8)) * unsigned(ga.NT));
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

}  // namespace moe
