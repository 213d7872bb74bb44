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
// of K the MFMA chain of the group adds
//     P_g = sum_{k in g} x_k (1 + q_k/16)             (fp32)
// to an accumulator kept in units of U = 16 s_g: before the chain the
// accumulator is multiplied by U_{g-1} / U_g (one multiply per output per
// group, and no second accumulator set), and after the K loop by the last U.
// The remaining sum_g (b_g - 16 s_g) X_g, X_g = sum_{k in g} x_k, runs on the
// MFMA as 8 extra K columns per group: the group's coefficient in the current
// unit, split into bf16 parts, against an exact three-part bf16 split of X_g
// (a side table); every second group one such MFMA per block covers the last
// two groups.
//
// Operand order. One 32-bit word holds codes k..k+7 (nibble i = code k+i); the
// AND/OR unpack yields the bf16 pairs (k, k+4), (k+1, k+5), (k+2, k+6),
// (k+3, k+7). Activations are therefore stored with every 8-element chunk in
// the order [0,4,1,5,2,6,3,7] (prep kernel / SwiGLU epilogue), so both MFMA
// operands list the same K indices in the same slots.
//
// Tiling (one workgroup = 4 wave64s = 256 threads, tile = up to 128 rows,
// two workgroups per CU):
//   each wave owns 64 output columns as two 32-column blocks and all rows of
//   the tile, as up to four 32-row MFMA blocks, so each activation fragment
//   read from LDS feeds two MFMAs; only row blocks that hold real rows are
//   computed (the kernel is instantiated per live-block count).
//   SwiGLU: wave w = gate columns 32w..32w+31 (block 0) and the same up
//           columns (block 1) of the workgroup's 128, so gate and up meet in
//           registers;
//   STORE_F32: wave w = columns 64w..64w+63 of the workgroup's 256.
//   MFMA v_mfma_f32_32x32x16_bf16: per 64-wide group a wave issues one chain
//   of 4 MFMAs per (row block, column block); one group's weight codes are
//   unpacked once and reused by every row block.
// Streaming: per group, the activation tile (128 or 160 rows x 64 bf16,
//   16-byte chunks XOR-swizzled by row) and the 256 columns' weight codes land
//   in a 2-slot LDS ring through buffer loads that write LDS directly (no
//   registers, one scalar offset per group), issued one group ahead (tiles of
//   at most 32 rows: 32-row activation tiles in a 5-slot ring, four groups
//   ahead); the scale and bias words of a group pair land in a 2-slot (3-slot)
//   ring with the even group's loads (global loads that write LDS), and the
//   rows' side-table entries of the current pair in a single slot, issued at
//   its even step. No load returns to registers: a register-returning load
//   would make the compiler wait for it with a count that ignores the
//   LDS-writing loads issued after it, i.e. stall on the loads just issued.
//   One s_waitcnt + s_barrier per group (small tiles: one more per pair
//   before the side table is read).
// Work mapping: each XCD takes a contiguous chunk of the tile list and runs
// all column slices of its tiles (see the kernel), so activation rows and
// expert weights are fetched into one XCD's L2 rather than into all eight.
#include "gemm_tiles.h"

namespace moe {

constexpr int kGemmWaves = 4;
constexpr int kGemmThreads = kGemmWaves * 64;
constexpr int kXpSlotBytes = 4096;       // side table of one group pair: 128 rows x 32 B (groups 2p, 2p+1)
constexpr int kSbWaveBytes = 256;        // scale/bias words of one group pair, one column block: 64 words

// LDS ring geometry. Group g's activation tile lives in A slot g % A_RING and
// its codes in code slot g % C_RING; activations are loaded DA steps ahead and
// codes DC steps ahead. The scale/bias words of pair p live in slot p % SBS.
//   full tiles (33..128 rows): 2 slots, each 128 activation rows then the
//     codes; group g issued at step g - 1 into the slot group g - 2 used (one
//     step of a full tile covers the round trip: three slots, two groups
//     ahead, measured 1% slower at T=4096 and the same at T=512);
//   small tiles (at most 32 rows): 5 slots of 32 activation rows and 6 code
//     slots; group g's activations issued at step g - 4, and both groups of a
//     pair's codes at the pair's even step 2p - 4, back to back, so the second
//     group's loads find the 128-byte lines the first group's brought into L1
//     (a column's codes of two groups are 64 contiguous bytes). Such a tile
//     does too little arithmetic per group to cover a memory round trip in two
//     steps; its activation tile is a quarter of a full one, so the same LDS
//     holds twice the groups in flight;
//   merged tiles (129..160 rows: an expert's last full tile together with a
//     remainder of at most 32 rows, in the layer's tile lists): the same with
//     160 activation rows. The
//     remainder rows then share the full tile's code unpacking instead of
//     unpacking the expert's weights again for a few rows (a tile of 1..32
//     rows costs ~35-45% of a full one).
//   one-column-block launches (NCB = 1: all tiles of at most 32 rows, each
//     wave one 32-column block): the small geometry with half the code
//     bytes per group, activations and codes two groups ahead (a code pair
//     at every even step), 31 KB, so that five workgroups fit per CU: at this
//     size more resident workgroups beat a deeper ring (T=512 layer, 32-row
//     tiles: 3 per CU with 4 groups ahead ~166 us, 4 per CU with activations
//     2 ahead ~158, 5 per CU ~151; 3 per CU with codes 6 ahead was slower).
enum RingMode { kRingFull = 0, kRingSmall = 1, kRingMerged = 2 };
template <int RM, int NCB = 2>
struct Ring {
  static constexpr bool SR = RM == kRingSmall;
  static constexpr int DC = SR ? (NCB == 1 ? 2 : 4) : 1;             // codes: groups ahead (even when SR)
  static constexpr int DA = SR ? (NCB == 1 ? 2 : 4) : 1;             // activations: groups ahead, DA <= DC
  static constexpr int AROWS = SR ? 32 : RM == kRingMerged ? 160 : 128;   // activation rows per slot
  static constexpr int ALOADS = AROWS / 32;               // activation loads per wave and group (8 rows each)
  static constexpr int A_RING = DA + 1;
  static constexpr int C_RING = SR ? DC + 2 : DC + 1;
  static constexpr int CODES = 4 * NCB * 1024;           // 4 waves x NCB column blocks x 64 lanes x 16 B
  static constexpr int A_SLOT = SR ? AROWS * 128 : AROWS * 128 + CODES;
  static constexpr int C_BASE = SR ? A_RING * A_SLOT : AROWS * 128;
  static constexpr int C_SLOT = SR ? CODES : A_SLOT;
  static constexpr int XP = SR ? C_BASE + C_RING * C_SLOT : A_RING * A_SLOT;
  // side-table slot of one pair: 32 B per row. Small tiles: rows 0..31, which
  // every wave loads into the same 1 KB (the same bytes); merged tiles load
  // rows 128..159 with a second load per wave (again the same bytes)
  static constexpr int XLOADS = AROWS > 128 ? 2 : 1;
  static constexpr int XP_BYTES = SR ? 1024 : XLOADS * kXpSlotBytes;
  static constexpr int SB = XP + XP_BYTES;
  static constexpr int SBS = SR ? DC / 2 + 1 : 2;      // pair p's words are read at step 2p, loaded at 2p - DC
  static constexpr int SB_SLOT = 4 * NCB * kSbWaveBytes;
  static constexpr int END = SB + SBS * SB_SLOT;
  static_assert(!SR || (DC % 2 == 0 && DA >= 1 && DA <= DC), "small ring distances");
};
constexpr int kLdsLoopFS = Ring<kRingFull>::END > Ring<kRingSmall>::END ? Ring<kRingFull>::END : Ring<kRingSmall>::END;
constexpr int kLdsLoop = kLdsLoopFS > Ring<kRingMerged>::END ? kLdsLoopFS : Ring<kRingMerged>::END;
constexpr int kMaxRows = 160;   // rows of a merged tile
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer descriptor flags (gfx9 family)
// A byte offset past every buffer descriptor's range here (num_records is
// 0x7FFFFFFF; with the per-group offsets of at most a few KB it stays below
// 2^32): a load at it is out of range and makes no memory access.
constexpr uint32_t kPastRange = 0x80000000u;
// s_waitcnt immediates (gfx9: vmcnt[3:0] and [15:14], expcnt[6:4],
// lgkmcnt[11:8]); only vmcnt waits.
constexpr int kWaitVm0 = 0x0F70;
// Scales below this magnitude count as zero (their products are below 2^-96
// of the activations): the running unit must stay a normal fp32 number.
constexpr float kMinUnit = 0x1p-96f;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

// Row m of an activation tile holds its 8 16-byte chunks permuted by
// c -> c ^ swz(m). Within any 16 consecutive rows, (m & 1, chunk slot) never
// repeats for a fixed c, and within any 8 consecutive rows the slots are all
// distinct, so a 16-lane (64-bank) or 8-lane (32-bank) group of one fragment
// read touches every bank once.
__device__ __forceinline__ int swz(int m) { return (m & 7) ^ ((m >> 3) & 1); }
__device__ __forceinline__ int a_chunk_off(int m, int c) { return (m * 8 + (c ^ swz(m))) * 16; }

__device__ __forceinline__ lds_ptr_t lds(void* p) { return (lds_ptr_t)p; }
__device__ __forceinline__ gbl_ptr_t gbl(const void* p) { return (gbl_ptr_t)const_cast<void*>(p); }

// One 16-byte-per-lane buffer load that writes LDS at dst + 16 * lane, and one
// 4-byte-per-lane global load that writes LDS at dst + 4 * lane. (Plain
// functions, so that the templates below reach the builtins only through
// them.)
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds(dst), 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void global_to_lds4(const uint32_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(gbl(src), lds(dst), 4, 0, 0);
}

// LDS of one workgroup: the two rings during the K loop; afterwards the h
// tile (SwiGLU: up to 160 x 128 bf16) or each wave's 128 x 32 fp32 staging
// block (STORE_F32, row stride 36 floats; a merged tile's last 32 rows take a
// second round).
constexpr int kF32StageStride = 36;
size_t gemm_lds_bytes(int /*K*/, int ncb = 2) {
  if (ncb == 1) {
    // the small ring, then 32 x 65 fp32 gate values + 32 x 64 bf16 h, or four
    // 32 x 36 fp32 staging blocks
    constexpr size_t ring = size_t(Ring<kRingSmall, 1>::END);
    constexpr size_t epi = 32 * 65 * 4 + 32 * 64 * 2;
    static_assert(ring <= 160 * 1024 / 5 && epi <= ring && size_t(kGemmWaves) * 32 * kF32StageStride * 4 <= ring,
                  "five workgroups per CU");
    return ring;
  }
  const size_t swiglu = size_t(kMaxRows) * 128 * 2;
  const size_t f32 = size_t(kGemmWaves) * kBlockRows * kF32StageStride * 4;
  size_t m = size_t(kLdsLoop);
  m = m > swiglu ? m : swiglu;
  return m > f32 ? m : f32;
}

// Per-wave streaming state: buffer descriptors, per-lane byte offsets, and the
// scale/bias pair addresses of the lane's two columns.
struct Stream {
  __amdgpu_buffer_rsrc_t ra, rb0, rb1, rxp;
  uint32_t va[5];    // activation chunk offsets (one per load; small tiles use va[0] only)
  uint32_t vb;       // code offset of the lane (same in both column blocks)
  uint32_t vxp;      // side-table offset of (row, half)
  uint32_t vxp2;     // merged tiles: the same for rows 128..159
  int gstride;       // bytes between a column's codes of consecutive groups (32, or N * 32 when packed)
  int sbstride;      // u32 words between a column's scale/bias pairs of consecutive pairs (1, or N when packed)
  const uint32_t* sbp[2];  // lanes 0-31: scale pairs, lanes 32-63: bias pairs of the lane's column (blocks 0, 1)
};

// Scale and bias pairs (groups 2p, 2p+1) of the lane's two columns.
struct SBPair {
  uint32_t s[2], b[2];
};

// Loads of group g: activations and codes into ring slot g % RING; for even g
// also the scale and bias pairs of groups g, g+1 into scale/bias slot
// (g/2) % SBS (per wave and column block: 32 scale words, then 32 bias
// words). Every load writes LDS directly, so the compiler tracks no register
// results of them and only the explicit waits order them.
template <int RM, int NCB>
__device__ __forceinline__ void issue_codes(const Stream& st, uint8_t* ring, int g, int wave) {
  using R = Ring<RM, NCB>;
  uint8_t* cs = ring + R::C_BASE + (g % R::C_RING) * R::C_SLOT;
  buffer_to_lds16(st.rb0, cs + (wave * NCB) * 1024, st.vb, g * st.gstride);
  if constexpr (NCB == 2) buffer_to_lds16(st.rb1, cs + (wave * 2 + 1) * 1024, st.vb, g * st.gstride);
}

// Activation loads of group g (ALOADS per wave).
template <int RM, int NCB>
__device__ __forceinline__ void issue_act(const Stream& st, uint8_t* ring, int g, int wave) {
  using R = Ring<RM, NCB>;
  uint8_t* slot = ring + (g % R::A_RING) * R::A_SLOT;
#pragma unroll
  for (int i = 0; i < R::ALOADS; ++i)
    buffer_to_lds16(st.ra, slot + (wave * R::ALOADS + i) * 1024, st.va[i], g * (kGroup * 2));
}

// Scale/bias words of pair p (NCB loads per wave).
template <int RM, int NCB>
__device__ __forceinline__ void issue_sb(const Stream& st, uint8_t* ring, int p, int wave) {
  using R = Ring<RM, NCB>;
  uint8_t* sbs = ring + R::SB + (p % R::SBS) * R::SB_SLOT + wave * (NCB * kSbWaveBytes);
  global_to_lds4(st.sbp[0] + p * st.sbstride, sbs);
  if constexpr (NCB == 2) global_to_lds4(st.sbp[1] + p * st.sbstride, sbs + kSbWaveBytes);
}

// Loads of one step's lookahead, in this order (which the waits count on):
//   full and merged rings (g = step + 1): activations and codes of g; for
//     even g the scale/bias words of pair g/2 (issue_group);
//   small ring (step j): activations of j + DA; at even j the codes of
//     j + DC, the scale/bias words of pair (j + DC)/2 and the codes of
//     j + DC + 1 (issue_codepair): both groups of a pair back to back.
template <int ODD, int RM, int NCB>
__device__ __forceinline__ void issue_group(const Stream& st, uint8_t* ring, int g, int wave) {
  issue_act<RM, NCB>(st, ring, g, wave);
  issue_codes<RM, NCB>(st, ring, g, wave);
  if (!ODD) issue_sb<RM, NCB>(st, ring, g >> 1, wave);
}
template <int RM, int NCB>
__device__ __forceinline__ void issue_codepair(const Stream& st, uint8_t* ring, int g, int wave) {
  issue_codes<RM, NCB>(st, ring, g, wave);
  issue_sb<RM, NCB>(st, ring, g >> 1, wave);
  issue_codes<RM, NCB>(st, ring, g + 1, wave);   // g + 1 < G: G is even
}

// Side-table entries of group pair p (groups 2p, 2p+1; every wave loads 32
// rows) into the side-table slot, issued at step 2p once every wave is past
// step 2p-1, the last reader of pair p-1.
template <int RM, int NCB>
__device__ __forceinline__ void issue_xp(const Stream& st, uint8_t* ring, int p, int wave) {
  using R = Ring<RM, NCB>;
  buffer_to_lds16(st.rxp, ring + R::XP + (R::SR ? 0 : wave * 1024), st.vxp, p * 32);
  if constexpr (R::XLOADS > 1) buffer_to_lds16(st.rxp, ring + R::XP + kXpSlotBytes, st.vxp2, p * 32);
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(kWaitVm0 | (N & 15) | ((N >> 4) << 14));
}

// The same with the count known only at run time (uniform): exact up to 30;
// a larger count waits until 31 are left, which waits for more loads than
// needed, never for fewer.
__device__ __forceinline__ void wait_vm_dyn(int n) {
  switch (n < 0 ? 0 : n) {
#define MOE_WAIT_CASE(N) \
  case N:                \
    wait_vm<N>();        \
    break;
    MOE_WAIT_CASE(0) MOE_WAIT_CASE(1) MOE_WAIT_CASE(2) MOE_WAIT_CASE(3) MOE_WAIT_CASE(4) MOE_WAIT_CASE(5)
    MOE_WAIT_CASE(6) MOE_WAIT_CASE(7) MOE_WAIT_CASE(8) MOE_WAIT_CASE(9) MOE_WAIT_CASE(10) MOE_WAIT_CASE(11)
    MOE_WAIT_CASE(12) MOE_WAIT_CASE(13) MOE_WAIT_CASE(14) MOE_WAIT_CASE(15) MOE_WAIT_CASE(16) MOE_WAIT_CASE(17)
    MOE_WAIT_CASE(18) MOE_WAIT_CASE(19) MOE_WAIT_CASE(20) MOE_WAIT_CASE(21) MOE_WAIT_CASE(22) MOE_WAIT_CASE(23)
    MOE_WAIT_CASE(24) MOE_WAIT_CASE(25) MOE_WAIT_CASE(26) MOE_WAIT_CASE(27) MOE_WAIT_CASE(28) MOE_WAIT_CASE(29)
    MOE_WAIT_CASE(30)
#undef MOE_WAIT_CASE
    default: wait_vm<31>(); break;
  }
}

__device__ __forceinline__ void scale_acc(f32x16& acc, float r) {
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] *= r;
}

// Step g of the K loop (P4 = g % 4, a compile-time constant: group parity and
// pair parity). Group g is in activation slot g % A_RING and code slot
// g % C_RING; the step's lookahead loads go into slots whose groups every wave
// has finished (the barrier after the top wait orders them).
//
// One accumulator per (row block, column block), kept in units of U = 16 s of
// the lane's column for the latest group with a nonzero scale: acc holds
// (result so far) / U. At group g the unit becomes U' = 16 s_g, acc is
// multiplied by U / U', and the group's chains add P_g straight into it. A
// group whose scale is 0 keeps the unit and zeroes its column's operand. The
// chains are issued level by level (level l = the l-th 16-wide slice of the
// group), so consecutive MFMAs never depend on each other. For odd g one more
// MFMA per block adds the bias terms of groups g-1 and g (lanes 0..31: group
// g-1, 32..63: group g) in the current unit: c = (b - 16 s) / U, split into
// bf16 parts (h, m, l), against the rows' side-table entries
// (Xh, Xm, Xl, Xh, Xm, Xh, 0, 0) as (h, h, h, m, m, l, 0, 0), i.e. X c up to
// terms of 2^-24 relative.
// Wait at the top of step g until this wave's loads that step g reads have
// landed (activations and codes of group g; at even g the scale/bias words of
// pair g/2). Loads complete in issue order for the count, so at most the loads
// issued after the last needed one may still be outstanding:
//   full and merged rings (one group ahead): none (at step g-1 the side table
//     was issued before group g);
//   small ring: step j issues the side table of pair j/2 (even j >= 0), the
//     activations of j + DA and, at even j, the code pair of j + DC (3 NCB
//     loads); the steps before the loop are j = -DC .. -1 without side
//     tables. With DA < DC the last needed load is the activations of g
//     (step g - DA); with DA == DC it is the pair's scale/bias words at even g
//     (the codes of g + 1 follow them) and the activations at odd g.
template <int RM, int NCB>
__device__ __forceinline__ int sr_step_loads(int j, int G) {
  using R = Ring<RM, NCB>;
  const bool even = (j & 1) == 0;
  return (even && j >= 0 ? 1 : 0) + (j + R::DA >= 0 && j + R::DA < G ? 1 : 0) +
         (even && j + R::DC < G ? 3 * NCB : 0);
}

template <int RM, int NCB>
__device__ __forceinline__ int sr_top_count(int g, int G) {
  using R = Ring<RM, NCB>;
  int n = 0;
#pragma unroll
  for (int d = R::DA - 1; d >= 1; --d) n += sr_step_loads<RM, NCB>(g - d, G);
  if constexpr (R::DA < R::DC) {
    if (((g - R::DA) & 1) == 0 && g - R::DA + R::DC < G) n += 3 * NCB;   // the code pair after them
  } else {
    if ((g & 1) == 0) n += NCB;
  }
  return n;
}

template <int ODD, int RM, int NCB>
__device__ __forceinline__ void wait_group(int g, int G) {
  if constexpr (!Ring<RM, NCB>::SR)
    wait_vm<0>();
  else
    wait_vm_dyn(sr_top_count<RM, NCB>(g, G));
}

template <int NRB, int P4, int RM, int NCB>
__device__ __forceinline__ void loop_step(const Stream& st, uint8_t* ring, int g, int G, int wave, int lane,
                                          SBPair& sb, float (&U)[2], f32x16 (&acc)[5][2]) {
  using R = Ring<RM, NCB>;
  constexpr bool SR = R::SR;
  constexpr int ODD = P4 & 1;
  const int l32 = lane & 31, half = lane >> 5;
  // this wave's loads of group g have landed; the barrier makes it so for
  // every wave, and orders every wave's reads of the slot of group g-1
  // (previous step) before its refill
  wait_group<ODD, RM, NCB>(g, G);
  __builtin_amdgcn_s_barrier();
  if (!ODD) issue_xp<RM, NCB>(st, ring, g >> 1, wave);
  if constexpr (SR) {
    if (g + R::DA < G) issue_act<RM, NCB>(st, ring, g + R::DA, wave);
    if (!ODD && g + R::DC < G) issue_codepair<RM, NCB>(st, ring, g + R::DC, wave);
  } else if (g + R::DC < G) {
    issue_group<(ODD + R::DC) & 1, RM, NCB>(st, ring, g + R::DC, wave);
  }
  const uint8_t* slot = ring + (g % R::A_RING) * R::A_SLOT;
  const uint8_t* cslot = ring + R::C_BASE + (g % R::C_RING) * R::C_SLOT;
  if (!ODD) {
    // this pair's scale and bias words of the lane's column
    const uint8_t* sbs = ring + R::SB + ((g >> 1) % R::SBS) * R::SB_SLOT + wave * (NCB * kSbWaveBytes);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      sb.s[cb] = *reinterpret_cast<const uint32_t*>(sbs + cb * kSbWaveBytes + l32 * 4);
      sb.b[cb] = *reinterpret_cast<const uint32_t*>(sbs + cb * kSbWaveBytes + 128 + l32 * 4);
    }
  }

  u32x4 w[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) w[cb] = *reinterpret_cast<const u32x4*>(cslot + (wave * NCB + cb) * 1024 + lane * 16);
  bf16x8 fa[2][NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
    fa[0][rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(slot + a_chunk_off(rb * 32 + l32, 4 * half)));
  // each column block's unit and the factor that moves acc into it
  float r[NCB];
  uint32_t nib[NCB], magic[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const float sf = 16.0f * __uint_as_float(ODD ? (sb.s[cb] & 0xFFFF0000u) : (sb.s[cb] << 16));
    const bool nz = __builtin_fabsf(sf) >= kMinUnit;
    const float Un = nz ? sf : U[cb];
    r[cb] = U[cb] * __builtin_amdgcn_rcpf(Un);
    U[cb] = Un;
    nib[cb] = nz ? kNib : 0u;
    magic[cb] = nz ? kMagic : 0u;
  }
#pragma unroll
  for (int l = 0; l < 4; ++l) {
    if (l + 1 < 4) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        fa[(l + 1) & 1][rb] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(slot + a_chunk_off(rb * 32 + l32, 4 * half + l + 1)));
    }
    bf16x8 bq[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) bq[cb] = unpack_word(w[cb][l], nib[cb], magic[cb]);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      if (l == 0) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) scale_acc(acc[rb][cb], r[cb]);
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[l & 1][rb], bq[cb], acc[rb][cb], 0, 0, 0);
    }
  }
  if (ODD) {
    // the side table of this pair was issued first at step g-1: every wave
    // waits for its part. One group ahead, the next load was group g's, which
    // this step's top wait and barrier already covered; the small ring has
    // later loads outstanding.
    if constexpr (SR) {
      // issued after the side table: the rest of step g-1's loads and step
      // g's
      wait_vm_dyn(sr_step_loads<RM, NCB>(g - 1, G) - 1 + sr_step_loads<RM, NCB>(g, G));
      __builtin_amdgcn_s_barrier();
    }
    const int sh = half << 4;
    bf16x8 bv[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const float sg = __uint_as_float(((sb.s[cb] >> sh) & 0xFFFFu) << 16);
      const float bg = __uint_as_float(((sb.b[cb] >> sh) & 0xFFFFu) << 16);
      const float c = (bg - 16.0f * sg) * __builtin_amdgcn_rcpf(U[cb]);
      uint16_t ch, cm, cl;
      split3_bf16(c, ch, cm, cl);
      const u32x4 pk = {uint32_t(ch) | (uint32_t(ch) << 16), uint32_t(ch) | (uint32_t(cm) << 16),
                        uint32_t(cm) | (uint32_t(cl) << 16), 0u};
      bv[cb] = __builtin_bit_cast(bf16x8, pk);
    }
    const uint8_t* xps = ring + R::XP;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const bf16x8 xa =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xps + (rb * 32 + l32) * 32 + half * 16));
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, bv[cb], acc[rb][cb], 0, 0, 0);
    }
  }
}

// G is even (K is a multiple of 128). RM: the ring geometry (small tiles:
// NRB == 1; merged tiles: NRB == 5).
template <int NRB, int RM, int NCB = 2>
__device__ __forceinline__ void main_loop(const Stream& st, uint8_t* ring, int G, int wave, int lane,
                                          SBPair& sb, f32x16 (&acc)[5][2]) {
  using R = Ring<RM, NCB>;
  if constexpr (R::SR) {
    // steps j = -DC .. -1 issue what step j of the loop would, without side
    // tables
#pragma unroll
    for (int j = -R::DC; j < 0; ++j) {
      if (j + R::DA >= 0 && j + R::DA < G) issue_act<RM, NCB>(st, ring, j + R::DA, wave);
      if ((j & 1) == 0 && j + R::DC < G) issue_codepair<RM, NCB>(st, ring, j + R::DC, wave);
    }
  } else {
    issue_group<0, RM, NCB>(st, ring, 0, wave);   // group 0 before the first step
  }
  float U[2] = {1.0f, 1.0f};   // any normal value: acc is zero until the first nonzero scale
  // unrolled by 4 so the group parity and the pair parity are constants
  for (int g = 0; g < G; g += 4) {
    loop_step<NRB, 0, RM, NCB>(st, ring, g, G, wave, lane, sb, U, acc);
    loop_step<NRB, 1, RM, NCB>(st, ring, g + 1, G, wave, lane, sb, U, acc);
    if (g + 2 < G) {
      loop_step<NRB, 2, RM, NCB>(st, ring, g + 2, G, wave, lane, sb, U, acc);
      loop_step<NRB, 3, RM, NCB>(st, ring, g + 3, G, wave, lane, sb, U, acc);
    }
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) scale_acc(acc[rb][cb], U[cb]);
  }
}

// Epilogue of a one-column-block workgroup (tile of at most 32 rows; acc is
// the wave's 32 x 32 block). F32: each wave stages its block in LDS (row
// stride 36 floats) and writes 128-byte row segments with non-temporal stores.
// SwiGLU: the gate waves (0, 1) leave their fp32 values in LDS, the up waves
// (2, 3) form h = silu(gate) * up in bf16, and one wave writes the 32 x 64 h
// block (and, internal layout, the group-sum entry of its one 64-wide group).
template <int EPI>
__device__ __forceinline__ void epilogue_ncb1(const GemmArgs& a, const TileInfo& ti, int nt, int nrows, bool live,
                                              int cbase, int wave, int lane, const f32x16& acc, uint8_t* ring) {
  const int l32 = lane & 31, half = lane >> 5;
  if constexpr (EPI == kEpiF32) {
    float* out = reinterpret_cast<float*>(a.out);
    float* stg = reinterpret_cast<float*>(ring) + wave * (32 * kF32StageStride);
#pragma unroll
    for (int r = 0; r < 16; ++r) stg[(8 * (r >> 2) + 4 * half + (r & 3)) * kF32StageStride + l32] = acc[r];
    __builtin_amdgcn_wave_barrier();
    if (live) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = i * 8 + (lane >> 3), c4 = (lane & 7) * 4;
        const f32x4 v = *reinterpret_cast<const f32x4*>(stg + m * kF32StageStride + c4);
        if (m < nrows) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(out + size_t(ti.r0 + m) * a.N + cbase + c4));
      }
    }
  } else {
    constexpr int kGs = 65;                                     // gate row stride (floats)
    float* gs = reinterpret_cast<float*>(ring);                 // [32][65] gate values
    uint16_t* hs = reinterpret_cast<uint16_t*>(ring + 32 * kGs * 4);   // [32][64] h
    const int col = (wave & 1) * 32 + l32;
    if (wave < 2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) gs[(8 * (r >> 2) + 4 * half + (r & 3)) * kGs + col] = acc[r];
    }
    __syncthreads();
    if (wave >= 2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 8 * (r >> 2) + 4 * half + (r & 3);
        const float gv = gs[m * kGs + col];
        const float hv = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * acc[r];
        hs[m * 64 + col] = uint16_t(f32_to_bf16_rne(hv));
      }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // unit u: row u/2, half u%2 = 32 columns; the two halves of a row are
      // the 64-wide group of h this workgroup produced (adjacent lanes)
      const int u = threadIdx.x;
      const int srow = u >> 1, sq = u & 1;
      const int row = ti.r0 + srow;
      uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
      u32x4 ch[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ch[i] = *reinterpret_cast<const u32x4*>(hs + srow * 64 + sq * 32 + 8 * i);
      if constexpr (EPI == kEpiSwigluInternal) {
        double part = 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i) part += chunk_sum_f64(ch[i]);
        const float X = float(part + __shfl_xor(part, 1, kWave));
        if (srow < nrows) {
          uint16_t* dst = out + size_t(row) * a.N + nt * 64 + sq * 32;
#pragma unroll
          for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(dst + 8 * i) = permute_chunk(ch[i]);
          if (sq == 0) {
            uint16_t h, m, l;
            split3_bf16(X, h, m, l);
            const u32x4 e = {uint32_t(h) | (uint32_t(m) << 16), uint32_t(l) | (uint32_t(h) << 16),
                             uint32_t(m) | (uint32_t(h) << 16), 0u};
            *reinterpret_cast<u32x4*>(a.out_part + size_t(row) * xpart_cols(a.N) + 8 * nt) = e;
          }
        }
      } else {
        if (srow < nrows && nt * 64 + sq * 32 < a.N) {
          uint16_t* dst = out + size_t(row) * a.N + nt * 64 + sq * 32;
#pragma unroll
          for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(dst + 8 * i) = ch[i];
        }
      }
    }
  }
}

// NCB = 2: every tile geometry, two workgroups per CU. NCB = 1: launches whose
// tiles all hold at most 32 rows (the host guarantees it), five per CU.
template <int EPI, int NCB>
__global__ __launch_bounds__(kGemmThreads, NCB == 1 ? 5 : 2) void gemm_q4_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int K = a.K;
  const int G = K / kGroup;
  const int KPx = xpart_cols(K);
  uint8_t* ring = smem;

  // XCD-aware work mapping: workgroups are dispatched round-robin over the 8
  // XCDs (blockIdx % 8). The tile list (shared tiles, then routed tiles in
  // expert order) is cut into 8 contiguous chunks, chunk x runs on XCD x, and
  // within a chunk the column slices of a tile are consecutive. So every
  // column slice of a row tile reads the activation rows from the same L2, and
  // consecutive tiles of one expert share its weights in that L2.
  const int ntot = a.n_shared_tiles + (a.routed_tiles ? *a.num_tiles : 0);
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

  // ---- this wave's 32-column blocks (two, or one with NCB = 1) -----------------
  // A block past the last column (N not a multiple of the workgroup's width)
  // streams the last 32 columns again and stores nothing.
  int cbase[2];
  const QStack* mat[2];
  if constexpr (NCB == 1) {
    // F32: wave w = columns 32w..32w+31 of the workgroup's 128; SwiGLU: waves
    // 0, 1 = gate columns 32w.. of the workgroup's 64 h columns, waves 2, 3 =
    // the same up columns (gate and up meet in LDS after the loop)
    if constexpr (EPI == kEpiF32) {
      cbase[0] = nt * 128 + wave * 32;
      mat[0] = &a.w0[stack];
    } else {
      cbase[0] = nt * 64 + (wave & 1) * 32;
      mat[0] = wave < 2 ? &a.w0[stack] : &a.w1[stack];
    }
    cbase[1] = cbase[0];
    mat[1] = mat[0];
  } else if constexpr (EPI == kEpiF32) {
    cbase[0] = nt * 256 + wave * 64;
    cbase[1] = cbase[0] + 32;
    mat[0] = mat[1] = &a.w0[stack];
  } else {
    cbase[0] = cbase[1] = nt * 128 + wave * 32;
    mat[0] = &a.w0[stack];
    mat[1] = &a.w1[stack];
  }
  bool live[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    live[cb] = cbase[cb] < a.N;
    cbase[cb] = live[cb] ? cbase[cb] : a.N - 32;
  }

  // ---- streaming descriptors and per-lane offsets -------------------------
  Stream st;
  st.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.A), 0, 0x7FFFFFFF, kRsrcWord3);
  st.rxp = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.Apart), 0, 0x7FFFFFFF, kRsrcWord3);
  // both matrices of a stack slot share its layout (checked on the host)
  const bool packed = mat[0]->packed != 0;
  {
    // descriptors based at the wave's first column of each block; the lane
    // (column l32, half) reads words 4*half..4*half+3 of the group's 8
    const uint32_t* q0 = packed ? mat[0]->q + (size_t(el) * G * a.N + cbase[0]) * 8
                                : mat[0]->q + (size_t(el) * a.N + cbase[0]) * size_t(K / 8);
    const uint32_t* q1 = packed ? mat[1]->q + (size_t(el) * G * a.N + cbase[1]) * 8
                                : mat[1]->q + (size_t(el) * a.N + cbase[1]) * size_t(K / 8);
    st.rb0 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(q0), 0, 0x7FFFFFFF, kRsrcWord3);
    st.rb1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(q1), 0, 0x7FFFFFFF, kRsrcWord3);
    st.vb = packed ? uint32_t((l32 * 8 + 4 * half) * 4) : uint32_t((l32 * (K / 8) + 4 * half) * 4);
    st.gstride = packed ? a.N * 32 : 32;
    st.sbstride = packed ? a.N : 1;
  }
  {
    // activation load i of wave w fills chunk positions (A w + i)*64 + lane,
    // A = activation loads per wave (4, or 1 in the small-tile ring): row
    // m = (A w + i)*8 + lane/8 and chunk slot lane%8, which holds logical
    // chunk (lane%8) ^ swz(m). Rows past the tile's last (the padding of its
    // last 32-row block) get an offset past the descriptor's range: the
    // buffer load makes no memory access for them, and their results are
    // never stored (with the side table's padding rows below, the T=512
    // layer ran ~3% faster than re-reading the last row)
    const int aloads = nrb == 1 ? Ring<kRingSmall>::ALOADS : nrb == 5 ? Ring<kRingMerged>::ALOADS
                                                                       : Ring<kRingFull>::ALOADS;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int m = (wave * aloads + i) * 8 + (lane >> 3);
      const int cidx = (lane & 7) ^ swz(m);
      const int r = ti.r0 + min(m, nrows - 1);
      st.va[i] = m < nrows ? uint32_t(src_row(a, r)) * uint32_t(K * 2) + uint32_t(cidx * 16) : kPastRange;
    }
    // side-table load of wave w: row w*32 + lane/2, 16-byte half lane%2;
    // padding rows, as above, past the range
    const int mx = (nrb == 1 ? 0 : wave * 32) + (lane >> 1);   // small tiles: rows 0..31 in every wave
    const int mx2 = kBlockRows + (lane >> 1);                  // merged tiles' second load
    st.vxp = mx < nrows ? uint32_t(src_row(a, ti.r0 + mx)) * uint32_t(KPx * 2) + uint32_t((lane & 1) * 16)
                        : kPastRange;
    st.vxp2 = mx2 < nrows ? uint32_t(src_row(a, ti.r0 + mx2)) * uint32_t(KPx * 2) + uint32_t((lane & 1) * 16)
                          : kPastRange;
  }
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    // the lane's column's G scales (lanes 32-63: biases) as G/2 pairs of groups
    const uint16_t* sb = half ? mat[cb]->b : mat[cb]->s;
    const int col = cbase[cb] + l32;
    st.sbp[cb] = packed ? reinterpret_cast<const uint32_t*>(sb) + size_t(el) * (G / 2) * a.N + col
                        : reinterpret_cast<const uint32_t*>(sb + (size_t(el) * a.N + col) * size_t(G));
  }

  SBPair sb;

  f32x16 acc[5][2];
#pragma unroll
  for (int rb = 0; rb < 5; ++rb) acc[rb][0] = acc[rb][1] = f32x16{};
  if constexpr (NCB == 1) {
    main_loop<1, kRingSmall, 1>(st, ring, G, wave, lane, sb, acc);   // every tile: at most 32 rows
  } else {
    switch (nrb) {
      case 1: main_loop<1, kRingSmall>(st, ring, G, wave, lane, sb, acc); break;
      case 2: main_loop<2, kRingFull>(st, ring, G, wave, lane, sb, acc); break;
      case 3: main_loop<3, kRingFull>(st, ring, G, wave, lane, sb, acc); break;
      case 4: main_loop<4, kRingFull>(st, ring, G, wave, lane, sb, acc); break;
      default: main_loop<5, kRingMerged>(st, ring, G, wave, lane, sb, acc); break;   // merged tiles only
    }
  }
  __syncthreads();   // every wave is done with the rings
  if constexpr (NCB == 1) {
    epilogue_ncb1<EPI>(a, ti, nt, nrows, live[0], cbase[0], wave, lane, acc[0][0], ring);
    return;
  }

  // ---- epilogues ------------------------------------------------------------
  if constexpr (EPI == kEpiF32) {
    // each wave stages one 128 x 32 column block at a time in its own LDS area
    // (row stride 36 floats) and writes whole 128-byte row segments, with
    // non-temporal stores (the rows are read once, by the combine; 1.5-2%
    // faster T=4096 layer with the combine's non-temporal loads)
    float* out = reinterpret_cast<float*>(a.out);
    float* stg = reinterpret_cast<float*>(ring) + wave * (kBlockRows * kF32StageStride);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = rb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          stg[m * kF32StageStride + l32] = acc[rb][cb][r];
        }
      __builtin_amdgcn_wave_barrier();
      if (live[cb]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = i * 8 + (lane >> 3), c4 = (lane & 7) * 4;
          const f32x4 v = *reinterpret_cast<const f32x4*>(stg + m * kF32StageStride + c4);
          if (m < nrows) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(out + size_t(ti.r0 + m) * a.N + cbase[cb] + c4));
        }
      }
      __builtin_amdgcn_wave_barrier();
      if (nrows > kBlockRows) {   // uniform: a merged tile's rows 128..159
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 8 * (r >> 2) + 4 * half + (r & 3);
          stg[m * kF32StageStride + l32] = acc[4][cb][r];
        }
        __builtin_amdgcn_wave_barrier();
        if (live[cb]) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = i * 8 + (lane >> 3), c4 = (lane & 7) * 4;
            const f32x4 v = *reinterpret_cast<const f32x4*>(stg + m * kF32StageStride + c4);
            if (kBlockRows + m < nrows)
              __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(out + size_t(ti.r0 + kBlockRows + m) * a.N + cbase[cb] + c4));
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
  } else {
    uint16_t* hs = reinterpret_cast<uint16_t*>(ring);   // [160][128] bf16
    const int col = wave * 32 + l32;
#pragma unroll
    for (int rb = 0; rb < 5; ++rb) {
      if (rb == 4 && nrows <= kBlockRows) break;   // uniform
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = rb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const float gv = acc[rb][0][r];
        const float hv = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * acc[rb][1][r];
        hs[m * 128 + col] = uint16_t(f32_to_bf16_rne(hv));
      }
    }
    __syncthreads();
    // unit u: row u/4, quarter u%4 = 32 columns; quarters (0,1) and (2,3) are
    // the two 64-wide groups of h this workgroup produced (units u and u^1 are
    // in adjacent lanes)
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      if (it == 2 && nrows <= kBlockRows) break;   // uniform: rows 128..159 of a merged tile
      const int u = tid + it * kGemmThreads;
      const int srow = u >> 2, sq = u & 3;
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
                             uint32_t(m) | (uint32_t(h) << 16), 0u};
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
}

hipError_t launch_gemm(const GemmArgs& ga, int epilogue, int max_row_tiles, hipStream_t stream, bool one_block) {
  // 8 chunks of at most ceil(max_row_tiles / 8) tiles, NT column slices each
  const dim3 grid(8u * unsigned(ceil_div(max_row_tiles, 8)) * unsigned(ga.NT));
  if (grid.x == 0) return hipSuccess;
  const size_t lds = gemm_lds_bytes(ga.K, one_block ? 1 : 2);
#define MOE_GEMM_LAUNCH(E)                                                                        \
  do {                                                                                            \
    if (one_block)                                                                                \
      hipLaunchKernelGGL((gemm_q4_kernel<E, 1>), grid, dim3(kGemmThreads), lds, stream, ga);      \
    else                                                                                          \
      hipLaunchKernelGGL((gemm_q4_kernel<E, 2>), grid, dim3(kGemmThreads), lds, stream, ga);      \
  } while (0)
  switch (epilogue) {
    case kEpiF32: MOE_GEMM_LAUNCH(kEpiF32); break;
    case kEpiSwigluNatural: MOE_GEMM_LAUNCH(kEpiSwigluNatural); break;
    default: MOE_GEMM_LAUNCH(kEpiSwigluInternal); break;
  }
#undef MOE_GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
