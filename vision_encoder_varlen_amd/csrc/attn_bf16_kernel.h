// Varlen (block-diagonal) attention, bf16 in/out, for gfx950: the kernel
// template, its configurations and its launch helper.  attn_bf16.hip
// instantiates the plain kernels, attn_bf16_fused.hip those that do part of
// the pre-pass themselves (two files, so they compile in parallel).
//
// Computes, for every work item (segment, q-tile) and head, the rows of
// softmax(Q K^T * scale) V restricted to the segment (vLLM page
// vllm.models.dots3_note.nvidia.vision_attention, VisionAttentionV2.forward;
// tokenspeed page mm_encoder_attention.py, vision_attn_fa3 with
// cu_seqlens_q = cu_seqlens_k).  The S x S mask of VisionAttention.forward is
// never formed: each workgroup only visits its own segment's keys.  The
// CAUSAL instantiation (is_causal of _VisionAttentionBase on the vLLM page)
// also drops keys after each query row, and a work item stops at the key tile
// holding its last row.
//
// Design (one workgroup = WAVES waves; each wave owns 32*QB query rows of
// one head; two waves share each SIMD so one's softmax overlaps the other's
// MFMA -- two 4-wave workgroups per CU, or one 8-wave workgroup, whose waves
// then share one K/V ring: half the global -> LDS copies per CU):
//  * Q fragments stay in VGPRs for the whole key loop.
//  * K and V tiles of BN keys are copied global -> LDS by the buffer unit
//    itself (buffer_load_dwordx4 ... lds) into a ring of STAGES buffers, issued
//    STAGES-1 tiles ahead.  No VGPRs hold tiles in flight and no VALU stores
//    them; each wave waits only on its own copies (vmcnt) and one barrier per
//    tile publishes the tile to all waves.  The buffer resource is bounded by
//    the segment, so keys past its end arrive as zeros.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the query index runs along the lanes, so the row
//    max and row sum of the online softmax are in-lane reductions plus one
//    exchange between the two 32-lane halves.
//  * K rows are placed in LDS with bits 2 and 3 of the key index swapped (the
//    copy picks which key each LDS row receives).  With that order the 32x32
//    accumulator layout hands each lane eight consecutive keys per 16-key step,
//    which is the B operand layout of the P V^T product, so P goes from the
//    score registers to the next MFMA without any cross-lane shuffle.
//  * V stays row-major in LDS; the A operand of O^T = V^T P^T (eight
//    consecutive keys of one head-dim column per lane) comes from two
//    ds_read_b64_tr_b16 transpose reads.
//  * LDS row strides, in 16-byte units (the LDS has 64 four-byte banks, 256
//    bytes per clock): K rows use an odd count (the sixteen rows a
//    ds_read_b128 serves together, read at the same column, hit distinct
//    banks); V rows use 4 mod 8 (a ds_read_b64_tr_b16 serves 32 lanes
//    together, four rows x 64 bytes, which then hit distinct banks).
//  * Softmax in base 2: p = 2^(s*c - m_ref) with c = scale*log2(e), one FMA
//    and one v_exp_f32 per score.  The reference max m_ref of a query row is
//    fixed for a whole pass over the keys (taken from the first key tile), so
//    O is never rescaled, the key loop touches the accumulators only through
//    MFMAs, and after the first tile no row max is computed at all.  If a
//    row's sum of p ends above 2^64 (some key scored far above the first
//    tile), the workgroup runs a max-only pass and repeats the unit with the
//    exact row max, where every p <= 1.  Below the limit no p or partial sum
//    can overflow fp32.
//  * QB > 1 gives a wave several 32-row query blocks, so each K and V
//    fragment read from LDS feeds QB MFMAs.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "vit_kernels.h"

namespace vit {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) const u16 lds_u16_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRestartLimit = 0x1p64f;  // a row sum above this triggers the exact-max repeat
// Tile modes of the key loop.
constexpr int kSetRef = 0, kPlain = 1, kMaxOnly = 2;
constexpr int kRsrcWord3 = 0x00020000;    // gfx9-family buffer descriptor word 3 (raw, 32-bit)
// Rotary coordinates below this come from a per-workgroup table of cos and
// sin (fused q/k kernels); larger ones are evaluated directly.
constexpr int kRopeCoords = 64;
// Output rows staged through LDS before the global stores (see the kernel's
// finalize step).
constexpr bool kStageOut = true;
// Byte offset for copy lanes that fill padding: past any segment's num_records
// (segments are limited to kMaxSegmentBytes) even after adding the tile offset.
constexpr unsigned kPadOffset = 0x40000000u;
static_assert(kMaxSegmentBytes <= (int64_t)kPadOffset, "pad offset must exceed every segment");
static_assert((int64_t)kPadOffset + kMaxSegmentBytes < (int64_t(1) << 32), "offsets must not wrap");

constexpr int odd_units(int u) { return (u & 1) ? u : u + 1; }
constexpr int units_4_mod_8(int u) { return u % 8 == 4 ? u : units_4_mod_8(u + 1); }

template <int D_, int WAVES_, int QB_, int BN_, int STAGES_, int OCC_, int PRE_ = 0>
struct Cfg {
  static constexpr int D = D_;
  static constexpr int WAVES = WAVES_;
  static constexpr int QB = QB_;                        // 32-row query blocks per wave
  static constexpr int BN = BN_;                        // keys per tile
  static constexpr int STAGES = STAGES_;                // LDS ring depth
  static constexpr int OCC = OCC_;                      // waves per SIMD the kernel is built for
  // PRE: which part of the pre-pass the kernel does itself.  0: none (or
  // q's, evaluated directly; the plain kernels).  1 (QT): q's, with the
  // rotary taken from a per-workgroup table and the first tiles issued before
  // the transform.  2 (KF, also QT): q's and k's; each K tile is normalised
  // and rotated in LDS before its fragments are read, and the tile's key
  // positions (8 bytes per key) ride along with its copies (dword copies, so
  // a segment's last key never shares a load with bytes past its end) into a
  // region of their own.
  static constexpr int PRE = PRE_;
  static constexpr bool QT = PRE_ >= 1;
  static constexpr bool KF = PRE_ == 2;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int WG_PER_CU = 4 * OCC / WAVES;     // resident workgroups per CU (4 SIMDs)
  static constexpr int BM = 32 * QB * WAVES;            // query rows per workgroup
  static constexpr int KB = BN / 32;                    // 32-key blocks per tile
  static constexpr int KSTEPS = D / 16;                 // 16-wide contraction steps of Q K^T
  static constexpr int DB = (D + 31) / 32;              // 32-row blocks of O^T
  static constexpr int DU = D / 8;                      // 16-byte units per row of data
  static constexpr int KSTR = odd_units(DU);            // K row stride (units)
  static constexpr int VSTR = units_4_mod_8(DU);        // V row stride (units)
  static constexpr int NK = (BN * KSTR + 63) / 64;      // copy instructions for K
  static constexpr int NV = (BN * VSTR + 63) / 64;      // copy instructions for V
  static constexpr int NP = KF ? BN / 32 : 0;           // dword copies of the keys' positions
  static constexpr int NT = NK + NV + NP;               // copy instructions per tile
  // Instruction i goes to wave i % WAVES: the first NT % WAVES waves issue
  // NI_HI copies per tile, the others NI_LO.
  static constexpr int NI_LO = NT / WAVES;
  static constexpr int NI_HI = (NT + WAVES - 1) / WAVES;
  static constexpr int KREG = NK * 64;                  // K region (units), instruction aligned
  // V region plus slack: the last copy instruction may run past the V rows,
  // and the transpose reads of head-dim columns D..32*DB-1 read at most one
  // row further.
  static constexpr int VREG = NV * 64 + VSTR;
  static constexpr int PREG = KF ? BN / 2 : 0;          // positions region (units), after V's
  static constexpr int STAGE_UNITS = KREG + VREG + PREG;
  static constexpr int LDS_BYTES = STAGES * STAGE_UNITS * 16;
  static_assert(D % 16 == 0, "head dim must be a multiple of 16");
  static_assert(BN % 32 == 0, "key tile must be a multiple of 32");
  static_assert(BN <= kMaxKeyTile, "key tile exceeds the padding the segment limit allows for");
  static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");
  static_assert(NI_HI * (STAGES - 2) <= 63, "vmcnt range");
  static_assert((4 * OCC) % WAVES == 0 && WG_PER_CU >= 1, "whole workgroups per CU");
  static_assert(LDS_BYTES * WG_PER_CU <= 160 * 1024, "LDS budget");
  template <int P>
  using WithPre = Cfg<D_, WAVES_, QB_, BN_, STAGES_, OCC_, P>;
};

// The value lane l ^ 32 holds (v_permlane32_swap: a VALU exchange of the two
// 32-lane halves, no LDS round trip).
__device__ __forceinline__ float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(threadIdx.x & 32 ? r[0] : r[1]);
}

__device__ __forceinline__ float bf16_bits_to_f32(u16 b) { return __uint_as_float(unsigned(b) << 16); }
__device__ __forceinline__ u16 f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(u16, (__bf16)x);  // round to nearest even
}

// Sum over aligned groups of N lanes (N = 2, 4 or 8) with DPP moves: lane
// pairs, then quads, then the two quads of each 8-lane half row (mirrored).
// Every lane of a group ends with the same bits (each step adds two values
// that the partner lane adds in the other order).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 2 || N == 4 || N == 8, "group size");
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
  if constexpr (N >= 4)
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
  if constexpr (N >= 8)
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
  return x;
}

__device__ __forceinline__ int swap_bits_2_3(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// vmcnt(n) only (expcnt and lgkmcnt at their no-wait maxima), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most `later` tiles of this wave's copies (NI instructions
// each) are still in flight.
template <int NI, int STAGES>
__device__ __forceinline__ void wait_copies(int later) {
  if constexpr (STAGES >= 4) {
    if (later >= 2) { wait_vmcnt<NI * 2>(); return; }
  }
  if constexpr (STAGES >= 3) {
    if (later >= 1) { wait_vmcnt<NI>(); return; }
  }
  wait_vmcnt<0>();
}

// One 64-lane global -> LDS copy of 16 bytes per lane: lane L writes LDS bytes
// [lds_byte + 16L, lds_byte + 16L + 16).  Issued from asm so the compiler's
// wait-counter pass does not drain it before every LDS read; the kernel waits
// for its own copies explicitly.
__device__ __forceinline__ void copy_to_lds(unsigned lds_byte, unsigned voffset, i32x4_t rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_byte), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}

// The same with 4 bytes per lane (LDS bytes [lds_byte + 4L, lds_byte + 4L + 4)):
// each dword is inside the buffer's range or past it as a whole.
__device__ __forceinline__ void copy_dword_to_lds(unsigned lds_byte, unsigned voffset, i32x4_t rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_byte), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}

__device__ __forceinline__ i32x4_t make_rsrc(const void* base, unsigned num_bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane(int(unsigned(a)));
  r.y = __builtin_amdgcn_readfirstlane(int(unsigned(a >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane(int(num_bytes));
  r.w = kRsrcWord3;
  return r;
}

// p must point into LDS (a __shared__ array); the cast only changes the
// address space the compiler sees.
__device__ __forceinline__ i16x4_t ds_read_tr16(lds_u16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
}

template <class C, bool POS_SCALE, bool CAUSAL>
__global__ __launch_bounds__(C::THREADS, C::OCC) void attn_bf16_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const int32_t* __restrict__ items, const int32_t* __restrict__ meta, long long list_cap,
    int u_batch, int u_seq_len, int H,
    float scale_log2, u16* __restrict__ out, float* __restrict__ lse, TokenStrides ts,
    QPrepass qpre) {
  constexpr int D = C::D, BN = C::BN, KB = C::KB, STAGES = C::STAGES, NI = C::NI_HI, QB = C::QB;
  // When D is not a multiple of 32 the last 32-row block of O^T has padding
  // rows; row D then collects the row sums of P (see the tile loop), and
  // lane kOnesLane (l&31) of that block is the one that reads it.
  constexpr bool kSumByMfma = C::DB * 32 > D;
  constexpr int kOnesLane = D - 32 * (C::DB - 1);
  constexpr bool kSoftmaxPrio = D == 128;
  __shared__ __align__(16) u16 smem[C::LDS_BYTES / 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const unsigned smem_base = static_cast<unsigned>((uintptr_t)(lds_u16_t*)smem);  // LDS address

  // Per-lane byte offsets of this wave's copy instructions relative to the
  // tile's first key.  Instruction i = wave + WAVES*j (K units first, then V
  // units, then with KF one for the keys' positions); lanes that fall on row
  // padding get an offset past num_records and write zeros.  With kSumByMfma
  // the head-dim padding units of the V rows are not copied at all (cp_skip):
  // they hold a constant 1 in dim D, written once below, so row D of V^T is
  // all ones without any per-tile work.
  const bool wave_hi = wave < C::NT % C::WAVES || C::NT % C::WAVES == 0;
  unsigned cp_off[NI];
  bool cp_is_k[NI];
  bool cp_is_p[NI];
  bool cp_skip[NI];
  unsigned cp_lds[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int i = wave + C::WAVES * j;
    const bool is_p = C::KF && i >= C::NK + C::NV;
    const bool is_k = i < C::NK;
    const int u = is_k ? i * 64 + lane : (i - C::NK) * 64 + lane;
    const int str = is_k ? C::KSTR : C::VSTR;
    const int row = u / str;
    const int col = u - row * str;
    const int key = is_k ? swap_bits_2_3(row) : row;
    const bool data = row < BN && col < C::DU;
    cp_off[j] = data ? (unsigned(key) * unsigned(is_k ? ts.k : ts.v) + unsigned(col) * 8u) * 2u
                     : kPadOffset;
    cp_is_k[j] = is_k;
    cp_is_p[j] = is_p;
    cp_skip[j] = kSumByMfma && !is_k && !is_p && row < BN && col >= C::DU;
    cp_lds[j] = unsigned((is_k ? i * 64 : C::KREG + (i - C::NK) * 64) * 16);
    if (is_p) {
      // dword L of copy pi: int32 L & 1 (row, col) of key 32 pi + L / 2
      const int pi = i - C::NK - C::NV;
      cp_off[j] = unsigned(pi * 256 + lane * 4);
      cp_lds[j] = unsigned((C::KREG + C::VREG) * 16 + pi * 256);
    }
  }
  // V row padding of every ring stage: unit DU starts with bf16 1.0 (dim D),
  // the rest are zero.  No copy writes these units (cp_skip), and the first
  // tile's barrier orders these stores before any read.  Written here, and
  // again at the start of every later unit when the previous unit's output
  // was staged through the ring.
  auto write_ones = [&]() __attribute__((always_inline)) {
    if constexpr (kSumByMfma) {
      static_assert(C::VSTR > C::DU && kOnesLane % 8 == 0, "dim D must open a padding unit");
      constexpr int kPadUnits = C::VSTR - C::DU;
      for (int i = tid; i < STAGES * BN * kPadUnits; i += C::THREADS) {
        const int stage = i / (BN * kPadUnits);
        const int r = (i / kPadUnits) % BN;
        const int pu = i % kPadUnits;
        u32x4_t val = u32x4_t{0u, 0u, 0u, 0u};
        if (pu == 0) val.x = 0x3f80u;  // dims D, D+1 = (1.0, 0) in the low dword
        *reinterpret_cast<u32x4_t*>(smem + (stage * C::STAGE_UNITS + C::KREG + r * C::VSTR + C::DU + pu) *
                                               8) = val;
      }
    }
  };
  write_ones();
  bool ring_staged = false;  // the previous unit's output went through the ring

  // Q-side pre-pass (when asked for): each unit's Q fragments are normalised
  // and rotated in registers right after they are loaded.  The tables hold
  // the norm weights and the rotary frequencies (turns per unit coordinate,
  // hi + lo).
  __shared__ float s_qw[D];
  __shared__ float s_kw[C::KF ? D : 1];
  __shared__ float2 s_rev[kMaxQFreqs];
  // Rotary table rows (one per coordinate) are D/4 + 2 entries apart, so
  // rows of different coordinates start 4 banks apart: lanes reading the
  // same frequency of different coordinates do not share banks.
  constexpr int kCsRow = D / 4 + 2;
  __shared__ float2 s_cs[C::QT ? kRopeCoords * kCsRow : 1];
  static_assert((C::LDS_BYTES + (C::KF ? 2 : 1) * D * 4 + kMaxQFreqs * 8 +
                 (C::QT ? kRopeCoords * kCsRow * 8 : 0)) * C::WG_PER_CU <= 160 * 1024,
                "LDS budget with the pre-pass tables");
  const bool q_pending = qpre.pos != nullptr || qpre.weight != nullptr;
  if (q_pending || C::KF) {
    for (int i = tid; i < D; i += C::THREADS) s_qw[i] = qpre.weight != nullptr ? qpre.weight[i] : 1.f;
    if constexpr (C::KF)
      for (int i = tid; i < D; i += C::THREADS)
        s_kw[i] = qpre.k_weight != nullptr ? qpre.k_weight[i] : 1.f;
    if (tid == 0)
      static_for<D / 4>([&](auto f_c) __attribute__((always_inline)) {
        constexpr int f = decltype(f_c)::value;
        s_rev[f] = make_float2(qpre.rev_hi[f], qpre.rev_lo[f]);
      });
    __syncthreads();
  }
  // QT: cos and sin of the angle of every (coordinate < kRopeCoords,
  // frequency) pair, once per workgroup, with the direct path's arithmetic.
  // Each head of a token needs the same angles, and a workgroup runs many
  // (item, head) units.
  if constexpr (C::QT) {
    if (qpre.pos != nullptr) {
      for (int e = tid; e < kRopeCoords * (D / 4); e += C::THREADS) {
        const float coord = float(e / (D / 4));
        const float2 rv = s_rev[e % (D / 4)];
        const float t = coord * rv.x;
        const float frac = (t - rintf(t)) + (fmaf(coord, rv.x, -t) + coord * rv.y);
        s_cs[(e / (D / 4)) * kCsRow + e % (D / 4)] =
            make_float2(__builtin_amdgcn_cosf(frac), __builtin_amdgcn_sinf(frac));
      }
      __syncthreads();
    }
  }

  // items == null: a uniform batch (u_batch segments of u_seq_len tokens).
  // Otherwise each unit reads its 16-byte item (segment, q-tile, first token,
  // length) in one load, with no dependent read of the list length or of
  // cu_seqlens; the list's capacity bounds the loop and the first item marked
  // with segment -1 ends it.
  //
  // Unit order.  A unit is an (item, head) pair.  Workgroup b runs on XCD
  // b % 8 (the dispatcher hands workgroups to the 8 XCDs in turn; the grid is
  // a multiple of 8, so a workgroup keeps its XCD from unit to unit), and
  // each XCD has its own L2.  With H a multiple of 8 the item-major order
  // (unit = item * H + head) gives XCD x the heads h = x (mod 8) of every
  // item, so its co-resident workgroups share those heads' K and V tiles.
  // With other head counts (12, say) that order would spread every head over
  // several XCDs; the units are then taken head-major (head * N + item, N
  // items) in 8 contiguous chunks, one per XCD, so each XCD streams about H/8
  // heads, one after another, and needs the list length N itself.
  const bool uniform = items == nullptr;
  const int uni_tiles = (u_seq_len + C::BM - 1) / C::BM;
  const bool head_major = (H & 7) != 0;
  const int64_t n_items =
      uniform ? int64_t(u_batch) * uni_tiles : (head_major ? int64_t(meta[0]) : list_cap);
  const int64_t nunits = n_items * H;
  const int64_t xcd_chunk = (nunits + 7) / 8;
  for (int64_t slot = blockIdx.x;; slot += gridDim.x) {
    // No drain here: the previous unit's output stores may still be in
    // flight.  Every copy wait below counts only copies issued after the
    // tile it waits for, and loads (global and global -> LDS) complete in
    // issue order, so older outstanding stores can only lengthen a wait,
    // never end it early.  (Letting the stores drain under this unit's
    // loads is 4% faster on batches of 64-token segments.)
    int item, h;
    if (head_major) {
      const int64_t s = slot >> 3;
      const int64_t u = int64_t(blockIdx.x & 7) * xcd_chunk + s;
      if (s >= xcd_chunk || u >= nunits) break;
      h = int(u / n_items);
      item = int(u - int64_t(h) * n_items);
    } else {
      if (slot >= nunits) break;
      item = int(slot / H);
      h = int(slot - int64_t(item) * H);
    }
    int qt, start, len;
    if (uniform) {
      const int seg = item / uni_tiles;
      qt = item - seg * uni_tiles;
      start = seg * u_seq_len;
      len = u_seq_len;
    } else {
      const int4 it = *reinterpret_cast<const int4*>(items + 4 * size_t(item));
      if (it.x < 0) break;  // past the list's last item
      qt = it.y;
      start = it.z;
      len = it.w;
    }
    // Causal: a segment's last q-tile visits the most keys, so its tiles are
    // taken last-first (the heaviest items start first, as in the list order).
    // An item past the segment's tiles (a list built for other boundaries)
    // is skipped, as it finds no rows without the reversal.
    if (CAUSAL) {
      const int nq = (len + C::BM - 1) / C::BM;
      if (qt >= nq) continue;
      qt = nq - 1 - qt;
    }
    // Offsets are 32-bit: a segment larger than the addressable span is skipped
    // (the host rejects the max_seqlen that would allow it).  Within the span,
    // every copy offset, padding rows of the last tile included, stays below
    // kPadOffset + kMaxSegmentBytes < 2^32.
    if (!segment_fits(len, ts.k > ts.v ? ts.k : ts.v)) continue;
    const int row0 = qt * C::BM + wave * 32 * QB;  // first query row of this wave
    const bool wave_active = row0 < len;
    const i32x4_t krs = make_rsrc(k + size_t(start) * ts.k + size_t(h) * D,
                                  unsigned(((len - 1) * ts.k + D) * 2));
    const i32x4_t vrs = make_rsrc(v + size_t(start) * ts.v + size_t(h) * D,
                                  unsigned(((len - 1) * ts.v + D) * 2));
    // KF: the segment's positions (8 bytes per key); without rotary a
    // resource of zero bytes, so that copy only writes zeros.
    i32x4_t prs{};
    if constexpr (C::KF)
      prs = qpre.pos != nullptr ? make_rsrc(qpre.pos + 2 * size_t(start), unsigned(len) * 8u)
                                : make_rsrc(k, 0u);

    // Q^T fragments (B operand of S^T = K Q^T): lane holds 8 dims of its row
    // in each of the wave's QB query blocks: dims 16*st + 8*half + 0..7.
    bf16x8_t qf[QB][C::KSTEPS];
    auto load_q = [&]() {
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const int row = row0 + 32 * b + l32;
        if (row < len) {
          const u16* qp = q + size_t(start + row) * ts.q + size_t(h) * D + half * 8;
#pragma unroll
          for (int st = 0; st < C::KSTEPS; ++st)
            qf[b][st] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(qp + st * 16));
        } else {
#pragma unroll
          for (int st = 0; st < C::KSTEPS; ++st) qf[b][st] = bf16x8_t{};
        }
      }
    };
    load_q();
    // QT: the query rows' positions are loaded with the rows, so the
    // transform waits for one round of loads.
    int2 q_pc[QB];
    if constexpr (C::QT) {
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const int row = row0 + 32 * b + l32;
        q_pc[b] = make_int2(0, 0);
        if (qpre.pos != nullptr && row < len)
          q_pc[b] = *reinterpret_cast<const int2*>(qpre.pos + 2 * (start + row));
      }
    }

    // The Q-side pre-pass on the fragments: RMSNorm then rotary in fp32,
    // rounded once to bf16 (the pre-pass kernel's arithmetic).  Lane (l32,
    // half) holds dims 16*st + 8*half + i of row l32.  Rotate-half pairs
    // (m, m + D/2): the partner of register st is register st + D/32 of the
    // same lane when D/2 is a multiple of 16; for D = 80 it sits in the other
    // half-wave (register st + 2 + half, read across with v_permlane32_swap).
    // Angle of pair m: the row coordinate for m < D/4, the column for the
    // rest, with frequency m mod D/4; it is reduced exactly to a fraction of
    // a turn before the hardware sine and cosine.  Complex pairs (2j, 2j+1)
    // lie in one dword of one lane.
    auto transform_q = [&]() {
      constexpr int HALF = D / 2, QUART = D / 4, KS = C::KSTEPS;
      constexpr bool kCross = HALF % 16 != 0;
      static_assert(HALF % 8 == 0, "rotary pairs must stay on the same element of a register");
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const int row = row0 + 32 * b + l32;
        float x[KS][8];
#pragma unroll
        for (int st = 0; st < KS; ++st)
#pragma unroll
          for (int i = 0; i < 8; ++i) x[st][i] = float(qf[b][st][i]);
        if (qpre.weight != nullptr) {
          float ss = 0.f;
#pragma unroll
          for (int st = 0; st < KS; ++st)
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = fmaf(x[st][i], x[st][i], ss);
          ss += other_half(ss);
          const float rinv = rsqrtf(ss * (1.f / D) + qpre.eps);
#pragma unroll
          for (int st = 0; st < KS; ++st)
#pragma unroll
            for (int i = 0; i < 8; ++i) x[st][i] = x[st][i] * rinv * s_qw[16 * st + 8 * half + i];
        }
        if (qpre.pos != nullptr) {
          int2 pc = make_int2(0, 0);
          if constexpr (C::QT) {
            pc = q_pc[b];
          } else {
            if (row < len) pc = *reinterpret_cast<const int2*>(qpre.pos + 2 * (start + row));
          }
          if constexpr (!C::QT) {
          // cos and sin of the angle of pair index m (< D/2)
          auto cossin = [&](int m, float& cs, float& sn) {
            const float coord = float(m < QUART ? pc.x : pc.y);
            const float2 rv = s_rev[m < QUART ? m : m - QUART];
            const float t = coord * rv.x;
            const float frac = (t - rintf(t)) + (fmaf(coord, rv.x, -t) + coord * rv.y);
            cs = __builtin_amdgcn_cosf(frac);
            sn = __builtin_amdgcn_sinf(frac);
          };
          float y[KS][8];
          if (qpre.rope_mode == 0) {
#pragma unroll
            for (int st = 0; st < KS; ++st) {
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                float partner;
                if constexpr (kCross) {
                  // each lane passes on the register its partner lane needs
                  const int A = (st + HALF / 16 + 1) % KS, B = (st + HALF / 16) % KS;
                  partner = other_half(half ? x[B][i] : x[A][i]);
                } else {
                  partner = x[(st + HALF / 16) % KS][i];
                }
                const int d = 16 * st + 8 * half + i;
                const bool first = d < HALF;
                float cs, sn;
                cossin(first ? d : d - HALF, cs, sn);
                y[st][i] = first ? x[st][i] * cs - partner * sn : x[st][i] * cs + partner * sn;
              }
            }
          } else {
#pragma unroll
            for (int st = 0; st < KS; ++st) {
#pragma unroll
              for (int i = 0; i < 8; i += 2) {
                float cs, sn;
                cossin((16 * st + 8 * half + i) / 2, cs, sn);
                y[st][i] = x[st][i] * cs - x[st][i + 1] * sn;
                y[st][i + 1] = x[st][i + 1] * cs + x[st][i] * sn;
              }
            }
          }
#pragma unroll
          for (int st = 0; st < KS; ++st)
#pragma unroll
            for (int i = 0; i < 8; ++i) x[st][i] = y[st][i];
          } else {
          // cos and sin of the angle of pair index m (< D/2)
          auto cossin_direct = [&](int m, float& cs, float& sn) {
            const float coord = float(m < QUART ? pc.x : pc.y);
            const float2 rv = s_rev[m < QUART ? m : m - QUART];
            const float t = coord * rv.x;
            const float frac = (t - rintf(t)) + (fmaf(coord, rv.x, -t) + coord * rv.y);
            cs = __builtin_amdgcn_cosf(frac);
            sn = __builtin_amdgcn_sinf(frac);
          };
          // QT: the same values from the workgroup's table when every row of
          // the wave has both coordinates below kRopeCoords.
          auto cossin_table = [&](int m, float& cs, float& sn) {
            const int coord = m < QUART ? pc.x : pc.y;
            const float2 v = s_cs[coord * kCsRow + (m < QUART ? m : m - QUART)];
            cs = v.x;
            sn = v.y;
          };
          auto rope_rows = [&](auto cossin) __attribute__((always_inline)) {
          float y[KS][8];
          if (qpre.rope_mode == 0) {
#pragma unroll
            for (int st = 0; st < KS; ++st) {
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                float partner;
                if constexpr (kCross) {
                  // each lane passes on the register its partner lane needs
                  const int A = (st + HALF / 16 + 1) % KS, B = (st + HALF / 16) % KS;
                  partner = other_half(half ? x[B][i] : x[A][i]);
                } else {
                  partner = x[(st + HALF / 16) % KS][i];
                }
                const int d = 16 * st + 8 * half + i;
                const bool first = d < HALF;
                float cs, sn;
                cossin(first ? d : d - HALF, cs, sn);
                y[st][i] = first ? x[st][i] * cs - partner * sn : x[st][i] * cs + partner * sn;
              }
            }
          } else {
#pragma unroll
            for (int st = 0; st < KS; ++st) {
#pragma unroll
              for (int i = 0; i < 8; i += 2) {
                float cs, sn;
                cossin((16 * st + 8 * half + i) / 2, cs, sn);
                y[st][i] = x[st][i] * cs - x[st][i + 1] * sn;
                y[st][i + 1] = x[st][i + 1] * cs + x[st][i] * sn;
              }
            }
          }
#pragma unroll
          for (int st = 0; st < KS; ++st)
#pragma unroll
            for (int i = 0; i < 8; ++i) x[st][i] = y[st][i];
          };
          // Table reads by runs: the 8 elements of register st hold 8
          // consecutive rotary pairs of one coordinate (rotate-half, D a
          // multiple of 32) or 4 (complex), so their cos and sin are one run
          // of the table (16-byte reads instead of one read and an address
          // per element).
          auto rope_rows_runs = [&]() __attribute__((always_inline)) {
            float y[KS][8];
            if (qpre.rope_mode == 0) {
              if constexpr (D % 32 == 0) {
#pragma unroll
                for (int st = 0; st < KS; ++st) {
                  // D/2 is a multiple of 16, so whether dims 16st + 8half ..
                  // + 7 are in the first half does not depend on half
                  constexpr int kFirstRegs = HALF / 16;
                  const bool first = st < kFirstRegs;
                  const int m0 = 16 * st + 8 * half - (first ? 0 : HALF);
                  const bool on_row = m0 < QUART;
                  const float2* tb = s_cs + (on_row ? pc.x : pc.y) * kCsRow + (on_row ? m0 : m0 - QUART);
#pragma unroll
                  for (int i = 0; i < 8; ++i) {
                    const float partner = x[(st + HALF / 16) % KS][i];
                    const float2 v = tb[i];
                    y[st][i] = first ? x[st][i] * v.x - partner * v.y : x[st][i] * v.x + partner * v.y;
                  }
                }
              }
            } else {
#pragma unroll
              for (int st = 0; st < KS; ++st) {
                const int j0 = 8 * st + 4 * half;
                const bool on_row = j0 < QUART;
                const float2* tb = s_cs + (on_row ? pc.x : pc.y) * kCsRow + (on_row ? j0 : j0 - QUART);
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                  const float2 v = tb[i / 2];
                  y[st][i] = x[st][i] * v.x - x[st][i + 1] * v.y;
                  y[st][i + 1] = x[st][i + 1] * v.x + x[st][i] * v.y;
                }
              }
            }
#pragma unroll
            for (int st = 0; st < KS; ++st)
#pragma unroll
              for (int i = 0; i < 8; ++i) x[st][i] = y[st][i];
          };
          static_assert(QUART % 4 == 0, "complex pairs of a register share a coordinate");
          if constexpr (C::QT) {
            if (__all(unsigned(pc.x) < unsigned(kRopeCoords) && unsigned(pc.y) < unsigned(kRopeCoords))) {
              if (D % 32 == 0 || qpre.rope_mode != 0)
                rope_rows_runs();
              else
                rope_rows(cossin_table);  // rotate-half at D = 80: runs cross the row/column split
            } else {
              rope_rows(cossin_direct);
            }
          } else {
            rope_rows(cossin_direct);
          }
          }
        }
#pragma unroll
        for (int st = 0; st < KS; ++st)
#pragma unroll
          for (int i = 0; i < 8; ++i) qf[b][st][i] = (__bf16)x[st][i];
      }
    };

    // Reference max per query row (log2 domain), fixed for a whole pass over
    // the keys: p = 2^(s*c - m_ref) needs no rescaling of O, so the key loop
    // never touches the accumulators outside the MFMAs, and after the first
    // tile it needs no row max either.  Pass 0 takes m_ref from the first key
    // tile.  A row whose sum of p then exceeds kRestartLimit = 2^64 (or is not
    // finite) means some later key scored far above that tile; the workgroup
    // then runs a max-only pass over the keys and repeats the unit with the
    // exact row max, where every p <= 1.
    float m_ref[QB], m_seen[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) m_ref[b] = m_seen[b] = -INFINITY;
    f32x16_t o[QB][C::DB];
    float l_run[QB];
    // Keys this unit visits: the whole segment, or with CAUSAL only keys up to
    // the unit's last query row.
    const int kv_end = CAUSAL ? min(len, (qt + 1) * C::BM) : len;
    const int ntiles = (kv_end + BN - 1) / BN;
    auto issue_tile = [&](int t) {
      const unsigned tile_off_k = unsigned(t) * unsigned(BN * 2) * unsigned(ts.k);
      const unsigned tile_off_v = unsigned(t) * unsigned(BN * 2) * unsigned(ts.v);
      const unsigned stage_lds = smem_base + unsigned((t % STAGES) * C::STAGE_UNITS * 16);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        if ((j < C::NI_LO || wave_hi) && !cp_skip[j]) {
          if constexpr (C::KF) {
            if (cp_is_p[j])
              copy_dword_to_lds(stage_lds + cp_lds[j], cp_off[j] + unsigned(t) * unsigned(BN * 8), prs);
            else
              copy_to_lds(stage_lds + cp_lds[j], cp_off[j] + (cp_is_k[j] ? tile_off_k : tile_off_v),
                          cp_is_k[j] ? krs : vrs);
          } else {
            copy_to_lds(stage_lds + cp_lds[j], cp_off[j] + (cp_is_k[j] ? tile_off_k : tile_off_v),
                        cp_is_k[j] ? krs : vrs);
          }
        }
    };
    // KF: RMSNorm then rotary on tile t's K rows in LDS, once per workgroup,
    // in place, with the arithmetic of transform_q (fp32, one rounding to
    // bf16).  CHP lanes share a key: lane c of them takes rotary pairs
    // 8c .. 8c + 7, which lie in two 16-byte units of the row (dims 8c.. and
    // D/2 + 8c.. for rotate-half, dims 16c .. 16c + 15 for complex), so every
    // unit is read and written once.  The key's sum of squares is joined
    // across its lanes with DPP.  Keys past the segment's end stay zero.  The
    // positions arrive with the tile's copies (8 bytes per key, key order).
    auto transform_k = [&](int t) __attribute__((always_inline)) {
      constexpr int CH = D / 16;
      constexpr int CHP = CH <= 2 ? 2 : (CH <= 4 ? 4 : 8);
      static_assert(CH <= 8 && (D / 2) % 8 == 0, "rotary pairs must fill whole 16-byte units");
      constexpr int ROUNDS = (BN * CHP + C::THREADS - 1) / C::THREADS;
      u16* const kst = smem + (t % STAGES) * C::STAGE_UNITS * 8;
      const int2* const kpos = reinterpret_cast<const int2*>(kst + (C::KREG + C::VREG) * 8);
      // One code path per rotary pairing (a uniform branch, taken once per
      // tile), so no element is computed both ways and selected.
      auto run = [&](auto neox_tag) __attribute__((always_inline)) {
      constexpr bool neox = decltype(neox_tag)::value;
#pragma unroll
      for (int rd = 0; rd < ROUNDS; ++rd) {
        const int w = tid + rd * C::THREADS;
        const int c = w % CHP;
        const int row = w / CHP < BN ? w / CHP : BN - 1;  // LDS row; it holds key swap(row)
        const int key = swap_bits_2_3(row);
        const bool act = w / CHP < BN && c < CH && t * BN + key < len;
        const int cc = c < CH ? c : CH - 1;  // idle lanes still compute, on valid indices
        const int u0 = neox ? cc : 2 * cc;
        const int u1 = neox ? cc + CH : 2 * cc + 1;
        u32x4_t* const p0 = reinterpret_cast<u32x4_t*>(kst + (row * C::KSTR + u0) * 8);
        u32x4_t* const p1 = reinterpret_cast<u32x4_t*>(kst + (row * C::KSTR + u1) * 8);
        u32x4_t a = u32x4_t{0u, 0u, 0u, 0u}, b = a;
        if (act) {
          a = *p0;
          b = *p1;
        }
        float x[16];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = __uint_as_float(a[e] << 16);
          x[2 * e + 1] = __uint_as_float(a[e] & 0xffff0000u);
          x[8 + 2 * e] = __uint_as_float(b[e] << 16);
          x[8 + 2 * e + 1] = __uint_as_float(b[e] & 0xffff0000u);
        }
        if (qpre.k_weight != nullptr) {
          float ss = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) ss = fmaf(x[i], x[i], ss);
          ss = group_sum<CHP>(ss);
          const float rinv = rsqrtf(ss * (1.f / D) + qpre.eps);
          const float* w0 = s_kw + (neox ? 8 * cc : 16 * cc);  // weights of x[0..7]
          const float* w1 = s_kw + (neox ? D / 2 + 8 * cc : 16 * cc + 8);  // of x[8..15]
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            x[i] = x[i] * rinv * w0[i];
            x[8 + i] = x[8 + i] * rinv * w1[i];
          }
        }
        if (qpre.pos != nullptr) {
          const int2 pc = act ? kpos[key] : make_int2(0, 0);
          // pair m = 8 cc + pr: the row coordinate for m < D/4, else the column
          auto rotate = [&](auto cossin) __attribute__((always_inline)) {
#pragma unroll
            for (int pr = 0; pr < 8; ++pr) {
              const int m = 8 * cc + pr;
              const bool on_row = m < D / 4;
              float cs, sn;
              cossin(pr, on_row ? pc.x : pc.y, on_row ? m : m - D / 4, cs, sn);
              if constexpr (neox) {
                const float lo = x[pr], hi = x[8 + pr];
                x[pr] = lo * cs - hi * sn;
                x[8 + pr] = hi * cs + lo * sn;
              } else {
                const float e0 = x[2 * pr], e1 = x[2 * pr + 1];
                x[2 * pr] = e0 * cs - e1 * sn;
                x[2 * pr + 1] = e1 * cs + e0 * sn;
              }
            }
          };
          if (__all(unsigned(pc.x) < unsigned(kRopeCoords) && unsigned(pc.y) < unsigned(kRopeCoords))) {
            // One 8-byte read per pair.  Reading a lane's eight pairs as one
            // 64-byte run was slower (ragged batch 908 against 692 us): the
            // lanes of a key then read runs 64 bytes apart, on the same banks.
            rotate([&](int, int ci, int f, float& cs, float& sn) {
              const float2 v = s_cs[ci * kCsRow + f];
              cs = v.x;
              sn = v.y;
            });
          } else {
            rotate([&](int, int ci, int f, float& cs, float& sn) {
              const float coord = float(ci);
              const float2 rv = s_rev[f];
              const float tt = coord * rv.x;
              const float frac = (tt - rintf(tt)) + (fmaf(coord, rv.x, -tt) + coord * rv.y);
              cs = __builtin_amdgcn_cosf(frac);
              sn = __builtin_amdgcn_sinf(frac);
            });
          }
        }
        if (act) {
          bf16x8_t y0, y1;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            y0[i] = (__bf16)x[i];
            y1[i] = (__bf16)x[8 + i];
          }
          *p0 = __builtin_bit_cast(u32x4_t, y0);
          *p1 = __builtin_bit_cast(u32x4_t, y1);
        }
      }
      };
      if (qpre.rope_mode == 0)
        run(std::true_type{});
      else
        run(std::false_type{});
    };

    // Sum of p over the whole row b (both lane halves).
    auto row_total = [&](int b) {
      if constexpr (kSumByMfma) {
        // O^T register r of block DB-1 holds dim 32(DB-1) + 8(r>>2) + 4half + (r&3).
        constexpr int rr = kOnesLane;  // offset of dim D inside the last block
        constexpr int r = 4 * (rr >> 3) + (rr & 3);
        const float v = o[b][C::DB - 1][r];
        const float w = other_half(v);
        return ((rr >> 2) & 1) == 0 ? (half == 0 ? v : w) : (half == 1 ? v : w);
      } else {
        return l_run[b] + other_half(l_run[b]);
      }
    };

    // One key tile.  MASKED: a tile with keys past the segment's end or (with
    // CAUSAL) after some query row of the unit.  MODE: kSetRef (tile 0
    // of pass 0: its max becomes m_ref), kPlain (exponentials and P V only),
    // kMaxOnly (scores and row max only).
    auto process_tile = [&](auto masked_tag, auto mode_tag, int t) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      constexpr int MODE = decltype(mode_tag)::value;
      // Own copies of tile t done: at most min(STAGES-2, ntiles-1-t) later
      // tiles' copies may still be in flight.
      const int later = min(ntiles - 1 - t, STAGES - 2);
      if (wave_hi) wait_copies<C::NI_HI, STAGES>(later);
      else wait_copies<C::NI_LO, STAGES>(later);
      __syncthreads();  // everyone's copies of tile t landed; tile t-1 is free
      if (t + STAGES - 1 < ntiles) issue_tile(t + STAGES - 1);
      if constexpr (C::KF) {
        transform_k(t);  // every wave takes part, active or not
        __syncthreads();  // tile t's K rows are normalised and rotated
      }
      if (!wave_active) return;
      const int kv0 = t * BN;
      // Causal: a tile that starts after this wave's last row adds nothing.
      if (CAUSAL && kv0 > row0 + 32 * QB - 1) return;

      const u16* stage = smem + (t % STAGES) * C::STAGE_UNITS * 8;
      // All LDS fragment reads of the tile are issued up front, K first, so
      // their latency is paid once and the V reads land during the scores
      // and the softmax.
      bf16x8_t kf[KB][C::KSTEPS];
      const u16* kt = stage + l32 * C::KSTR * 8 + half * 8;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int st = 0; st < C::KSTEPS; ++st)
          kf[kb][st] = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(kt + kb * 32 * C::KSTR * 8 + st * 16));
      // Transpose-read lane l (group g = l>>4, j = l&15) addresses V row (key)
      // kb*32 + 16*s2 + 8*half + 4*qh + (j>>2), dims 32d + 16*(g&1) +
      // 4*(j&3) .. +3, and receives keys kb*32 + 16*s2 + 8*half + 4*qh + 0..3
      // of dim 32d + (l&31).  One LDS-space base; the per-read offsets are
      // constants the compiler folds into the instructions.
      i16x4_t vf[KB][2][C::DB][2];
      if constexpr (MODE != kMaxOnly) {
        lds_u16_t* const vbase = (lds_u16_t*)(stage + C::KREG * 8) +
                                 (8 * half + ((lane & 15) >> 2)) * C::VSTR * 8 +
                                 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int d = 0; d < C::DB; ++d) {
              lds_u16_t* base = vbase + (kb * 32 + 16 * s2) * C::VSTR * 8 + 32 * d;
              vf[kb][s2][d][0] = ds_read_tr16(base);
              vf[kb][s2][d][1] = ds_read_tr16(base + 4 * C::VSTR * 8);
            }
      }
      __builtin_amdgcn_sched_barrier(0);
      // With kSumByMfma, head-dim row D of V^T is all ones in LDS, so row D of
      // O^T accumulates the row sums of P.

      // S^T = K Q^T for every query block (each K fragment feeds QB MFMAs).
      f32x16_t sc[QB][KB];
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          sc[b][kb] = f32x16_t{};
#pragma unroll
          for (int st = 0; st < C::KSTEPS; ++st)
            sc[b][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb][st], qf[b][st], sc[b][kb], 0, 0, 0);
        }

      // Softmax.  Register r of block kb holds key
      // kv0 + 32kb + 16(r>>3) + 8half + (r&7) for query row l32.  Block kb's
      // exponentials need only m_ref, so they and its P V products overlap
      // the MFMAs of the neighbouring blocks.
      // D = 128: the softmax and the P V MFMAs issue at raised priority, the
      // dependent chain of S MFMAs at normal priority, so of the two waves on
      // a SIMD the one in its softmax goes first while the other's S chain
      // runs (2.5-3% faster on the 1 x 16384-token batch, 0.6-1% on the
      // ragged one; neutral at D = 80 and 2% slower at D = 64, so only here).
      if constexpr (kSoftmaxPrio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        if constexpr (MASKED || !POS_SCALE) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              float x = POS_SCALE ? sc[b][kb][r] : sc[b][kb][r] * scale_log2;
              if constexpr (MASKED) {
                const int key = kv0 + kb * 32 + 16 * (r >> 3) + 8 * half + (r & 7);
                if (key >= len) x = -INFINITY;
                if (CAUSAL && key > row0 + 32 * b + l32) x = -INFINITY;
              }
              sc[b][kb][r] = x;
            }
        }
        if constexpr (MODE != kPlain) {
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[b][kb][r]);
          mx = fmaxf(mx, other_half(mx));
          const float mt = POS_SCALE ? mx * scale_log2 : mx;  // tile max, log2 domain
          if constexpr (MODE == kSetRef) m_ref[b] = mt;
          if constexpr (MODE == kMaxOnly) m_seen[b] = fmaxf(m_seen[b], mt);
        }
        if constexpr (MODE != kMaxOnly) {
          const float neg_m = -m_ref[b];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            bf16x8_t p[2];
            float part[4] = {0.f, 0.f, 0.f, 0.f};  // four independent partial sums
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float e = POS_SCALE ? __builtin_amdgcn_exp2f(fmaf(sc[b][kb][r], scale_log2, neg_m))
                                        : __builtin_amdgcn_exp2f(sc[b][kb][r] + neg_m);
              if constexpr (!kSumByMfma) part[r & 3] += e;
              p[r >> 3][r & 7] = (__bf16)e;
            }
            if constexpr (!kSumByMfma) l_run[b] += (part[0] + part[1]) + (part[2] + part[3]);

            // O^T += V^T P^T (each V fragment feeds QB MFMAs).
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
              for (int d = 0; d < C::DB; ++d)
                o[b][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8_t, vf[kb][s2][d]), p[s2], o[b][d], 0, 0, 0);
          }
        }
      }
      if constexpr (kSoftmaxPrio) __builtin_amdgcn_s_setprio(0);
    };

    // One pass over the keys: tile 0 in mode M0, the others in mode M.
    // The previous unit's (or pass's) last tile must no longer be read, then
    // the pass's first tiles are issued.  The Q loads may still be in flight:
    // loads complete in issue order, so a copy wait (vmcnt) also covers the
    // older Q loads, and the first tiles' copies overlap them.
    auto start_pass = [&]() {
      __syncthreads();
      if constexpr (kStageOut && kSumByMfma) {
        if (ring_staged) {  // every wave has read its staged rows back (barrier above)
          write_ones();
          ring_staged = false;
        }
      }
#pragma unroll
      for (int t = 0; t < STAGES - 1; ++t)
        if (t < ntiles) issue_tile(t);
    };
    // The Q-side pre-pass runs before the pass's first tiles are issued: its
    // register spills at D = 80 and 96 go through scratch, and a scratch
    // reload issued behind the tile copies would wait for them (loads
    // complete in order).  With QT the first tiles go out first, so the query
    // rows, their positions and the tiles arrive in one round trip instead of
    // two (with KF the K transform needs the tiles anyway).
    if constexpr (C::QT) {
      start_pass();
      if (q_pending && wave_active) transform_q();  // a wave past the rows has none to prepare
    } else {
      if (q_pending) transform_q();
      start_pass();
    }

    auto run_pass = [&](auto m0_tag, auto m_tag, bool started) {
      if (!started) start_pass();
#pragma unroll
      for (int b = 0; b < QB; ++b) {
#pragma unroll
        for (int d = 0; d < C::DB; ++d) o[b][d] = f32x16_t{};
        l_run[b] = 0.f;  // this lane's partial row sum
      }
      // Tiles before nfull need no mask: every key is inside the segment and
      // (causal) at or before the unit's first query row.  The rest are masked.
      const int nfull = CAUSAL ? min(len, qt * C::BM + 1) / BN : len / BN;
      // With KF the tile body outgrows the inliner's budget; its calls are
      // inlined by force (the other kernels' code is left as it was).
      auto tile = [&](auto masked_tag, auto mode_tag, int t) __attribute__((always_inline)) {
        if constexpr (C::KF) {
          [[clang::always_inline]] process_tile(masked_tag, mode_tag, t);
        } else {
          process_tile(masked_tag, mode_tag, t);
        }
      };
      if (nfull == 0) {
        tile(std::true_type{}, m0_tag, 0);
      } else {
        tile(std::false_type{}, m0_tag, 0);
        for (int t = 1; t < nfull; ++t) tile(std::false_type{}, m_tag, t);
      }
      for (int t = nfull > 1 ? nfull : 1; t < ntiles; ++t) tile(std::true_type{}, m_tag, t);
    };

    run_pass(std::integral_constant<int, kSetRef>{}, std::integral_constant<int, kPlain>{}, true);
    bool repeat = false;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const float lt = row_total(b);  // every lane takes part in the half exchange
      repeat |= wave_active && row0 + 32 * b + l32 < len && !(lt <= kRestartLimit);
    }
    // Every wave shares the copy ring, so the workgroup repeats together.
    if (__syncthreads_or(repeat)) {
      run_pass(std::integral_constant<int, kMaxOnly>{}, std::integral_constant<int, kMaxOnly>{}, false);
#pragma unroll
      for (int b = 0; b < QB; ++b) m_ref[b] = m_seen[b];
      run_pass(std::integral_constant<int, kPlain>{}, std::integral_constant<int, kPlain>{}, false);
    }

    // Finalize: O^T register r of block d holds dim 32d + 8(r>>2) + 4half + (r&3).
    // With kStageOut the normalised rows go through LDS first (the ring is
    // free once every wave is past its last tile) and leave as whole 16-byte
    // pieces, lane-consecutive along each row; written straight from the
    // accumulators, each store instruction would put 16 bytes into each of 32
    // rows.
    if constexpr (kStageOut) {
      constexpr int kORow = D * 2 + 16;    // staged row stride, bytes
      constexpr int kCPR = D / 8;          // 16-byte pieces per row
      static_assert(C::WAVES * 32 * QB * kORow <= C::LDS_BYTES, "output staging fits the ring");
      static_assert((32 * QB * kCPR) % 64 == 0, "whole store rounds per wave");
      __syncthreads();  // every wave is past its last tile: the ring is free
      ring_staged = true;
      char* const ost = reinterpret_cast<char*>(smem) + wave * (32 * QB * kORow);
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const int row = row0 + 32 * b + l32;
        const float l_tot = row_total(b);
        // Log-sum-exp of the row's scores, natural log: p = 2^(x - m_ref)
        // with x = scale * log2(e) * score, so sum_b e^(scale*score) = 2^m_ref * l.
        if (lse != nullptr && row < len)
          lse[size_t(start + row) * H + h] = (m_ref[b] + log2f(l_tot)) * kLn2;
        const float inv = 1.f / l_tot;  // rows past the segment are staged, never stored
        char* const orow = ost + (32 * b + l32) * kORow;
#pragma unroll
        for (int d = 0; d < C::DB; ++d) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d0 = d * 32 + 8 * g + 4 * half;
            if (d0 < D) {
              __bf16 w[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[b][d][4 * g + e] * inv);
              *reinterpret_cast<u32x2_t*>(orow + d0 * 2) = __builtin_bit_cast(u32x2_t, w);
            }
          }
        }
      }
      // A wave reads back only what it wrote, and a wave's LDS accesses are
      // carried out in order.
#pragma unroll
      for (int it = 0; it < 32 * QB * kCPR / 64; ++it) {
        const int c = it * 64 + lane;
        const int r = c / kCPR, col = c - r * kCPR;
        const u32x4_t val = *reinterpret_cast<const u32x4_t*>(ost + r * kORow + col * 16);
        if (row0 + r < len)
          *reinterpret_cast<u32x4_t*>(out + size_t(start + row0 + r) * ts.o + size_t(h) * D + col * 8) =
              val;
      }
    } else {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int row = row0 + 32 * b + l32;
      const float l_tot = row_total(b);
      // Log-sum-exp of the row's scores, natural log: p = 2^(x - m_ref) with
      // x = scale * log2(e) * score, so sum_b e^(scale*score) = 2^m_ref * l.
      if (lse != nullptr && row < len)
        lse[size_t(start + row) * H + h] = (m_ref[b] + log2f(l_tot)) * kLn2;
      if (row < len) {
        const float inv = 1.f / l_tot;
        u16* op = out + size_t(start + row) * ts.o + size_t(h) * D;
#pragma unroll
        for (int d = 0; d < C::DB; ++d) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d0 = d * 32 + 8 * g + 4 * half;
            if (d0 < D) {
              __bf16 w[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[b][d][4 * g + e] * inv);
              *reinterpret_cast<u32x2_t*>(op + d0) = __builtin_bit_cast(u32x2_t, w);
            }
          }
        }
      }
    }
    }
  }
}

template <class C>
auto pick_kernel(bool causal, bool pos_scale) {
  return causal ? (pos_scale ? attn_bf16_kernel<C, true, true> : attn_bf16_kernel<C, false, true>)
                : (pos_scale ? attn_bf16_kernel<C, true, false> : attn_bf16_kernel<C, false, false>);
}

template <class C>
hipError_t launch_cfg(const void* q, const void* k, const void* v, const Schedule& sch, int H,
                      float scale, bool causal, const QPrepass* qp, void* out, float* lse,
                      TokenStrides ts, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  QPrepass qpre{};
  if (qp != nullptr) qpre = *qp;
  const int64_t items = sch.items != nullptr
                            ? sch.cap
                            : int64_t(sch.batch) * ((sch.seq_len + C::BM - 1) / C::BM);
  const int64_t units = items * int64_t(H);
  if (units <= 0) return hipSuccess;
  static_assert(kWorklistSentinelSpan >= kMaxAttnGridBf16, "every workgroup must meet a marked item");
  static_assert(kMaxAttnGridBf16 % 8 == 0, "the grid is a whole number of XCD rounds");
  // A multiple of 8 workgroups, so each keeps its XCD across its units.
  const int64_t grid = ((units < kMaxAttnGridBf16 ? units : kMaxAttnGridBf16) + 7) / 8 * 8;
  const float c = scale * kLog2e;
  auto kern = pick_kernel<C>(causal, c > 0.f);
  hipExtLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(C::THREADS), 0, stream, e0, e1, 0,
                     static_cast<const u16*>(q), static_cast<const u16*>(k),
                     static_cast<const u16*>(v), sch.items, sch.meta, (long long)sch.cap, sch.batch,
                     sch.seq_len, H, c, static_cast<u16*>(out), lse, ts, qpre);
  return hipGetLastError();
}

// Per head dim: (waves, query blocks per wave, keys per tile, ring depth,
// waves per SIMD).  Rows per workgroup must equal bf16_block_m_const(D).
// D = 80 takes 8-wave workgroups: one K/V ring per CU instead of two halves
// the copies into LDS, and the 4 x 1024-token batch runs 7% faster (31 us
// instead of 33); at D = 128 the 256-row q-tiles lose more on the ragged
// batch's short segments than the shared ring gains.
template <int D> struct Choice;
template <> struct Choice<32> { using C = Cfg<32, 4, 1, 64, 2, 2>; };
template <> struct Choice<64> { using C = Cfg<64, 4, 1, 64, 2, 2>; };
template <> struct Choice<80> { using C = Cfg<80, 8, 1, 64, 2, 2>; };
template <> struct Choice<96> { using C = Cfg<96, 4, 1, 64, 2, 2>; };
template <> struct Choice<128> { using C = Cfg<128, 4, 1, 32, 2, 2>; };

}  // namespace
}  // namespace vit
