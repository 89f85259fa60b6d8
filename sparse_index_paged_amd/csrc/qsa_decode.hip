// qsa_decode.hip -- packed QSA decode kernel for gfx950 (MI355X).
//
// What it computes is stated in include/qsa.h.  The design follows the
// page "fix(qsa): restore SM121 correctness with Humanize and Kernel Design
// Agent", section "Optimized kernel": the 12 Q heads that share a KV head
// live in one workgroup so every gathered K/V row is read once for all of
// them; QK and PV run as bf16 matrix products with fp32 online-softmax state;
// long lists are split across workgroups, and the last split to finish merges
// the fp32 partials in a fixed order and resets its counter in the same
// launch.  Dequantization of fp8 / int8 / int4 pools happens in the gather
// itself (page "feat(qsa): quantized KV pools with dequant-on-gather
// (fp8/int8/int4)", part 4 "Motivation").
//
// Mapping onto CDNA4:
//   * workgroup = 4 waves = one (row b, KV head g, split s).  Each wave owns
//     a contiguous slice of the list and runs its own online softmax over
//     16-entry tiles; the 4 wave states are merged through LDS at the end.
//   * Gather: each wave instruction loads 1 KB of whole K (or V) rows with
//     16-byte loads, so the rows of a 16-entry tile arrive fully coalesced;
//     they are dequantized to bf16 into the wave's LDS tiles while the next
//     tile's rows are in flight.
//   * QK as S^T = K . Q^T with v_mfma_f32_16x16x32_bf16: the A operand is 16
//     K rows read from the LDS tile (row = lane % 16, 8 channels per lane
//     per MFMA), the B operand is Q from a tile shared by the workgroup
//     (heads 12..15 zero).
//     The result holds, in lane l, head l % 16 for list entries
//     4*(l/16) + 0..3 -- the entries whose P values the lane then feeds to
//     the PV product, so P never moves between lanes.
//   * PV as O^T = V^T . P^T with v_mfma_f32_16x16x32_bf16: V^T is read
//     from the wave's LDS copy of the V tile with transposing LDS reads.
//     The accumulator O^T keeps head l % 16 in lane l, the same lane that
//     owns that head's running max and sum, so the rescale by
//     exp(m_old - m_new) needs no shuffle.
//   * P enters the PV product as a hi + lo bf16 pair, so the product sees P
//     to ~16 bits instead of bf16's 8: the 32 k-slots of one product hold
//     the tile's 16 entries twice, with P's hi parts against the first copy
//     of V and its lo parts against the second.  Quantized codes are
//     converted exactly to bf16; their fp32 scales are applied outside the
//     MFMA (K scales on the QK partial of each channel group, V scales folded
//     into P).  8-wave workgroups stage int4 codes as the exact values
//     12 + code / 2, one instruction per code, and take the offset out in
//     fp32 (int4_offset_bf16x8).
//   * The online softmax keeps a running max per head that moves only when
//     a tile's max exceeds it by more than 2^8, so the accumulators are
//     rescaled on a few tiles only.
//   * Tiered pools (same page, tiered pool bullet): entry j reads ring row
//     r = sel_j & (R-1) (int8, 64-channel scales) when owner[r] == sel_j,
//     else its int4 row (32-channel scales).  The owner ids join the
//     pipeline one stage before the rows: slot ids of tile t+3D, owner ids
//     of tile t+2D, rows of tile t+D.  Every lane dequantizes 16 channels of
//     either tier into the same LDS place (an int4 lane loads the aligned
//     16 bytes holding its 8 bytes), and the scales are staged per 32
//     channels (a ring scale twice).
//   * Wave priorities for two waves on a SIMD: a tiered wave raises its
//     priority while it stages a tile and issues the next loads, so the
//     dependent chain of slot ids, owner ids and rows advances first.  An
//     int4 wave raises its priority for the tile's products instead, so
//     their dependent chain goes first and the other wave's unpacking
//     fills the gaps.
//   * All splits of one (row, KV head) are given workgroup ids congruent mod
//     8, so they are dispatched to the same XCD and their partials stay in
//     one L2; with quantized pools all KV heads of a row share the XCD as
//     well, so the scale lines they both read come from memory once.  bf16
//     workgroups, once the library has checked the device's dispatch, take
//     their pair slot from the XCD they read in XCC_ID rather than from
//     blockIdx % 8, which keeps the two KV heads of a row on neighbouring
//     XCDs whichever XCD the dispatcher starts at (qsa_internal.h,
//     decode_workgroups).
#include <type_traits>

#include "qsa_internal.h"

namespace qsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));


// s_getreg_b32 operand for the XCC_ID hardware register (hwreg 20, bits
// 0..3): the XCD the wave runs on
constexpr int kHwRegXccId = (3 << 11) | (0 << 6) | 20;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kScaleLog2 = kLog2e / 16.0f;  // softmax scale 1/16 in log2 units
constexpr float kLazyLog2 = 8.0f;              // weights below 2^8 against a stale max

// ---- per-format gather geometry --------------------------------------------
// Rows are gathered with fully coalesced 16-byte loads: one wave instruction
// covers 1 KB = kRPI whole rows (kLPR lanes per row), and a 16-row tile takes
// kNI instructions.  Lane l serves rows (l / kLPR) * kNI + i, i < kNI, so its
// slot ids are contiguous in the list.  Part is the storage of 8 codes.
template <int FMT> struct Fmt;
template <> struct Fmt<kFmtBF16> { using Part = uint4;    static constexpr int kRowBytes = 512; };
template <> struct Fmt<kFmtFP8>  { using Part = uint2;    static constexpr int kRowBytes = 256; };
template <> struct Fmt<kFmtINT8> { using Part = uint2;    static constexpr int kRowBytes = 256; };
template <> struct Fmt<kFmtINT4> { using Part = uint32_t; static constexpr int kRowBytes = 128; };
// tiered: the int8 ring row's geometry; an int4 row's 16 channels of a
// lane are the half of a 16-byte load selected in stage()
template <> struct Fmt<kFmtTIERED> { using Part = uint2; static constexpr int kRowBytes = 256; };
template <int FMT> struct Geo {
  static constexpr int kLPR = Fmt<FMT>::kRowBytes / 16;  // lanes per row
  static constexpr int kRPI = 64 / kLPR;                 // rows per instruction
  static constexpr int kNI = 16 / kRPI;                  // instructions per tile
  static constexpr int kParts = 16 / sizeof(typename Fmt<FMT>::Part);  // 8-code parts per lane
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest even bf16 (one v_cvt_pk_bf16_f32 on
// gfx950): a in bits 0..15, b in bits 16..31.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Two exact values as a bf16 pair: the high halves of their fp32 bits
// (lo in bits 0..15, hi in bits 16..31).  Exact because every value
// converted here (int8 / int4 codes) has at most 8 significant bits.
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// 8 codes -> 8 bf16 values packed in a uint4 (element e in half e%2 of word e/2)
template <int FMT> __device__ __forceinline__ uint4 to_bf16x8(typename Fmt<FMT>::Part r);

template <> __device__ __forceinline__ uint4 to_bf16x8<kFmtBF16>(uint4 r) { return r; }

// OCP e4m3fn -> bf16 with the gfx950 conversion (scale 1): exact for every
// non-NaN code, two codes per instruction.
template <> __device__ __forceinline__ uint4 to_bf16x8<kFmtFP8>(uint2 r) {
  auto lo = [](uint32_t src) {  // codes in bytes 0, 1
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(src), 1.0f, false));
  };
  auto hi = [](uint32_t src) {  // codes in bytes 2, 3
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(src), 1.0f, true));
  };
  return make_uint4(lo(r.x), hi(r.x), lo(r.y), hi(r.y));
}

template <> __device__ __forceinline__ uint4 to_bf16x8<kFmtINT8>(uint2 r) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t src = (i < 2) ? r.x : r.y;
    const int sh = (i & 1) * 16;
    const float a = static_cast<float>(static_cast<int8_t>(src >> sh));
    const float b = static_cast<float>(static_cast<int8_t>(src >> (sh + 8)));
    w[i] = pack_bf16_exact(a, b);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <> __device__ __forceinline__ uint4 to_bf16x8<kFmtINT4>(uint32_t r) {
  // byte i holds channel 2i (low nibble) and 2i+1 (high nibble), code =
  // nibble - 8, which is the nibble with its top bit flipped read as a
  // 4-bit two's-complement number
  const uint32_t x = r ^ 0x88888888u;
  auto nib = [&](int k) {  // signed 4-bit field k of x
    return static_cast<float>(static_cast<int32_t>(x << (28 - 4 * k)) >> 28);
  };
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16_exact(nib(2 * i), nib(2 * i + 1));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// int8 codes as exact bf16 in the channel order 0, 2, 4, 6, 1, 3, 5, 7 of
// int4_offset_bf16x8 (the ring rows of a tiered pool share the LDS tiles
// with its int4 rows)
__device__ __forceinline__ uint4 int8_bf16x8_permuted(uint2 r) {
  auto code = [](uint32_t src, int byte) { return static_cast<float>(static_cast<int8_t>(src >> (8 * byte))); };
  return make_uint4(pack_bf16_exact(code(r.x, 0), code(r.x, 2)), pack_bf16_exact(code(r.y, 0), code(r.y, 2)),
                    pack_bf16_exact(code(r.x, 1), code(r.x, 3)), pack_bf16_exact(code(r.y, 1), code(r.y, 3)));
}

// int4 codes of 8-wave workgroups: nibble n = code + 8
// becomes the top four of the seven mantissa bits of a bf16 whose exponent
// is 3 (bits 0x4100 | n << 3), the exact value 8 + n / 2 = 12 + code / 2.
// Eight codes cost two shift-and-masks and four byte permutes, and come out
// in the order 0, 2, 4, 6, 1, 3, 5, 7 of their channels.  The kernel stores
// Q's channels in the same order, stages the scales of such rows doubled
// (exact), and takes the offset out with the group sums of Q (QK) and of the
// scaled weights (PV).
__device__ __forceinline__ uint4 int4_offset_bf16x8(uint32_t r) {
  const uint32_t ev = (r << 3) & 0x78787878u;  // byte i: nibble 2i << 3
  const uint32_t od = (r >> 1) & 0x78787878u;  // byte i: nibble 2i+1 << 3
  constexpr uint32_t kHi = 0x41414141u;        // sign and exponent byte
  return make_uint4(__builtin_amdgcn_perm(kHi, ev, 0x04010400u), __builtin_amdgcn_perm(kHi, ev, 0x04030402u),
                    __builtin_amdgcn_perm(kHi, od, 0x04010400u), __builtin_amdgcn_perm(kHi, od, 0x04030402u));
}

// Q chunk (8 bf16, channels 0..7) in the order of int4_offset_bf16x8
__device__ __forceinline__ uint4 int4_channel_order(uint4 q) {
  return make_uint4(__builtin_amdgcn_perm(q.y, q.x, 0x05040100u), __builtin_amdgcn_perm(q.w, q.z, 0x05040100u),
                    __builtin_amdgcn_perm(q.y, q.x, 0x07060302u), __builtin_amdgcn_perm(q.w, q.z, 0x07060302u));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// LDS rows of the V and Q tiles are padded from 512 to 528 bytes: the
// 16-byte row-wise writes of 8 consecutive rows then fall into 8 different
// bank groups, and every LDS address stays base + immediate.
constexpr int kLdsRow = kHeadDim * 2 + 16;

// Rows of the merge's accumulator table are padded from 256 to 260 floats:
// the 16 lanes of a 16-byte write then cover 16 different 4-bank groups
// (unpadded, rows 1 KB apart put all 16 into the same banks)
constexpr int kAccRow = kHeadDim + 4;

// Maximum of x over the four 16-lane groups of the wave (lanes l, l ^ 16,
// l ^ 32, l ^ 48), with the gfx950 row-swap permutes instead of LDS
// permutes: with both operands x, v_permlane16_swap returns rows (0,0,2,2)
// and (1,1,3,3) of x, and v_permlane32_swap halves (0,0) and (1,1).
__device__ __forceinline__ float max_over_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float m16 = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const uint32_t v = __float_as_uint(m16);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS layout for a workgroup of W waves.  During the loop each wave owns a
// K tile and a V tile [16][528 B] (dequantized to bf16) plus their scale
// rows, and all waves share Q [16][528 B]; afterwards each of waves 0..3
// puts its state (m[16], l[16], acc[12][260]) into its own loop area, and
// the split merge's per-wave weight tables [4][64][16] reuse the start of
// the buffer.  A workgroup of 8 waves first folds waves 4..7 into 0..3
// through [4][16 f32x4][64 lanes].
template <int W, bool FLAGS> struct Lds {
  static constexpr int kTileB = kTile * kLdsRow;               // one bf16 tile [16][528 B]
  static constexpr int kScaleFloats = kTile * 8;               // up to 8 groups per row
  static constexpr int kFlagFloats = FLAGS ? kTile : 0;        // tiered: 1 for an int4 row
  static constexpr int kWave = 2 * kTileB + (2 * kScaleFloats + kFlagFloats) * 4;
  static constexpr int kLoop = W * kWave;
  static constexpr int kQ = 16 * kLdsRow;
  static_assert(4 * 64 * 16 * 4 <= kLoop, "split-merge weight tables exceed the loop area");
  static constexpr int kFold = (W > 4) ? 4 * (16 * 64 * 16 + 2 * 64 * 4) : 0;
  static constexpr int kBytes = (kLoop + kQ) > kFold ? (kLoop + kQ) : kFold;
};

// Phase stamp k of this workgroup (the measurement build only; see
// kStampSlots).  s_memrealtime reads the constant 100 MHz clock; the stamp
// is written with a vector store.
__device__ __forceinline__ void phase_stamp(const Params &p, int tid, int k) {
#ifdef QSA_PHASE_STAMPS
  if (tid == 0 && p.stamps != nullptr)
    p.stamps[static_cast<int64_t>(blockIdx.x) * kStampSlots + k] = __builtin_amdgcn_s_memrealtime();
#else
  (void)p, (void)tid, (void)k;
#endif
}

__device__ void write_nan_rows(const Params &p, int b, int g, int tid, int nthreads) {
  const __bf16 nan = __builtin_bit_cast(__bf16, static_cast<uint16_t>(0x7FC0u));
  for (int i = tid; i < kGqa * kHeadDim; i += nthreads)
    p.out[b * p.o_sb + (g * kGqa + i / kHeadDim) * p.o_sh + (i % kHeadDim)] = nan;
  if (tid < kGqa) p.lse[b * p.l_sb + (g * kGqa + tid) * p.l_sh] = __builtin_nanf("");
}

// The values the first loads depend on (the cu_seqlens and slot-id arrays,
// the sizes that map a workgroup to its row) come as leading scalar
// arguments, which the build asks the dispatcher to preload into scalar
// registers at wave launch: the cu_seqlens -> slot ids chain then starts
// at once, while the rest of the argument block is still being fetched.
template <int FMT, int G, int W, bool SF16, bool A32>
__global__ void __launch_bounds__(64 * W, 8 / W)
    qsa_decode_kernel(const int32_t *__restrict__ cu_lead, const int32_t *__restrict__ sel_lead, int bs_lead,
                      int hkv_lead, int nsplit_lead, int msk_lead, int nsel_lead, int xcc_lead,
                      const Params p) {
  using Part = typename Fmt<FMT>::Part;
  using GEO = Geo<FMT>;
  constexpr bool TIER = FMT == kFmtTIERED;
  // int4 codes (of int4 pools and of the int4 rows of tiered pools) staged
  // as 12 + code / 2 in permuted channel order (int4_offset_bf16x8) by
  // 8-wave workgroups; the 4-wave instances, which keep more tiles in
  // flight, have no registers left for the offsets
  constexpr bool I4OFF = (FMT == kFmtINT4 || TIER) && W > 4;
  using LDS = Lds<W, I4OFF && TIER>;
  using Scale = typename std::conditional<SF16, _Float16, float>::type;
  static_assert(!TIER || (G == 32 && SF16), "tiered pools: f16 scales staged per 32 channels");
  static_assert(!I4OFF || (G >= 32 && G < kHeadDim), "int4 rows: 2 to 8 channel groups");
  constexpr int kThr = 64 * W;
  constexpr int NG = (FMT == kFmtBF16) ? 0 : kHeadDim / G;   // scale groups per row
  constexpr int NI = GEO::kNI;
  // tiles in flight: with 4-wave workgroups as many as fit the register
  // budget of one bf16 tile (8 row loads per lane for K and for V), so
  // narrower formats keep as many bytes in flight per wave as bf16 does;
  // 8-wave workgroups (two waves per SIMD) and tiered pools keep one (more
  // was slower for every format: the second wave covers the wait, and a
  // tiered pool's owner ids and tier selects take the registers)
  constexpr int D = (TIER || W > 4) ? 1 : 8 / NI;
  // wave priorities, which order two waves of a SIMD (8-wave workgroups, or
  // two 4-wave workgroups on a CU); see the loop
  constexpr bool kPrioStage = TIER;
  constexpr bool kPrioProcess = FMT == kFmtINT4 && !TIER;

  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS::kBytes];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave loop bounds scalar
  const int r16 = lane & 15;  // MFMA row / head
  const int qg = lane >> 4;   // lane group 0..3
  const int ldrow = (lane / GEO::kLPR) * NI;  // first tile row this lane loads
  const int lchunk = lane % GEO::kLPR;       // its 16-byte chunk of each row

  // ---- workgroup -> (row b, KV head g, split); the splits of a pair
  // share blockIdx % 8 (the XCD), and with quantized pools so do all KV
  // heads of a row; with xcc_lead a bf16 workgroup takes slot x of its
  // group of 8 pairs from the XCD it runs on (decode_workgroups)
  const int wg = blockIdx.x;
  const int local = wg >> 3;
  const int pp = local / nsplit_lead;
  const int split = local - pp * nsplit_lead;
  int b, g;
  if constexpr (rows_share_xcd(FMT)) {
    const int rb = (hkv_lead == 2) ? (pp >> 1) : pp;
    g = pp - rb * hkv_lead;
    b = rb * 8 + (wg & 7);
    if (b >= bs_lead) return;
  } else {
    const int x = xcc_lead ? (__builtin_amdgcn_s_getreg(kHwRegXccId) & 7) : (wg & 7);
    const int pair8 = pp * 8 + x;
    if (pair8 >= bs_lead * hkv_lead) return;
    b = (hkv_lead == 2) ? (pair8 >> 1) : pair8;
    g = pair8 - b * hkv_lead;
  }
  const int pair = b * hkv_lead + g;
  phase_stamp(p, tid, 0);

  // ---- live row length from device cu_seqlens
  const int c0 = cu_lead[b];
  const int c1 = cu_lead[b + 1];
  const int L = c1 - c0;
  if (c0 < 0 || L < 0 || L > kMaxSel || c1 > nsel_lead) {
    if (split == 0) {
      write_nan_rows(p, b, g, tid, kThr);
      if (tid == 0) atomicOr(p.err, kErrRowRange);
    }
    return;
  }
  int n_active = (L + msk_lead - 1) / msk_lead;
  n_active = n_active < 1 ? 1 : (n_active > nsplit_lead ? nsplit_lead : n_active);
  if (split >= n_active) return;
  phase_stamp(p, tid, 1);

  // ---- this wave's contiguous slice of the list
  const int nw = n_active * W;
  const int wi = split * W + wave;
  const int k0 = (L * wi) / nw;
  const int nkeys = (L * (wi + 1)) / nw - k0;
  const int ntile = (nkeys + kTile - 1) / kTile;

  unsigned char *qlds = smem + LDS::kLoop;
  unsigned char *wlds = smem + wave * LDS::kWave;
  unsigned char *kt = wlds;                                          // [16][528 B]
  unsigned char *vt = wlds + LDS::kTileB;                            // [16][528 B]
  float *ksc = reinterpret_cast<float *>(wlds + 2 * LDS::kTileB);    // [16][NG]
  float *vsc = ksc + LDS::kScaleFloats;                              // [16][NG]
  float *i4row = vsc + LDS::kScaleFloats;                            // tiered: [16] 1 = int4 row

  // Row addresses.  With A32 (every pool byte within 4 GiB of the pool
  // start, slot ids and strides below 2^24) a row's address is a
  // workgroup-uniform base plus one 24-bit multiply-add per lane (a 32-bit
  // offset the load adds to a scalar base); otherwise 64-bit arithmetic.
  const uint8_t *kpool = p.k + g * p.k_sh;
  const uint8_t *vpool = p.v + g * p.v_sh;
  const uint8_t *kbase = kpool + 16 * lchunk;
  const uint8_t *vbase = vpool + 16 * lchunk;
  const uint32_t k_ss32 = static_cast<uint32_t>(p.k_ss), v_ss32 = static_cast<uint32_t>(p.v_ss);
  const uint32_t lane16 = 16u * static_cast<uint32_t>(lchunk);
  // every lane loads a scale (lanes past the row's NG groups re-read group
  // 0, so no load is conditional); only lanes lchunk < NG store them
  const int sgrp = (NG > 0 && lchunk < NG) ? lchunk : 0;
  const uint8_t *kspool = (NG > 0) ? p.ks + g * p.ks_sh : nullptr;
  const uint8_t *vspool = (NG > 0) ? p.vs + g * p.vs_sh : nullptr;
  const uint8_t *ksbase = (NG > 0) ? kspool + sgrp * sizeof(Scale) : nullptr;
  const uint8_t *vsbase = (NG > 0) ? vspool + sgrp * sizeof(Scale) : nullptr;
  const uint32_t ks_ss32 = static_cast<uint32_t>(p.ks_ss), vs_ss32 = static_cast<uint32_t>(p.vs_ss);
  const uint32_t sgrpb = static_cast<uint32_t>(sgrp * sizeof(Scale));
  const int32_t *selw = sel_lead + c0 + k0;
  const uint32_t slots = static_cast<uint32_t>(p.slots > 0x7FFFFFFF ? 0x7FFFFFFF : p.slots);
  // tiered: ring rows of KV head g; a cold lane reads the 16 bytes at
  // 16 * (lchunk / 2) of the int4 row and a hot lane 16 * lchunk of the ring
  // row; scale group sgrp of a cold row is group sgrp / 2 of a ring row
  const uint8_t *rkbase = TIER ? p.ring.k + g * p.ring.k_sh + 16 * lchunk : nullptr;
  const uint8_t *rvbase = TIER ? p.ring.v + g * p.ring.v_sh + 16 * lchunk : nullptr;
  const uint8_t *ckbase = TIER ? kpool + 16 * (lchunk >> 1) : nullptr;
  const uint8_t *cvbase = TIER ? vpool + 16 * (lchunk >> 1) : nullptr;
  const uint8_t *rksbase = TIER ? p.ring.ks + g * p.ring.ks_sh + (sgrp >> 1) * 2 : nullptr;
  const uint8_t *rvsbase = TIER ? p.ring.vs + g * p.ring.vs_sh + (sgrp >> 1) * 2 : nullptr;
  const uint32_t rmask = TIER ? p.ring.mask : 0u;
  // tiered with A32: one uniform base per array; a row's address is that
  // base plus a 32-bit offset, d*r (ring) or d*c (int4 pool) plus a 24-bit
  // product, the tier chosen per lane by a select on the offset
  auto delta = [](const uint8_t *p0, const uint8_t *base) {
    return static_cast<uint32_t>(static_cast<uint64_t>(p0 - base));
  };
  constexpr bool T32 = TIER && A32;
  const uint32_t dkr = T32 ? delta(rkbase, p.ring.kb) : 0u, dkc = T32 ? delta(ckbase, p.ring.kb) : 0u;
  const uint32_t dvr = T32 ? delta(rvbase, p.ring.vb) : 0u, dvc = T32 ? delta(cvbase, p.ring.vb) : 0u;
  const uint32_t dksr = T32 ? delta(rksbase, p.ring.ksb) : 0u, dksc = T32 ? delta(ksbase, p.ring.ksb) : 0u;
  const uint32_t dvsr = T32 ? delta(rvsbase, p.ring.vsb) : 0u, dvsc = T32 ? delta(vsbase, p.ring.vsb) : 0u;
  const uint32_t rk_ss32 = static_cast<uint32_t>(p.ring.k_ss), rv_ss32 = static_cast<uint32_t>(p.ring.v_ss);
  const uint32_t rks_ss32 = static_cast<uint32_t>(p.ring.ks_ss), rvs_ss32 = static_cast<uint32_t>(p.ring.vs_ss);

  // per-lane online-softmax state for head r16 (replicated over lane groups)
  float m_run = -INFINITY;
  float l_run = 0.0f;  // partial sum over this lane's 4 entries per tile
  f32x4 acc[16];
#pragma unroll
  for (int mt = 0; mt < 16; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool bad_slot = false;

  // LDS row layout of the K and V tiles.  A lane stages P = kParts chunks
  // of 8 channels (16 B of bf16) per row, chunk c of lane l being channel
  // chunk m = P*l + c.  Chunk m is stored at byte (m % P) * kPartB +
  // (m / P) * 16, so the lanes of one 16-byte LDS write are 16 B apart (no
  // bank conflicts); for bf16 (P = 1) this is the plain row.  With P = 2
  // the second part starts 16 B past mid-row, so that the column reads of
  // the V operand (channels c and c + 8 in one instruction) fall into
  // different banks; the row still fits the 528-byte pitch.
  constexpr int P = GEO::kParts;
  constexpr int kPartB = (P == 2) ? 512 / P + 16 : 512 / P;
  static_assert((P - 1) * kPartB + 512 / P <= kLdsRow, "parts exceed the LDS row pitch");
  // Transposed V operand: lane (r16, qg) needs V[4*qg + e][16*mt + r16],
  // e = 0..3.  ds_read_b64_tr_b16 gives lane i of a 16-lane group element
  // i % 4 of the 8 bytes read by lane 4*e + i / 4 of the group, so lane
  // r16 of group qg reads channels 16*mt + 4*(r16 & 3) .. + 3 of entry
  // 4*qg + (r16 >> 2): chunk 2*mt + ((r16 >> 1) & 1), byte 8*(r16 & 1) in
  // the chunk -- a lane base plus the per-mt constant
  // (2*mt % P) * kPartB + (2*mt / P) * 16.
  const int vhalf = (r16 >> 1) & 1;
  const unsigned char *vtr = vt + (4 * qg + (r16 >> 2)) * kLdsRow + (vhalf % P) * kPartB +
                             (vhalf / P) * 16 + 8 * (r16 & 1);

  // The K / V rows (and scales) of the next D tiles are in flight in D
  // register sets; set u is emptied into the LDS tiles at the start of step
  // t = u (mod D) and refilled with tile t + D.
  uint4 kraw[D][NI], vraw[D][NI];
  Scale ksr[D][NI], vsr[D][NI];  // converted to fp32 when staged
  bool hot[D][NI];               // tiered: the row came from the ring

  // Every load of the pipeline is unconditional and its value is used as
  // loaded, so the compiler's load counting never has to assume a skipped
  // load (or wait early for a value it post-processes) and wait for every
  // load in flight: tiles past the end re-read the last entry (cache hits),
  // and a wave with no entries reads cu[0] as its "slot id" (checked below
  // without raising the error bit; its rows are never processed).
  const int32_t *ids = (nkeys > 0) ? selw : cu_lead;
  const int jmax = (nkeys > 0) ? nkeys - 1 : 0;
  auto fetch_slots = [&](int t, int32_t (&sl)[NI]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = kTile * t + ldrow + i;
      sl[i] = ids[j < jmax ? j : jmax];
    }
  };
  auto checked = [&](int32_t s) -> uint32_t {
    const bool bad = static_cast<uint32_t>(s) >= slots;
    bad_slot = bad_slot || (bad && nkeys > 0);
    return bad ? 0u : static_cast<uint32_t>(s);
  };
  // tiered: owner ids of the ring rows the slot ids map to (always in range)
  auto fetch_owners = [&](const int32_t (&sl)[NI], int32_t (&ow)[NI]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) ow[i] = p.ring.owner[static_cast<uint32_t>(sl[i]) & rmask];
  };
  auto issue_tiered = [&](int u, const int32_t (&sl)[NI], const int32_t (&ow)[NI]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t cs = checked(sl[i]);
      const uint32_t r = static_cast<uint32_t>(sl[i]) & rmask;
      const bool h = ow[i] == sl[i];
      hot[u][i] = h;
      if constexpr (A32) {
        auto at = [&](const uint8_t *base, uint32_t ro, uint32_t co) {
          return base + static_cast<uint64_t>(h ? ro : co);
        };
        kraw[u][i] = *reinterpret_cast<const uint4 *>(
            at(p.ring.kb, __umul24(r, rk_ss32) + dkr, __umul24(cs, k_ss32) + dkc));
        vraw[u][i] = *reinterpret_cast<const uint4 *>(
            at(p.ring.vb, __umul24(r, rv_ss32) + dvr, __umul24(cs, v_ss32) + dvc));
        ksr[u][i] = *reinterpret_cast<const Scale *>(
            at(p.ring.ksb, __umul24(r, rks_ss32) + dksr, __umul24(cs, ks_ss32) + dksc));
        vsr[u][i] = *reinterpret_cast<const Scale *>(
            at(p.ring.vsb, __umul24(r, rvs_ss32) + dvsr, __umul24(cs, vs_ss32) + dvsc));
      } else {
        const int64_t ro = static_cast<int64_t>(r), co = static_cast<int64_t>(cs);
        kraw[u][i] = *reinterpret_cast<const uint4 *>(h ? rkbase + ro * p.ring.k_ss : ckbase + co * p.k_ss);
        vraw[u][i] = *reinterpret_cast<const uint4 *>(h ? rvbase + ro * p.ring.v_ss : cvbase + co * p.v_ss);
        ksr[u][i] = *reinterpret_cast<const Scale *>(h ? rksbase + ro * p.ring.ks_ss : ksbase + co * p.ks_ss);
        vsr[u][i] = *reinterpret_cast<const Scale *>(h ? rvsbase + ro * p.ring.vs_ss : vsbase + co * p.vs_ss);
      }
    }
  };
  auto issue = [&](int u, const int32_t (&sl)[NI]) {
    uint32_t slot[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) slot[i] = checked(sl[i]);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      kraw[u][i] = A32 ? *reinterpret_cast<const uint4 *>(kpool + static_cast<uint64_t>(__umul24(slot[i], k_ss32) + lane16))
                       : *reinterpret_cast<const uint4 *>(kbase + static_cast<int64_t>(slot[i]) * p.k_ss);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      vraw[u][i] = A32 ? *reinterpret_cast<const uint4 *>(vpool + static_cast<uint64_t>(__umul24(slot[i], v_ss32) + lane16))
                       : *reinterpret_cast<const uint4 *>(vbase + static_cast<int64_t>(slot[i]) * p.v_ss);
    if constexpr (NG > 0) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        ksr[u][i] = A32 ? *reinterpret_cast<const Scale *>(kspool + static_cast<uint64_t>(__umul24(slot[i], ks_ss32) + sgrpb))
                        : *reinterpret_cast<const Scale *>(ksbase + static_cast<int64_t>(slot[i]) * p.ks_ss);
        vsr[u][i] = A32 ? *reinterpret_cast<const Scale *>(vspool + static_cast<uint64_t>(__umul24(slot[i], vs_ss32) + sgrpb))
                        : *reinterpret_cast<const Scale *>(vsbase + static_cast<int64_t>(slot[i]) * p.vs_ss);
      }
    }
  };

  // ---- prologue: the slot ids of tiles 0..2D-1 and Q are in flight
  // together, then the rows of tiles 0..D-1; Q of the 12 heads of KV head g
  // goes to LDS [16 heads][528 B] (heads 12..15 zero), where each QK MFMA
  // reads its B operand.  snext[u] holds the slot ids of the tile that
  // register set u loads next.
  int32_t snext[D][NI];
  int32_t onext[D][NI], s2[D][NI];  // tiered: owner ids of snext; slot ids one tile set further
  {
    int32_t s0[D][NI], o0[D][NI];
#pragma unroll
    for (int u = 0; u < D; ++u) fetch_slots(u, s0[u]);
#pragma unroll
    for (int u = 0; u < D; ++u) fetch_slots(D + u, snext[u]);
    if constexpr (TIER) {
#pragma unroll
      for (int u = 0; u < D; ++u) fetch_slots(2 * D + u, s2[u]);
#pragma unroll
      for (int u = 0; u < D; ++u) fetch_owners(s0[u], o0[u]);
#pragma unroll
      for (int u = 0; u < D; ++u) fetch_owners(snext[u], onext[u]);
    }
    constexpr int CPT = 512 / kThr;  // 16-byte Q chunks per thread
    uint4 qv[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid * CPT + i;
      const int h = idx >> 5, c = idx & 31;
      qv[i] = make_uint4(0, 0, 0, 0);
      if (h < kGqa)
        qv[i] = reinterpret_cast<const uint4 *>(p.q + b * p.q_sb + (g * kGqa + h) * p.q_sh)[c];
    }
#pragma unroll
    for (int u = 0; u < D; ++u) {
      if constexpr (TIER)
        issue_tiered(u, s0[u], o0[u]);
      else
        issue(u, s0[u]);
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid * CPT + i;
      *reinterpret_cast<uint4 *>(qlds + (idx >> 5) * kLdsRow + (idx & 31) * 16) =
          I4OFF ? int4_channel_order(qv[i]) : qv[i];
    }
  }
  __syncthreads();
  // Q's B operands do not change over the loop: instances with register
  // room keep all 8 in registers (32 VGPRs), which takes 8 KB of LDS reads
  // off every tile -- those without per-group K scales, and every 8-wave
  // instance (one tile in flight per wave leaves the room); the 4-wave
  // group-scale and tiered instances re-read them from LDS
  constexpr bool QREG = (NG <= 1 && !TIER) || W > 4;
  bf16x8 qreg[QREG ? 8 : 1];
  if constexpr (QREG) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qreg[kk] = as_bf16x8(*reinterpret_cast<const uint4 *>(qlds + r16 * kLdsRow + (4 * kk + qg) * 16));
  }
  auto qfrag = [&](int kk) -> bf16x8 {
    if constexpr (QREG) return qreg[kk];
    return as_bf16x8(*reinterpret_cast<const uint4 *>(qlds + r16 * kLdsRow + (4 * kk + qg) * 16));
  };
  // int4 rows: 12 x the sum of head r16's Q over each channel group (the QK
  // offset of int4_offset_bf16x8); chunk 4*kk + qg of this lane lies in
  // group 32*kk / G, and the four lane groups hold the other chunks
  float qoff[I4OFF ? NG : 1];
  if constexpr (I4OFF) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) qoff[gi] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8 f = qfrag(kk);
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += static_cast<float>(f[i]);
      qoff[32 * kk / G] += sum;
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      qoff[gi] += __shfl_xor(qoff[gi], 16);
      qoff[gi] += __shfl_xor(qoff[gi], 32);
      qoff[gi] *= 12.0f;
    }
  }
  // int4 rows: running sum over this lane's int4 entries of the weights
  // times the (doubled) V scale of each channel group (the PV offset),
  // rescaled with the accumulators
  float voff[I4OFF ? NG : 1];
#pragma unroll
  for (int gi = 0; gi < (I4OFF ? NG : 1); ++gi) voff[gi] = 0.0f;
  // K operand: channel chunk 4*kk + qg of row r16
  const unsigned char *krow = kt + r16 * kLdsRow + (qg % P) * kPartB + (qg / P) * 16;
  auto kfrag = [&](int kk) -> bf16x8 {
    return as_bf16x8(*reinterpret_cast<const uint4 *>(krow + (4 * kk / P) * 16));
  };

  // 1. register set u (one tile's K and V rows, dequantized to bf16, and
  // their scale rows) into the wave's LDS tiles
  auto stage = [&](int u) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int off = (ldrow + i) * kLdsRow + lchunk * 16;
      if constexpr (TIER) {
        uint4 k0, k1, v0, v1;
        auto ring8 = [](uint32_t a, uint32_t b) {
          if constexpr (I4OFF) return int8_bf16x8_permuted(make_uint2(a, b));
          return to_bf16x8<kFmtINT8>(make_uint2(a, b));
        };
        auto pool4 = [](uint32_t a) {
          if constexpr (I4OFF) return int4_offset_bf16x8(a);
          return to_bf16x8<kFmtINT4>(a);
        };
        if (hot[u][i]) {
          k0 = ring8(kraw[u][i].x, kraw[u][i].y);
          k1 = ring8(kraw[u][i].z, kraw[u][i].w);
          v0 = ring8(vraw[u][i].x, vraw[u][i].y);
          v1 = ring8(vraw[u][i].z, vraw[u][i].w);
        } else {
          const bool odd = lchunk & 1;
          k0 = pool4(odd ? kraw[u][i].z : kraw[u][i].x);
          k1 = pool4(odd ? kraw[u][i].w : kraw[u][i].y);
          v0 = pool4(odd ? vraw[u][i].z : vraw[u][i].x);
          v1 = pool4(odd ? vraw[u][i].w : vraw[u][i].y);
        }
        *reinterpret_cast<uint4 *>(kt + off) = k0;
        *reinterpret_cast<uint4 *>(kt + off + kPartB) = k1;
        *reinterpret_cast<uint4 *>(vt + off) = v0;
        *reinterpret_cast<uint4 *>(vt + off + kPartB) = v1;
      } else {
#pragma unroll
        for (int c = 0; c < P; ++c) {
          const Part kp = reinterpret_cast<const Part *>(&kraw[u][i])[c];
          const Part vp = reinterpret_cast<const Part *>(&vraw[u][i])[c];
          if constexpr (I4OFF) {
            *reinterpret_cast<uint4 *>(kt + off + c * kPartB) = int4_offset_bf16x8(kp);
            *reinterpret_cast<uint4 *>(vt + off + c * kPartB) = int4_offset_bf16x8(vp);
          } else {
            *reinterpret_cast<uint4 *>(kt + off + c * kPartB) = to_bf16x8<FMT>(kp);
            *reinterpret_cast<uint4 *>(vt + off + c * kPartB) = to_bf16x8<FMT>(vp);
          }
        }
      }
    }
    if constexpr (NG > 0) {
      if (lchunk < NG) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          float ks = static_cast<float>(ksr[u][i]), vs = static_cast<float>(vsr[u][i]);
          if constexpr (I4OFF) {  // rows staged as 12 + code / 2: scales doubled
            const float f = (TIER && hot[u][i]) ? 1.0f : 2.0f;
            ks *= f;
            vs *= f;
          }
          ksc[(ldrow + i) * NG + lchunk] = ks;
          vsc[(ldrow + i) * NG + lchunk] = vs;
        }
      }
      if constexpr (I4OFF && TIER) {
        if (lchunk == 0) {
#pragma unroll
          for (int i = 0; i < NI; ++i) i4row[ldrow + i] = hot[u][i] ? 0.0f : 1.0f;
        }
      }
    }
  };

  auto process = [&](int t) {
    // 2. S^T = K . Q^T  (lane: head r16, entries 4*qg + e)
    wave_lds_fence();
    f32x4 s;
    if constexpr (NG <= 1) {
      // two accumulation chains of 4 products (even and odd channel
      // blocks) instead of one of 8, added at the end
      f32x4 s_even = f32x4{0.f, 0.f, 0.f, 0.f}, s_odd = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 8; kk += 2) {
        s_even = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag(kk), qfrag(kk), s_even, 0, 0, 0);
        s_odd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag(kk + 1), qfrag(kk + 1), s_odd, 0, 0, 0);
      }
      s = s_even + s_odd;
    }
    // tiered: which of this lane's entries are int4 rows
    f32x4 i4f = f32x4{1.f, 1.f, 1.f, 1.f};
    if constexpr (I4OFF && TIER) i4f = *reinterpret_cast<const f32x4 *>(i4row + 4 * qg);
    if constexpr (NG == 1) {
      const f32x4 k4 = *reinterpret_cast<const f32x4 *>(ksc + 4 * qg);
      s *= k4;
    } else if constexpr (NG > 1) {
      constexpr int KPG = G / 32;  // QK MFMAs per scale group
      s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < KPG; ++u) {
          const int kk = gi * KPG + u;
          part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag(kk), qfrag(kk), part, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float t = part[e];
          if constexpr (I4OFF) t = TIER ? fmaf(-i4f[e], qoff[gi], t) : t - qoff[gi];
          s[e] += ksc[(4 * qg + e) * NG + gi] * t;
        }
      }
    }

    // 3. online softmax in log2 units
    const int jbase = kTile * t + 4 * qg;
    float s2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) s2[e] = (jbase + e < nkeys) ? s[e] * kScaleLog2 : -INFINITY;
    const float mx = max_over_groups(fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3])));
    // The running max moves only when some head's tile max exceeds it by
    // more than kLazyLog2; then every head takes its new max and the state
    // is rescaled once.  Otherwise the weights are taken against the older
    // max and may reach 2^kLazyLog2, which the fp32 sums and the hi + lo
    // split of P carry at the same relative precision.  After the first
    // tiles almost no tile rescales.
    if (__any(mx > m_run + kLazyLog2)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) acc[mt] *= alpha;
      if constexpr (I4OFF) {
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) voff[gi] *= alpha;
      }
    }
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = __builtin_amdgcn_exp2f(s2[e] - m_run);
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);

    // 4. O^T += V^T . P^T with P as hi + lo bf16
    auto split_p = [&](const float (&pv)[4], i16x4 &hi, i16x4 &lo) {
      const uint32_t h01 = bf16x2_rne(pv[0], pv[1]);
      const uint32_t h23 = bf16x2_rne(pv[2], pv[3]);
      const uint32_t l01 = bf16x2_rne(pv[0] - __uint_as_float(h01 << 16), pv[1] - __uint_as_float(h01 & 0xFFFF0000u));
      const uint32_t l23 = bf16x2_rne(pv[2] - __uint_as_float(h23 << 16), pv[3] - __uint_as_float(h23 & 0xFFFF0000u));
      hi = __builtin_bit_cast(i16x4, make_uint2(h01, h23));
      lo = __builtin_bit_cast(i16x4, make_uint2(l01, l23));
    };
    // One 16x16x32 product per channel block: in lane group qg the eight
    // k-slots hold entries 4*qg .. 4*qg+3 twice, with the V values
    // duplicated in A and P's hi parts then lo parts in B, so the product
    // adds V^T . P_hi + V^T . P_lo.
    auto pv_mfma = [&](int mt, const i16x4 &hi, const i16x4 &lo) {
      const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4 *)(vtr + (2 * mt % P) * kPartB + (2 * mt / P) * 16));
      const i16x8 a2 = __builtin_shufflevector(a, a, 0, 1, 2, 3, 0, 1, 2, 3);
      const i16x8 b2 = __builtin_shufflevector(hi, lo, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a2),
                                                        __builtin_bit_cast(bf16x8, b2), acc[mt], 0, 0, 0);
    };
    if constexpr (NG <= 1) {
      float pv[4];
      if constexpr (NG == 1) {
        const f32x4 v4 = *reinterpret_cast<const f32x4 *>(vsc + 4 * qg);
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = pr[e] * v4[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = pr[e];
      }
      i16x4 hi, lo;
      split_p(pv, hi, lo);
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) pv_mfma(mt, hi, lo);
    } else {
      constexpr int MPG = G / 16;  // PV MFMAs per scale group
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = pr[e] * vsc[(4 * qg + e) * NG + gi];
        if constexpr (I4OFF) {
          if constexpr (TIER)
            voff[gi] += (i4f[0] * pv[0] + i4f[1] * pv[1]) + (i4f[2] * pv[2] + i4f[3] * pv[3]);
          else
            voff[gi] += (pv[0] + pv[1]) + (pv[2] + pv[3]);
        }
        i16x4 hi, lo;
        split_p(pv, hi, lo);
#pragma unroll
        for (int u = 0; u < MPG; ++u) pv_mfma(gi * MPG + u, hi, lo);
      }
    }
    wave_lds_fence();  // reads of this tile finish before the next tile's writes
  };

  // ---- software pipeline: the rows of tiles t+1 .. t+D are in flight
  // while tile t is processed.  Step t (u = t mod D): K/V(t) -> LDS, issue
  // K/V(t+D) into the freed register set u, fetch the slot ids of t+2D into
  // snext[u], then QK / softmax / PV of tile t.  Slot ids are fetched D
  // steps before their rows are issued, so that waiting for them (loads
  // complete in issue order) never waits for rows still in flight.
  // The loop runs whole groups of D steps; a step past the last tile stages
  // and loads (the clamped rows) but skips the processing, so no load sits
  // behind a branch and the compiler's load counting never has to assume a
  // skipped load and wait for every load in flight.  The last group is
  // peeled off the loop and issues no loads.
  int t0 = 0;
  for (; t0 + D < ntile; t0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int t = t0 + u;
      // tiered pools, two waves on a SIMD: the wave that converts its rows
      // and issues the next loads goes first.  Its row
      // loads end a chain of dependent loads (slot ids, then owner ids, then
      // rows), and this lets the chain advance before the other wave's
      // products; the tile's own products then yield.
      if constexpr (kPrioStage) __builtin_amdgcn_s_setprio(2);
      stage(u);
      if (t == 0) phase_stamp(p, tid, 2);
      if constexpr (TIER) {
        // owner ids of tile t+2D from its slot ids fetched D steps ago; the
        // same slot ids are fetched again (cache hits) for the row issue D
        // steps later, so no loaded register is copied
        issue_tiered(u, snext[u], onext[u]);
        fetch_owners(s2[u], onext[u]);
        fetch_slots(t + 2 * D, snext[u]);
        fetch_slots(t + 3 * D, s2[u]);
      } else {
        issue(u, snext[u]);
        fetch_slots(t + 2 * D, snext[u]);
      }
      if constexpr (kPrioStage) __builtin_amdgcn_s_setprio(0);
      // int4 pools, two waves on a SIMD: a tile's products go first.  Their
      // chain of dependent steps (QK products, group scales, softmax, P
      // splits, PV products) then keeps moving, and the other wave's
      // unpacking, which depends on nothing in flight, fills the gaps.
      if constexpr (kPrioProcess) __builtin_amdgcn_s_setprio(1);
      if (t < ntile) process(t);
      if constexpr (kPrioProcess) __builtin_amdgcn_s_setprio(0);
    }
  }
  // the last group: its rows are in flight already and nothing more is
  // loaded, so the epilogue never waits for rows that would not be used
  if (t0 < ntile) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int t = t0 + u;
      if (t < ntile) {
        stage(u);
        if (t == 0) phase_stamp(p, tid, 2);
        process(t);
      }
    }
  }

  phase_stamp(p, tid, 3);

  // ---- int4 rows: the accumulators hold sum_j P'_j (12 + code_j / 2) over
  // them (P' with the doubled V scale) in the permuted channel order; take
  // out the offset (12 x the weight sum of the channel's group over the
  // int4 rows, over all four lane groups), then give every lane channels
  // 16*mt + 4*qg + 0..3 again.  Lane groups 2i and
  // 2i+1 hold one 8-channel chunk between them, the even channels in the
  // first and the odd ones in the second; one row swap per pair of
  // accumulator elements restores the channel order.
  if constexpr (I4OFF) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      voff[gi] += __shfl_xor(voff[gi], 16);
      voff[gi] += __shfl_xor(voff[gi], 32);
      voff[gi] *= 12.0f;
    }
    auto swap_rows = [](float a, float b, float &x, float &y) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
      x = __uint_as_float(r[0]);
      y = __uint_as_float(r[1]);
    };
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
      const float off = voff[16 * mt / G];
      f32x4 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = acc[mt][e] - off;
      float o0, o1, o2, o3;
      swap_rows(a[0], a[2], o0, o1);
      swap_rows(a[1], a[3], o2, o3);
      acc[mt] = f32x4{o0, o1, o2, o3};
    }
  }

  // ---- wave result: full sum per head over the 4 lane groups
  float l_w = l_run + __shfl_xor(l_run, 16);
  l_w += __shfl_xor(l_w, 32);
  if (__any(bad_slot)) {
    l_w = __builtin_nanf("");
    if (lane == 0) atomicOr(p.err, kErrSlot);
  }

  // ---- 8-wave workgroups: fold waves 4..7 into waves 0..3 (same lane
  // layout, so the fold is element-wise per lane)
  if constexpr (W > 4) {
    __syncthreads();
    f32x4 *fold = reinterpret_cast<f32x4 *>(smem);               // [4][16][64]
    float *fold_ml = reinterpret_cast<float *>(smem + 4 * 16 * 64 * 16);  // [4][2][64]
    if (wave >= 4) {
      const int slot = wave - 4;
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) fold[(slot * 16 + mt) * 64 + lane] = acc[mt];
      fold_ml[(slot * 2 + 0) * 64 + lane] = m_run;
      fold_ml[(slot * 2 + 1) * 64 + lane] = l_w;
    }
    __syncthreads();
    if (wave < 4) {
      const float m2 = fold_ml[(wave * 2 + 0) * 64 + lane];
      const float l2 = fold_ml[(wave * 2 + 1) * 64 + lane];
      const float M = fmaxf(m_run, m2);
      const float f1 = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
      const float f2 = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) acc[mt] = acc[mt] * f1 + fold[(wave * 16 + mt) * 64 + lane] * f2;
      l_w = l_w * f1 + l2 * f2;
      m_run = M;
    }
    __syncthreads();
  }

  // ---- merge the (up to) 4 wave states of this workgroup through LDS.
  // Wave w's state (m[16], l[16], acc[12][260]) goes into its own loop
  // area, which no other wave reads, so a wave writes it as soon as its
  // loop is done and one barrier suffices.
  auto wstate = [&](int w) { return reinterpret_cast<float *>(smem + w * LDS::kWave); };
  static_assert((32 + kGqa * kAccRow) * 4 <= LDS::kWave, "a wave state exceeds the wave's loop area");
  if (wave < 4) {
    float *ws = wstate(wave);
    if (qg == 0) {
      ws[r16] = m_run;
      ws[16 + r16] = l_w;
    }
    if (r16 < kGqa) {
#pragma unroll
      for (int mt = 0; mt < 16; ++mt)
        *reinterpret_cast<f32x4 *>(ws + 32 + r16 * kAccRow + 16 * mt + 4 * qg) = acc[mt];
    }
  }
  __syncthreads();

  // From here wave wv < 4 owns heads wv, wv + 4, wv + 8 and lane l owns
  // channels 4l .. 4l + 3 of each; the waves 4..7 of an 8-wave workgroup
  // only take part in the barriers.  Weights are computed redundantly per
  // wave: lane j = 16 w + h holds state w of head h, so the merged max, sum
  // and reciprocal of head h end up in lanes h, h + 16, h + 32, h + 48 and
  // are read out with readlane (no extra barrier).
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int sq = lane >> 4;  // state (wave or split) index within a group of 4
  const int hh = lane & 15;  // head
  auto bcast = [](float x, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), src));
  };
  auto weights4 = [&](float mj, float lj, float &Mj, float &sj) {
    Mj = fmaxf(mj, __shfl_xor(mj, 16));
    Mj = fmaxf(Mj, __shfl_xor(Mj, 32));
    const float fj = (mj == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mj - Mj);
    sj = fj * lj;
    sj += __shfl_xor(sj, 16);
    sj += __shfl_xor(sj, 32);
    return fj;
  };
  auto recip = [](float s) { return (s > 0.f || s != s) ? 1.0f / s : 0.f; };
  auto lse_of = [](float M, float s) { return (s > 0.f || s != s) ? (M + __log2f(s)) * kLn2 : -INFINITY; };
  auto store_out = [&](int h, const f32x4 &o, float inv) {
    uint2 w;
    w.x = bf16x2_rne(o[0] * inv, o[1] * inv);
    w.y = bf16x2_rne(o[2] * inv, o[3] * inv);
    *reinterpret_cast<uint2 *>(p.out + b * p.o_sb + (g * kGqa + h) * p.o_sh + 4 * lane) = w;
  };
  float *lrow = p.lse + b * p.l_sb + (g * kGqa) * p.l_sh;

  float Mw = 0.f, sw = 0.f;
  f32x4 o[3];
  if (wv < 4) {
    const float fj = weights4(wstate(sq)[hh], wstate(sq)[16 + hh], Mw, sw);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int h = 4 * k + wv;
      o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w)
        o[k] += bcast(fj, 16 * w + h) *
                *reinterpret_cast<const f32x4 *>(wstate(w) + 32 + h * kAccRow + 4 * lane);
    }
  }

  phase_stamp(p, tid, 4);
  if (n_active == 1) {
    if (wv < 4) {
      const float invj = recip(sw);
#pragma unroll
      for (int k = 0; k < 3; ++k) store_out(4 * k + wv, o[k], bcast(invj, 4 * k + wv));
      if (wv == 0 && lane < kGqa) lrow[lane * p.l_sh] = lse_of(Mw, sw);
    }
    phase_stamp(p, tid, 6);
    return;
  }

  // ---- split partial, then the last arriver merges all splits in order.
  // A partial is m[16], l[16] (log2 domain) and the unnormalised
  // accumulator laid out [head][4][64 lanes], so every store and load of a
  // wave covers 256 contiguous bytes.  Partials are written and read with
  // device-scope (sc1) accesses, which are coherent across XCDs without
  // writing back or invalidating whole L2 caches; each wave waits for its
  // stores to be acknowledged before the workgroup barrier, and one
  // device-scope atomic per workgroup counts the arrivals.  The split that
  // sees count n_active - 1 is the last one.
  auto st = [](float *ptr, float x) { __hip_atomic_store(ptr, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  auto ld = [](const float *ptr) { return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  const float *pbase = p.part + static_cast<int64_t>(pair) * nsplit_lead * kPartFloats;
  if (wv < 4) {
    float *part = p.part + (static_cast<int64_t>(pair) * nsplit_lead + split) * kPartFloats;
    if (wv == 0 && lane < 16) {
      st(part + lane, Mw);
      st(part + 16 + lane, sw);
    }
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) st(part + 32 + ((4 * k + wv) * 4 + i) * 64 + lane, o[k][i]);
  }
  // s_waitcnt vmcnt(0) (expcnt, lgkmcnt unconstrained); as a builtin, the
  // compiler's own wait tracking knows that no load is outstanding after it
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(p.ctr + pair * kCtrStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == static_cast<uint32_t>(n_active - 1)) ? 1 : 0;
  }
  __syncthreads();
  phase_stamp(p, tid, 5);
  if (!s_last || wv >= 4) return;

  // (a) m and l of every split: lane j = 16 s' + h of round r holds split
  // 4r + s' (at most 64 splits = 16 rounds; rounds past the last split
  // re-read the last split and are masked), then the accumulators of the
  // first kBatch splits.  Round 0 always exists and is straight-line code; the
  // other rounds sit behind one branch, so the common case of at most 4
  // splits issues all its loads back to back.
  constexpr int kBatch = 12;  // splits whose accumulators are loaded in one round trip
  const int nround = (n_active + 3) >> 2;
  float mr[16], lr[16];
  {
    const int s = min(sq, n_active - 1);
    mr[0] = ld(pbase + s * kPartFloats + hh);
    lr[0] = ld(pbase + s * kPartFloats + 16 + hh);
  }
  if (nround > 1) {
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      if (r < nround) {
        const int s = min(4 * r + sq, n_active - 1);
        mr[r] = ld(pbase + s * kPartFloats + hh);
        lr[r] = ld(pbase + s * kPartFloats + 16 + hh);
      }
    }
  }
  const float *pacc = pbase + 32 + wv * 4 * 64 + lane;
  auto acc_ld = [&](int s, int k) {
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = ld(pacc + s * kPartFloats + (16 * k + i) * 64);
    return r;
  };
  // (a split's registers are only written and read when the split exists)
  f32x4 a[kBatch][3];
#pragma unroll
  for (int u = 0; u < kBatch; ++u)
    if (u < n_active) {
#pragma unroll
      for (int k = 0; k < 3; ++k) a[u][k] = acc_ld(u, k);
    }

  // (b) per head: merged max, each split's weight (into this wave's LDS
  // table wf[split][16] beyond 4 splits), sum and reciprocal
  float M = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r < nround) {
      if (4 * r + sq >= n_active) mr[r] = -INFINITY;
      M = fmaxf(M, mr[r]);
    }
  }
  M = fmaxf(M, __shfl_xor(M, 16));
  M = fmaxf(M, __shfl_xor(M, 32));
  // (with at most 4 splits the weights stay in registers: lane 16 s + h
  // holds split s's weight for head h and is read out with readlane)
  const bool few = n_active <= 4;
  float *wf = reinterpret_cast<float *>(smem) + wv * 64 * 16;
  float ssum = 0.f, f0 = 0.f;
  if (few) {
    f0 = (mr[0] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mr[0] - M);
    ssum = f0 * lr[0];
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (r < nround) {
        const float f = (mr[r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mr[r] - M);
        wf[r * 64 + lane] = f;
        ssum += f * lr[r];
      }
    }
    wave_lds_fence();
  }
  ssum += __shfl_xor(ssum, 16);
  ssum += __shfl_xor(ssum, 32);

  // (c) out = (sum_s w_s acc_s) / l with the splits in index order
  f32x4 acc_o[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) acc_o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (few) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u < n_active) {
#pragma unroll
        for (int k = 0; k < 3; ++k) acc_o[k] += bcast(f0, 16 * u + 4 * k + wv) * a[u][k];
      }
  } else {
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (u < n_active) {
#pragma unroll
        for (int k = 0; k < 3; ++k) acc_o[k] += wf[u * 16 + 4 * k + wv] * a[u][k];
      }
  }
  for (int s0 = kBatch; s0 < n_active; s0 += kBatch) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (s0 + u < n_active) {
#pragma unroll
        for (int k = 0; k < 3; ++k) a[u][k] = acc_ld(s0 + u, k);
      }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (s0 + u < n_active) {
#pragma unroll
        for (int k = 0; k < 3; ++k) acc_o[k] += wf[(s0 + u) * 16 + 4 * k + wv] * a[u][k];
      }
  }
  const float invj = recip(ssum);
#pragma unroll
  for (int k = 0; k < 3; ++k) store_out(4 * k + wv, acc_o[k], bcast(invj, 4 * k + wv));
  if (wv == 0 && lane < kGqa) lrow[lane * p.l_sh] = lse_of(M, ssum);
  if (tid == 0) __hip_atomic_store(p.ctr + pair * kCtrStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  phase_stamp(p, tid, 6);
}

// XCC_ID of every workgroup of the dispatch check's probe launches
__device__ int32_t xcc_probe_out[kXccProbeWords];

__global__ void xcc_probe_kernel(int base) {
  if (threadIdx.x == 0) xcc_probe_out[base + blockIdx.x] = __builtin_amdgcn_s_getreg(kHwRegXccId) & 15;
}

__global__ void fill_u32_kernel(uint32_t *dst, int64_t n, uint32_t value) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = value;
}

__global__ void audit_kernel(const uint32_t *ctr, int n, uint32_t *accum) {
  __shared__ uint32_t part[256];
  uint32_t s = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) s += ctr[i];
  part[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int i = 0; i < static_cast<int>(blockDim.x); ++i) t += part[i];
    atomicAdd(accum, t);
  }
}

template <int FMT, int G, bool SF16, bool A32>
void launch_waves(const Params &p, dim3 grid, hipStream_t stream) {
  const int nsel = p.n_sel > 0x7FFFFFFF ? 0x7FFFFFFF : static_cast<int>(p.n_sel);
  if (p.waves == 8)
    hipLaunchKernelGGL((qsa_decode_kernel<FMT, G, 8, SF16, A32>), grid, dim3(512), 0, stream, p.cu, p.sel,
                       p.bs, p.hkv, p.nsplit, p.min_split_keys, nsel, p.xcc_lanes, p);
  else
    hipLaunchKernelGGL((qsa_decode_kernel<FMT, G, 4, SF16, A32>), grid, dim3(256), 0, stream, p.cu, p.sel,
                       p.bs, p.hkv, p.nsplit, p.min_split_keys, nsel, p.xcc_lanes, p);
}

template <int FMT, int G, bool SF16>
void launch_addr(const Params &p, dim3 grid, hipStream_t stream) {
  if (p.a32)
    launch_waves<FMT, G, SF16, true>(p, grid, stream);
  else
    launch_waves<FMT, G, SF16, false>(p, grid, stream);
}

template <int FMT, int G>
hipError_t launch_one(const Params &p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(decode_workgroups(FMT, p.bs, p.hkv, p.nsplit)));
  if constexpr (FMT == kFmtBF16) {
    launch_addr<FMT, G, false>(p, grid, stream);
  } else {
    if (p.scale_f16)
      launch_addr<FMT, G, true>(p, grid, stream);
    else
      launch_addr<FMT, G, false>(p, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const Params &p, int fmt, int group, hipStream_t stream) {
  switch (fmt) {
    case kFmtBF16: return launch_one<kFmtBF16, 256>(p, stream);
    case kFmtFP8:
      if (group == 256) return launch_one<kFmtFP8, 256>(p, stream);
      if (group == 64) return launch_one<kFmtFP8, 64>(p, stream);
      if (group == 32) return launch_one<kFmtFP8, 32>(p, stream);
      break;
    case kFmtINT8:
      if (group == 256) return launch_one<kFmtINT8, 256>(p, stream);
      if (group == 64) return launch_one<kFmtINT8, 64>(p, stream);
      if (group == 32) return launch_one<kFmtINT8, 32>(p, stream);
      break;
    case kFmtINT4:
      if (group == 64) return launch_one<kFmtINT4, 64>(p, stream);
      if (group == 32) return launch_one<kFmtINT4, 32>(p, stream);
      break;
    case kFmtTIERED:
      launch_addr<kFmtTIERED, 32, true>(
          p, dim3(static_cast<unsigned>(decode_workgroups(kFmtTIERED, p.bs, p.hkv, p.nsplit))), stream);
      return hipGetLastError();
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_audit(const uint32_t *ctr, int n, uint32_t *accum, hipStream_t stream) {
  hipLaunchKernelGGL(audit_kernel, dim3(1), dim3(256), 0, stream, ctr, n, accum);
  return hipGetLastError();
}

hipError_t launch_xcc_probe(int base, int blocks, hipStream_t stream) {
  if (base < 0 || blocks <= 0 || base + blocks > kXccProbeWords) return hipErrorInvalidValue;
  hipLaunchKernelGGL(xcc_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(64), 0, stream, base);
  return hipGetLastError();
}

hipError_t read_xcc_probe(int32_t *host, int n, hipStream_t stream) {
  if (n < 0 || n > kXccProbeWords) return hipErrorInvalidValue;
  return hipMemcpyFromSymbolAsync(host, HIP_SYMBOL(xcc_probe_out), static_cast<size_t>(n) * sizeof(int32_t), 0,
                                  hipMemcpyDeviceToHost, stream);
}

hipError_t launch_fill_u32(uint32_t *dst, int64_t n, uint32_t value, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream,
                     dst, n, value);
  return hipGetLastError();
}

}  // namespace qsa
