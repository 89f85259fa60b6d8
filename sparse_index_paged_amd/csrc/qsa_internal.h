// qsa_internal.h -- types shared by the decode kernel and the host API of
// libqsa.so (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

constexpr int kHeadDim = 256;
constexpr int kGqa = 12;          // Q heads per KV head
constexpr int kMaxSel = 2055;     // list entries per row
constexpr int kMaxBs = 128;
// Arrival counters sit one per 128-byte line: the device-scope adds of the
// splits of different pairs then never meet at one line.
constexpr int kCtrStride = 32;
constexpr int kTile = 16;         // list entries per wave iteration

// One split partial: m[16] and l[16] (log2 domain, 12 used) then the
// unnormalised accumulator [12][256].
constexpr int kPartFloats = 32 + kGqa * kHeadDim;

// kFmtTIERED: an int8 ring (64-channel f16 scales) of 2^k rows with an
// owner table over an int4 pool (32-channel f16 scales); the int4 pool sits
// in the plain pool fields, the ring in Params::ring.
enum KvFormat : int { kFmtBF16 = 0, kFmtFP8 = 1, kFmtINT8 = 2, kFmtINT4 = 3, kFmtTIERED = 4 };

// Workgroup placement.  Workgroup w runs on XCD w % 8 (round-robin
// dispatch), and every split of one (row, KV head) pair gets ids congruent
// mod 8, so its partials stay in one L2.  bf16 pools deal the pairs out in
// order: pair p = b * hkv + g on XCD p % 8.  Quantized pools put all KV
// heads of row b on XCD b % 8: a slot's scales of every KV head share one
// 128-byte line of the scale arrays, which the heads' workgroups then fetch
// from that XCD's L2 once instead of from memory once per head.  The rows
// are rounded up to a multiple of 8 for that, so the grid can hold up to
// 8 * hkv idle pair slots more than the bf16 one.
//
// Which XCD a workgroup lands on depends on where the dispatcher starts its
// round-robin, which differs between launches (graph replays start one XCD
// further than eager launches here), while the bf16 order is fastest with
// the two KV heads of a row on XCDs 2k and 2k + 1.  With Params::xcc_lanes
// each bf16 workgroup therefore takes the pair slot of the XCD it reads from
// its XCC_ID register instead of blockIdx % 8.  That stays a one-to-one
// assignment only while every aligned block of 8 workgroups covers the 8
// XCDs, so the library sets it only on a device that reports 8 XCDs and has
// passed a dispatch check (xcc_dispatch_check).
constexpr bool rows_share_xcd(int fmt) { return fmt != kFmtBF16; }

inline int64_t decode_workgroups(int fmt, int bs, int hkv, int splits) {
  const int64_t pairs8 = rows_share_xcd(fmt) ? ((static_cast<int64_t>(bs) + 7) / 8) * 8 * hkv
                                             : ((static_cast<int64_t>(bs) * hkv + 7) / 8) * 8;
  return pairs8 * splits;
}

// Device-side error bits (sticky, OR-ed into Params::err).
constexpr uint32_t kErrRowRange = 1u;   // cu_seqlens out of range / row > 2055
constexpr uint32_t kErrSlot = 2u;       // a slot id outside [0, slots)
constexpr uint32_t kErrStoreSlot = 4u;  // a store's slot id outside [0, slots)

struct Params {
  const __bf16 *q;          // [bs, hq, 256]
  int64_t q_sb, q_sh;       // element strides
  const uint8_t *k, *v;     // pools (byte pointers)
  int64_t k_ss, k_sh;       // byte strides (slot, kv head)
  int64_t v_ss, v_sh;
  const uint8_t *ks, *vs;   // scales [slots, hkv, 256/G] (f32 or f16) or null
  int64_t ks_ss, ks_sh;     // byte strides
  int64_t vs_ss, vs_sh;
  int scale_f16;            // scales are f16 (else f32)
  int a32;                  // every row / scale address fits a 24-bit slot x 24-bit stride
                            // product below 2^32 bytes from its pool's start
  const int32_t *sel;
  int64_t n_sel;
  const int32_t *cu;
  __bf16 *out;
  int64_t o_sb, o_sh;
  float *lse;
  int64_t l_sb, l_sh;
  int64_t slots;
  struct Ring {             // tiered pools only
    const uint8_t *k, *v;   // int8 codes [R, hkv, 256]
    int64_t k_ss, k_sh, v_ss, v_sh;      // byte strides
    const uint8_t *ks, *vs; // f16 scales [R, hkv, 4]
    int64_t ks_ss, ks_sh, vs_ss, vs_sh;  // byte strides
    const int32_t *owner;   // [R]
    uint32_t mask;          // R - 1
    // with Params::a32: per array a base from which every ring and int4
    // row (and scale row) lies within 4 GiB, for 32-bit lane offsets
    const uint8_t *kb, *vb, *ksb, *vsb;
  } ring;
  int bs, hkv;
  int nsplit;               // splits per (row, kv head) in the grid
  int waves;                // waves per workgroup: 4 or 8
  int min_split_keys;       // entries per split before another is used
  int xcc_lanes;            // bf16 placement from the workgroup's own XCD (decode_workgroups)
  float *part;              // [npairs][nsplit][kPartFloats]
  uint32_t *ctr;            // pair i's counter at ctr[i * kCtrStride], zero at rest
  uint32_t *err;            // sticky error word
#ifdef QSA_PHASE_STAMPS
  uint64_t *stamps;         // [grid][kStampSlots] wall-clock stamps, or null
#endif
};

// Phase stamps (measurement build libqsa_stamps.so only): per workgroup,
// thread 0 writes the 100 MHz wall clock at kernel entry, once cu_seqlens
// has arrived, once its first tile's rows have arrived, at the end of its
// loop, after the workgroup's wave merge, after the split arrival count, and
// when it has written the output (slots 0..6; slots it does not reach keep
// the value the host put there).
constexpr int kStampSlots = 8;

// One quantize + scatter call: rows t of k_new / v_new go to pool slot loc[t].
struct StoreParams {
  const __bf16 *k, *v;      // new rows [n, hkv, 256]
  int64_t k_st, k_sh;       // element strides (token, kv head)
  int64_t v_st, v_sh;
  const void *loc;          // [n] int32 or int64 slot ids
  int loc_i64;
  int64_t n;
  uint8_t *kp, *vp;         // code pools (byte pointers)
  int64_t kp_ss, kp_sh;     // byte strides (slot, kv head)
  int64_t vp_ss, vp_sh;
  uint8_t *ks, *vs;         // scale pools or null (bf16 pools)
  int64_t ks_ss, ks_sh;     // byte strides
  int64_t vs_ss, vs_sh;
  int scale_f16;
  int group;                // channels per scale: 32, 64 or 256
  int64_t slots;
  int hkv;
  uint32_t *err;            // sticky error word
  // ring write of a tiered pool (null otherwise): token t goes to ring row
  // loc[t] & ring_mask only if claim[row] == t + 1 (the last token of the
  // call naming that row), which then stamps owner[row] = loc[t] and
  // clears claim[row]
  int32_t *claim;
  int32_t *owner;
  uint32_t ring_mask;
};

constexpr uint32_t kErrIndexRow = 8u;  // an indexer row's context length / block table entry out of range

// One indexer call: block scores of every row, then per row the top
// budget / c blocks, expanded to KV slots and packed.
struct IndexParams {
  const __bf16 *q;          // [bs, hi, di]
  int64_t q_sb, q_sh;       // element strides
  const float *w;           // [bs, hi] or null (all 1)
  int64_t w_sb;
  const __bf16 *k;          // key pool [n_k, di]
  int64_t k_ss;             // element stride between key rows
  int64_t n_k;
  const int32_t *bt;        // block table [bs, max_blocks]
  int64_t bt_sb;
  int max_blocks;
  const int32_t *r2t;       // token -> KV slot [bs, max_tokens]
  int64_t r2t_sb;
  int max_tokens;
  const int32_t *ctx;       // [bs] context lengths
  int bs, hi, di;
  int budget, c;
  float *scores;            // scratch [bs, max_blocks]
  int32_t *sel;             // packed output
  int32_t *cu;              // [bs + 1]
  uint32_t *err;
};

// Score kernel then select/expand kernel on `stream`.
hipError_t launch_index(const IndexParams &p, hipStream_t stream);

// Launch the decode kernel for one call (grid = 8 * ceil(npairs/8) * nsplit).
hipError_t launch_decode(const Params &p, int fmt, int group, hipStream_t stream);
// Dispatch check probe (no allocation): `blocks` workgroups of 64 threads,
// workgroup i writing the XCC_ID of its XCD to entry base + i of a
// kXccProbeWords-entry device array, which read_xcc_probe copies to the host
// in stream order on `stream` (the caller synchronises the stream before
// reading `host`).
constexpr int kXccProbeWords = 2 * 1024 + 3;
hipError_t launch_xcc_probe(int base, int blocks, hipStream_t stream);
hipError_t read_xcc_probe(int32_t *host, int n, hipStream_t stream);

// Launch the quantize + scatter kernel (one wave per (token, kv head)).
hipError_t launch_store(const StoreParams &p, int fmt, hipStream_t stream);

// Ring claims of a tiered write: claim[loc[t] & ring_mask] = max(.., t + 1)
// for every in-range slot id (p.claim, p.loc, p.n, p.slots).
hipError_t launch_claim(const StoreParams &p, hipStream_t stream);

// Zero n words at dst with a small kernel (no memset node in captured graphs).
hipError_t launch_fill_u32(uint32_t *dst, int64_t n, uint32_t value, hipStream_t stream);

// *accum += sum of ctr[0..n) (one workgroup).
hipError_t launch_audit(const uint32_t *ctr, int n, uint32_t *accum, hipStream_t stream);

}  // namespace qsa
