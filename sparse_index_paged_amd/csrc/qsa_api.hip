// qsa_api.hip -- host side of libqsa.so: contract validation, split plan,
// per-device workspace and the single launch of qsa_decode.
//
// The contract (page "fix(qsa): restore SM121 correctness with Humanize and
// Kernel Design Agent", sections "Changes" and the integration update): bf16,
// head dim 256, 12:1 GQA as 24 Q / 2 KV or 12 Q / 1 KV heads, one query per
// row, 1 <= bs <= 128, at most 2055 selected entries per row; calls outside
// it fail with a descriptive error and nothing is launched.  Lengths are only
// read on the device, so a captured graph replays correctly when cu_seqlens
// changes.  Counters are kept across calls and are zero at rest.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/qsa.h"
#ifdef QSA_PHASE_STAMPS
#include "../../include/qsa_stamps.h"
#endif
#include "qsa_internal.h"

namespace {

// The message of the last failed call on this thread (a fixed buffer, so
// reporting an error allocates nothing).
thread_local char g_last_error[512];

qsa_status fail(qsa_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
qsa_status fail(qsa_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

qsa_status ok() {
  g_last_error[0] = '\0';
  return QSA_OK;
}

// ---- options ---------------------------------------------------------------
std::atomic<int64_t> g_split_target{0};  // 0: cost model below
std::atomic<int64_t> g_max_splits{16};
std::atomic<int64_t> g_min_split_keys{256};
std::atomic<int64_t> g_waves{0};  // 0: chosen per call (waves_for)
std::atomic<int64_t> g_splits{0};     // > 0: exactly this many splits (tuning)
std::atomic<int64_t> g_xcc_lanes{1};  // 1: XCD-read bf16 placement where checked, 0: never

// Splits per (row, KV head) pair.  The plan depends on (bs, hkv) and the
// options only -- never on live lengths -- so captured graphs stay valid.
//
// Default: a cost model of one launch with every list at full capacity on
// a 256-CU MI355X (8 XCDs of 32 CUs), fitted to graph-replayed saturated
// calls at every bs 1..128 in both layouts and every split count.  All
// splits of pair p run on XCD p % 8 (the launch gives them workgroup ids
// congruent mod 8), so the busiest XCD holds ceil(P/8) pairs and
// ceil(P/8)*n workgroups on its 32 CUs.  With n splits a launch costs
//   max(busiest CU's entries / 40 per us, P * 2055 * 1 KB / 7 TB/s)
//   + (6 + 0.5 n) us of split merge when n > 1
//   + 20 us for each workgroup per CU beyond the two resident ones,
// where the busiest CU's entries are ceil(ceil(P/8)*n/32) * ceil(2055/n):
// more splits shorten each workgroup's dependent chain of tiles until the
// gather is bound by HBM, and each one lengthens the merge.  Only split
// counts a full row can activate are priced.
// (Quantized pools place rows, not pairs, on the XCDs: with Hkv = 2 and bs
// mod 8 in 1..4 their busiest XCD holds one pair more than the model's
// ceil(P/8); the plan is the same for every format.)
// split_target > 0 replaces the model by "about split_target workgroups";
// splits > 0 fixes the split count.
int plan_splits(int bs, int hkv) {
  const int64_t npairs = static_cast<int64_t>(bs) * hkv;
  const int64_t smax = g_max_splits.load();
  const int64_t target = g_split_target.load();
  const int64_t forced = g_splits.load();
  if (forced > 0) return static_cast<int>(forced < smax ? forced : smax);
  if (target > 0) {
    const int64_t npairs8 = ((npairs + 7) / 8) * 8;
    int64_t s = (target + npairs8 - 1) / npairs8;
    if (s > smax) s = smax;
    if (s < 1) s = 1;
    return static_cast<int>(s);
  }
  // a row never activates more than ceil(2055 / min_split_keys) splits, so
  // the model only prices split counts that can all be active (a larger
  // grid would be costed for short workgroups that never run)
  const int64_t msk = g_min_split_keys.load() > 4096 ? 4096 : g_min_split_keys.load();
  const int64_t sact = (qsa::kMaxSel + msk - 1) / msk;
  const int64_t nmax = smax < sact ? smax : sact;
  int best = 1;
  double best_cost = 1e30;
  const double hbm_us = static_cast<double>(npairs) * qsa::kMaxSel * 1024.0 / 7.0e6;
  for (int n = 1; n <= nmax; ++n) {
    const int64_t per_cu = (((npairs + 7) / 8) * n + 31) / 32;
    const double lat_us = static_cast<double>(per_cu) * ((qsa::kMaxSel + n - 1) / n) / 40.0;
    const double cost = (lat_us > hbm_us ? lat_us : hbm_us) + (n > 1 ? 6.0 + 0.5 * n : 0.0) +
                        20.0 * static_cast<double>(per_cu > 2 ? per_cu - 2 : 0);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = n;
    }
  }
  return best;
}

// Workgroups of a launch over bf16 pools (quantized pools: decode_workgroups)
int64_t plan_workgroups(int bs, int hkv, int splits) {
  return qsa::decode_workgroups(qsa::kFmtBF16, bs, hkv, splits);
}

// Waves per workgroup.  4-wave workgroups leave two resident per CU, which
// with at most one workgroup per CU is one wave per SIMD.  The quantized
// formats are bound by per-tile ALU work (dequantization, and for the
// tiered pool the tier selection), so they run as 8-wave workgroups: two
// waves per SIMD overlap one wave's dequantization with the other's memory
// wait, and each wave keeps one tile in flight.  Measured on MI355X (bs=128 /
// 96 / 64 / 32 TP1, 4 -> 8 waves): fp8 59.8 -> 60.1 / 53.6 -> 48.5 / 36.7 ->
// 36.4 / 25.8 -> 24.3 us, int8 g64 68.7 -> 65.1 / 64.3 -> 52.1 / 40.6 -> 39.6 /
// 29.3 -> 26.0 us, int4 g32 73.2 -> 58.0 / 71.9 -> 56.0 / 44.7 -> 37.9 / 31.3 ->
// 27.9 us (two int4 tiles in flight then; one is faster again: bs=128 / 64 /
// 32 TP1 54.2 -> 52.8 / 35.1 -> 33.9 / 25.8 -> 25.0 us); bf16 is faster with
// 4.  More tiles in flight with 8 waves was slower at every measured point
// (bs=128 TP1 fp8 59.3 -> 60.8, int4 55.8 -> 61.0 us).  An 8-wave workgroup
// takes 151 KB of LDS, so only one fits on a CU: grids of more than 256
// workgroups (two per CU) keep 4 waves.
int waves_for(int fmt, int64_t workgroups) {
  const int64_t forced = g_waves.load();
  if (forced == 4 || forced == 8) return static_cast<int>(forced);
  if (fmt != qsa::kFmtBF16 && workgroups <= 256) return 8;
  return 4;
}

// ---- workspaces ------------------------------------------------------------
// A workspace holds the split partials, the split counters followed by the
// sticky error word, and the indexer's block scores.  Each device has one
// shared workspace, used by every stream without one of its own, and up to
// kMaxAttached private workspaces, each bound to one stream by
// qsa_workspace_attach.  Calls on different streams run concurrently only
// when their workspaces differ.
//
// Captured graphs keep the device addresses of the buffers their calls
// used, so nothing a capture may reference is freed before the workspace
// itself goes (qsa_workspace_detach / qsa_workspace_release):
//   * the counters and the error word are one fixed-size allocation made
//     when the workspace is created; they never move, so the error word
//     stays sticky and an audit pointer stays valid;
//   * when the partials or the index scores grow, the new buffer replaces
//     the old one for later calls and the old one is retired, not freed.
// Growth is geometric (at least doubling), so a workspace retires at most
// a few dozen buffers over its life.
constexpr int kMaxDevices = 64;
constexpr int kMaxAttached = 64;
constexpr int kMaxRetired = 64;

struct Workspace {
  float *part = nullptr;
  int64_t part_floats = 0;
  uint32_t *words = nullptr;  // [kMaxBs * 2 counters][1 error word]
  int64_t n_ctr = 0;
  float *iscores = nullptr;   // indexer block scores
  int64_t iscore_floats = 0;
  void *retired[kMaxRetired] = {};  // replaced buffers, freed with the workspace
  int n_retired = 0;
  int64_t retired_bytes = 0;
};

struct DeviceWorkspaces {
  Workspace shared;
  bool used[kMaxAttached] = {};
  hipStream_t stream[kMaxAttached] = {};
  Workspace own[kMaxAttached];
};

std::mutex g_ws_mutex;
DeviceWorkspaces g_ws[kMaxDevices];

constexpr int64_t kCtrWords = static_cast<int64_t>(qsa::kMaxBs) * 2 * qsa::kCtrStride;

int64_t part_floats_needed(int max_bs, int hkv) {
  int64_t worst = 0;
  for (int bs = 1; bs <= max_bs; ++bs) {
    const int64_t n = static_cast<int64_t>(bs) * hkv * plan_splits(bs, hkv);
    if (n > worst) worst = n;
  }
  return worst * qsa::kPartFloats;
}

bool stream_capturing(hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) != hipSuccess) return false;
  return st != hipStreamCaptureStatusNone;
}

// ---- bf16 placement by the workgroup's own XCD (decode_workgroups) --------
std::mutex g_xcc_mutex;
int g_xcc_state[kMaxDevices];  // 0: not checked yet, 1: not used, 2: used

// Every workgroup of a probe launch of n ran on XCD (i + r) % 8 for one r.
bool xcc_round_robin(const int32_t *xcc, int n) {
  const int r = xcc[0] & 7;
  for (int i = 0; i < n; ++i)
    if (xcc[i] != ((i + r) & 7)) return false;
  return true;
}

// Whether device `dev` may place bf16 workgroups by their XCC_ID: it reports
// 8 XCDs, and two probe launches of 1024 workgroups, one before and one after
// a launch of 3 workgroups (which moves where the dispatcher starts), each
// ran workgroup i on XCD (i + r) % 8 for a single r.  Runs once per device,
// outside capture, allocating nothing; it synchronises `stream`.
bool xcc_dispatch_check(int dev, hipStream_t stream) {
  int nx = 0;
  if (hipDeviceGetAttribute(&nx, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || nx != 8) {
    (void)hipGetLastError();
    return false;
  }
  constexpr int kN = 1024;
  static_assert(2 * kN + 3 <= qsa::kXccProbeWords, "probe launches exceed the probe array");
  static int32_t host[qsa::kXccProbeWords];
  bool ok = qsa::launch_xcc_probe(0, kN, stream) == hipSuccess &&
            qsa::launch_xcc_probe(2 * kN, 3, stream) == hipSuccess &&
            qsa::launch_xcc_probe(kN, kN, stream) == hipSuccess &&
            qsa::read_xcc_probe(host, 2 * kN, stream) == hipSuccess &&
            hipStreamSynchronize(stream) == hipSuccess;
  ok = ok && xcc_round_robin(host, kN) && xcc_round_robin(host + kN, kN);
  (void)hipGetLastError();
  return ok;
}

// Params::xcc_lanes of a launch on `stream` (the device is checked at its
// first call outside capture; a captured call before that one places
// workgroups by blockIdx).
int xcc_lanes_for(hipStream_t stream) {
  if (g_xcc_lanes.load() == 0) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lock(g_xcc_mutex);
  if (g_xcc_state[dev] == 0) {
    if (stream_capturing(stream)) return 0;
    g_xcc_state[dev] = xcc_dispatch_check(dev, stream) ? 2 : 1;
  }
  return g_xcc_state[dev] == 2 ? 1 : 0;
}

// ---- phase stamps (the measurement build libqsa_stamps.so only) ----------
#ifdef QSA_PHASE_STAMPS
std::atomic<uint64_t *> g_stamps{nullptr};
std::atomic<int64_t> g_stamp_words{0};
// A launch writes its stamps when the buffer holds kStampSlots words per
// workgroup of its grid.
void stamp_launch(qsa::Params *p, int fmt) {
  const int64_t need = qsa::decode_workgroups(fmt, p->bs, p->hkv, p->nsplit) * qsa::kStampSlots;
  p->stamps = g_stamp_words.load() >= need ? g_stamps.load() : nullptr;
}
#else
inline void stamp_launch(qsa::Params *, int) {}
#endif

// Index of the private workspace bound to `stream` on `dev`, or -1 (the
// caller holds g_ws_mutex).
int attached_slot(int dev, hipStream_t stream) {
  const DeviceWorkspaces &d = g_ws[dev];
  for (int i = 0; i < kMaxAttached; ++i)
    if (d.used[i] && d.stream[i] == stream) return i;
  return -1;
}

// The workspace that calls on `stream` use (the caller holds g_ws_mutex).
// Slots never move, so the reference stays valid until a detach or release.
Workspace &workspace_of(int dev, hipStream_t stream, bool *own = nullptr) {
  const int i = attached_slot(dev, stream);
  if (own) *own = i >= 0;
  return i >= 0 ? g_ws[dev].own[i] : g_ws[dev].shared;
}

// Free every buffer of a workspace, retired ones included (the caller has
// synchronised whatever could still use it).
void free_workspace(Workspace &ws) {
  if (ws.part) (void)hipFree(ws.part);
  if (ws.words) (void)hipFree(ws.words);
  if (ws.iscores) (void)hipFree(ws.iscores);
  for (int i = 0; i < ws.n_retired; ++i) (void)hipFree(ws.retired[i]);
  ws = Workspace{};
}

// Replace *buf (of *have floats) by a new buffer of at least `need` floats,
// retiring the old one.  Growth at least doubles the size.
template <typename T>
qsa_status grow_buffer(Workspace &ws, T **buf, int64_t *have, int64_t need, const char *fn,
                       const char *what) {
  if (*buf != nullptr && ws.n_retired >= kMaxRetired)
    return fail(QSA_ERR_WORKSPACE, "%s: the workspace has replaced its %s %d times; "
                "call qsa_workspace_reserve with the largest size first", fn, what, kMaxRetired);
  int64_t n = need;
  if (*buf != nullptr && n < 2 * *have) n = 2 * *have;
  void *ptr = nullptr;
  if (hipMalloc(&ptr, static_cast<size_t>(n) * sizeof(T)) != hipSuccess) {
    (void)hipGetLastError();
    return fail(QSA_ERR_HIP, "%s: hipMalloc of %lld bytes for the %s failed", fn,
                static_cast<long long>(n * static_cast<int64_t>(sizeof(T))), what);
  }
  if (*buf != nullptr) {
    ws.retired[ws.n_retired++] = *buf;
    ws.retired_bytes += *have * static_cast<int64_t>(sizeof(T));
  }
  *buf = static_cast<T *>(ptr);
  *have = n;
  return QSA_OK;
}

// Ensure the workspace `stream` uses on `dev` exists (counters and error
// word) and holds `floats` partial floats.
qsa_status ensure_workspace(int dev, int64_t floats, hipStream_t stream, bool allow_alloc,
                            Workspace **out, const char *fn = "qsa_decode") {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  bool own = false;
  Workspace &ws = workspace_of(dev, stream, &own);
  if (ws.words != nullptr && ws.part_floats >= floats) {
    *out = &ws;
    return QSA_OK;
  }
  if (!allow_alloc)
    return fail(QSA_ERR_WORKSPACE,
                "%s: the stream is capturing and the %s workspace of device %d holds %lld "
                "partial floats, %lld needed; call qsa_workspace_reserve before capture",
                fn, own ? "stream's own" : "shared", dev, static_cast<long long>(ws.part_floats),
                static_cast<long long>(floats));
  if (ws.words == nullptr) {
    void *words = nullptr;
    if (hipMalloc(&words, static_cast<size_t>(kCtrWords + 1) * sizeof(uint32_t)) != hipSuccess) {
      (void)hipGetLastError();
      return fail(QSA_ERR_HIP, "%s: hipMalloc of the workspace counters failed", fn);
    }
    ws.words = static_cast<uint32_t *>(words);
    ws.n_ctr = kCtrWords;
    if (qsa::launch_fill_u32(ws.words, kCtrWords + 1, 0u, stream) != hipSuccess)
      return fail(QSA_ERR_HIP, "%s: zeroing the workspace counters failed", fn);
  }
  if (ws.part_floats < floats) {
    qsa_status st = grow_buffer(ws, &ws.part, &ws.part_floats, floats, fn, "split partials");
    if (st != QSA_OK) return st;
  }
  *out = &ws;
  return QSA_OK;
}

// The indexer score scratch of the workspace `stream` uses, holding at least
// `floats` (the counters and error word are created with it when missing).
qsa_status ensure_index_scores(int dev, int64_t floats, hipStream_t stream, bool allow_alloc,
                               Workspace **out, const char *fn) {
  qsa_status st = ensure_workspace(dev, 0, stream, allow_alloc, out, fn);
  if (st != QSA_OK) return st;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  bool own = false;
  Workspace &ws = workspace_of(dev, stream, &own);
  if (ws.iscore_floats >= floats && (floats == 0 || ws.iscores != nullptr)) return QSA_OK;
  if (!allow_alloc)
    return fail(QSA_ERR_WORKSPACE,
                "%s: the stream is capturing and the %s workspace of device %d holds %lld index "
                "score floats, %lld needed; call qsa_index_reserve before capture", fn,
                own ? "stream's own" : "shared", dev, static_cast<long long>(ws.iscore_floats),
                static_cast<long long>(floats));
  if ((st = grow_buffer(ws, &ws.iscores, &ws.iscore_floats, floats, fn, "index scores")) != QSA_OK)
    return st;
  *out = &ws;
  return QSA_OK;
}

// ---- descriptor checks -----------------------------------------------------
const char *dtype_name(int32_t dt) {
  switch (dt) {
    case QSA_DTYPE_BF16: return "bf16";
    case QSA_DTYPE_F16: return "f16";
    case QSA_DTYPE_F32: return "f32";
    case QSA_DTYPE_I32: return "i32";
    case QSA_DTYPE_FP8_E4M3FN: return "fp8_e4m3fn";
    case QSA_DTYPE_I8: return "i8";
    case QSA_DTYPE_U4X2: return "u4x2";
    case QSA_DTYPE_I64: return "i64";
    default: return "unknown";
  }
}

int64_t dtype_bytes(int32_t dt) {
  switch (dt) {
    case QSA_DTYPE_BF16:
    case QSA_DTYPE_F16: return 2;
    case QSA_DTYPE_F32:
    case QSA_DTYPE_I32: return 4;
    case QSA_DTYPE_I64: return 8;
    case QSA_DTYPE_FP8_E4M3FN:
    case QSA_DTYPE_I8:
    case QSA_DTYPE_U4X2: return 1;
    default: return 0;
  }
}

qsa_status check_tensor(const qsa_tensor *t, const char *name, int32_t dtype, int ndim,
                        bool last_dim_contiguous = true, const char *fn = "qsa_decode") {
  if (t == nullptr) return fail(QSA_ERR_ARG, "%s: %s is NULL", fn, name);
  if (t->data == nullptr) return fail(QSA_ERR_ARG, "%s: %s.data is NULL", fn, name);
  if (t->dtype != dtype)
    return fail(QSA_ERR_CONTRACT, "%s: %s must be %s, got %s", fn, name, dtype_name(dtype),
                dtype_name(t->dtype));
  if (t->ndim != ndim)
    return fail(QSA_ERR_CONTRACT, "%s: %s must have %d dimensions, got %d", fn, name, ndim,
                t->ndim);
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] < 0) return fail(QSA_ERR_CONTRACT, "%s: %s.shape[%d] < 0", fn, name, i);
    if (t->stride[i] < 0) return fail(QSA_ERR_CONTRACT, "%s: %s.stride[%d] < 0", fn, name, i);
  }
  if (last_dim_contiguous && t->stride[ndim - 1] != 1 && t->shape[ndim - 1] > 1)
    return fail(QSA_ERR_CONTRACT, "%s: %s must be contiguous in its last dimension", fn, name);
  return QSA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A pair of K/V pools and their scales, as validated for decode and store.
struct PoolDesc {
  int32_t dtype = 0;
  int fmt = qsa::kFmtBF16, group = QSA_HEAD_DIM;
  int64_t slots = 0, hkv = 0, eb = 0;  // eb: bytes per pool element
  const qsa_tensor *k = nullptr, *v = nullptr;
  uint8_t *ks = nullptr, *vs = nullptr;
  int64_t ks_ss = 0, ks_sh = 0, vs_ss = 0, vs_sh = 0;  // bytes
  int scale_f16 = 0;
};

// Pools: bf16 | fp8_e4m3fn | i8 [slots, Hkv, 256] or u4x2 [slots, Hkv, 128],
// one format for K and V, Hkv 1 or 2, rows on 16-byte boundaries.  Scales:
// absent for bf16, else f32 or f16 [slots, Hkv, 256 / group] for both.
qsa_status check_pools(const char *fn, const qsa_tensor *k_pool, const qsa_tensor *v_pool,
                       const qsa_kv_scales *kv_scales, PoolDesc *d) {
  qsa_status st;
  if (k_pool == nullptr || v_pool == nullptr) return fail(QSA_ERR_ARG, "%s: a pool is NULL", fn);
  const int32_t pdt = k_pool->dtype;
  if (pdt != QSA_DTYPE_BF16 && pdt != QSA_DTYPE_FP8_E4M3FN && pdt != QSA_DTYPE_I8 &&
      pdt != QSA_DTYPE_U4X2)
    return fail(QSA_ERR_CONTRACT, "%s: k_pool dtype %s is not bf16, fp8_e4m3fn, i8 or u4x2", fn,
                dtype_name(pdt));
  if (v_pool->dtype != pdt)
    return fail(QSA_ERR_CONTRACT, "%s: k_pool (%s) and v_pool (%s) must share a format", fn,
                dtype_name(pdt), dtype_name(v_pool->dtype));
  if ((st = check_tensor(k_pool, "k_pool", pdt, 3, true, fn)) != QSA_OK) return st;
  if ((st = check_tensor(v_pool, "v_pool", pdt, 3, true, fn)) != QSA_OK) return st;
  const int64_t slots = k_pool->shape[0], hkv = k_pool->shape[1];
  const int64_t row_elems = (pdt == QSA_DTYPE_U4X2) ? QSA_HEAD_DIM / 2 : QSA_HEAD_DIM;
  if (hkv != 1 && hkv != 2)
    return fail(QSA_ERR_CONTRACT, "%s: pools must hold 1 or 2 KV heads, got %lld", fn,
                static_cast<long long>(hkv));
  if (k_pool->shape[2] != row_elems || v_pool->shape[2] != row_elems)
    return fail(QSA_ERR_CONTRACT, "%s: pool rows must hold %lld %s elements (head dim 256)", fn,
                static_cast<long long>(row_elems), dtype_name(pdt));
  if (v_pool->shape[0] != slots || v_pool->shape[1] != hkv)
    return fail(QSA_ERR_CONTRACT, "%s: k_pool and v_pool shapes differ", fn);
  if (slots < 1) return fail(QSA_ERR_CONTRACT, "%s: the pools hold no slots", fn);
  if (slots > 0x7FFFFFFFLL)
    return fail(QSA_ERR_CONTRACT, "%s: more than 2^31-1 slots cannot be named by int32 ids", fn);
  const int64_t eb = dtype_bytes(pdt);
  if (!aligned16(k_pool->data) || !aligned16(v_pool->data) || (k_pool->stride[0] * eb) % 16 ||
      (k_pool->stride[1] * eb) % 16 || (v_pool->stride[0] * eb) % 16 || (v_pool->stride[1] * eb) % 16)
    return fail(QSA_ERR_CONTRACT, "%s: pool rows must start on 16-byte boundaries", fn);

  *d = PoolDesc{};
  d->dtype = pdt;
  d->slots = slots;
  d->hkv = hkv;
  d->eb = eb;
  d->k = k_pool;
  d->v = v_pool;
  if (pdt == QSA_DTYPE_BF16) {
    if (kv_scales != nullptr)
      return fail(QSA_ERR_CONTRACT, "%s: bf16 pools take no scales (kv_scales must be NULL)", fn);
    return QSA_OK;
  }
  d->fmt = pdt == QSA_DTYPE_FP8_E4M3FN ? qsa::kFmtFP8 : pdt == QSA_DTYPE_I8 ? qsa::kFmtINT8 : qsa::kFmtINT4;
  if (kv_scales == nullptr) return fail(QSA_ERR_CONTRACT, "%s: %s pools need kv_scales", fn, dtype_name(pdt));
  const int group = kv_scales->group_size;
  const bool g_ok = (d->fmt == qsa::kFmtINT4) ? (group == 32 || group == 64)
                                              : (group == 32 || group == 64 || group == 256);
  if (!g_ok)
    return fail(QSA_ERR_CONTRACT, "%s: group_size %d is not supported for %s pools "
                "(fp8/i8: 32, 64, 256; u4x2: 32, 64)", fn, group, dtype_name(pdt));
  d->group = group;
  const int32_t sdt = kv_scales->k_scale.dtype;
  if (sdt != QSA_DTYPE_F32 && sdt != QSA_DTYPE_F16)
    return fail(QSA_ERR_CONTRACT, "%s: k_scale must be f32 or f16, got %s", fn, dtype_name(sdt));
  if ((st = check_tensor(&kv_scales->k_scale, "k_scale", sdt, 3, true, fn)) != QSA_OK) return st;
  if ((st = check_tensor(&kv_scales->v_scale, "v_scale", sdt, 3, true, fn)) != QSA_OK) return st;
  const int64_t ng = QSA_HEAD_DIM / group;
  for (const qsa_tensor *t : {&kv_scales->k_scale, &kv_scales->v_scale})
    if (t->shape[0] != slots || t->shape[1] != hkv || t->shape[2] != ng)
      return fail(QSA_ERR_CONTRACT, "%s: scales must be [slots, Hkv, 256/group] = "
                  "[%lld, %lld, %lld]", fn, static_cast<long long>(slots),
                  static_cast<long long>(hkv), static_cast<long long>(ng));
  const int64_t sb = dtype_bytes(sdt);
  if ((reinterpret_cast<uintptr_t>(kv_scales->k_scale.data) % sb) ||
      (reinterpret_cast<uintptr_t>(kv_scales->v_scale.data) % sb))
    return fail(QSA_ERR_CONTRACT, "%s: scale data must be aligned to its element size", fn);
  d->scale_f16 = sdt == QSA_DTYPE_F16;
  d->ks = static_cast<uint8_t *>(kv_scales->k_scale.data);
  d->vs = static_cast<uint8_t *>(kv_scales->v_scale.data);
  d->ks_ss = kv_scales->k_scale.stride[0] * sb;
  d->ks_sh = kv_scales->k_scale.stride[1] * sb;
  d->vs_ss = kv_scales->v_scale.stride[0] * sb;
  d->vs_sh = kv_scales->v_scale.stride[1] * sb;
  return QSA_OK;
}


// True when every row and scale the decode can read lies within 4 GiB of
// its pool's (KV head's) start and the offset is a 24-bit x 24-bit product:
// slot ids and byte strides below 2^24, (slots - 1) * stride + row bytes
// below 2^32.  The kernel then forms addresses with 32-bit arithmetic.
bool addresses_fit_32(const PoolDesc &pd, const qsa_tensor *k_pool, const qsa_tensor *v_pool) {
  constexpr int64_t k24 = int64_t{1} << 24, k32 = int64_t{1} << 32;
  if (pd.slots >= k24) return false;
  auto fits = [&](int64_t ss, int64_t row) { return ss < k24 && (pd.slots - 1) * ss + row < k32; };
  const int64_t row = (pd.fmt == qsa::kFmtINT4 ? 128 : 256) * pd.eb;
  if (!fits(k_pool->stride[0] * pd.eb, row) || !fits(v_pool->stride[0] * pd.eb, row)) return false;
  if (pd.ks != nullptr) {
    const int64_t srow = (QSA_HEAD_DIM / pd.group) * (pd.scale_f16 ? 2 : 4);
    if (!fits(pd.ks_ss, srow) || !fits(pd.vs_ss, srow)) return false;
  }
  return true;
}

// The query's dtype, rank, head dim and batch size (checked before the pools).
qsa_status check_query(const char *fn, const qsa_tensor *q) {
  qsa_status st;
  if ((st = check_tensor(q, "q", QSA_DTYPE_BF16, 3, true, fn)) != QSA_OK) return st;
  if (q->shape[2] != QSA_HEAD_DIM)
    return fail(QSA_ERR_CONTRACT, "%s: head dim must be 256, q.shape[2] = %lld", fn,
                static_cast<long long>(q->shape[2]));
  if (q->shape[0] < 1 || q->shape[0] > QSA_MAX_BS)
    return fail(QSA_ERR_CONTRACT, "%s: bs must be in [1, 128], got %lld", fn,
                static_cast<long long>(q->shape[0]));
  return QSA_OK;
}

// Query, outputs and index lists of one decode call and the pool- and
// scratch-independent launch parameters (pool fields are left to the
// caller, the split scratch to attach_workspace / the scratch array).
qsa_status prepare_decode(const char *fn, const qsa_tensor *q, int64_t hkv,
                          const qsa_tensor *sel_indices, const qsa_tensor *cu_seqlens,
                          qsa_tensor *out, qsa_tensor *lse, qsa::Params *pp) {
  qsa_status st;
  if ((st = check_query(fn, q)) != QSA_OK) return st;
  const int64_t bs = q->shape[0], hq = q->shape[1];
  if (!((hq == 24 && hkv == 2) || (hq == 12 && hkv == 1)))
    return fail(QSA_ERR_CONTRACT,
                "%s: (Hq, Hkv) must be (24, 2) or (12, 1) (12:1 GQA), got (%lld, %lld)", fn,
                static_cast<long long>(hq), static_cast<long long>(hkv));
  if (!aligned16(q->data) || q->stride[0] % 8 || q->stride[1] % 8)
    return fail(QSA_ERR_CONTRACT, "%s: q rows must start on 16-byte boundaries", fn);

  if ((st = check_tensor(out, "out", QSA_DTYPE_BF16, 3, true, fn)) != QSA_OK) return st;
  if (out->shape[0] != bs || out->shape[1] != hq || out->shape[2] != QSA_HEAD_DIM)
    return fail(QSA_ERR_CONTRACT, "%s: out must be [bs, Hq, 256] like q", fn);
  if (!aligned16(out->data) || out->stride[0] % 8 || out->stride[1] % 8)
    return fail(QSA_ERR_CONTRACT, "%s: out rows must start on 16-byte boundaries", fn);
  // lse is written one float at a time: any strides
  if ((st = check_tensor(lse, "lse", QSA_DTYPE_F32, 2, false, fn)) != QSA_OK) return st;
  if (lse->shape[0] != bs || lse->shape[1] != hq)
    return fail(QSA_ERR_CONTRACT, "%s: lse must be [bs, Hq]", fn);

  if ((st = check_tensor(sel_indices, "sel_indices", QSA_DTYPE_I32, 1, true, fn)) != QSA_OK) return st;
  if ((st = check_tensor(cu_seqlens, "cu_seqlens", QSA_DTYPE_I32, 1, true, fn)) != QSA_OK) return st;
  if (cu_seqlens->shape[0] != bs + 1)
    return fail(QSA_ERR_CONTRACT, "%s: cu_seqlens must have bs + 1 = %lld entries, got %lld", fn,
                static_cast<long long>(bs + 1), static_cast<long long>(cu_seqlens->shape[0]));

  qsa::Params &p = *pp;
  p.q = static_cast<const __bf16 *>(q->data);
  p.q_sb = q->stride[0];
  p.q_sh = q->stride[1];
  p.sel = static_cast<const int32_t *>(sel_indices->data);
  p.n_sel = sel_indices->shape[0];
  p.cu = static_cast<const int32_t *>(cu_seqlens->data);
  p.out = static_cast<__bf16 *>(out->data);
  p.o_sb = out->stride[0];
  p.o_sh = out->stride[1];
  p.lse = static_cast<float *>(lse->data);
  p.l_sb = lse->stride[0];
  p.l_sh = lse->stride[1];
  p.bs = static_cast<int>(bs);
  p.hkv = static_cast<int>(hkv);
  p.nsplit = plan_splits(p.bs, p.hkv);
  p.min_split_keys = static_cast<int>(g_min_split_keys.load() > 4096 ? 4096 : g_min_split_keys.load());
  return QSA_OK;
}

// Split partials the plan of a prepared call needs.
int64_t partial_floats_of(const qsa::Params &p) {
  return static_cast<int64_t>(p.bs) * p.hkv * p.nsplit * qsa::kPartFloats;
}

// The split scratch of the workspace `stream` uses (created or grown
// outside capture) into a prepared call.
qsa_status attach_workspace(const char *fn, hipStream_t stream, qsa::Params *p) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QSA_ERR_HIP, "%s: no HIP device", fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(QSA_ERR_HIP, "%s: device id out of range", fn);
  Workspace *ws = nullptr;
  qsa_status st = ensure_workspace(dev, partial_floats_of(*p), stream, !stream_capturing(stream), &ws, fn);
  if (st != QSA_OK) return st;
  p->part = ws->part;
  p->ctr = ws->words;
  p->err = ws->words + kCtrWords;
  return QSA_OK;
}

// A tiered pool as validated for decode and store: the int8 ring (R rows,
// 64-channel f16 scales, owner table, and for a store the claim table) and
// the int4 pool (32-channel f16 scales).
struct TieredDesc {
  PoolDesc ring, cold;
};

qsa_status check_tiered(const char *fn, const qsa_tiered_pool *tp, bool want_claim, TieredDesc *d) {
  if (tp == nullptr) return fail(QSA_ERR_ARG, "%s: pool is NULL", fn);
  qsa_status st;
  if (tp->ring_k.dtype != QSA_DTYPE_I8 || tp->ring_v.dtype != QSA_DTYPE_I8)
    return fail(QSA_ERR_CONTRACT, "%s: ring_k / ring_v must be i8", fn);
  if (tp->cold_k.dtype != QSA_DTYPE_U4X2 || tp->cold_v.dtype != QSA_DTYPE_U4X2)
    return fail(QSA_ERR_CONTRACT, "%s: cold_k / cold_v must be u4x2", fn);
  for (const qsa_tensor *t : {&tp->ring_k_scale, &tp->ring_v_scale, &tp->cold_k_scale, &tp->cold_v_scale})
    if (t->dtype != QSA_DTYPE_F16)
      return fail(QSA_ERR_CONTRACT, "%s: tiered pool scales must be f16, got %s", fn, dtype_name(t->dtype));
  const qsa_kv_scales rs{tp->ring_k_scale, tp->ring_v_scale, 64};
  const qsa_kv_scales cs{tp->cold_k_scale, tp->cold_v_scale, 32};
  if ((st = check_pools(fn, &tp->ring_k, &tp->ring_v, &rs, &d->ring)) != QSA_OK) return st;
  if ((st = check_pools(fn, &tp->cold_k, &tp->cold_v, &cs, &d->cold)) != QSA_OK) return st;
  const int64_t r = d->ring.slots;
  if ((r & (r - 1)) != 0)
    return fail(QSA_ERR_CONTRACT, "%s: the ring must hold a power of two rows, got %lld", fn,
                static_cast<long long>(r));
  if (d->ring.hkv != d->cold.hkv)
    return fail(QSA_ERR_CONTRACT, "%s: ring and int4 pool hold different KV head counts", fn);
  if ((st = check_tensor(&tp->owner, "owner", QSA_DTYPE_I32, 1, true, fn)) != QSA_OK) return st;
  if (tp->owner.shape[0] != r)
    return fail(QSA_ERR_CONTRACT, "%s: owner must have one entry per ring row (%lld)", fn,
                static_cast<long long>(r));
  if (want_claim) {
    if ((st = check_tensor(&tp->claim, "claim", QSA_DTYPE_I32, 1, true, fn)) != QSA_OK) return st;
    if (tp->claim.shape[0] != r)
      return fail(QSA_ERR_CONTRACT, "%s: claim must have one entry per ring row (%lld)", fn,
                  static_cast<long long>(r));
  }
  return QSA_OK;
}

// New rows, slot ids and error word of one store call (pool fields are
// left to set_store_pool).
qsa_status prepare_store(const char *fn, const qsa_tensor *k_new, const qsa_tensor *v_new,
                         const qsa_tensor *loc, int64_t hkv, hipStream_t stream,
                         qsa::StoreParams *pp) {
  qsa_status st;
  if ((st = check_tensor(k_new, "k_new", QSA_DTYPE_BF16, 3, true, fn)) != QSA_OK) return st;
  if ((st = check_tensor(v_new, "v_new", QSA_DTYPE_BF16, 3, true, fn)) != QSA_OK) return st;
  const int64_t n = k_new->shape[0];
  for (const qsa_tensor *t : {k_new, v_new}) {
    if (t->shape[0] != n || t->shape[1] != hkv || t->shape[2] != QSA_HEAD_DIM)
      return fail(QSA_ERR_CONTRACT, "%s: k_new and v_new must be [n, Hkv, 256] = [%lld, %lld, 256]",
                  fn, static_cast<long long>(n), static_cast<long long>(hkv));
    if (!aligned16(t->data) || t->stride[0] % 8 || t->stride[1] % 8)
      return fail(QSA_ERR_CONTRACT, "%s: k_new / v_new rows must start on 16-byte boundaries", fn);
  }
  if (loc == nullptr) return fail(QSA_ERR_ARG, "%s: loc is NULL", fn);
  if (loc->dtype != QSA_DTYPE_I32 && loc->dtype != QSA_DTYPE_I64)
    return fail(QSA_ERR_CONTRACT, "%s: loc must be i32 or i64, got %s", fn, dtype_name(loc->dtype));
  if ((st = check_tensor(loc, "loc", loc->dtype, 1, true, fn)) != QSA_OK) return st;
  if (loc->shape[0] != n)
    return fail(QSA_ERR_CONTRACT, "%s: loc must have n = %lld entries, got %lld", fn,
                static_cast<long long>(n), static_cast<long long>(loc->shape[0]));
  if ((n * hkv + 3) / 4 > 0x7FFFFFFFLL)
    return fail(QSA_ERR_CONTRACT, "%s: n = %lld rows is too many for one launch", fn,
                static_cast<long long>(n));

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QSA_ERR_HIP, "%s: no HIP device", fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(QSA_ERR_HIP, "%s: device id out of range", fn);
  Workspace *ws = nullptr;  // only its sticky error word is used
  if ((st = ensure_workspace(dev, 0, stream, !stream_capturing(stream), &ws, fn)) != QSA_OK) return st;

  qsa::StoreParams &p = *pp;
  p.k = static_cast<const __bf16 *>(k_new->data);
  p.v = static_cast<const __bf16 *>(v_new->data);
  p.k_st = k_new->stride[0];
  p.k_sh = k_new->stride[1];
  p.v_st = v_new->stride[0];
  p.v_sh = v_new->stride[1];
  p.loc = loc->data;
  p.loc_i64 = loc->dtype == QSA_DTYPE_I64;
  p.n = n;
  p.hkv = static_cast<int>(hkv);
  p.err = ws->words + kCtrWords;
  return QSA_OK;
}

void set_store_pool(qsa::StoreParams *p, const PoolDesc &pd, const qsa_tensor *k_pool,
                    const qsa_tensor *v_pool) {
  p->kp = static_cast<uint8_t *>(k_pool->data);
  p->vp = static_cast<uint8_t *>(v_pool->data);
  p->kp_ss = k_pool->stride[0] * pd.eb;
  p->kp_sh = k_pool->stride[1] * pd.eb;
  p->vp_ss = v_pool->stride[0] * pd.eb;
  p->vp_sh = v_pool->stride[1] * pd.eb;
  p->ks = pd.ks;
  p->vs = pd.vs;
  p->ks_ss = pd.ks_ss;
  p->ks_sh = pd.ks_sh;
  p->vs_ss = pd.vs_ss;
  p->vs_sh = pd.vs_sh;
  p->scale_f16 = pd.scale_f16;
  p->group = pd.group;
  p->slots = pd.slots;
}

// Tiered pools: true when, for each of K, V and their scales, every ring
// and int4 row lies within 4 GiB above the lower of the two arrays' starts
// and row offsets are 24-bit x 24-bit products; then sets the common bases
// and the kernel addresses rows with 32-bit offsets.
bool tiered_fits_32(const qsa_tiered_pool *tp, const TieredDesc &td, qsa::Params *p) {
  constexpr int64_t k24 = int64_t{1} << 24, k32 = int64_t{1} << 32;
  if (td.ring.slots > k24 || td.cold.slots > k24) return false;
  const int64_t hkv = td.cold.hkv;
  struct Span {
    uintptr_t lo, hi;
  };
  // byte span of an array of `rows` rows (slot stride ss, head stride sh)
  auto span = [&](const void *data, int64_t rows, int64_t ss, int64_t sh, int64_t row, bool *ok) {
    if (ss >= k24) *ok = false;
    const uintptr_t lo = reinterpret_cast<uintptr_t>(data);
    return Span{lo, lo + static_cast<uintptr_t>((rows - 1) * ss + (hkv - 1) * sh + row)};
  };
  const uint8_t *bases[4];
  const qsa_tensor *rt[4] = {&tp->ring_k, &tp->ring_v, &tp->ring_k_scale, &tp->ring_v_scale};
  const qsa_tensor *ct[4] = {&tp->cold_k, &tp->cold_v, &tp->cold_k_scale, &tp->cold_v_scale};
  const int64_t eb[4] = {1, 1, 2, 2};
  const int64_t rrow[4] = {256, 256, 8, 8}, crow[4] = {128, 128, 16, 16};
  for (int a = 0; a < 4; ++a) {
    bool ok = true;
    const Span r = span(rt[a]->data, td.ring.slots, rt[a]->stride[0] * eb[a], rt[a]->stride[1] * eb[a], rrow[a], &ok);
    const Span c = span(ct[a]->data, td.cold.slots, ct[a]->stride[0] * eb[a], ct[a]->stride[1] * eb[a], crow[a], &ok);
    const uintptr_t lo = r.lo < c.lo ? r.lo : c.lo;
    const uintptr_t hi = r.hi > c.hi ? r.hi : c.hi;
    if (!ok || hi - lo > static_cast<uintptr_t>(k32)) return false;
    bases[a] = reinterpret_cast<const uint8_t *>(lo);
  }
  p->ring.kb = bases[0];
  p->ring.vb = bases[1];
  p->ring.ksb = bases[2];
  p->ring.vsb = bases[3];
  return true;
}

// Validated pools + the prepared call of qsa_decode / qsa_decode_noalloc
// (everything but the split scratch).
qsa_status prepare_pooled_decode(const char *fn, const qsa_tensor *q, const qsa_tensor *k_pool,
                                 const qsa_tensor *v_pool, const qsa_kv_scales *kv_scales,
                                 const qsa_tensor *sel_indices, const qsa_tensor *cu_seqlens,
                                 qsa_tensor *out, qsa_tensor *lse, qsa::Params *pp, PoolDesc *pd) {
  qsa_status st;
  if ((st = check_query(fn, q)) != QSA_OK) return st;
  if ((st = check_pools(fn, k_pool, v_pool, kv_scales, pd)) != QSA_OK) return st;
  if ((st = prepare_decode(fn, q, pd->hkv, sel_indices, cu_seqlens, out, lse, pp)) != QSA_OK) return st;
  qsa::Params &p = *pp;
  p.k = static_cast<const uint8_t *>(k_pool->data);
  p.v = static_cast<const uint8_t *>(v_pool->data);
  p.k_ss = k_pool->stride[0] * pd->eb;
  p.k_sh = k_pool->stride[1] * pd->eb;
  p.v_ss = v_pool->stride[0] * pd->eb;
  p.v_sh = v_pool->stride[1] * pd->eb;
  p.ks = pd->ks;
  p.vs = pd->vs;
  p.ks_ss = pd->ks_ss;
  p.ks_sh = pd->ks_sh;
  p.vs_ss = pd->vs_ss;
  p.vs_sh = pd->vs_sh;
  p.scale_f16 = pd->scale_f16;
  p.a32 = addresses_fit_32(*pd, k_pool, v_pool) ? 1 : 0;
  p.slots = pd->slots;
  p.waves = waves_for(pd->fmt, qsa::decode_workgroups(pd->fmt, p.bs, p.hkv, p.nsplit));
  return QSA_OK;
}

// ---- the scratch of qsa_decode_noalloc -------------------------------------
// A file-scope device array: split partials for at most kScratchPartFloats
// floats (8 MiB, enough for the default split plan of every bs and head
// layout: at most 6.2 MB), then the split counters and an error word.  The
// loader zero-fills it on every device, each split's counter is back at zero
// when its launch ends, and the first call on a device zeroes the words once
// more.  In host code `scratch` only names the array: its device address on
// each device comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is handed to kernels.
constexpr int64_t kScratchPartFloats = int64_t{2} << 20;
constexpr int64_t kScratchBytes = kScratchPartFloats * 4 + (kCtrWords + 1) * 4;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
uint8_t *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (taken, and its words
// zeroed on `stream`, on the first call per device; refused under capture).
qsa_status scratch_of_device(const char *fn, hipStream_t stream, uint8_t **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QSA_ERR_HIP, "%s: no HIP device", fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(QSA_ERR_HIP, "%s: device id out of range", fn);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    if (stream_capturing(stream))
      return fail(QSA_ERR_WORKSPACE, "%s: the first call on device %d must not be captured "
                  "(it sets up the device's scratch); call it once outside capture", fn, dev);
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(QSA_ERR_HIP, "%s: hipGetSymbolAddress of the scratch failed on device %d: %s", fn,
                  dev, hipGetErrorString(e));
    uint32_t *words = reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(ptr) + kScratchPartFloats * 4);
    if (qsa::launch_fill_u32(words, kCtrWords + 1, 0u, stream) != hipSuccess)
      return fail(QSA_ERR_HIP, "%s: zeroing the scratch counters failed", fn);
    g_scratch_ptr[dev] = static_cast<uint8_t *>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return QSA_OK;
}

}  // namespace

extern "C" {

int qsa_abi_version(void) { return QSA_ABI_VERSION; }

const char *qsa_last_error(void) { return g_last_error; }

qsa_status qsa_set_option(const char *name, int64_t value) {
  if (name == nullptr) return fail(QSA_ERR_ARG, "qsa_set_option: name is NULL");
  if (value < 0 || (value == 0 && strcmp(name, "split_target") != 0 && strcmp(name, "waves_per_workgroup") != 0 &&
                     strcmp(name, "splits") != 0 && strcmp(name, "xcc_lanes") != 0))
    return fail(QSA_ERR_ARG, "qsa_set_option: %s must be >= 1", name);
  if (!strcmp(name, "split_target")) {
    g_split_target = value;  // 0 restores the cost model
  } else if (!strcmp(name, "max_splits")) {
    if (value > 64) return fail(QSA_ERR_ARG, "qsa_set_option: max_splits must be <= 64");
    g_max_splits = value;
  } else if (!strcmp(name, "min_split_keys")) {
    g_min_split_keys = value;
  } else if (!strcmp(name, "waves_per_workgroup")) {
    if (value != 0 && value != 4 && value != 8) return fail(QSA_ERR_ARG, "qsa_set_option: waves_per_workgroup must be 0, 4 or 8");
    g_waves = value;
  } else if (!strcmp(name, "splits")) {
    if (value > 64) return fail(QSA_ERR_ARG, "qsa_set_option: splits must be <= 64");
    g_splits = value;
  } else if (!strcmp(name, "xcc_lanes")) {
    if (value > 1) return fail(QSA_ERR_ARG, "qsa_set_option: xcc_lanes must be 0 or 1");
    g_xcc_lanes = value;
  } else {
    return fail(QSA_ERR_ARG, "qsa_set_option: unknown option '%s'", name);
  }
  return ok();
}

qsa_status qsa_get_option(const char *name, int64_t *value) {
  if (name == nullptr || value == nullptr) return fail(QSA_ERR_ARG, "qsa_get_option: NULL argument");
  if (!strcmp(name, "split_target")) *value = g_split_target;
  else if (!strcmp(name, "max_splits")) *value = g_max_splits;
  else if (!strcmp(name, "min_split_keys")) *value = g_min_split_keys;
  else if (!strcmp(name, "waves_per_workgroup")) *value = g_waves;
  else if (!strcmp(name, "splits")) *value = g_splits;
  else if (!strcmp(name, "xcc_lanes")) *value = g_xcc_lanes;
  else if (!strcmp(name, "xcc_lanes_active")) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
      return fail(QSA_ERR_HIP, "qsa_get_option: no HIP device");
    std::lock_guard<std::mutex> lock(g_xcc_mutex);
    *value = g_xcc_state[dev] - 1;  // -1: not checked yet, 0: not used, 1: used
  }
  else return fail(QSA_ERR_ARG, "qsa_get_option: unknown option '%s'", name);
  return ok();
}

qsa_status qsa_plan(int bs, int hkv, int *splits, int *workgroups) {
  if (bs < 1 || bs > QSA_MAX_BS) return fail(QSA_ERR_CONTRACT, "qsa_plan: bs must be in [1, 128]");
  if (hkv != 1 && hkv != 2) return fail(QSA_ERR_CONTRACT, "qsa_plan: Hkv must be 1 or 2");
  const int s = plan_splits(bs, hkv);
  if (splits) *splits = s;
  if (workgroups) *workgroups = static_cast<int>(plan_workgroups(bs, hkv, s));
  return ok();
}

qsa_status qsa_decode(const qsa_tensor *q, const qsa_tensor *k_pool, const qsa_tensor *v_pool,
                      const qsa_kv_scales *kv_scales, const qsa_tensor *sel_indices,
                      const qsa_tensor *cu_seqlens, qsa_tensor *out, qsa_tensor *lse,
                      hipStream_t stream) {
  static const char *fn = "qsa_decode";
  qsa::Params p{};
  PoolDesc pd;
  qsa_status st = prepare_pooled_decode(fn, q, k_pool, v_pool, kv_scales, sel_indices, cu_seqlens,
                                        out, lse, &p, &pd);
  if (st != QSA_OK) return st;
  if ((st = attach_workspace(fn, stream, &p)) != QSA_OK) return st;
  p.xcc_lanes = xcc_lanes_for(stream);
  stamp_launch(&p, pd.fmt);
  const hipError_t e = qsa::launch_decode(p, pd.fmt, pd.group, stream);
  if (e != hipSuccess) return fail(QSA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

qsa_status qsa_decode_noalloc(const qsa_tensor *q, const qsa_tensor *k_pool,
                              const qsa_tensor *v_pool, const qsa_kv_scales *kv_scales,
                              const qsa_tensor *sel_indices, const qsa_tensor *cu_seqlens,
                              qsa_tensor *out, qsa_tensor *lse, hipStream_t stream) {
  static const char *fn = "qsa_decode_noalloc";
  qsa::Params p{};
  PoolDesc pd;
  qsa_status st = prepare_pooled_decode(fn, q, k_pool, v_pool, kv_scales, sel_indices, cu_seqlens,
                                        out, lse, &p, &pd);
  if (st != QSA_OK) return st;
  const int64_t need = partial_floats_of(p);
  if (need > kScratchPartFloats)
    return fail(QSA_ERR_WORKSPACE,
                "%s: the split plan (bs %d, %d KV heads, %d splits) needs %lld bytes of split "
                "partials, more than the %lld-byte scratch of this entry point; use qsa_decode",
                fn, p.bs, p.hkv, p.nsplit, static_cast<long long>(need * 4),
                static_cast<long long>(kScratchPartFloats * 4));
  uint8_t *base = nullptr;
  if ((st = scratch_of_device(fn, stream, &base)) != QSA_OK) return st;
  p.part = reinterpret_cast<float *>(base);
  p.ctr = reinterpret_cast<uint32_t *>(base + kScratchPartFloats * sizeof(float));
  p.err = p.ctr + kCtrWords;
  p.xcc_lanes = xcc_lanes_for(stream);
  stamp_launch(&p, pd.fmt);
  const hipError_t e = qsa::launch_decode(p, pd.fmt, pd.group, stream);
  if (e != hipSuccess) return fail(QSA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

qsa_status qsa_decode_tiered(const qsa_tensor *q, const qsa_tiered_pool *pool,
                             const qsa_tensor *sel_indices, const qsa_tensor *cu_seqlens,
                             qsa_tensor *out, qsa_tensor *lse, hipStream_t stream) {
  static const char *fn = "qsa_decode_tiered";
  qsa_status st;
  if ((st = check_query(fn, q)) != QSA_OK) return st;
  TieredDesc td;
  if ((st = check_tiered(fn, pool, false, &td)) != QSA_OK) return st;
  qsa::Params p{};
  if ((st = prepare_decode(fn, q, td.cold.hkv, sel_indices, cu_seqlens, out, lse, &p)) != QSA_OK)
    return st;
  if ((st = attach_workspace(fn, stream, &p)) != QSA_OK) return st;
  p.k = static_cast<const uint8_t *>(pool->cold_k.data);
  p.v = static_cast<const uint8_t *>(pool->cold_v.data);
  p.k_ss = pool->cold_k.stride[0];
  p.k_sh = pool->cold_k.stride[1];
  p.v_ss = pool->cold_v.stride[0];
  p.v_sh = pool->cold_v.stride[1];
  p.ks = td.cold.ks;
  p.vs = td.cold.vs;
  p.ks_ss = td.cold.ks_ss;
  p.ks_sh = td.cold.ks_sh;
  p.vs_ss = td.cold.vs_ss;
  p.vs_sh = td.cold.vs_sh;
  p.scale_f16 = 1;
  p.slots = td.cold.slots;
  p.ring.k = static_cast<const uint8_t *>(pool->ring_k.data);
  p.ring.v = static_cast<const uint8_t *>(pool->ring_v.data);
  p.ring.k_ss = pool->ring_k.stride[0];
  p.ring.k_sh = pool->ring_k.stride[1];
  p.ring.v_ss = pool->ring_v.stride[0];
  p.ring.v_sh = pool->ring_v.stride[1];
  p.ring.ks = td.ring.ks;
  p.ring.vs = td.ring.vs;
  p.ring.ks_ss = td.ring.ks_ss;
  p.ring.ks_sh = td.ring.ks_sh;
  p.ring.vs_ss = td.ring.vs_ss;
  p.ring.vs_sh = td.ring.vs_sh;
  p.ring.owner = static_cast<const int32_t *>(pool->owner.data);
  p.ring.mask = static_cast<uint32_t>(td.ring.slots - 1);
  p.a32 = tiered_fits_32(pool, td, &p) ? 1 : 0;
  p.waves = waves_for(qsa::kFmtTIERED, qsa::decode_workgroups(qsa::kFmtTIERED, p.bs, p.hkv, p.nsplit));
  p.xcc_lanes = xcc_lanes_for(stream);
  stamp_launch(&p, qsa::kFmtTIERED);
  const hipError_t e = qsa::launch_decode(p, qsa::kFmtTIERED, 32, stream);
  if (e != hipSuccess) return fail(QSA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

qsa_status qsa_kv_store(const qsa_tensor *k_new, const qsa_tensor *v_new, const qsa_tensor *loc,
                        qsa_tensor *k_pool, qsa_tensor *v_pool, const qsa_kv_scales *kv_scales,
                        hipStream_t stream) {
  static const char *fn = "qsa_kv_store";
  qsa_status st;
  PoolDesc pd;
  if ((st = check_pools(fn, k_pool, v_pool, kv_scales, &pd)) != QSA_OK) return st;
  qsa::StoreParams p{};
  if ((st = prepare_store(fn, k_new, v_new, loc, pd.hkv, stream, &p)) != QSA_OK) return st;
  set_store_pool(&p, pd, k_pool, v_pool);
  const hipError_t e = qsa::launch_store(p, pd.fmt, stream);
  if (e != hipSuccess) return fail(QSA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

qsa_status qsa_kv_store_tiered(const qsa_tensor *k_new, const qsa_tensor *v_new,
                               const qsa_tensor *loc, qsa_tiered_pool *pool, hipStream_t stream) {
  static const char *fn = "qsa_kv_store_tiered";
  qsa_status st;
  TieredDesc td;
  if ((st = check_tiered(fn, pool, true, &td)) != QSA_OK) return st;
  qsa::StoreParams p{};
  if ((st = prepare_store(fn, k_new, v_new, loc, td.cold.hkv, stream, &p)) != QSA_OK) return st;
  if (p.n > 0x7FFFFFFELL)
    return fail(QSA_ERR_CONTRACT, "%s: n = %lld tokens cannot be ranked in the int32 claim table",
                fn, static_cast<long long>(p.n));
  // 1. every token into the int4 pool
  set_store_pool(&p, td.cold, &pool->cold_k, &pool->cold_v);
  hipError_t e = qsa::launch_store(p, qsa::kFmtINT4, stream);
  // 2. the last token of the call per ring row claims it
  qsa::StoreParams r = p;
  r.claim = static_cast<int32_t *>(pool->claim.data);
  r.owner = static_cast<int32_t *>(pool->owner.data);
  r.ring_mask = static_cast<uint32_t>(td.ring.slots - 1);
  if (e == hipSuccess) e = qsa::launch_claim(r, stream);
  // 3. the claimed rows into the ring, with their owner stamps
  set_store_pool(&r, td.ring, &pool->ring_k, &pool->ring_v);
  r.slots = td.cold.slots;  // slot ids are checked against the full pool
  if (e == hipSuccess) e = qsa::launch_store(r, qsa::kFmtINT8, stream);
  if (e != hipSuccess) return fail(QSA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

qsa_status qsa_index(const qsa_tensor *q_index, const qsa_tensor *head_weights,
                     const qsa_tensor *k_index_pool, const qsa_tensor *block_table,
                     const qsa_tensor *req_to_token, const qsa_tensor *context_lens, int budget,
                     int compress_ratio, qsa_tensor *sel_out, qsa_tensor *cu_out,
                     hipStream_t stream) {
  static const char *fn = "qsa_index";
  qsa_status st;
  if ((st = check_tensor(q_index, "q_index", QSA_DTYPE_BF16, 3, true, fn)) != QSA_OK) return st;
  const int64_t bs = q_index->shape[0], hi = q_index->shape[1], di = q_index->shape[2];
  if (bs < 1 || bs > QSA_MAX_BS)
    return fail(QSA_ERR_CONTRACT, "%s: bs must be in [1, 128], got %lld", fn, static_cast<long long>(bs));
  if (hi < 1 || hi > 64)
    return fail(QSA_ERR_CONTRACT, "%s: index heads must be in [1, 64], got %lld", fn, static_cast<long long>(hi));
  if (di != 64 && di != 128)
    return fail(QSA_ERR_CONTRACT, "%s: index head dim must be 64 or 128, got %lld", fn, static_cast<long long>(di));
  if (!aligned16(q_index->data) || q_index->stride[0] % 8 || q_index->stride[1] % 8)
    return fail(QSA_ERR_CONTRACT, "%s: q_index rows must start on 16-byte boundaries", fn);
  if (head_weights != nullptr) {
    if ((st = check_tensor(head_weights, "head_weights", QSA_DTYPE_F32, 2, true, fn)) != QSA_OK) return st;
    if (head_weights->shape[0] != bs || head_weights->shape[1] != hi)
      return fail(QSA_ERR_CONTRACT, "%s: head_weights must be [bs, index heads]", fn);
  }
  if ((st = check_tensor(k_index_pool, "k_index_pool", QSA_DTYPE_BF16, 2, true, fn)) != QSA_OK) return st;
  if (k_index_pool->shape[0] < 1)
    return fail(QSA_ERR_CONTRACT, "%s: k_index_pool holds no rows", fn);
  if (k_index_pool->shape[1] != di)
    return fail(QSA_ERR_CONTRACT, "%s: k_index_pool rows must hold %lld elements like q_index", fn,
                static_cast<long long>(di));
  if (!aligned16(k_index_pool->data) || k_index_pool->stride[0] % 8)
    return fail(QSA_ERR_CONTRACT, "%s: k_index_pool rows must start on 16-byte boundaries", fn);
  if ((st = check_tensor(block_table, "block_table", QSA_DTYPE_I32, 2, true, fn)) != QSA_OK) return st;
  if ((st = check_tensor(req_to_token, "req_to_token", QSA_DTYPE_I32, 2, true, fn)) != QSA_OK) return st;
  if ((st = check_tensor(context_lens, "context_lens", QSA_DTYPE_I32, 1, true, fn)) != QSA_OK) return st;
  if (block_table->shape[0] != bs || req_to_token->shape[0] != bs || context_lens->shape[0] != bs)
    return fail(QSA_ERR_CONTRACT, "%s: block_table, req_to_token and context_lens need one row per q_index row", fn);
  if (req_to_token->shape[1] > QSA_INDEX_MAX_TOKENS)
    return fail(QSA_ERR_CONTRACT, "%s: req_to_token holds more than %d tokens per row", fn, QSA_INDEX_MAX_TOKENS);
  const int c = compress_ratio;
  if (c < 1 || c > 64)
    return fail(QSA_ERR_CONTRACT, "%s: compress_ratio must be in [1, 64], got %d", fn, c);
  if (budget < c || budget % c != 0 || budget + c - 1 > QSA_MAX_SEL)
    return fail(QSA_ERR_CONTRACT, "%s: budget must be a positive multiple of compress_ratio with "
                "budget + compress_ratio - 1 <= 2055, got budget %d, ratio %d", fn, budget, c);
  if (block_table->shape[1] > QSA_INDEX_MAX_TOKENS)
    return fail(QSA_ERR_CONTRACT, "%s: block_table holds more than %d blocks per row", fn, QSA_INDEX_MAX_TOKENS);
  if ((st = check_tensor(sel_out, "sel_out", QSA_DTYPE_I32, 1, true, fn)) != QSA_OK) return st;
  if (sel_out->shape[0] < bs * (budget + c - 1))
    return fail(QSA_ERR_CONTRACT, "%s: sel_out must hold bs * (budget + compress_ratio - 1) = %lld entries", fn,
                static_cast<long long>(bs * (budget + c - 1)));
  if ((st = check_tensor(cu_out, "cu_out", QSA_DTYPE_I32, 1, true, fn)) != QSA_OK) return st;
  if (cu_out->shape[0] != bs + 1)
    return fail(QSA_ERR_CONTRACT, "%s: cu_out must have bs + 1 entries", fn);

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QSA_ERR_HIP, "%s: no HIP device", fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(QSA_ERR_HIP, "%s: device id out of range", fn);
  const int64_t max_blocks = block_table->shape[1];
  Workspace *ws = nullptr;
  if ((st = ensure_index_scores(dev, bs * max_blocks, stream, !stream_capturing(stream), &ws, fn)) != QSA_OK)
    return st;

  qsa::IndexParams p{};
  p.q = static_cast<const __bf16 *>(q_index->data);
  p.q_sb = q_index->stride[0];
  p.q_sh = q_index->stride[1];
  p.w = head_weights ? static_cast<const float *>(head_weights->data) : nullptr;
  p.w_sb = head_weights ? head_weights->stride[0] : 0;
  p.k = static_cast<const __bf16 *>(k_index_pool->data);
  p.k_ss = k_index_pool->stride[0];
  p.n_k = k_index_pool->shape[0];
  p.bt = static_cast<const int32_t *>(block_table->data);
  p.bt_sb = block_table->stride[0];
  p.max_blocks = static_cast<int>(max_blocks);
  p.r2t = static_cast<const int32_t *>(req_to_token->data);
  p.r2t_sb = req_to_token->stride[0];
  p.max_tokens = static_cast<int>(req_to_token->shape[1]);
  p.ctx = static_cast<const int32_t *>(context_lens->data);
  p.bs = static_cast<int>(bs);
  p.hi = static_cast<int>(hi);
  p.di = static_cast<int>(di);
  p.budget = budget;
  p.c = c;
  p.scores = ws->iscores;
  p.sel = static_cast<int32_t *>(sel_out->data);
  p.cu = static_cast<int32_t *>(cu_out->data);
  p.err = ws->words + kCtrWords;
  const hipError_t e = qsa::launch_index(p, stream);
  if (e != hipSuccess) return fail(QSA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

qsa_status qsa_index_reserve(int max_bs, int max_blocks, hipStream_t stream) {
  static const char *fn = "qsa_index_reserve";
  if (max_bs < 1 || max_bs > QSA_MAX_BS) return fail(QSA_ERR_CONTRACT, "%s: max_bs must be in [1, 128]", fn);
  if (max_blocks < 0 || max_blocks > QSA_INDEX_MAX_TOKENS)
    return fail(QSA_ERR_CONTRACT, "%s: max_blocks must be in [0, %d]", fn, QSA_INDEX_MAX_TOKENS);
  if (stream_capturing(stream)) return fail(QSA_ERR_WORKSPACE, "%s: called while the stream is capturing", fn);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return fail(QSA_ERR_HIP, "%s: no HIP device", fn);
  Workspace *ws = nullptr;
  qsa_status st = ensure_index_scores(dev, static_cast<int64_t>(max_bs) * max_blocks, stream, true, &ws, fn);
  return st == QSA_OK ? ok() : st;
}

qsa_status qsa_workspace_reserve(int max_bs, int hq, int hkv, hipStream_t stream) {
  if (max_bs < 1 || max_bs > QSA_MAX_BS)
    return fail(QSA_ERR_CONTRACT, "qsa_workspace_reserve: max_bs must be in [1, 128]");
  if (!((hq == 24 && hkv == 2) || (hq == 12 && hkv == 1)))
    return fail(QSA_ERR_CONTRACT, "qsa_workspace_reserve: (Hq, Hkv) must be (24, 2) or (12, 1)");
  if (stream_capturing(stream))
    return fail(QSA_ERR_WORKSPACE, "qsa_workspace_reserve: called while the stream is capturing");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(QSA_ERR_HIP, "qsa_workspace_reserve: no HIP device");
  Workspace *ws = nullptr;
  qsa_status st = ensure_workspace(dev, part_floats_needed(max_bs, hkv), stream, true, &ws);
  if (st != QSA_OK) return st;
  if (qsa::launch_fill_u32(ws->words, kCtrWords + 1, 0u, stream) != hipSuccess)
    return fail(QSA_ERR_HIP, "qsa_workspace_reserve: zeroing the counters failed");
  return ok();
}

qsa_status qsa_workspace_attach(hipStream_t stream) {
  static const char *fn = "qsa_workspace_attach";
  if (stream_capturing(stream)) return fail(QSA_ERR_WORKSPACE, "%s: called while the stream is capturing", fn);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(QSA_ERR_HIP, "%s: no HIP device", fn);
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  if (attached_slot(dev, stream) >= 0) return ok();
  DeviceWorkspaces &d = g_ws[dev];
  for (int i = 0; i < kMaxAttached; ++i) {
    if (d.used[i]) continue;
    d.own[i] = Workspace{};
    d.stream[i] = stream;
    d.used[i] = true;
    return ok();
  }
  return fail(QSA_ERR_WORKSPACE, "%s: device %d already has %d streams with their own workspace", fn,
              dev, kMaxAttached);
}

qsa_status qsa_workspace_detach(hipStream_t stream) {
  static const char *fn = "qsa_workspace_detach";
  if (stream_capturing(stream)) return fail(QSA_ERR_WORKSPACE, "%s: called while the stream is capturing", fn);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(QSA_ERR_HIP, "%s: no HIP device", fn);
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  const int i = attached_slot(dev, stream);
  if (i < 0) return ok();
  DeviceWorkspaces &d = g_ws[dev];
  if (d.own[i].words != nullptr || d.own[i].iscores != nullptr) {
    if (hipStreamSynchronize(stream) != hipSuccess) return fail(QSA_ERR_HIP, "%s: hipStreamSynchronize failed", fn);
    free_workspace(d.own[i]);
  }
  d.used[i] = false;
  d.stream[i] = nullptr;
  return ok();
}

qsa_status qsa_workspace_reset(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(QSA_ERR_HIP, "qsa_workspace_reset: no HIP device");
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace &ws = workspace_of(dev, stream);
  if (ws.words == nullptr) return ok();
  if (qsa::launch_fill_u32(ws.words, kCtrWords + 1, 0u, stream) != hipSuccess)
    return fail(QSA_ERR_HIP, "qsa_workspace_reset: zeroing the counters failed");
  return ok();
}

qsa_status qsa_workspace_release(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) cur = -1;
  for (int dev = 0; dev < kMaxDevices; ++dev) {
    DeviceWorkspaces &d = g_ws[dev];
    bool any = d.shared.words != nullptr || d.shared.iscores != nullptr;
    for (int i = 0; i < kMaxAttached; ++i) any = any || d.used[i];
    if (!any) continue;
    if (hipSetDevice(dev) == hipSuccess && hipDeviceSynchronize() == hipSuccess) {
      free_workspace(d.shared);
      for (int i = 0; i < kMaxAttached; ++i) free_workspace(d.own[i]);
    }
    d = DeviceWorkspaces{};
  }
  if (cur >= 0) (void)hipSetDevice(cur);
  return ok();
}

int64_t qsa_workspace_bytes(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  auto bytes = [](const Workspace &ws) {
    return ws.part_floats * 4 + (ws.words ? (kCtrWords + 1) * 4 : 0) + ws.iscore_floats * 4 +
           ws.retired_bytes;
  };
  const DeviceWorkspaces &d = g_ws[dev];
  int64_t total = bytes(d.shared);
  for (int i = 0; i < kMaxAttached; ++i)
    if (d.used[i]) total += bytes(d.own[i]);
  return total;
}

qsa_status qsa_debug_counters(const uint32_t **dev_ptr, int *n, hipStream_t stream) {
  if (dev_ptr == nullptr || n == nullptr) return fail(QSA_ERR_ARG, "qsa_debug_counters: NULL argument");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(QSA_ERR_HIP, "qsa_debug_counters: no HIP device");
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  const Workspace &ws = workspace_of(dev, stream);
  if (ws.words == nullptr) return fail(QSA_ERR_WORKSPACE, "qsa_debug_counters: no workspace yet");
  *dev_ptr = ws.words;
  *n = static_cast<int>(ws.n_ctr);
  return ok();
}

qsa_status qsa_debug_read_counters(uint32_t *host, int n, hipStream_t stream) {
  const uint32_t *ctr = nullptr;
  int total = 0;
  qsa_status st = qsa_debug_counters(&ctr, &total, stream);
  if (st != QSA_OK) return st;
  if (host == nullptr || n < 0 || n > total)
    return fail(QSA_ERR_ARG, "qsa_debug_read_counters: n must be in [0, %d]", total);
  if (hipMemcpyAsync(host, ctr, sizeof(uint32_t) * n, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail(QSA_ERR_HIP, "qsa_debug_read_counters: copy failed");
  return ok();
}

qsa_status qsa_debug_audit_counters(uint32_t *dev_accum, hipStream_t stream) {
  const uint32_t *ctr = nullptr;
  int total = 0;
  qsa_status st = qsa_debug_counters(&ctr, &total, stream);
  if (st != QSA_OK) return st;
  if (dev_accum == nullptr) return fail(QSA_ERR_ARG, "qsa_debug_audit_counters: NULL accumulator");
  if (qsa::launch_audit(ctr, total, dev_accum, stream) != hipSuccess)
    return fail(QSA_ERR_HIP, "qsa_debug_audit_counters: launch failed");
  return ok();
}

qsa_status qsa_debug_device_error(uint32_t *host_word, hipStream_t stream) {
  if (host_word == nullptr) return fail(QSA_ERR_ARG, "qsa_debug_device_error: NULL argument");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(QSA_ERR_HIP, "qsa_debug_device_error: no HIP device");
  uint32_t *word = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    const Workspace &ws = workspace_of(dev, stream);
    if (ws.words == nullptr) {
      *host_word = 0;
      return ok();
    }
    word = ws.words + kCtrWords;
  }
  if (hipMemcpyAsync(host_word, word, sizeof(uint32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail(QSA_ERR_HIP, "qsa_debug_device_error: copy failed");
  return ok();
}

#ifdef QSA_PHASE_STAMPS
int qsa_debug_set_phase_stamps(void *buf, int64_t words) {
  g_stamps = static_cast<uint64_t *>(buf);
  g_stamp_words = buf != nullptr && words > 0 ? words : 0;
  return 0;
}
#endif

}  // extern "C"
