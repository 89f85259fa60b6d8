// abi_host_check.hip -- drives the host side of libqsa (contract checks,
// split plan, options, workspace bookkeeping, error strings) in a process
// built with AddressSanitizer and UndefinedBehaviorSanitizer on the host
// code.  The kernels are not linked: the launch functions below stand in
// for them and only count calls, so the check runs without a GPU (without
// one, every call that passes validation stops at its first HIP call with
// QSA_ERR_HIP).  Exit status 0 when every expectation holds.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "qsa.h"
#include "../../sparse_index_paged_amd/csrc/qsa_internal.h"

namespace qsa {
static int g_launches = 0;
hipError_t launch_decode(const Params &, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_store(const StoreParams &, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_claim(const StoreParams &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_index(const IndexParams &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fill_u32(uint32_t *, int64_t, uint32_t, hipStream_t) { return hipSuccess; }
hipError_t launch_audit(const uint32_t *, int, uint32_t *, hipStream_t) { return hipSuccess; }
hipError_t launch_xcc_probe(int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t read_xcc_probe(int32_t *, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace qsa

static int g_fail = 0;
#define EXPECT(cond, ...)                                        \
  do {                                                           \
    if (!(cond)) {                                               \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);  \
      std::fprintf(stderr, __VA_ARGS__);                         \
      std::fprintf(stderr, "\n");                                \
      ++g_fail;                                                  \
    }                                                            \
  } while (0)

// Fake device addresses: 16-byte aligned host memory the library never reads.
static unsigned char g_fake[1 << 16] __attribute__((aligned(256)));

static qsa_tensor T(std::initializer_list<int64_t> shape, int32_t dtype, void *data = g_fake) {
  qsa_tensor t{};
  t.data = data;
  t.dtype = dtype;
  t.ndim = static_cast<int32_t>(shape.size());
  int i = 0;
  for (int64_t n : shape) t.shape[i++] = n;
  int64_t acc = 1;
  for (int d = t.ndim - 1; d >= 0; --d) {
    t.stride[d] = acc;
    acc *= t.shape[d];
  }
  return t;
}

struct Decode {
  qsa_tensor q = T({4, 24, 256}, QSA_DTYPE_BF16);
  qsa_tensor k = T({64, 2, 256}, QSA_DTYPE_BF16);
  qsa_tensor v = T({64, 2, 256}, QSA_DTYPE_BF16);
  qsa_tensor sel = T({100}, QSA_DTYPE_I32);
  qsa_tensor cu = T({5}, QSA_DTYPE_I32);
  qsa_tensor out = T({4, 24, 256}, QSA_DTYPE_BF16);
  qsa_tensor lse = T({4, 24}, QSA_DTYPE_F32);
  qsa_kv_scales sc{};
  bool scales = false;
  qsa_status run() {
    return qsa_decode(&q, &k, &v, scales ? &sc : nullptr, &sel, &cu, &out, &lse, nullptr);
  }
};

static void expect_status(qsa_status got, qsa_status want, const char *what, const char *needle) {
  EXPECT(got == want, "%s: status %d, expected %d (%s)", what, got, want, qsa_last_error());
  if (needle != nullptr && got != QSA_OK)
    EXPECT(std::strstr(qsa_last_error(), needle) != nullptr, "%s: message '%s' lacks '%s'", what,
           qsa_last_error(), needle);
  if (got != QSA_OK) EXPECT(qsa_last_error()[0] != '\0', "%s: empty error message", what);
}

// A call that passes validation: QSA_OK with a device, QSA_ERR_HIP without.
static bool accepted(qsa_status st) { return st == QSA_OK || st == QSA_ERR_HIP; }

static void decode_contract() {
  { Decode d; qsa_status st = d.run(); EXPECT(accepted(st), "valid bf16 call: %d %s", st, qsa_last_error()); }
  { Decode d; d.q.dtype = QSA_DTYPE_F16; expect_status(d.run(), QSA_ERR_CONTRACT, "q dtype", "q must be bf16"); }
  { Decode d; d.q.shape[2] = 128; expect_status(d.run(), QSA_ERR_CONTRACT, "head dim", "head dim"); }
  { Decode d; d.q.shape[0] = 0; expect_status(d.run(), QSA_ERR_CONTRACT, "bs 0", "bs must be"); }
  { Decode d; d.q.shape[0] = 129; expect_status(d.run(), QSA_ERR_CONTRACT, "bs 129", "bs must be"); }
  { Decode d; d.q.shape[1] = 12; expect_status(d.run(), QSA_ERR_CONTRACT, "gqa", "(Hq, Hkv)"); }
  { Decode d; d.v.dtype = QSA_DTYPE_I8; expect_status(d.run(), QSA_ERR_CONTRACT, "mixed pools", "share a format"); }
  { Decode d; d.k.shape[1] = 3; d.v.shape[1] = 3; expect_status(d.run(), QSA_ERR_CONTRACT, "hkv 3", "1 or 2 KV heads"); }
  { Decode d; d.k.data = g_fake + 8; expect_status(d.run(), QSA_ERR_CONTRACT, "pool align", "16-byte"); }
  { Decode d; d.q.data = nullptr; expect_status(d.run(), QSA_ERR_ARG, "null q", "NULL"); }
  { Decode d; expect_status(qsa_decode(&d.q, nullptr, &d.v, nullptr, &d.sel, &d.cu, &d.out, &d.lse, nullptr),
                            QSA_ERR_ARG, "null pool", "NULL"); }
  { Decode d; d.cu.shape[0] = 4; expect_status(d.run(), QSA_ERR_CONTRACT, "cu length", "cu_seqlens"); }
  { Decode d; d.sel.dtype = QSA_DTYPE_I64; expect_status(d.run(), QSA_ERR_CONTRACT, "sel dtype", "sel_indices"); }
  { Decode d; d.out.shape[1] = 12; expect_status(d.run(), QSA_ERR_CONTRACT, "out shape", "out must be"); }
  { Decode d; d.lse.shape[0] = 3; expect_status(d.run(), QSA_ERR_CONTRACT, "lse shape", "lse must be"); }
  { Decode d; d.q.stride[2] = 2; expect_status(d.run(), QSA_ERR_CONTRACT, "q last dim", "contiguous"); }
  { Decode d; d.k.dtype = d.v.dtype = QSA_DTYPE_FP8_E4M3FN; expect_status(d.run(), QSA_ERR_CONTRACT, "fp8 no scales", "kv_scales"); }
  { Decode d; d.scales = true; d.sc.k_scale = T({64, 2, 1}, QSA_DTYPE_F32); d.sc.v_scale = d.sc.k_scale;
    d.sc.group_size = 256; expect_status(d.run(), QSA_ERR_CONTRACT, "bf16 with scales", "no scales"); }
  for (int fmt : {QSA_DTYPE_FP8_E4M3FN, QSA_DTYPE_I8, QSA_DTYPE_U4X2}) {
    for (int group : {16, 32, 64, 128, 256}) {
      for (int sdt : {QSA_DTYPE_F32, QSA_DTYPE_F16, QSA_DTYPE_BF16}) {
        Decode d;
        const int64_t row = fmt == QSA_DTYPE_U4X2 ? 128 : 256;
        d.k = T({64, 2, row}, fmt);
        d.v = T({64, 2, row}, fmt);
        d.scales = true;
        d.sc.k_scale = T({64, 2, 256 / group}, sdt);
        d.sc.v_scale = T({64, 2, 256 / group}, sdt);
        d.sc.group_size = group;
        const bool gok = fmt == QSA_DTYPE_U4X2 ? (group == 32 || group == 64)
                                               : (group == 32 || group == 64 || group == 256);
        const bool ok = gok && sdt != QSA_DTYPE_BF16;
        const qsa_status st = d.run();
        if (ok)
          EXPECT(accepted(st), "fmt %d g%d sdt %d: %d %s", fmt, group, sdt, st, qsa_last_error());
        else
          EXPECT(st == QSA_ERR_CONTRACT, "fmt %d g%d sdt %d accepted", fmt, group, sdt);
      }
    }
  }
}

// qsa_decode_noalloc validates exactly like qsa_decode, and refuses plans
// whose partials exceed its fixed scratch.
static void noalloc_contract() {
  Decode d;
  qsa_status st = qsa_decode_noalloc(&d.q, &d.k, &d.v, nullptr, &d.sel, &d.cu, &d.out, &d.lse, nullptr);
  EXPECT(accepted(st), "noalloc valid call: %d %s", st, qsa_last_error());
  d.q.shape[0] = 0;
  expect_status(qsa_decode_noalloc(&d.q, &d.k, &d.v, nullptr, &d.sel, &d.cu, &d.out, &d.lse, nullptr),
                QSA_ERR_CONTRACT, "noalloc bs 0", "bs must be");
  Decode big;
  big.q = T({128, 24, 256}, QSA_DTYPE_BF16);
  big.out = T({128, 24, 256}, QSA_DTYPE_BF16);
  big.lse = T({128, 24}, QSA_DTYPE_F32);
  big.cu = T({129}, QSA_DTYPE_I32);
  EXPECT(qsa_set_option("splits", 64) == QSA_OK && qsa_set_option("max_splits", 64) == QSA_OK, "options");
  expect_status(qsa_decode_noalloc(&big.q, &big.k, &big.v, nullptr, &big.sel, &big.cu, &big.out, &big.lse, nullptr),
                QSA_ERR_WORKSPACE, "noalloc over the scratch", "scratch");
  EXPECT(qsa_set_option("splits", 0) == QSA_OK && qsa_set_option("max_splits", 16) == QSA_OK, "options");
  // the default plan of every bs fits the scratch
  for (int bs = 1; bs <= 128; ++bs)
    for (int hkv = 1; hkv <= 2; ++hkv) {
      int s = 0;
      EXPECT(qsa_plan(bs, hkv, &s, nullptr) == QSA_OK, "plan");
      EXPECT(static_cast<int64_t>(bs) * hkv * s * qsa::kPartFloats <= (int64_t{2} << 20),
             "default plan bs %d hkv %d exceeds the noalloc scratch", bs, hkv);
    }
}

static void store_contract() {
  qsa_tensor kn = T({8, 2, 256}, QSA_DTYPE_BF16), vn = kn;
  qsa_tensor kp = T({64, 2, 256}, QSA_DTYPE_I8), vp = kp;
  qsa_kv_scales sc{T({64, 2, 4}, QSA_DTYPE_F16), T({64, 2, 4}, QSA_DTYPE_F16), 64};
  for (int dt : {QSA_DTYPE_I32, QSA_DTYPE_I64, QSA_DTYPE_F32}) {
    qsa_tensor loc = T({8}, dt);
    qsa_status st = qsa_kv_store(&kn, &vn, &loc, &kp, &vp, &sc, nullptr);
    if (dt == QSA_DTYPE_F32)
      expect_status(st, QSA_ERR_CONTRACT, "loc f32", "loc must be");
    else
      EXPECT(accepted(st), "store loc dtype %d: %d %s", dt, st, qsa_last_error());
  }
  qsa_tensor loc = T({7}, QSA_DTYPE_I32);
  expect_status(qsa_kv_store(&kn, &vn, &loc, &kp, &vp, &sc, nullptr), QSA_ERR_CONTRACT, "loc length", "loc must have");
  qsa_tensor kn1 = T({8, 1, 256}, QSA_DTYPE_BF16);
  loc = T({8}, QSA_DTYPE_I32);
  expect_status(qsa_kv_store(&kn1, &vn, &loc, &kp, &vp, &sc, nullptr), QSA_ERR_CONTRACT, "k_new heads", "k_new");
  qsa_tensor empty = T({0, 2, 256}, QSA_DTYPE_BF16), loc0 = T({0}, QSA_DTYPE_I32);
  EXPECT(accepted(qsa_kv_store(&empty, &empty, &loc0, &kp, &vp, &sc, nullptr)), "n = 0 store");
}

static qsa_tiered_pool tiered(int64_t ring_rows) {
  qsa_tiered_pool tp{};
  tp.ring_k = T({ring_rows, 2, 256}, QSA_DTYPE_I8);
  tp.ring_v = tp.ring_k;
  tp.ring_k_scale = T({ring_rows, 2, 4}, QSA_DTYPE_F16);
  tp.ring_v_scale = tp.ring_k_scale;
  tp.owner = T({ring_rows}, QSA_DTYPE_I32);
  tp.claim = T({ring_rows}, QSA_DTYPE_I32);
  tp.cold_k = T({512, 2, 128}, QSA_DTYPE_U4X2);
  tp.cold_v = tp.cold_k;
  tp.cold_k_scale = T({512, 2, 8}, QSA_DTYPE_F16);
  tp.cold_v_scale = tp.cold_k_scale;
  return tp;
}

static void tiered_contract() {
  Decode d;
  qsa_tiered_pool tp = tiered(64);
  EXPECT(accepted(qsa_decode_tiered(&d.q, &tp, &d.sel, &d.cu, &d.out, &d.lse, nullptr)), "tiered decode: %s", qsa_last_error());
  qsa_tiered_pool bad = tiered(48);
  expect_status(qsa_decode_tiered(&d.q, &bad, &d.sel, &d.cu, &d.out, &d.lse, nullptr), QSA_ERR_CONTRACT,
                "ring 48", "power of two");
  bad = tiered(64);
  bad.owner.shape[0] = 32;
  expect_status(qsa_decode_tiered(&d.q, &bad, &d.sel, &d.cu, &d.out, &d.lse, nullptr), QSA_ERR_CONTRACT,
                "owner length", "owner");
  bad = tiered(64);
  bad.cold_k_scale.dtype = QSA_DTYPE_F32;
  expect_status(qsa_decode_tiered(&d.q, &bad, &d.sel, &d.cu, &d.out, &d.lse, nullptr), QSA_ERR_CONTRACT,
                "f32 scales", "f16");
  qsa_tensor kn = T({8, 2, 256}, QSA_DTYPE_BF16), loc = T({8}, QSA_DTYPE_I64);
  EXPECT(accepted(qsa_kv_store_tiered(&kn, &kn, &loc, &tp, nullptr)), "tiered store: %s", qsa_last_error());
  bad = tiered(64);
  bad.claim.shape[0] = 63;
  expect_status(qsa_kv_store_tiered(&kn, &kn, &loc, &bad, nullptr), QSA_ERR_CONTRACT, "claim length", "claim");
  expect_status(qsa_decode_tiered(&d.q, nullptr, &d.sel, &d.cu, &d.out, &d.lse, nullptr), QSA_ERR_ARG,
                "null pool", "NULL");
}

static void index_contract() {
  qsa_tensor q = T({4, 8, 128}, QSA_DTYPE_BF16), w = T({4, 8}, QSA_DTYPE_F32);
  qsa_tensor k = T({1000, 128}, QSA_DTYPE_BF16), bt = T({4, 300}, QSA_DTYPE_I32);
  qsa_tensor r2t = T({4, 1200}, QSA_DTYPE_I32), ctx = T({4}, QSA_DTYPE_I32);
  qsa_tensor sel = T({4 * 2051}, QSA_DTYPE_I32), cu = T({5}, QSA_DTYPE_I32);
  EXPECT(accepted(qsa_index(&q, &w, &k, &bt, &r2t, &ctx, 2048, 4, &sel, &cu, nullptr)), "index: %s", qsa_last_error());
  EXPECT(accepted(qsa_index(&q, nullptr, &k, &bt, &r2t, &ctx, 2048, 4, &sel, &cu, nullptr)), "index no w");
  expect_status(qsa_index(&q, &w, &k, &bt, &r2t, &ctx, 2050, 4, &sel, &cu, nullptr), QSA_ERR_CONTRACT,
                "budget", "budget");
  expect_status(qsa_index(&q, &w, &k, &bt, &r2t, &ctx, 2048, 65, &sel, &cu, nullptr), QSA_ERR_CONTRACT,
                "ratio", "compress_ratio");
  qsa_tensor q96 = T({4, 8, 96}, QSA_DTYPE_BF16);
  expect_status(qsa_index(&q96, &w, &k, &bt, &r2t, &ctx, 2048, 4, &sel, &cu, nullptr), QSA_ERR_CONTRACT,
                "di", "head dim");
  qsa_tensor small = T({100}, QSA_DTYPE_I32);
  expect_status(qsa_index(&q, &w, &k, &bt, &r2t, &ctx, 2048, 4, &small, &cu, nullptr), QSA_ERR_CONTRACT,
                "sel_out", "sel_out");
  EXPECT(qsa_index_reserve(0, 10, nullptr) == QSA_ERR_CONTRACT, "index reserve bs 0");
}

static void plan_and_options() {
  for (int bs = 1; bs <= 128; ++bs)
    for (int hkv = 1; hkv <= 2; ++hkv) {
      int s = 0, w = 0;
      EXPECT(qsa_plan(bs, hkv, &s, &w) == QSA_OK, "plan %d %d", bs, hkv);
      EXPECT(s >= 1 && s <= 9 && w == ((bs * hkv + 7) / 8) * 8 * s, "plan %d %d = %d %d", bs, hkv, s, w);
    }
  EXPECT(qsa_plan(0, 2, nullptr, nullptr) == QSA_ERR_CONTRACT, "plan bs 0");
  EXPECT(qsa_plan(4, 3, nullptr, nullptr) == QSA_ERR_CONTRACT, "plan hkv 3");
  int64_t v = -1;
  EXPECT(qsa_set_option("splits", 7) == QSA_OK && qsa_get_option("splits", &v) == QSA_OK && v == 7, "splits option");
  int s = 0;
  EXPECT(qsa_plan(128, 2, &s, nullptr) == QSA_OK && s == 7, "forced splits");
  EXPECT(qsa_set_option("splits", 0) == QSA_OK, "reset splits");
  EXPECT(qsa_set_option("nope", 1) == QSA_ERR_ARG, "unknown option");
  EXPECT(qsa_set_option(nullptr, 1) == QSA_ERR_ARG, "null option");
  EXPECT(qsa_set_option("max_splits", 65) == QSA_ERR_ARG, "max_splits 65");
  EXPECT(qsa_set_option("waves_per_workgroup", 6) == QSA_ERR_ARG, "waves 6");
  EXPECT(qsa_get_option("nope", &v) == QSA_ERR_ARG, "get unknown");
  EXPECT(qsa_get_option("splits", nullptr) == QSA_ERR_ARG, "get null");
}

static void workspace_and_debug() {
  EXPECT(qsa_workspace_reserve(0, 24, 2, nullptr) == QSA_ERR_CONTRACT, "reserve bs 0");
  EXPECT(qsa_workspace_reserve(8, 24, 1, nullptr) == QSA_ERR_CONTRACT, "reserve heads");
  EXPECT(qsa_workspace_release() == QSA_OK, "release");
  EXPECT(qsa_workspace_bytes() >= 0, "bytes");
  EXPECT(qsa_debug_counters(nullptr, nullptr, nullptr) == QSA_ERR_ARG, "counters null");
  EXPECT(qsa_debug_device_error(nullptr, nullptr) == QSA_ERR_ARG, "device error null");
  EXPECT(qsa_debug_audit_counters(nullptr, nullptr) != QSA_OK, "audit null");
  EXPECT(qsa_abi_version() == QSA_ABI_VERSION, "abi version");
}

// The error message is thread-local: threads failing in different ways
// each read back their own message.
static void thread_local_errors() {
  std::vector<std::thread> threads;
  std::vector<int> bad(8, 0);
  for (int i = 0; i < 8; ++i)
    threads.emplace_back([i, &bad] {
      for (int r = 0; r < 200; ++r) {
        Decode d;
        d.q.shape[0] = (i % 2) ? 0 : 129;
        const char *want = "bs must be";
        if (i % 4 == 2) { d.q.shape[0] = 4; d.q.shape[2] = 64; want = "head dim"; }
        if (d.run() != QSA_ERR_CONTRACT || std::strstr(qsa_last_error(), want) == nullptr) ++bad[i];
        int s = 0;
        if (qsa_plan(1 + (r % 128), 1 + (i % 2), &s, nullptr) != QSA_OK || qsa_last_error()[0] != '\0') ++bad[i];
      }
    });
  for (auto &t : threads) t.join();
  for (int i = 0; i < 8; ++i) EXPECT(bad[i] == 0, "thread %d saw %d wrong results", i, bad[i]);
}

int main() {
  decode_contract();
  noalloc_contract();
  store_contract();
  tiered_contract();
  index_contract();
  plan_and_options();
  workspace_and_debug();
  thread_local_errors();
  std::printf("abi_host_check: %s (%d failures, %d stub launches)\n", g_fail ? "FAILED" : "ok", g_fail,
              qsa::g_launches);
  return g_fail ? 1 : 0;
}
