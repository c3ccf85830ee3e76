// Host side of the C ABI declared in include/rlk.h: argument validation,
// workspace layout and kernel launches.  Everything is enqueued on the
// caller's stream; nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "rlk.h"
#include "rlk_bench.h"
#include "rlk_kernels.h"
#include "rlk_tiles_w8.h"

namespace {

thread_local std::string g_last_error;

rlk_status fail(rlk_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
rlk_status fail(rlk_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

rlk_status ok() {
  g_last_error.clear();
  return RLK_OK;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Limits that keep every 32-bit index inside the kernels in range.
constexpr int64_t kMaxT = int64_t(1) << 24;
constexpr int64_t kMaxH = 1 << 16;
constexpr int64_t kMaxV = 8000000;  // 32 splits x chunks stay within one grid dimension
constexpr int64_t kMaxGemmMN = int64_t(1) << 24;
constexpr int64_t kMaxGemmK = int64_t(1) << 20;  // 255 rows x K x 2 bytes stay below 2^32

struct Geom {
  int64_t V, S, cps, S_pad;
};

Geom geom_of(int64_t V_global) {
  Geom g;
  g.V = V_global;
  g.S = ceil_div(V_global, rlk::kNSplit);
  g.cps = ceil_div(g.S, rlk::kChunk);
  g.S_pad = g.cps * rlk::kChunk;
  return g;
}

// --- workspace layouts -------------------------------------------------------
struct FwdWs {
  size_t idx, yA, n_act, zt, hA, rec, total;
  int64_t rec_chunks, T_pad;
};

// Record slots: one per (chunk of the full vocabulary of V rows, row).
FwdWs fwd_layout(int64_t T, int64_t H, int64_t V) {
  FwdWs w;
  w.T_pad = ceil_div(std::max<int64_t>(T, 1), rlk::kBM) * rlk::kBM;
  size_t off = 0;
  w.idx = off;
  off = align256(off + sizeof(int32_t) * T);
  w.yA = off;
  off = align256(off + sizeof(int32_t) * T);
  w.n_act = off;
  off = align256(off + sizeof(int32_t));
  w.zt = off;
  off = align256(off + sizeof(float) * T);
  w.hA = off;
  off = align256(off + 2 * (size_t)w.T_pad * H);
  w.rec_chunks = rlk::kNSplit * geom_of(V).cps;
  w.rec = off;
  off = align256(off + sizeof(float2) * (size_t)w.rec_chunks * (size_t)T);
  w.total = off;
  return w;
}

// Splits per backward group: the largest power of two G <= 32 whose dz
// block (T_pad x G x S_pad bf16) fits the budget (default 2.5 GiB, env
// RLK_DZ_BUDGET_MB overrides it, at most 3.5 GiB).  G changes no result
// bit, only the workspace size and the number of launches.  The cap keeps
// the per-lane byte offsets of a 256-row dz tile (255 rows x G x S_pad x
// 2 B, less than the block since T_pad >= 256) inside the 32 unsigned bits
// the tile loaders use.
int64_t dz_budget_bytes() {
  constexpr int64_t kMaxBudget = int64_t(3584) << 20;
  const char* e = std::getenv("RLK_DZ_BUDGET_MB");
  if (e && *e) {
    const long long mb = std::atoll(e);
    if (mb > 0) return std::min<int64_t>((int64_t)mb << 20, kMaxBudget);
  }
  return (int64_t)2560 << 20;
}

struct BwdWs {
  size_t idx, n_act, rowinfo, hA, dZ, ghacc, total;
  int64_t T_pad, S_pad, G;
};

BwdWs bwd_layout(int64_t T, int64_t H, int64_t V) {
  const Geom g = geom_of(V);
  BwdWs w;
  w.T_pad = ceil_div(std::max<int64_t>(T, 1), rlk::kBM) * rlk::kBM;
  w.S_pad = ceil_div(g.S, 64) * 64;
  const int64_t per_split = 2 * w.T_pad * w.S_pad;
  const int64_t budget = dz_budget_bytes();
  w.G = 1;
  while (w.G < rlk::kNSplit && 2 * w.G * per_split <= budget) w.G *= 2;
  size_t off = 0;
  w.idx = off;
  off = align256(off + sizeof(int32_t) * T);
  w.n_act = off;
  off = align256(off + sizeof(int32_t));
  w.rowinfo = off;
  off = align256(off + 16 * (size_t)w.T_pad);
  w.hA = off;
  off = align256(off + 2 * (size_t)w.T_pad * H);
  w.dZ = off;
  off = align256(off + (size_t)per_split * w.G);
  w.ghacc = off;
  if (w.G < rlk::kNSplit) off = align256(off + 4 * (size_t)T * H);
  w.total = off;
  return w;
}

// --- device check ----------------------------------------------------------------
std::mutex g_dev_mu;
int g_dev_ok[64];   // 0 unknown, 1 gfx950, -1 other
int g_dev_cus[64];  // compute units of a checked device

rlk_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RLK_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(RLK_ERR_UNSUPPORTED_DEVICE, "device index %d", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(RLK_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    g_dev_ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_dev_cus[dev] = prop.multiProcessorCount;
    if (g_dev_ok[dev] < 0) return fail(RLK_ERR_UNSUPPORTED_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  }
  if (g_dev_ok[dev] < 0) return fail(RLK_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
  return RLK_OK;
}

// Compute units of the current device (after check_device succeeded on it).
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  return g_dev_cus[dev] > 0 ? g_dev_cus[dev] : 256;
}

// grad_h in two row passes (gradh_tile's kPart) when its whole tiles would
// leave most compute units idle while each runs the vocabulary-long chain:
// a pass's chain takes ~70 % of a tile's and the passes add ~40 % to
// grad_h's work, which pays while three times the tile count fits on the
// units (the grad_W tiles fill the rest).  The environment variable
// RLK_GRAD_H_PASSES = 0 / 1 forces either form (results are the same bits;
// tests use it).
bool grad_h_passes(int64_t row_tiles, int64_t n_tiles) {
  const char* e = std::getenv("RLK_GRAD_H_PASSES");
  if (e && *e) return std::atoi(e) != 0;
  return 3 * row_tiles * n_tiles <= device_cus();
}

// Tile grids stay within the 2^31 - 1 threads a launch holds along x
// (checked for the larger of the two block sizes).  Row-wise kernels take
// at most kRowBlocks blocks and stride over the rows.
constexpr int64_t kRowBlocks = int64_t(1) << 22;  // 256-thread blocks: 2^30 threads
constexpr int64_t kRowBlocksY = 65535;            // the limit along y
rlk_status check_grid(int64_t blocks) {
  if (blocks * std::max(rlk::kThreads, rlk::kThreadsW8) > (int64_t)INT32_MAX)
    return fail(RLK_ERR_BAD_SHAPE, "problem needs %lld tile blocks, more than one launch holds", (long long)blocks);
  return RLK_OK;
}

rlk_status launched(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RLK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return RLK_OK;
}

// --- optional per-kernel timing (rlk_profile_begin / rlk_profile_end) ---------
struct ProfRec {
  const char* name;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
// read without the lock on every launch: when timing is off (the normal
// case) a launch takes no lock at all
std::atomic<bool> g_prof_on{false};
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one launch with events on its stream when timing is enabled.
struct ProfScope {
  const char* name;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
  ProfScope(const char* n, hipStream_t s) : name(n), st(s) {
    if (!g_prof_on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on.load(std::memory_order_relaxed)) return;
    a = prof_event();
    b = prof_event();
    if (a && b) {
      (void)hipEventRecord(a, st);
    } else {  // event creation failed: this launch goes untimed
      if (a) g_prof_pool.push_back(a);
      if (b) g_prof_pool.push_back(b);
      a = b = nullptr;
    }
  }
  ~ProfScope() {
    if (!a || !b) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    (void)hipEventRecord(b, st);
    g_prof_recs.push_back(ProfRec{name, a, b});
  }
};

#define RLK_TRY(x)                  \
  do {                              \
    rlk_status _s = (x);            \
    if (_s != RLK_OK) return _s;    \
  } while (0)

// Launch a kernel on stream `st`, timed when profiling is on; return on error.
#define RLK_LAUNCH(kern, grid, block, st, ...)                        \
  do {                                                                \
    {                                                                 \
      ProfScope _ps(#kern, st);                                       \
      hipLaunchKernelGGL(rlk::kern, grid, block, 0, st, __VA_ARGS__); \
    }                                                                 \
    RLK_TRY(launched(#kern));                                         \
  } while (0)

// Same for a kernel given as a function pointer, timed under `name`.
#define RLK_LAUNCH_FN(name, fn, grid, block, st, ...)           \
  do {                                                          \
    {                                                           \
      ProfScope _ps(name, st);                                  \
      hipLaunchKernelGGL(fn, grid, block, 0, st, __VA_ARGS__);  \
    }                                                           \
    RLK_TRY(launched(name));                                    \
  } while (0)

// Same for a launch made by a launcher of the eight-wave unit
// (rlk_tiles_w8.h), timed under `name`.
#define RLK_LAUNCH_W8(name, launcher, grid, st, args) \
  do {                                                \
    {                                                 \
      ProfScope _ps(name, st);                        \
      rlk::launcher(grid, st, args);                  \
    }                                                 \
    RLK_TRY(launched(name));                          \
  } while (0)

// Shapes first; with T == 0 there is nothing to read or write, so the
// pointers are not checked (empty tensors may carry NULL).
rlk_status check_common(const void* h, const void* W, const int32_t* y, int64_t T, int64_t H, int64_t V) {
  if (T < 0 || T > kMaxT) return fail(RLK_ERR_BAD_SHAPE, "T=%lld out of [0, 2^24]", (long long)T);
  if (H <= 0 || H > kMaxH || H % 64 != 0)
    return fail(RLK_ERR_BAD_SHAPE, "H=%lld must be a positive multiple of 64 up to 65536", (long long)H);
  if (V <= 0 || V > kMaxV) return fail(RLK_ERR_BAD_SHAPE, "V=%lld out of [1, 8000000]", (long long)V);
  if (T == 0) return RLK_OK;
  if (!h || !W || !y) return fail(RLK_ERR_NULL_ARG, "h, W and y are required");
  if (!aligned16(h) || !aligned16(W) || !aligned16(y)) return fail(RLK_ERR_BAD_ALIGNMENT, "h, W, y must be 16-byte aligned");
  return RLK_OK;
}

// Split range [s0, s0 + n) of an aligned vocabulary block, or an error.
rlk_status split_range(int64_t vocab_start, int64_t vocab_len, int64_t V_global, int* s0, int* n) {
  const Geom g = geom_of(V_global);
  if (vocab_start < 0 || vocab_len <= 0 || vocab_start + vocab_len > V_global)
    return fail(RLK_ERR_UNALIGNED_VOCAB_RANGE, "range [%lld, +%lld) not inside [0, %lld)", (long long)vocab_start,
                (long long)vocab_len, (long long)V_global);
  int64_t nn = 1;
  while (nn * g.S < vocab_len) nn <<= 1;
  if (nn > rlk::kNSplit || vocab_start % (nn * g.S) != 0 ||
      vocab_len != std::min(vocab_start + nn * g.S, V_global) - vocab_start)
    return fail(RLK_ERR_UNALIGNED_VOCAB_RANGE,
                "range [%lld, +%lld) is not an aligned block of splits (split width %lld)", (long long)vocab_start,
                (long long)vocab_len, (long long)g.S);
  *s0 = (int)(vocab_start / g.S);
  *n = (int)nn;
  return RLK_OK;
}

// Shared forward body: statistics of splits [s0, s0+n) then the epilogue.
rlk_status run_forward(const void* h, const void* W, const int32_t* y, int64_t T, int64_t H, int64_t V_global,
                       int32_t ignore_index, int s0, int nsplit, int64_t vocab_start, int64_t vocab_len, int mode,
                       float* logp, float* lse, rlk_lse_partial_t* pout, void* ws, hipStream_t st,
                       float* zsave = nullptr, int64_t ldzs = 0, const rlk::RlLossArgs* rl = nullptr) {
  const Geom g = geom_of(V_global);
  const FwdWs L = fwd_layout(T, H, V_global);
  char* base = static_cast<char*>(ws);
  int32_t* idx = reinterpret_cast<int32_t*>(base + L.idx);
  int32_t* yA = reinterpret_cast<int32_t*>(base + L.yA);
  int32_t* n_act = reinterpret_cast<int32_t*>(base + L.n_act);
  float* zt = reinterpret_cast<float*>(base + L.zt);
  uint16_t* hA = reinterpret_cast<uint16_t*>(base + L.hA);
  float2* rec = reinterpret_cast<float2*>(base + L.rec);
  rlk::PartialRec* pr = reinterpret_cast<rlk::PartialRec*>(pout);

  RLK_LAUNCH(compact_rows, dim3(1), dim3(1024), st, y, (int)T, ignore_index, idx, yA, n_act,
             mode == 0 ? logp : nullptr, mode == 0 ? lse : nullptr, mode == 1 ? pr : nullptr,
             rl ? rl->loss : nullptr, rl ? rl->g : nullptr);
  RLK_LAUNCH(gather_rows, dim3((unsigned)std::min(L.T_pad, kRowBlocks)), dim3(256), st,
             static_cast<const uint16_t*>(h), idx, n_act, (int)L.T_pad, (int)H, (int)V_global, y, nullptr, nullptr, hA,
             nullptr);

  rlk::SplitGeom gm;
  gm.V = (int)g.V;
  gm.S = (int)g.S;
  gm.cps = (int)g.cps;
  gm.s0 = s0;
  gm.vocab_start = (int)vocab_start;
  rlk::FwdArgs fa;
  fa.hA = hA;
  fa.W = static_cast<const uint16_t*>(W);
  fa.yA = yA;
  fa.idx = idx;
  fa.n_act = n_act;
  fa.H = (int)H;
  fa.nsplit = nsplit;
  fa.gm = gm;
  fa.tg.tps = (int)ceil_div(g.S, rlk::kBN);
  fa.rec_stride = (size_t)T;
  fa.rec = rec;
  fa.zt = zt;
  // grid: every row tile of T (the kernel keeps those of active rows)
  const int64_t fwd_blocks = 8 * ceil_div(ceil_div(T, rlk::kBM) * nsplit * fa.tg.tps, 8);
  RLK_TRY(check_grid(fwd_blocks));
  fa.zsave = zsave;
  fa.ldzs = ldzs;
  fa.zs_spad = (int)ceil_div(g.S, 64) * 64;
  // batches of at most 96 rows: one row tile whose rows >= 32 * skinny are
  // padding (the same bits, less work; see gemm_kk).  Not for 97..128 rows:
  // there the first wave row does all its MFMAs anyway, and merging the
  // full accumulator set across the per-wave engine copies spills.
  const int skinny = (!zsave && rlk::kWaves == 4 && T <= 3 * 32) ? (int)ceil_div(T, 32) : 0;
  const dim3 grid((unsigned)fwd_blocks), block(rlk::kThreads);
  if (zsave) RLK_LAUNCH_FN("fwd_tiles", (rlk::fwd_tiles<true, 0>), grid, block, st, fa);
  else if (skinny == 1) RLK_LAUNCH_FN("fwd_tiles", (rlk::fwd_tiles<false, 1>), grid, block, st, fa);
  else if (skinny == 2) RLK_LAUNCH_FN("fwd_tiles", (rlk::fwd_tiles<false, 2>), grid, block, st, fa);
  else if (skinny == 3) RLK_LAUNCH_FN("fwd_tiles", (rlk::fwd_tiles<false, 3>), grid, block, st, fa);
  else RLK_LAUNCH_W8("fwd_tiles", launch_fwd_tiles_w8, grid, st, fa);

  rlk::RlLossArgs rla{};  // no fused objective unless rl is given
  if (rl) rla = *rl;
  RLK_LAUNCH(merge_splits, dim3((unsigned)ceil_div(T, rlk::kMergeRows)), dim3(rlk::kMergeRows * rlk::kNSplit), st, rec,
             (size_t)T, zt, idx, n_act, y, gm, nsplit, mode, (int)vocab_start, (int)(vocab_start + vocab_len), logp, lse,
             pr, rla);
  return RLK_OK;
}

}  // namespace

extern "C" {

// Version 2: 16 x 16 x 32 MFMA steps (the default engine); 1: 32 x 32 x 16.
int32_t rlk_contract_version(void) { return rlk::kBlk == 16 ? 2 : 1; }
static_assert(rlk::kBlk != 16 || RLK_CONTRACT_VERSION == 2, "the default build implements the header's version");

const char* rlk_status_string(rlk_status s) {
  switch (s) {
    case RLK_OK: return "ok";
    case RLK_ERR_NULL_ARG: return "a required pointer is NULL";
    case RLK_ERR_BAD_SHAPE: return "invalid shape";
    case RLK_ERR_BAD_ALIGNMENT: return "pointer not 16-byte aligned";
    case RLK_ERR_UNALIGNED_VOCAB_RANGE: return "vocabulary range is not an aligned block of splits";
    case RLK_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case RLK_ERR_HIP: return "HIP runtime error";
    case RLK_ERR_UNSUPPORTED_DEVICE: return "device is not gfx950";
    case RLK_ERR_BAD_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

const char* rlk_last_error_message(void) { return g_last_error.c_str(); }

size_t rlk_workspace_bytes(int32_t op, int64_t T, int64_t H, int64_t V) {
  if (T < 0 || T > kMaxT || H <= 0 || H > kMaxH || H % 64 != 0 || V <= 0 || V > kMaxV) return 0;
  switch (op) {
    case RLK_OP_FWD:
    case RLK_OP_PARTIAL: return fwd_layout(T, H, V).total;
    case RLK_OP_BWD: return bwd_layout(T, H, V).total;
    default: return 0;
  }
}

rlk_status rlk_linear_logp_fwd(const void* h, const void* W, const int32_t* y, int64_t T, int64_t H, int64_t V,
                               int32_t ignore_index, float* logp, float* lse, void* ws, size_t ws_bytes,
                               void* stream) {
  RLK_TRY(check_common(h, W, y, T, H, V));
  if (T == 0) return ok();
  if (!logp || !ws) return fail(RLK_ERR_NULL_ARG, "logp and ws are required");
  if (!aligned16(logp) || (lse && !aligned16(lse)) || !aligned16(ws))
    return fail(RLK_ERR_BAD_ALIGNMENT, "logp, lse, ws must be 16-byte aligned");
  if (ws_bytes < fwd_layout(T, H, V).total)
    return fail(RLK_ERR_WORKSPACE_TOO_SMALL, "need %zu bytes, got %zu", fwd_layout(T, H, V).total, ws_bytes);
  RLK_TRY(check_device());
  RLK_TRY(run_forward(h, W, y, T, H, V, ignore_index, 0, rlk::kNSplit, 0, V, 0, logp, lse, nullptr, ws,
                      static_cast<hipStream_t>(stream)));
  return ok();
}

rlk_status rlk_lse_partial(const void* h, const void* W_shard, const int32_t* y, int64_t T, int64_t H,
                           int64_t vocab_start, int64_t vocab_len, int64_t V_global, int32_t ignore_index,
                           rlk_lse_partial_t* out, void* ws, size_t ws_bytes, void* stream) {
  RLK_TRY(check_common(h, W_shard, y, T, H, V_global));
  int s0 = 0, n = 0;
  RLK_TRY(split_range(vocab_start, vocab_len, V_global, &s0, &n));
  if (T == 0) return ok();
  if (!out || !ws) return fail(RLK_ERR_NULL_ARG, "out and ws are required");
  if (!aligned16(out) || !aligned16(ws)) return fail(RLK_ERR_BAD_ALIGNMENT, "out, ws must be 16-byte aligned");
  if (ws_bytes < fwd_layout(T, H, V_global).total)
    return fail(RLK_ERR_WORKSPACE_TOO_SMALL, "need %zu bytes, got %zu", fwd_layout(T, H, V_global).total, ws_bytes);
  RLK_TRY(check_device());
  RLK_TRY(run_forward(h, W_shard, y, T, H, V_global, ignore_index, s0, n, vocab_start, vocab_len, 1, nullptr, nullptr,
                      out, ws, static_cast<hipStream_t>(stream)));
  return ok();
}

rlk_status rlk_lse_merge(const rlk_lse_partial_t* parts, int32_t n_parts, const int32_t* y, int64_t T,
                         int32_t ignore_index, float* logp, float* lse, void* stream) {
  if (n_parts < 1 || n_parts > rlk::kNSplit) return fail(RLK_ERR_BAD_ARG, "n_parts=%d out of [1, 32]", n_parts);
  if (T < 0 || T > kMaxT) return fail(RLK_ERR_BAD_SHAPE, "T=%lld out of [0, 2^24]", (long long)T);
  if (T == 0) return ok();
  if (!parts || !y || !logp) return fail(RLK_ERR_NULL_ARG, "parts, y and logp are required");
  if (!aligned16(parts) || !aligned16(y) || !aligned16(logp) || (lse && !aligned16(lse)))
    return fail(RLK_ERR_BAD_ALIGNMENT, "parts, y, logp, lse must be 16-byte aligned");
  RLK_TRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  RLK_LAUNCH(merge_parts, dim3((unsigned)ceil_div(T, 256)), dim3(256), st,
             reinterpret_cast<const rlk::PartialRec*>(parts), n_parts, (int)T, y, ignore_index, logp, lse);
  return ok();
}

}  // extern "C"

namespace {

// Shared backward body: dz per group of splits (recomputed tiles, or from
// the forward's saved logits when zsave != NULL), then grad_h / grad_W.
rlk_status run_backward(const void* h, const void* W, const int32_t* y, const float* lse, const float* g,
                        const float* zsave, int64_t ldzs, int64_t T, int64_t H, int64_t V, int32_t ignore_index,
                        void* grad_h, float* grad_W, void* ws, size_t ws_bytes, void* stream) {
  RLK_TRY(check_common(h, W, y, T, H, V));
  if (T == 0) return ok();
  if (!lse || !g || !ws) return fail(RLK_ERR_NULL_ARG, "lse, g and ws are required");
  if (!aligned16(lse) || !aligned16(g) || !aligned16(ws) || (grad_h && !aligned16(grad_h)) ||
      (grad_W && !aligned16(grad_W)))
    return fail(RLK_ERR_BAD_ALIGNMENT, "lse, g, ws, grad_h, grad_W must be 16-byte aligned");
  const BwdWs L = bwd_layout(T, H, V);
  if (ws_bytes < L.total) return fail(RLK_ERR_WORKSPACE_TOO_SMALL, "need %zu bytes, got %zu", L.total, ws_bytes);
  if (!grad_h && !grad_W) return ok();
  RLK_TRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Geom gg = geom_of(V);
  char* base = static_cast<char*>(ws);
  int32_t* idx = reinterpret_cast<int32_t*>(base + L.idx);
  int32_t* n_act = reinterpret_cast<int32_t*>(base + L.n_act);
  float4* rowinfo = reinterpret_cast<float4*>(base + L.rowinfo);
  uint16_t* dZ = reinterpret_cast<uint16_t*>(base + L.dZ);
  uint16_t* hA = reinterpret_cast<uint16_t*>(base + L.hA);
  float* ghacc = reinterpret_cast<float*>(base + L.ghacc);
  const uint16_t* hb = static_cast<const uint16_t*>(h);
  const uint16_t* Wb = static_cast<const uint16_t*>(W);

  RLK_LAUNCH(compact_rows, dim3(1), dim3(1024), st, y, (int)T, ignore_index, idx, nullptr, n_act, nullptr, nullptr,
             nullptr, nullptr, nullptr);
  RLK_LAUNCH(gather_rows, dim3((unsigned)std::min(L.T_pad, kRowBlocks)), dim3(256), st, hb, idx, n_act, (int)L.T_pad,
             (int)H, (int)V, y, lse, g, hA, rowinfo);
  if (grad_h) {
    RLK_LAUNCH(zero_rows, dim3((unsigned)std::min(T, kRowBlocks)), dim3(256), st, y, (int)T, ignore_index, (int)H,
               static_cast<uint16_t*>(grad_h));
  }
  rlk::SplitGeom gm;
  gm.V = (int)gg.V;
  gm.S = (int)gg.S;
  gm.cps = (int)gg.cps;
  gm.s0 = 0;
  gm.vocab_start = 0;
  int last_split = 0;
  for (int c = 0; c < rlk::kNSplit; ++c)
    if ((int64_t)c * gg.S < V) last_split = c;
  const int tps = (int)ceil_div(gg.S, rlk::kBN);
  const int64_t row_tiles = ceil_div(T, rlk::kBM);
  const int n_tiles = (int)ceil_div(H, rlk::kBN);
  const int G = (int)L.G;
  // grids: every row tile of T (the kernels keep those of active rows)
  const int64_t dz_blocks = 8 * ceil_div(row_tiles * G * tps, 8);
  const bool passes = grad_h && grad_h_passes(row_tiles, n_tiles);
  const int64_t gh_blocks = grad_h ? 8 * ceil_div(row_tiles * n_tiles * (passes ? 2 : 1), 8) : 0;
  const int64_t gw_blocks = grad_W ? 8 * ceil_div((int64_t)n_tiles * G * tps, 8) : 0;
  RLK_TRY(check_grid(dz_blocks));
  RLK_TRY(check_grid(gh_blocks + gw_blocks));
  for (int c_lo = 0; c_lo <= last_split; c_lo += G) {
    rlk::BwdGeom bg;
    bg.c_lo = c_lo;
    bg.G = G;
    bg.S_pad = (int)L.S_pad;
    bg.ldz = (int)(G * L.S_pad);
    bg.T_pad = (int)L.T_pad;

    rlk::DzArgs da;
    da.hA = hA;
    da.W = Wb;
    da.rowinfo = rowinfo;
    da.n_act = n_act;
    da.H = (int)H;
    da.gm = gm;
    da.tg.tps = tps;
    da.bg = bg;
    da.dZ = dZ;
    if (zsave)
      RLK_LAUNCH(dz_saved, dim3((unsigned)ceil_div(bg.ldz / 8, 256), (unsigned)std::min(L.T_pad, kRowBlocksY)),
                 dim3(256), st, zsave, ldzs, idx, rowinfo, n_act, gm, bg, dZ);
    else
      RLK_LAUNCH_W8("dz_tiles", launch_dz_tiles_w8, dim3((unsigned)dz_blocks), st, da);

    rlk::GradWArgs wa;
    wa.dZ = dZ;
    wa.hA = hA;
    wa.n_act = n_act;
    wa.H = (int)H;
    wa.gm = gm;
    wa.bg = bg;
    wa.tps = tps;
    wa.n_tiles = n_tiles;
    wa.grad_W = grad_W;
    rlk::GradHArgs ha;
    ha.dZ = dZ;
    ha.W = Wb;
    ha.idx = idx;
    ha.n_act = n_act;
    ha.H = (int)H;
    ha.gm = gm;
    ha.bg = bg;
    ha.n_tiles = n_tiles;
    ha.ghacc = ghacc;
    ha.grad_h = static_cast<uint16_t*>(grad_h);
    const bool first = c_lo == 0, last = c_lo + G > last_split;
    {
      ProfScope _ps("grad_tiles", st);
      rlk::launch_grad_tiles_w8(first, last, passes, dim3((unsigned)(gh_blocks + gw_blocks)), st, ha, wa);
    }
    RLK_TRY(launched("grad_tiles"));
  }
  return ok();
}

}  // namespace

extern "C" {

rlk_status rlk_linear_logp_bwd(const void* h, const void* W, const int32_t* y, const float* lse, const float* g,
                               int64_t T, int64_t H, int64_t V, int32_t ignore_index, void* grad_h, float* grad_W,
                               void* ws, size_t ws_bytes, void* stream) {
  return run_backward(h, W, y, lse, g, nullptr, 0, T, H, V, ignore_index, grad_h, grad_W, ws, ws_bytes, stream);
}

int64_t rlk_saved_logits_ld(int64_t V) {
  if (V <= 0 || V > kMaxV) return 0;
  return rlk::kNSplit * ceil_div(geom_of(V).S, 64) * 64;
}

rlk_status rlk_linear_logp_fwd_save(const void* h, const void* W, const int32_t* y, int64_t T, int64_t H, int64_t V,
                                    int32_t ignore_index, float* logp, float* lse, float* zsave, int64_t ldzs,
                                    void* ws, size_t ws_bytes, void* stream) {
  RLK_TRY(check_common(h, W, y, T, H, V));
  if (T == 0) return ok();
  if (!logp || !lse || !zsave || !ws) return fail(RLK_ERR_NULL_ARG, "logp, lse, zsave and ws are required");
  if (!aligned16(logp) || !aligned16(lse) || !aligned16(zsave) || !aligned16(ws))
    return fail(RLK_ERR_BAD_ALIGNMENT, "logp, lse, zsave, ws must be 16-byte aligned");
  if (ldzs < rlk_saved_logits_ld(V) || ldzs % 4 != 0)
    return fail(RLK_ERR_BAD_SHAPE, "ldzs=%lld must be a multiple of 4 and >= %lld", (long long)ldzs,
                (long long)rlk_saved_logits_ld(V));
  if (ws_bytes < fwd_layout(T, H, V).total)
    return fail(RLK_ERR_WORKSPACE_TOO_SMALL, "need %zu bytes, got %zu", fwd_layout(T, H, V).total, ws_bytes);
  RLK_TRY(check_device());
  RLK_TRY(run_forward(h, W, y, T, H, V, ignore_index, 0, rlk::kNSplit, 0, V, 0, logp, lse, nullptr, ws,
                      static_cast<hipStream_t>(stream), zsave, ldzs));
  return ok();
}

rlk_status rlk_linear_logp_bwd_saved(const void* h, const void* W, const int32_t* y, const float* lse, const float* g,
                                     const float* zsave, int64_t ldzs, int64_t T, int64_t H, int64_t V,
                                     int32_t ignore_index, void* grad_h, float* grad_W, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (T > 0) {
    if (!zsave) return fail(RLK_ERR_NULL_ARG, "zsave is required");
    if (!aligned16(zsave)) return fail(RLK_ERR_BAD_ALIGNMENT, "zsave must be 16-byte aligned");
    if (ldzs < rlk_saved_logits_ld(V) || ldzs % 4 != 0)
      return fail(RLK_ERR_BAD_SHAPE, "ldzs=%lld must be a multiple of 4 and >= %lld", (long long)ldzs,
                  (long long)rlk_saved_logits_ld(V));
  }
  return run_backward(h, W, y, lse, g, zsave, ldzs, T, H, V, ignore_index, grad_h, grad_W, ws, ws_bytes, stream);
}

rlk_status rlk_gemm_bf16_nt(const void* A, const void* B, int64_t M, int64_t N, int64_t K, void* C, int64_t ldc,
                            int32_t c_dtype, void* stream) {
  if (M < 0 || N < 0 || M > kMaxGemmMN || N > kMaxGemmMN)
    return fail(RLK_ERR_BAD_SHAPE, "M=%lld N=%lld out of [0, 2^24]", (long long)M, (long long)N);
  if (K <= 0 || K % 64 != 0 || K > kMaxGemmK)
    return fail(RLK_ERR_BAD_SHAPE, "K=%lld must be a positive multiple of 64 up to 2^20", (long long)K);
  if (c_dtype != RLK_DT_F32 && c_dtype != RLK_DT_BF16) return fail(RLK_ERR_BAD_ARG, "c_dtype=%d", c_dtype);
  if (M == 0 || N == 0) return ok();
  if (ldc < N || ldc % 4 != 0) return fail(RLK_ERR_BAD_SHAPE, "ldc=%lld must be >= N and a multiple of 4", (long long)ldc);
  if (!A || !B || !C) return fail(RLK_ERR_NULL_ARG, "A, B and C are required");
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return fail(RLK_ERR_BAD_ALIGNMENT, "A, B, C must be 16-byte aligned");
  RLK_TRY(check_device());
  rlk::GemmArgs ga;
  ga.A = static_cast<const uint16_t*>(A);
  ga.B = static_cast<const uint16_t*>(B);
  ga.M = (int)M;
  ga.N = (int)N;
  ga.K = (int)K;
  ga.rtiles = (int)ceil_div(M, rlk::kBM);
  ga.ctiles = (int)ceil_div(N, rlk::kBN);
  ga.ldc = ldc;
  ga.c_bf16 = c_dtype == RLK_DT_BF16;
  ga.C = C;
  const int64_t blocks = 8 * ceil_div((int64_t)ga.rtiles * ga.ctiles, 8);
  RLK_TRY(check_grid(blocks));
  RLK_LAUNCH(gemm_tiles, dim3((unsigned)blocks), dim3(rlk::kThreads), static_cast<hipStream_t>(stream), ga);
  return ok();
}

namespace {

// Host checks of the RL objective's arguments (shared by the standalone
// call and the fused forward).
rlk_status check_rl_args(int64_t T, const float* logp_old, const float* adv, const float* logp_ref, float eps_low,
                         float eps_high, float beta, float scale) {
  if (T < 0 || T > kMaxT) return fail(RLK_ERR_BAD_SHAPE, "T=%lld out of [0, 2^24]", (long long)T);
  if (!(eps_low >= 0.f && eps_low < 1.f) || !(eps_high >= 0.f) || !(beta >= 0.f) || !(scale == scale))
    return fail(RLK_ERR_BAD_ARG, "need 0 <= eps_low < 1, eps_high >= 0, beta >= 0, scale not NaN");
  if (T > 0 && (!logp_old || !adv || (beta != 0.f && !logp_ref)))
    return fail(RLK_ERR_NULL_ARG, "logp_old, adv (and logp_ref when beta > 0) are required");
  return RLK_OK;
}

}  // namespace

rlk_status rlk_rl_token_loss(const float* logp, const float* logp_old, const float* adv, const float* logp_ref,
                             const int32_t* y, int64_t T, int32_t ignore_index, float eps_low, float eps_high,
                             float beta, float scale, float* loss, float* g, void* stream) {
  RLK_TRY(check_rl_args(T, logp_old, adv, logp_ref, eps_low, eps_high, beta, scale));
  if (T == 0) return ok();
  if (!logp || !y) return fail(RLK_ERR_NULL_ARG, "logp and y are required");
  if (!loss && !g) return ok();
  RLK_TRY(check_device());
  rlk::RlLossArgs ra;
  ra.logp = logp;
  ra.logp_old = logp_old;
  ra.adv = adv;
  ra.logp_ref = logp_ref;
  ra.y = y;
  ra.T = (int)T;
  ra.ignore_index = ignore_index;
  ra.eps_low = eps_low;
  ra.eps_high = eps_high;
  ra.beta = beta;
  ra.scale = scale;
  ra.loss = loss;
  ra.g = g;
  RLK_LAUNCH(rl_token_loss, dim3((unsigned)ceil_div(T, 256)), dim3(256), static_cast<hipStream_t>(stream), ra);
  return ok();
}

rlk_status rlk_linear_logp_fwd_rl(const void* h, const void* W, const int32_t* y, int64_t T, int64_t H, int64_t V,
                                  int32_t ignore_index, const float* logp_old, const float* adv,
                                  const float* logp_ref, float eps_low, float eps_high, float beta, float scale,
                                  float* logp, float* lse, float* loss, float* g, void* ws, size_t ws_bytes,
                                  void* stream) {
  RLK_TRY(check_common(h, W, y, T, H, V));
  RLK_TRY(check_rl_args(T, logp_old, adv, logp_ref, eps_low, eps_high, beta, scale));
  if (T == 0) return ok();
  if (!logp || !ws || (!loss && !g)) return fail(RLK_ERR_NULL_ARG, "logp, ws and loss or g are required");
  if (!aligned16(logp) || (lse && !aligned16(lse)) || !aligned16(ws))
    return fail(RLK_ERR_BAD_ALIGNMENT, "logp, lse, ws must be 16-byte aligned");
  if (ws_bytes < fwd_layout(T, H, V).total)
    return fail(RLK_ERR_WORKSPACE_TOO_SMALL, "need %zu bytes, got %zu", fwd_layout(T, H, V).total, ws_bytes);
  RLK_TRY(check_device());
  rlk::RlLossArgs ra;
  ra.logp = logp;
  ra.logp_old = logp_old;
  ra.adv = adv;
  ra.logp_ref = logp_ref;
  ra.y = y;
  ra.T = (int)T;
  ra.ignore_index = ignore_index;
  ra.eps_low = eps_low;
  ra.eps_high = eps_high;
  ra.beta = beta;
  ra.scale = scale;
  ra.loss = loss;
  ra.g = g;
  RLK_TRY(run_forward(h, W, y, T, H, V, ignore_index, 0, rlk::kNSplit, 0, V, 0, logp, lse, nullptr, ws,
                      static_cast<hipStream_t>(stream), nullptr, 0, &ra));
  return ok();
}

rlk_status rlk_bench_mfma_ceiling(const void* src, float* out, int32_t blocks, int32_t iters, void* stream) {
  if (blocks <= 0 || blocks > 65536 || iters <= 0) return fail(RLK_ERR_BAD_ARG, "blocks in [1, 65536], iters > 0");
  if (!src || !out) return fail(RLK_ERR_NULL_ARG, "src and out are required");
  if (!aligned16(src)) return fail(RLK_ERR_BAD_ALIGNMENT, "src must be 16-byte aligned");
  RLK_TRY(check_device());
  RLK_LAUNCH(mfma_ceiling, dim3((unsigned)blocks), dim3(rlk::kCeilThreads), static_cast<hipStream_t>(stream),
             static_cast<const rlk::u32x4*>(src), out, (int)iters);
  return ok();
}

rlk_status rlk_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof_recs) {
    g_prof_pool.push_back(r.start);
    g_prof_pool.push_back(r.stop);
  }
  g_prof_recs.clear();
  g_prof_on.store(true);
  return ok();
}

rlk_status rlk_profile_end(rlk_kernel_time_t* out, int32_t max_entries, int32_t* n_entries) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on.store(false);
  std::vector<rlk_kernel_time_t> acc;
  rlk_status st = RLK_OK;
  for (auto& r : g_prof_recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess && st == RLK_OK) st = fail(RLK_ERR_HIP, "profile events: %s", hipGetErrorString(e));
    size_t k = 0;
    while (k < acc.size() && std::strcmp(acc[k].name, r.name) != 0) ++k;
    if (k == acc.size()) {
      rlk_kernel_time_t t{};
      std::snprintf(t.name, sizeof(t.name), "%s", r.name);
      acc.push_back(t);
    }
    acc[k].launches += 1;
    acc[k].total_ms += ms;
    g_prof_pool.push_back(r.start);
    g_prof_pool.push_back(r.stop);
  }
  g_prof_recs.clear();
  if (n_entries) *n_entries = (int32_t)acc.size();
  for (size_t k = 0; out && k < acc.size() && (int32_t)k < max_entries; ++k) out[k] = acc[k];
  return st == RLK_OK ? ok() : st;
}

}  // extern "C"


// --- forward with a fixed device scratch (rlk_linear_logp_fwd_noalloc) --------
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops): the forward's workspace lives in this
// file-scope device array instead of a caller buffer.  Every GPU the library
// runs on holds one copy of it until the process ends.  In host code the name
// `scratch` is only a stand-in: its device address on the current GPU comes
// from hipGetSymbolAddress, looked up once per device and kept below.
__device__ __align__(256) unsigned char scratch[RLK_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_dev[64];  // device address of `scratch` per device; NULL until looked up

// Device address of `scratch` on the current device (looked up on the first
// call on that device, with the device current).
rlk_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RLK_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(RLK_ERR_UNSUPPORTED_DEVICE, "device index %d", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(RLK_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return RLK_OK;
}

}  // namespace

extern "C" {

rlk_status rlk_linear_logp_fwd_noalloc(const void* h, const void* W, const int32_t* y, int64_t T, int64_t H,
                                       int64_t V, int32_t ignore_index, float* logp, float* lse, void* stream) {
  RLK_TRY(check_common(h, W, y, T, H, V));
  if (T == 0) return ok();
  if (!logp) return fail(RLK_ERR_NULL_ARG, "logp is required");
  if (!aligned16(logp) || (lse && !aligned16(lse))) return fail(RLK_ERR_BAD_ALIGNMENT, "logp, lse must be 16-byte aligned");
  const size_t need = fwd_layout(T, H, V).total;
  if (need > (size_t)RLK_NOALLOC_SCRATCH_BYTES)
    return fail(RLK_ERR_WORKSPACE_TOO_SMALL,
                "T=%lld H=%lld V=%lld needs %zu bytes of scratch; the fixed device scratch holds %zu "
                "(use rlk_linear_logp_fwd with a workspace)",
                (long long)T, (long long)H, (long long)V, need, (size_t)RLK_NOALLOC_SCRATCH_BYTES);
  RLK_TRY(check_device());
  void* ws = nullptr;
  RLK_TRY(scratch_address(&ws));
  RLK_TRY(run_forward(h, W, y, T, H, V, ignore_index, 0, rlk::kNSplit, 0, V, 0, logp, lse, nullptr, ws,
                      static_cast<hipStream_t>(stream)));
  return ok();
}

}  // extern "C"
