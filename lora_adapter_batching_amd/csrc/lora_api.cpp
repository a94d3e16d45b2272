// lora_api.cpp -- C ABI, host-side validation, token bookkeeping, the work
// planner (segment scheduler) and launch orchestration of the MI355X
// multi-adapter LoRA library. See include/lora_sgmv.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unistd.h>
#include <vector>

#include "../../include/lora_sgmv.h"
#include "lora_inspect.h"
#include "lora_internal.h"
#include "lora_plan.h"

namespace lora {
hipError_t launch_fwd(const FwdPlan& P, int rbmax, hipStream_t stream, const uint64_t* wptr,
                      const uint64_t* vptr, const int32_t* rows, int n_rows);
hipError_t launch_transpose(const TransposePlan& P, hipStream_t stream);
hipError_t launch_wgrad(const WgradPlan& P, int grid, hipStream_t stream);
hipError_t launch_wgrad_reduce(const WgradReducePlan& R, hipStream_t stream);
hipError_t launch_dev_plan(const DevPlanArgs& a, hipStream_t stream);
int wgrad_items_for_rank(int rank, int h_in, int h_out);
}  // namespace lora

using namespace lora;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

// ---------------------------------------------------------------------------
// Tunables of the planner
// ---------------------------------------------------------------------------
constexpr int kMaxKs = 16;            // largest split of the shrink reduction
constexpr int kMaxDepTiles = 1024 - kCtrTiles;  // counter slots
constexpr size_t kCounterBytes = kStampOffset + (size_t)kMaxPartials * kStampStride;  // tile counters, then the part stamps
constexpr int kShrinkChunk = 512;     // k elements per item of a split shrink
constexpr int kExpandBlocks = 48;     // 32-column blocks per expand item of medium batches
constexpr int kMaxSlots = kMaxJobs;   // adapters per backward group

struct DeviceInfo {
  int cus = 256;
  int wall_khz = 100000;
  int xccs = 8;  // XCDs of the device (workgroup b runs on XCD b % xccs)
};

DeviceInfo device_info() {
  static std::mutex mu;
  static DeviceInfo cache[64];
  static bool have[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DeviceInfo{};
  std::lock_guard<std::mutex> lock(mu);
  if (!have[dev]) {
    DeviceInfo d;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      d.cus = v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev) == hipSuccess && v > 0)
      d.wall_khz = v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && v > 0)
      d.xccs = v;
    cache[dev] = d;
    have[dev] = true;
  }
  return cache[dev];
}

// Where the launches of a call go: the HIP stream, or (for the host-only
// plan inspection entry) a recorder that keeps the plans and launches
// nothing. Every planning decision is taken by the same code either way.
struct Launcher {
  virtual ~Launcher() = default;
  virtual DeviceInfo dev() = 0;
  // rows (host, n_rows entries) or null: the token-row table a small launch
  // carries in its arguments
  virtual hipError_t fwd(const FwdPlan& P, int rbmax, const uint64_t* wptr, const uint64_t* vptr,
                         const int32_t* rows, int n_rows) = 0;
  virtual hipError_t transpose(const TransposePlan& P) = 0;
  virtual hipError_t wgrad(const WgradPlan& P, int grid) = 0;
  virtual hipError_t reduce(const WgradReducePlan& R) = 0;
  virtual hipError_t dev_plan(const DevPlanArgs& a) = 0;
};

struct HipLauncher final : Launcher {
  hipStream_t stream;
  explicit HipLauncher(void* s) : stream(static_cast<hipStream_t>(s)) {}
  DeviceInfo dev() override { return device_info(); }
  hipError_t fwd(const FwdPlan& P, int rbmax, const uint64_t* wptr, const uint64_t* vptr, const int32_t* rows,
                 int n_rows) override {
    return launch_fwd(P, rbmax, stream, wptr, vptr, rows, n_rows);
  }
  hipError_t transpose(const TransposePlan& P) override { return launch_transpose(P, stream); }
  hipError_t wgrad(const WgradPlan& P, int grid) override { return launch_wgrad(P, grid, stream); }
  hipError_t reduce(const WgradReducePlan& R) override { return launch_wgrad_reduce(R, stream); }
  hipError_t dev_plan(const DevPlanArgs& a) override { return launch_dev_plan(a, stream); }
};

int round_up(int a, int b) { return (a + b - 1) / b * b; }
// Row length of a split-K partial tile: the kernels write 32 * RB rows with
// RB = 1, 2 or 4 rank blocks of 32.
int rpad_for(int rmax) { return rmax <= 32 ? 32 : (rmax <= 64 ? 64 : 128); }
int64_t round_up64(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
int cdiv(int a, int b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct ActiveSeg {
  int tok0, ntok, adapter, rank;
  float scale;
  int proj = 0;  // projection of a multi-projection call
};

// ---------------------------------------------------------------------------
// Validation (host mirrors only; no HIP call)
// ---------------------------------------------------------------------------
int check_adapters(const lora_adapters_t* a) {
  if (!a) return fail(LORA_INVALID_ARGUMENT, "adapters is NULL");
  if (a->num_adapters < 1) return fail(LORA_INVALID_ARGUMENT, "num_adapters must be >= 1");
  if (a->h_in <= 0 || a->h_out <= 0)
    return fail(LORA_INVALID_ARGUMENT, "h_in and h_out must be positive");
  if ((a->h_in & 7) || (a->h_out & 7))
    return fail(LORA_INVALID_ARGUMENT, "h_in (%d) and h_out (%d) must be multiples of 8", a->h_in,
                a->h_out);
  if (!a->ranks || !a->scales) return fail(LORA_INVALID_ARGUMENT, "ranks/scales host arrays are NULL");
  for (int i = 0; i < a->num_adapters; ++i) {
    if (a->ranks[i] < 0) return fail(LORA_INVALID_ARGUMENT, "rank of adapter %d is negative", i);
    if (a->ranks[i] > LORA_MAX_RANK)
      return fail(LORA_UNSUPPORTED, "rank %d of adapter %d exceeds %d", a->ranks[i], i, LORA_MAX_RANK);
    if (!std::isfinite(a->scales[i])) return fail(LORA_INVALID_ARGUMENT, "scale of adapter %d is not finite", i);
  }
  return LORA_OK;
}

int check_segments(const lora_segments_t* s, int N) {
  if (!s) return fail(LORA_INVALID_ARGUMENT, "segments is NULL");
  if (s->num_tokens < 0 || s->num_segments < 0)
    return fail(LORA_INVALID_ARGUMENT, "num_tokens and num_segments must be >= 0");
  if (s->num_segments == 0) {
    if (s->num_tokens != 0) return fail(LORA_INVALID_ARGUMENT, "tokens present but no segments");
    return LORA_OK;
  }
  if (!s->seg_starts || !s->seg_adapter)
    return fail(LORA_INVALID_ARGUMENT, "seg_starts/seg_adapter host arrays are NULL");
  if (s->seg_starts[0] != 0) return fail(LORA_INVALID_ARGUMENT, "seg_starts[0] must be 0");
  for (int g = 0; g < s->num_segments; ++g) {
    if (s->seg_starts[g + 1] < s->seg_starts[g])
      return fail(LORA_INVALID_ARGUMENT, "seg_starts decreases at segment %d", g);
    const int a = s->seg_adapter[g];
    if (a < -1 || a >= N) return fail(LORA_INVALID_ARGUMENT, "seg_adapter[%d] = %d outside [-1, %d)", g, a, N);
  }
  if (s->seg_starts[s->num_segments] != s->num_tokens)
    return fail(LORA_INVALID_ARGUMENT, "seg_starts[S] = %d differs from num_tokens = %d",
                s->seg_starts[s->num_segments], s->num_tokens);
  return LORA_OK;
}

std::vector<ActiveSeg> active_segments(const lora_adapters_t* a, const lora_segments_t* s) {
  std::vector<ActiveSeg> v;
  for (int g = 0; g < s->num_segments; ++g) {
    const int ad = s->seg_adapter[g];
    const int n = s->seg_starts[g + 1] - s->seg_starts[g];
    if (ad < 0 || n == 0 || a->ranks[ad] == 0) continue;
    v.push_back(ActiveSeg{s->seg_starts[g], n, ad, a->ranks[ad], a->scales[ad]});
  }
  return v;
}

int check_rows(const void* p, int64_t ld, int width, const char* name, bool needed) {
  if (!needed) return LORA_OK;
  if (!p) return fail(LORA_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned16(p)) return fail(LORA_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  if (ld < width) return fail(LORA_INVALID_ARGUMENT, "row stride of %s (%lld) is below its width %d", name,
                              (long long)ld, width);
  if (ld & 7) return fail(LORA_INVALID_ARGUMENT, "row stride of %s (%lld) is not a multiple of 8", name,
                          (long long)ld);
  return LORA_OK;
}

// With a token-row table the kernels address a whole matrix from its base
// through one buffer resource of kGatherSpan bytes. The rows of a batch are
// distinct, so its largest row is at least T - 1: a batch whose T rows cannot
// fit in that span is refused here (a row past the span would be read as
// zero and not written).
int check_gather(const lora_segments_t* s, int64_t ld, int width, const char* name, bool needed) {
  if (!needed || (!s->token_rows && !s->token_rows_host) || s->num_tokens == 0) return LORA_OK;
  const int64_t span = ((int64_t)(s->num_tokens - 1) * ld + width) * 2;
  if (span > kGatherSpan)
    return fail(LORA_INVALID_ARGUMENT,
                "%s: with token_rows, %d rows of stride %lld span %lld bytes, above the %lld-byte gather limit",
                name, s->num_tokens, (long long)ld, (long long)span, (long long)kGatherSpan);
  return LORA_OK;
}

// A call given only the host copy of the row table (no device table) must
// fit in one small launch, which carries the rows in its arguments.
int check_host_rows(const lora_segments_t* s, size_t n_active, const char* what) {
  if (!s->token_rows_host || s->token_rows) return LORA_OK;
  if (n_active > (size_t)kSmallSeg || s->num_tokens > kPlanRows)
    return fail(LORA_INVALID_ARGUMENT,
                "%s: token_rows is NULL and the host copy alone serves only batches of at most %d segments "
                "and %d tokens (this one: %zu segments, %d tokens)",
                what, kSmallSeg, kPlanRows, n_active, s->num_tokens);
  return LORA_OK;
}

int check_u(const float* u, int64_t ldu, int rmax, const char* name) {
  if (!u) return fail(LORA_INVALID_ARGUMENT, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(u) & 3u) return fail(LORA_INVALID_ARGUMENT, "%s is not 4-byte aligned", name);
  if (ldu < rmax) return fail(LORA_INVALID_ARGUMENT, "row stride of %s (%lld) is below the largest rank used (%d)",
                              name, (long long)ldu, rmax);
  return LORA_OK;
}

int max_rank_all(const lora_adapters_t* a) {
  int r = 0;
  for (int i = 0; i < a->num_adapters; ++i) r = std::max(r, a->ranks[i]);
  return r;
}
int max_rank_used(const std::vector<ActiveSeg>& v) {
  int r = 0;
  for (const auto& s : v) r = std::max(r, s.rank);
  return r;
}

// ---------------------------------------------------------------------------
// Workspace layout
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t counters = 0, partials = 0, du = 0, urec = 0, bt = 0, at = 0, wpart = 0, total = 0;
  int64_t lddu = 0;
  int64_t bt_slot = 0, at_slot = 0;  // elements per slot
  int64_t wpart_stride = 0;          // floats per weight-gradient partial slot
  int wpart_slots = 0;               // partial slots of split weight-gradient jobs
};

// Partial slots for token-range splits of the weight gradients: one slot
// holds one adapter's dB and dA at the largest rank. A part covers at least
// kSplitMinSteps 32-token steps, so a batch of T tokens has at most
// T / (32 kSplitMinSteps) parts; the slots together stay under
// kSplitBudgetBytes.
constexpr int kSplitMinSteps = 8;
constexpr size_t kSplitBudgetBytes = (size_t)64 << 20;
int64_t wpart_stride_for(const lora_adapters_t* a, int rmax) {
  return round_up64((int64_t)(a->h_in + a->h_out) * std::max(rmax, 1), 64);
}
int wpart_slots_for(const lora_adapters_t* a, int rmax, int64_t T) {
  const int64_t per = wpart_stride_for(a, rmax) * (int64_t)sizeof(float);
  int64_t n = std::min<int64_t>({(int64_t)kMaxJobs, T / (kTileM * kSplitMinSteps),
                                 (int64_t)(kSplitBudgetBytes / (size_t)per)});
  return n >= 2 ? (int)n : 0;
}

WsLayout ws_layout(int op, const lora_adapters_t* a, const lora_segments_t* s) {
  WsLayout L;
  const int rmax = max_rank_all(a);
  const int rpad = rpad_for(rmax);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) / 256 * 256;
    return o;
  };
  if (op == LORA_OP_EXPAND) {
    L.total = 0;
    return L;
  }
  L.counters = take(kCounterBytes);
  // parts of one launch: at most kMaxKs per tile, and a batch has at most
  // ceil(T / 32) + S tiles (each segment adds at most one ragged tile)
  int64_t parts = kMaxPartials;
  if (s) parts = std::min<int64_t>(parts, ((int64_t)cdiv(s->num_tokens, kTileM) + s->num_segments) * kMaxKs);
  L.partials = take((size_t)std::max<int64_t>(parts, 1) * kTileM * rpad * sizeof(float));
  if (op == LORA_OP_BACKWARD) {
    const int64_t T = s ? s->num_tokens : 0;
    L.lddu = round_up(std::max(rmax, 1), 4);
    L.du = take((size_t)T * L.lddu * sizeof(float));
    L.urec = take((size_t)T * L.lddu * sizeof(float));
    const int slots = std::min(a->num_adapters, kMaxSlots);
    L.bt_slot = round_up64((int64_t)rmax * a->h_out, 8);
    L.at_slot = round_up64((int64_t)a->h_in * round_up(std::max(rmax, 1), 8), 8);
    L.bt = take((size_t)slots * L.bt_slot * 2);
    L.at = take((size_t)slots * L.at_slot * 2);
    L.wpart_stride = wpart_stride_for(a, rmax);
    L.wpart_slots = wpart_slots_for(a, rmax, T);
    L.wpart = take((size_t)L.wpart_slots * L.wpart_stride * sizeof(float));
  }
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// Planner: forward-style launches
// ---------------------------------------------------------------------------
// Orders segments so that heavy work items are dispatched first. Workgroups
// are handed out in launch order to whichever CU frees up first, so the
// order is a longest-processing-time-first list schedule when it runs by
// the cost of one ITEM (a 32-token tile's share of x or y plus its adapter's
// weights, larger for larger ranks), not by a segment's total: a long
// segment of a small-rank adapter must not hold back a short one of a
// large rank. With room in the plan, the ragged last tile of a segment
// becomes an entry of its own, so that these lighter items go to the end
// of the order too.
void order_by_cost(std::vector<ActiveSeg>& v, int K, int N, bool split_ragged) {
  if (split_ragged) {
    size_t extra = 0;
    for (const auto& s : v) extra += (s.ntok > kTileM && s.ntok % kTileM) ? 1 : 0;
    if (v.size() + extra <= (size_t)kMaxSeg) {
      std::vector<ActiveSeg> w;
      w.reserve(v.size() + extra);
      for (const auto& s : v) {
        const int full = s.ntok / kTileM * kTileM;
        if (s.ntok > kTileM && full < s.ntok) {
          ActiveSeg a = s, b = s;
          a.ntok = full;
          b.tok0 = s.tok0 + full;
          b.ntok = s.ntok - full;
          w.push_back(a);
          w.push_back(b);
        } else {
          w.push_back(s);
        }
      }
      v.swap(w);
    }
  }
  auto item_cost = [&](const ActiveSeg& s) {
    const double rows = std::min(s.ntok, kTileM);
    return rows * (2.0 * K + 4.0 * N) + 2.0 * s.rank * (double)(K + N);
  };
  std::stable_sort(v.begin(), v.end(),
                   [&](const ActiveSeg& x, const ActiveSeg& y) { return item_cost(x) > item_cost(y); });
}

struct FwdCall {
  int mode_op;  // LORA_OP_SHRINK / EXPAND / FUSED
  const uint16_t* X;
  int64_t ldx;
  uint16_t* Y;
  int64_t ldy;
  float* U;
  int64_t ldu;
  bool write_u;
  const uint64_t* Wtab;
  const uint64_t* Vtab;
  const uint64_t* Wtab_host;  // host copies of the tables, or null
  const uint64_t* Vtab_host;
  const uint16_t* Wslots;
  const uint16_t* Vslots;
  int64_t w_slot_elems, v_slot_elems;
  int v_round;
  int scale_in_shrink;
  int K, N;
  const int32_t* token_rows;
  const int32_t* rows_host;  // host copy of the row table (small launches carry it), or null
  int n_rows;                // its entries (the batch's tokens)
  float* partials;
  int32_t* counters;
  int rmax;  // largest rank of the adapters (partials row length)
  // multi-projection calls: projections 1 .. n_proj-1 (projection 0 is Y,
  // ldy, N, Wtab, Vtab and their host copies above)
  int n_proj;
  uint16_t* proj_Y[kMaxProj];
  int64_t proj_ldy[kMaxProj];
  int proj_N[kMaxProj];
  const uint64_t* proj_Wtab[kMaxProj];
  const uint64_t* proj_Vtab[kMaxProj];
  const uint64_t* proj_Wtab_host[kMaxProj];
  const uint64_t* proj_Vtab_host[kMaxProj];
};

// Optional planner override for tuning, read once from LORA_SGMV_FORCE:
// "tile:NC" forces the on-chip fused mode with NC column chunks per tile,
// "dep:KS:NC" the split-shrink mode, "loc:KS:NC" the split-shrink mode with
// every item of a tile on one XCD. A third field ("dep:KS:NC:TICKS") sets how
// long an expand waits for the parts before it computes the shrink itself
// (0: one look, so most expands take that path). Applies to fused calls only.
struct ForcePlan {
  int mode = -1, ks = 0, nc = 0, local = 0, spin = -1;
};
ForcePlan force_plan() {
  static ForcePlan f = [] {
    ForcePlan r;
    const char* e = std::getenv("LORA_SGMV_FORCE");
    if (!e) return r;
    int a = 0, b = 0, t = -1;
    if (std::sscanf(e, "tile:%d", &a) == 1 && a > 0) { r.mode = kModeFusedTile; r.nc = a; }
    else if (std::sscanf(e, "dep:%d:%d:%d", &a, &b, &t) >= 2 && a > 0 && b > 0) { r.mode = kModeFusedDep; r.ks = a; r.nc = b; }
    else if (std::sscanf(e, "loc:%d:%d:%d", &a, &b, &t) >= 2 && a > 0 && b > 0) { r.mode = kModeFusedDep; r.ks = a; r.nc = b; r.local = 1; }
    if (r.mode == kModeFusedDep && t >= 0) r.spin = t;
    return r;
  }();
  return f;
}

// XCD-aware item order for the on-chip fused mode. Workgroup b runs on XCD
// b % 8, and with the remap the items of one tile (which all read the tile's
// x rows and its adapter's weights) land on one XCD, so that data enters one
// L2 instead of eight. On by default for small batches, where it cuts the
// fetched bytes about threefold; off for large ones, where it was measured
// slower. LORA_SGMV_XCD=0/1 forces it off/on.
bool xcd_remap_enabled(bool small_batch) {
  static const int env = [] {
    const char* e = std::getenv("LORA_SGMV_XCD");
    return e ? (e[0] == '1' ? 1 : 0) : -1;
  }();
  return env >= 0 ? env == 1 : small_batch;
}

// Byte budget of dy per backward adapter group (LORA_SGMV_BWD_GROUP_MB; 0:
// groups limited only by the kMaxSlots adapters a transpose pass holds).
int64_t bwd_group_bytes() {
  static const int64_t v = [] {
    const char* e = std::getenv("LORA_SGMV_BWD_GROUP_MB");
    return e ? (int64_t)std::atoll(e) << 20 : (int64_t)0;
  }();
  return v;
}

// A launch id that no earlier launch of any process used with the same
// workspace: split-shrink parts are stamped with it, so a stamp left in the
// workspace by an earlier call can never be taken for a current one.
uint64_t next_launch_id() {
  static std::atomic<uint64_t> next{[] {
    const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    return ((t << 12) ^ ((uint64_t)getpid() << 36)) & ((1ull << 56) - 1);
  }()};
  uint64_t id;
  do {
    id = next.fetch_add(1, std::memory_order_relaxed) & ((1ull << 56) - 1);
  } while (id == 0);
  return id;
}

// XCD-local split layout: the items of tile g (its ks shrink parts, then its
// nc expands) run on XCD g % 8, in dispatch order parts before expands.
// Returns the grid (8 x the largest per-XCD item count).
int local_grid(int tiles, int ks, int nc) {
  const int per_xcd_tiles = (tiles + 7) / 8;
  return 8 * per_xcd_tiles * (ks + nc);
}

// A batch whose expand moves more than four times the bytes of its shrink
// per tile, for the widest output (32 tokens of y read and written plus the
// expand weights, against 32 tokens of x plus the shrink weights; rank r).
bool expand_heavy(int K, int n_widest, int r) {
  const double expand = (double)n_widest * (4.0 * kTileM + 2.0 * r);
  const double shrink = (double)K * (2.0 * kTileM + 2.0 * r);
  return expand > 4.0 * shrink;
}

// Layout of a fused launch over `tiles` 32-token tiles whose largest rank
// is rmax_l and whose widest output has `nblocks` 32-column blocks: mode,
// k split, column chunks and grid (the layouts and their measurements are
// described at each branch).
void fused_layout(FwdPlan& P, const FwdCall& c, int tiles, int rmax_l, int nblocks, const DeviceInfo& dev) {
  const int cus = dev.cus;
  const int slots = 2 * cus;  // resident workgroups at the kernels' occupancy
  const ForcePlan fp = force_plan();
  if (fp.mode == kModeFusedTile) {
    P.mode = kModeFusedTile;
    P.ks = 1;
    P.kchunk = round_up(c.K, 64);
    P.nblk = cdiv(nblocks, std::min(fp.nc, nblocks));
    P.nc = cdiv(nblocks, P.nblk);
    P.n_items_a = tiles * P.nc;
    P.xcd_remap = xcd_remap_enabled(false) ? 1 : 0;
    P.grid = P.xcd_remap ? round_up(P.n_items_a, 8) : P.n_items_a;
  } else if (fp.mode == kModeFusedDep && fp.ks <= kMaxKs && tiles * fp.ks <= kMaxPartials) {
    P.mode = kModeFusedDep;
    P.kchunk = round_up(cdiv(c.K, fp.ks), 64);
    P.ks = cdiv(c.K, P.kchunk);
    P.nblk = cdiv(nblocks, std::min(fp.nc, nblocks));
    P.nc = cdiv(nblocks, P.nblk);
    P.n_items_a = tiles * P.ks;
    P.n_items_b = tiles * P.nc;
    P.xcd_local = fp.local && dev.xccs == 8 ? 1 : 0;
    P.grid = P.xcd_local ? local_grid(tiles, P.ks, P.nc) : P.n_items_a + P.n_items_b;
    if (fp.spin >= 0) P.spin_ticks = fp.spin;
  } else if (4 * tiles <= cus && expand_heavy(c.K, nblocks * 32, rmax_l)) {
    // small batch whose expand moves far more bytes than its shrink
    // (e.g. an MLP-up projection): the split layout with the items of
    // every tile spread over all XCDs, so that the expand's y and weight
    // traffic is shared by every XCD's L2 and fabric port rather than
    // concentrated on the XCDs that hold two tiles; the parts go through
    // device-scope stores and loads. Parts of about 320 columns, at most
    // as many as one batch of the expand's part loads takes (8, 4, 2
    // for rank <= 32, 64, 128), and the expand items of each tile fill
    // about two workgroups per CU. (Measured on the decode gate_up
    // projection, 2560 -> 19456 with 11 tiles: 16.8 us against 18.7 us
    // for the XCD-local layout; parts of 256 columns: 19.1-19.9 us.)
    P.mode = kModeFusedDep;
    const int rb = rmax_l <= 32 ? 1 : (rmax_l <= 64 ? 2 : 4);
    int ks = std::max(1, std::min({8 / rb, cdiv(c.K, 320), kMaxPartials / tiles}));
    P.kchunk = round_up(cdiv(c.K, ks), 64);
    P.ks = cdiv(c.K, P.kchunk);
    const int nc = std::max(1, std::min(nblocks, slots / tiles - P.ks));
    P.nblk = cdiv(nblocks, nc);
    P.nc = cdiv(nblocks, P.nblk);
    P.n_items_a = tiles * P.ks;
    P.n_items_b = tiles * P.nc;
    P.grid = P.n_items_a + P.n_items_b;
  } else if (4 * tiles <= cus && dev.xccs == 8 && xcd_remap_enabled(true)) {
    // small batch: each tile's shrink is split along k into parts and its
    // expand into column chunks, all on one XCD, so the parts reach the
    // expands with plain accesses through that XCD's L2 (the item order
    // assumes 8 XCDs). About two workgroups per CU.
    P.mode = kModeFusedDep;
    const int per_xcd_tiles = (tiles + 7) / 8;
    const int slots_per_xcd = 2 * cus / 8;
    int ks = std::max(1, std::min({kMaxKs, cdiv(c.K, 512), kMaxPartials / tiles}));
    P.kchunk = round_up(cdiv(c.K, ks), 64);
    P.ks = cdiv(c.K, P.kchunk);
    const int nc = std::max(1, std::min(nblocks, slots_per_xcd / per_xcd_tiles - P.ks));
    P.nblk = cdiv(nblocks, nc);
    P.nc = cdiv(nblocks, P.nblk);
    P.n_items_a = tiles * P.ks;
    P.n_items_b = tiles * P.nc;
    P.xcd_local = 1;
    P.grid = local_grid(tiles, P.ks, P.nc);
  } else if (4 * tiles <= cus) {
    // small batch without the XCD-local layout: each item computes its
    // tile's full shrink on chip and one column chunk of the expand
    P.mode = kModeFusedTile;
    P.ks = 1;
    P.kchunk = round_up(c.K, 64);
    P.nblk = cdiv(nblocks, std::max(1, std::min(nblocks, cus / tiles)));
    P.nc = cdiv(nblocks, P.nblk);
    P.n_items_a = tiles * P.nc;
    P.grid = P.n_items_a;
  } else if (tiles >= 2 * cus || 2 * tiles > kMaxPartials) {
    // the tiles alone fill every resident slot: keep u on chip, one item
    // per tile (measured on the packed-training forward, 2048 tiles:
    // 318 us, against 356 us with one shrink and two expand items per tile)
    P.mode = kModeFusedTile;
    P.ks = 1;
    P.kchunk = round_up(c.K, 64);
    P.nc = 1;
    P.nblk = nblocks;
    P.n_items_a = tiles;
    P.xcd_remap = xcd_remap_enabled(false) ? 1 : 0;
    P.grid = P.xcd_remap ? round_up(tiles, 8) : tiles;
  } else {
    // medium batch: each tile's shrink in one or two k-parts and its
    // expand in column items of about kExpandBlocks 32-column blocks (at
    // least about three workgroups per CU in all) that wait for the
    // parts, so every CU has work without repeating the shrink. Measured
    // (prefill 8192 tok 4096->4096: 64 -> 56 us; MLP-up 4096 tok
    // 4096->14336: 105 -> 85 us) against one item per tile and against
    // narrower expand items.
    P.mode = kModeFusedDep;
    const int ks = c.K >= 2048 ? 2 : 1;
    P.kchunk = round_up(cdiv(c.K, ks), 64);
    P.ks = cdiv(c.K, P.kchunk);
    int nc = std::max({2, (nblocks + kExpandBlocks / 2) / kExpandBlocks, 3 * cus / tiles - 1});
    // a multiple of 8 column items per tile puts column chunk c of every
    // tile on one XCD (workgroup b runs on XCD b % 8), so the tiles of an
    // adapter re-read that chunk's expand-weight slice from one L2
    // (MLP-up 4096 tok, 32 adapters r8..r128: 8 items 85 us, 9 items 88 us)
    if (nc >= 6) nc = std::max(8, (nc + 4) / 8 * 8);
    nc = std::min(nblocks, nc);
    P.nblk = cdiv(nblocks, nc);
    P.nc = cdiv(nblocks, P.nblk);
    P.n_items_a = tiles * P.ks;
    P.n_items_b = tiles * P.nc;
    P.grid = P.n_items_a + P.n_items_b;
  }
}

int run_fwd(const FwdCall& c, std::vector<ActiveSeg> segs, const std::vector<int>& slot_of,
            Launcher& launcher) {
  if (segs.empty()) return LORA_OK;
  const DeviceInfo dev = launcher.dev();
  const int cus = dev.cus;
  {
    int tiles_all = 0;
    for (const auto& sg : segs) tiles_all += cdiv(sg.ntok, kTileM);
    order_by_cost(segs, c.K, c.N, 4 * tiles_all > dev.cus);
  }
  // split into launches of at most kMaxSeg segments
  for (size_t base = 0; base < segs.size(); base += kMaxSeg) {
    const int ns = (int)std::min<size_t>(kMaxSeg, segs.size() - base);
    FwdPlan P;
    std::memset(&P, 0, sizeof(P));
    P.X = c.X; P.ldx = c.ldx; P.Y = c.Y; P.ldy = c.ldy; P.U = c.U; P.ldu = c.ldu;
    P.Wtab = c.Wtab; P.Vtab = c.Vtab; P.Wslots = c.Wslots; P.Vslots = c.Vslots;
    P.w_slot_elems = c.w_slot_elems; P.v_slot_elems = c.v_slot_elems;
    P.token_rows = c.token_rows; P.partials = c.partials; P.counters = c.counters;
    P.stamps = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(c.counters) + kStampOffset);
    P.launch_id = next_launch_id();
    P.K = c.K; P.N = c.N; P.v_round = c.v_round; P.scale_in_shrink = c.scale_in_shrink;
    P.write_u = c.write_u ? 1 : 0;
    P.rpad = rpad_for(c.rmax);
    for (int q = 1; q < std::max(1, c.n_proj); ++q) {
      P.proj_Y[q] = c.proj_Y[q]; P.proj_ldy[q] = c.proj_ldy[q]; P.proj_N[q] = c.proj_N[q];
      P.proj_Wtab[q] = c.proj_Wtab[q]; P.proj_Vtab[q] = c.proj_Vtab[q];
    }
    int tiles = 0;
    for (int i = 0; i < ns; ++i) {
      const ActiveSeg& s = segs[base + i];
      P.seg_tok0[i] = s.tok0;
      P.seg_ntok[i] = s.ntok;
      P.seg_tile0[i] = tiles;
      P.seg_adapter[i] = s.adapter;
      P.seg_scale[i] = s.scale;
      P.seg_rank[i] = (uint8_t)s.rank;
      P.seg_slot[i] = (uint8_t)(slot_of.empty() ? 0 : slot_of[s.adapter]);
      P.seg_proj[i] = (uint8_t)s.proj;
      tiles += cdiv(s.ntok, kTileM);
    }
    P.n_seg = ns;
    P.n_tiles = tiles;
    // column blocks of the widest projection: the item count per tile is
    // chosen for it, and every projection splits its own width into as many
    // items (some of a narrow projection's may be empty)
    int n_widest = c.N;
    for (int q = 1; q < c.n_proj; ++q) n_widest = std::max(n_widest, c.proj_N[q]);
    const int nblocks = cdiv(n_widest, 32);
    const int slots = 2 * cus;  // resident workgroups at the kernels' occupancy
    // split of a shrink-only call's reduction: none when the tiles alone fill
    // the GPU, otherwise chunks of about kShrinkChunk elements
    auto choose_ks = [&]() {
      int ks = 1;
      if (tiles < cus) ks = cdiv(c.K, kShrinkChunk);
      ks = std::min({ks, kMaxKs, std::max(1, kMaxPartials / tiles)});
      ks = std::max(ks, 1);
      P.kchunk = round_up(cdiv(c.K, ks), 64);
      P.ks = cdiv(c.K, P.kchunk);
    };
    // column chunks per tile: enough items for about two per resident slot,
    // at least one 32-column block per wave
    auto choose_nc = [&]() {
      int nc = std::max(1, cdiv(2 * slots, tiles));
      nc = std::min(nc, std::max(1, nblocks / 4));
      P.nblk = cdiv(nblocks, nc);
      P.nc = cdiv(nblocks, P.nblk);
    };
    P.spin_ticks = (int)std::min<int64_t>((int64_t)dev.wall_khz * 1000 / 5000, 1 << 30);  // 200 us
    if (c.mode_op == LORA_OP_SHRINK) {
      P.mode = kModeShrink;
      choose_ks();
      if (P.ks > 1 && tiles > kMaxDepTiles) { P.ks = 1; P.kchunk = round_up(c.K, 64); }
      P.n_items_a = tiles * P.ks;
      P.grid = P.n_items_a;
    } else if (c.mode_op == LORA_OP_EXPAND) {
      P.mode = kModeExpand;
      choose_nc();
      P.n_items_a = tiles * P.nc;
      P.grid = P.n_items_a;
    } else {
      int rmax_l = 0;
      for (int i = 0; i < ns; ++i) rmax_l = std::max(rmax_l, (int)P.seg_rank[i]);
      fused_layout(P, c, tiles, rmax_l, nblocks, dev);
    }
    if (P.grid <= 0) continue;
    if (c.n_proj > 1) {
      P.nblk = cdiv(cdiv(c.N, 32), P.nc);
      for (int q = 1; q < c.n_proj; ++q) P.proj_nblk[q] = cdiv(cdiv(c.proj_N[q], 32), P.nc);
    }
    int rmax_launch = 0;
    for (int i = 0; i < ns; ++i) rmax_launch = std::max(rmax_launch, (int)P.seg_rank[i]);
    const int rbmax = rmax_launch <= 32 ? 1 : (rmax_launch <= 64 ? 2 : 4);
    // small plans take the weight addresses from the host copies of the
    // tables (when the call uses tables and has the copies of those it uses)
    uint64_t wq[kSmallSeg], vq[kSmallSeg];
    const bool need_w = c.mode_op != LORA_OP_EXPAND, need_v = c.mode_op != LORA_OP_SHRINK;
    bool host_tabs = (c.Wtab || c.Vtab) && (!need_w || (c.Wtab && c.Wtab_host)) &&
                     (!need_v || (c.Vtab && c.Vtab_host));
    for (int q = 1; q < c.n_proj; ++q)
      host_tabs = host_tabs && c.proj_Wtab_host[q] && c.proj_Vtab_host[q];
    if (ns <= kSmallSeg && host_tabs) {
      for (int i = 0; i < ns; ++i) {
        const ActiveSeg& sg = segs[base + i];
        const uint64_t* wt = sg.proj ? c.proj_Wtab_host[sg.proj] : c.Wtab_host;
        const uint64_t* vt = sg.proj ? c.proj_Vtab_host[sg.proj] : c.Vtab_host;
        wq[i] = need_w ? wt[sg.adapter] : 0;
        vq[i] = need_v ? vt[sg.adapter] : 0;
      }
      P.ptrs_in_plan = 1;
    }
    // a small launch over at most kPlanRows positions carries the rows from
    // the caller's host copy: no device table is read, none need be uploaded
    const bool rows_in_plan = c.rows_host && ns <= kSmallSeg && c.n_rows <= kPlanRows;
    if (rows_in_plan) P.token_rows = nullptr;
    else if (c.rows_host && !c.token_rows)
      return fail(LORA_INVALID_ARGUMENT, "internal planner error (host row table on a large launch)");
    const int32_t* rows = rows_in_plan ? c.rows_host : nullptr;
    const int n_rows = rows_in_plan ? c.n_rows : 0;
    const hipError_t e = P.ptrs_in_plan ? launcher.fwd(P, rbmax, wq, vq, rows, n_rows)
                                        : launcher.fwd(P, rbmax, nullptr, nullptr, rows, n_rows);
    if (e != hipSuccess) return fail(LORA_DEVICE_ERROR, "kernel launch failed: %s", hipGetErrorString(e));
  }
  return LORA_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need)
    return fail(LORA_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is below the %zu needed", ws_bytes, need);
  if (need > 0 && !ws) return fail(LORA_INVALID_ARGUMENT, "workspace is NULL");
  if (need > 0 && (reinterpret_cast<uintptr_t>(ws) & 255u))
    return fail(LORA_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  return LORA_OK;
}

}  // namespace

namespace lora {
int set_error(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}
}  // namespace lora

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* lora_status_string(int status) {
  switch (status) {
    case LORA_OK: return "ok";
    case LORA_INVALID_ARGUMENT: return "invalid argument";
    case LORA_UNSUPPORTED: return "unsupported";
    case LORA_WORKSPACE_TOO_SMALL: return "workspace too small";
    case LORA_DEVICE_ERROR: return "device error";
    default: return "unknown status";
  }
}

const char* lora_last_error(void) { return g_last_error.c_str(); }

int lora_version(void) { return 200; }

int lora_segments_from_ids(const int32_t* ids, int32_t T, int32_t N, int32_t* perm,
                           int32_t* seg_starts, int32_t* seg_adapter) {
  g_last_error.clear();
  if (T < 0 || N < 1) return fail(LORA_INVALID_ARGUMENT, "num_tokens must be >= 0 and num_adapters >= 1");
  if ((T > 0 && (!ids || !perm)) || !seg_starts || !seg_adapter)
    return fail(LORA_INVALID_ARGUMENT, "NULL array");
  // stable counting sort; key N stands for "no adapter" (-1) and sorts last
  std::vector<int32_t> count((size_t)N + 2, 0);
  for (int32_t t = 0; t < T; ++t) {
    const int32_t id = ids[t];
    if (id < -1 || id >= N) return fail(LORA_INVALID_ARGUMENT, "ids[%d] = %d outside [-1, %d)", t, id, N);
    count[(size_t)(id < 0 ? N : id) + 1]++;
  }
  for (int32_t k = 0; k <= N; ++k) count[(size_t)k + 1] += count[(size_t)k];
  for (int32_t k = 0; k <= N + 1; ++k) seg_starts[k] = count[(size_t)k];
  for (int32_t k = 0; k < N; ++k) seg_adapter[k] = k;
  seg_adapter[N] = -1;
  for (int32_t t = 0; t < T; ++t) {
    const int32_t key = ids[t] < 0 ? N : ids[t];
    perm[count[(size_t)key]++] = t;
  }
  return LORA_OK;
}

int lora_workspace_size(int op, const lora_adapters_t* adapters, const lora_segments_t* segments,
                        size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(LORA_INVALID_ARGUMENT, "bytes is NULL");
  if (op < LORA_OP_SHRINK || op > LORA_OP_BACKWARD) return fail(LORA_INVALID_ARGUMENT, "unknown op %d", op);
  int st = check_adapters(adapters);
  if (st) return st;
  if (op == LORA_OP_BACKWARD) {
    if (!segments) return fail(LORA_INVALID_ARGUMENT, "segments is NULL");
    if (segments->num_tokens < 0) return fail(LORA_INVALID_ARGUMENT, "num_tokens must be >= 0");
  }
  *bytes = ws_layout(op, adapters, segments).total;
  return LORA_OK;
}

static int common_checks(const lora_adapters_t* adapters, const lora_segments_t* segments) {
  int st = check_adapters(adapters);
  if (st) return st;
  return check_segments(segments, adapters->num_adapters);
}

static int sgmv_shrink_impl(const void* x, int64_t ldx, const lora_adapters_t* adapters,
                            const lora_segments_t* segments, float* u, int64_t ldu, void* ws,
                            size_t ws_bytes, Launcher& launcher) {
  int st = common_checks(adapters, segments);
  if (st) return st;
  const auto segs = active_segments(adapters, segments);
  if (segs.empty()) return LORA_OK;
  if ((st = check_rows(x, ldx, adapters->h_in, "x", true))) return st;
  if ((st = check_gather(segments, ldx, adapters->h_in, "x", true))) return st;
  if ((st = check_u(u, ldu, max_rank_used(segs), "u"))) return st;
  if (!adapters->A_ptrs) return fail(LORA_INVALID_ARGUMENT, "A_ptrs is NULL");
  if ((st = check_host_rows(segments, segs.size(), "lora_sgmv_shrink"))) return st;
  const WsLayout L = ws_layout(LORA_OP_SHRINK, adapters, segments);
  if ((st = check_ws(ws, ws_bytes, L.total))) return st;
  FwdCall c{};
  c.mode_op = LORA_OP_SHRINK;
  c.X = static_cast<const uint16_t*>(x); c.ldx = ldx;
  c.U = u; c.ldu = ldu;
  c.Wtab = adapters->A_ptrs; c.v_round = 1;
  if (adapters->A_ptrs_host && adapters->B_ptrs_host) c.Wtab_host = adapters->A_ptrs_host;
  c.K = adapters->h_in; c.N = adapters->h_out;
  c.token_rows = segments->token_rows;
  c.rows_host = segments->token_rows_host; c.n_rows = segments->num_tokens;
  c.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + L.partials);
  c.counters = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.counters);
  c.rmax = max_rank_all(adapters);
  return run_fwd(c, segs, {}, launcher);
}

static int sgmv_expand_impl(const float* u, int64_t ldu, const lora_adapters_t* adapters,
                            const lora_segments_t* segments, void* y, int64_t ldy, Launcher& launcher) {
  int st = common_checks(adapters, segments);
  if (st) return st;
  const auto segs = active_segments(adapters, segments);
  if (segs.empty()) return LORA_OK;
  if ((st = check_rows(y, ldy, adapters->h_out, "y", true))) return st;
  if ((st = check_gather(segments, ldy, adapters->h_out, "y", true))) return st;
  if ((st = check_u(u, ldu, max_rank_used(segs), "u"))) return st;
  if (!adapters->B_ptrs) return fail(LORA_INVALID_ARGUMENT, "B_ptrs is NULL");
  if ((st = check_host_rows(segments, segs.size(), "lora_sgmv_expand"))) return st;
  FwdCall c{};
  c.mode_op = LORA_OP_EXPAND;
  c.Y = static_cast<uint16_t*>(y); c.ldy = ldy;
  c.U = const_cast<float*>(u); c.ldu = ldu;
  c.Vtab = adapters->B_ptrs; c.v_round = 1;
  if (adapters->A_ptrs_host && adapters->B_ptrs_host) c.Vtab_host = adapters->B_ptrs_host;
  c.K = adapters->h_in; c.N = adapters->h_out;
  c.token_rows = segments->token_rows;
  c.rows_host = segments->token_rows_host; c.n_rows = segments->num_tokens;
  c.rmax = max_rank_all(adapters);
  return run_fwd(c, segs, {}, launcher);
}

static int sgmv_fused_impl(const void* x, int64_t ldx, const lora_adapters_t* adapters,
                           const lora_segments_t* segments, void* y, int64_t ldy, float* u_save,
                           int64_t ldu, void* ws, size_t ws_bytes, Launcher& launcher,
                           WsSource* src = nullptr) {
  int st = common_checks(adapters, segments);
  if (st) return st;
  const auto segs = active_segments(adapters, segments);
  if (segs.empty()) return LORA_OK;
  if ((st = check_rows(x, ldx, adapters->h_in, "x", true))) return st;
  if ((st = check_rows(y, ldy, adapters->h_out, "y", true))) return st;
  if ((st = check_gather(segments, ldx, adapters->h_in, "x", true))) return st;
  if ((st = check_gather(segments, ldy, adapters->h_out, "y", true))) return st;
  if (u_save && (st = check_u(u_save, ldu, max_rank_used(segs), "u_save"))) return st;
  if ((st = check_host_rows(segments, segs.size(), "lora_sgmv_fused"))) return st;
  if (!adapters->A_ptrs || !adapters->B_ptrs) return fail(LORA_INVALID_ARGUMENT, "A_ptrs/B_ptrs is NULL");
  const WsLayout L = ws_layout(LORA_OP_FUSED, adapters, segments);
  if (src) {
    if (L.total > src->cap)
      return fail(LORA_UNSUPPORTED,
                  "this batch needs %zu bytes of hand-off scratch and the library's static scratch holds %zu "
                  "(call lora_sgmv_fused with a workspace instead)",
                  L.total, src->cap);
    ws = src->get();
    if (!ws) return LORA_DEVICE_ERROR;
    ws_bytes = src->cap;
  }
  if ((st = check_ws(ws, ws_bytes, L.total))) return st;
  FwdCall c{};
  c.mode_op = LORA_OP_FUSED;
  c.X = static_cast<const uint16_t*>(x); c.ldx = ldx;
  c.Y = static_cast<uint16_t*>(y); c.ldy = ldy;
  c.U = u_save; c.ldu = ldu; c.write_u = u_save != nullptr;
  c.Wtab = adapters->A_ptrs; c.Vtab = adapters->B_ptrs; c.v_round = 1;
  if (adapters->A_ptrs_host && adapters->B_ptrs_host) {
    c.Wtab_host = adapters->A_ptrs_host;
    c.Vtab_host = adapters->B_ptrs_host;
  }
  c.K = adapters->h_in; c.N = adapters->h_out;
  c.token_rows = segments->token_rows;
  c.rows_host = segments->token_rows_host; c.n_rows = segments->num_tokens;
  c.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + L.partials);
  c.counters = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.counters);
  c.rmax = max_rank_all(adapters);
  return run_fwd(c, segs, {}, launcher);
}

int lora_sgmv_shrink(const void* x, int64_t ldx, const lora_adapters_t* adapters,
                     const lora_segments_t* segments, float* u, int64_t ldu, void* ws,
                     size_t ws_bytes, void* stream) {
  g_last_error.clear();
  HipLauncher launcher(stream);
  return sgmv_shrink_impl(x, ldx, adapters, segments, u, ldu, ws, ws_bytes, launcher);
}

int lora_sgmv_expand(const float* u, int64_t ldu, const lora_adapters_t* adapters,
                     const lora_segments_t* segments, void* y, int64_t ldy, void* ws,
                     size_t ws_bytes, void* stream) {
  g_last_error.clear();
  (void)ws;
  (void)ws_bytes;
  HipLauncher launcher(stream);
  return sgmv_expand_impl(u, ldu, adapters, segments, y, ldy, launcher);
}

int lora_sgmv_fused(const void* x, int64_t ldx, const lora_adapters_t* adapters,
                    const lora_segments_t* segments, void* y, int64_t ldy, float* u_save,
                    int64_t ldu, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  HipLauncher launcher(stream);
  return sgmv_fused_impl(x, ldx, adapters, segments, y, ldy, u_save, ldu, ws, ws_bytes, launcher);
}

// ---------------------------------------------------------------------------
// Several projections over one x in one launch
// ---------------------------------------------------------------------------
// Checks shared by the multi-projection calls; on success *rmax is the
// largest rank over every projection's adapters.
static int multi_checks(int32_t num_proj, const lora_adapters_t* const* adapters,
                        const lora_segments_t* segments, int* rmax) {
  if (num_proj < 1 || num_proj > kMaxProj)
    return fail(LORA_INVALID_ARGUMENT, "num_proj must be in [1, %d], got %d", kMaxProj, num_proj);
  if (!adapters) return fail(LORA_INVALID_ARGUMENT, "adapters is NULL");
  *rmax = 0;
  for (int p = 0; p < num_proj; ++p) {
    if (!adapters[p]) return fail(LORA_INVALID_ARGUMENT, "adapters[%d] is NULL", p);
    int st = common_checks(adapters[p], segments);
    if (st) return st;
    if (adapters[p]->num_adapters != adapters[0]->num_adapters || adapters[p]->h_in != adapters[0]->h_in)
      return fail(LORA_INVALID_ARGUMENT, "adapters[%d]: every projection needs the same num_adapters and h_in", p);
    *rmax = std::max(*rmax, max_rank_all(adapters[p]));
  }
  return LORA_OK;
}

// Hand-off words and split-shrink partials of a multi-projection launch:
// the tiles of every projection share one part budget.
static size_t multi_ws_bytes(int32_t num_proj, int rmax, const lora_segments_t* s) {
  const int64_t tiles = (int64_t)cdiv(s->num_tokens, kTileM) + s->num_segments;
  const int64_t parts = std::max<int64_t>(1, std::min<int64_t>(kMaxPartials, num_proj * tiles * kMaxKs));
  const size_t part_off = (kCounterBytes + 255) / 256 * 256;
  return part_off + (size_t)parts * kTileM * rpad_for(rmax) * sizeof(float);
}

int lora_workspace_size_multi(int32_t num_proj, const lora_adapters_t* const* adapters,
                              const lora_segments_t* segments, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(LORA_INVALID_ARGUMENT, "bytes is NULL");
  int rmax = 0;
  int st = multi_checks(num_proj, adapters, segments, &rmax);
  if (st) return st;
  *bytes = multi_ws_bytes(num_proj, rmax, segments);
  return LORA_OK;
}

static int sgmv_fused_multi_impl(const void* x, int64_t ldx, int32_t num_proj,
                                 const lora_adapters_t* const* adapters, const lora_segments_t* segments,
                                 void* const* y, const int64_t* ldy, void* ws, size_t ws_bytes,
                                 Launcher& launcher) {
  int rmax = 0;
  int st = multi_checks(num_proj, adapters, segments, &rmax);
  if (st) return st;
  if (!y || !ldy) return fail(LORA_INVALID_ARGUMENT, "y / ldy is NULL");
  std::vector<ActiveSeg> segs;
  for (int p = 0; p < num_proj; ++p) {
    auto v = active_segments(adapters[p], segments);
    if (v.empty()) continue;
    char name[16];
    std::snprintf(name, sizeof(name), "y[%d]", p);
    if ((st = check_rows(y[p], ldy[p], adapters[p]->h_out, name, true))) return st;
    if ((st = check_gather(segments, ldy[p], adapters[p]->h_out, name, true))) return st;
    if (!adapters[p]->A_ptrs || !adapters[p]->B_ptrs)
      return fail(LORA_INVALID_ARGUMENT, "adapters[%d]: A_ptrs/B_ptrs is NULL", p);
    for (auto& a : v) a.proj = p;
    segs.insert(segs.end(), v.begin(), v.end());
  }
  if (segs.empty()) return LORA_OK;
  if ((st = check_rows(x, ldx, adapters[0]->h_in, "x", true))) return st;
  if ((st = check_gather(segments, ldx, adapters[0]->h_in, "x", true))) return st;
  if ((st = check_host_rows(segments, segs.size(), "lora_sgmv_fused_multi"))) return st;
  // every output is written: no two may share a base address, and none may be x
  for (int p = 0; p < num_proj; ++p) {
    if (y[p] == x) return fail(LORA_INVALID_ARGUMENT, "y[%d] is x: outputs must not overlap x", p);
    for (int q = 0; q < p; ++q)
      if (y[p] == y[q]) return fail(LORA_INVALID_ARGUMENT, "y[%d] and y[%d] are the same buffer", q, p);
  }
  if ((st = check_ws(ws, ws_bytes, multi_ws_bytes(num_proj, rmax, segments)))) return st;
  FwdCall c{};
  c.mode_op = LORA_OP_FUSED;
  c.X = static_cast<const uint16_t*>(x); c.ldx = ldx;
  c.Y = static_cast<uint16_t*>(y[0]); c.ldy = ldy[0];
  c.Wtab = adapters[0]->A_ptrs; c.Vtab = adapters[0]->B_ptrs; c.v_round = 1;
  if (adapters[0]->A_ptrs_host && adapters[0]->B_ptrs_host) {
    c.Wtab_host = adapters[0]->A_ptrs_host;
    c.Vtab_host = adapters[0]->B_ptrs_host;
  }
  c.K = adapters[0]->h_in; c.N = adapters[0]->h_out;
  c.n_proj = num_proj;
  for (int p = 1; p < num_proj; ++p) {
    c.proj_Y[p] = static_cast<uint16_t*>(y[p]); c.proj_ldy[p] = ldy[p];
    c.proj_N[p] = adapters[p]->h_out;
    c.proj_Wtab[p] = adapters[p]->A_ptrs; c.proj_Vtab[p] = adapters[p]->B_ptrs;
    if (adapters[p]->A_ptrs_host && adapters[p]->B_ptrs_host) {
      c.proj_Wtab_host[p] = adapters[p]->A_ptrs_host;
      c.proj_Vtab_host[p] = adapters[p]->B_ptrs_host;
    }
  }
  c.token_rows = segments->token_rows;
  c.rows_host = segments->token_rows_host; c.n_rows = segments->num_tokens;
  const size_t part_off = (kCounterBytes + 255) / 256 * 256;
  c.counters = reinterpret_cast<int32_t*>(ws);
  c.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + part_off);
  c.rmax = rmax;
  return run_fwd(c, segs, {}, launcher);
}

int lora_sgmv_fused_multi(const void* x, int64_t ldx, int32_t num_proj,
                          const lora_adapters_t* const* adapters, const lora_segments_t* segments,
                          void* const* y, const int64_t* ldy, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  HipLauncher launcher(stream);
  return sgmv_fused_multi_impl(x, ldx, num_proj, adapters, segments, y, ldy, ws, ws_bytes, launcher);
}

static int packed_backward_impl(const void* x, int64_t ldx, const void* dy, int64_t lddy, const float* u,
                                int64_t ldu, const lora_adapters_t* adapters,
                                const lora_segments_t* segments, void* dx, int64_t lddx,
                                const uint64_t* dA_ptrs, const uint64_t* dB_ptrs, uint32_t flags,
                                void* ws, size_t ws_bytes, Launcher& launcher) {
  int st = common_checks(adapters, segments);
  if (st) return st;
  if (flags & ~LORA_GRAD_ACCUMULATE) return fail(LORA_INVALID_ARGUMENT, "unknown flags 0x%x", flags);
  const bool accumulate = (flags & LORA_GRAD_ACCUMULATE) != 0;
  const int N = adapters->num_adapters;
  const auto segs = active_segments(adapters, segments);
  // adapters whose gradients this call writes
  std::vector<int> with_tokens(N, 0);
  for (const auto& s : segs) with_tokens[s.adapter] = 1;
  bool any_zero_fill = false;
  if (!accumulate)
    for (int i = 0; i < N; ++i)
      if (adapters->ranks[i] > 0 && !with_tokens[i]) any_zero_fill = true;
  if (segs.empty() && !any_zero_fill) return LORA_OK;
  if (!dA_ptrs || !dB_ptrs) return fail(LORA_INVALID_ARGUMENT, "dA_ptrs/dB_ptrs is NULL");
  if (!segs.empty()) {
    if ((st = check_rows(x, ldx, adapters->h_in, "x", true))) return st;
    if ((st = check_rows(dy, lddy, adapters->h_out, "dy", true))) return st;
    if ((st = check_rows(dx, lddx, adapters->h_in, "dx", dx != nullptr))) return st;
    if ((st = check_gather(segments, ldx, adapters->h_in, "x", true))) return st;
    if ((st = check_gather(segments, lddy, adapters->h_out, "dy", true))) return st;
    if ((st = check_gather(segments, lddx, adapters->h_in, "dx", dx != nullptr))) return st;
    if (segments->token_rows_host && !segments->token_rows)
      return fail(LORA_INVALID_ARGUMENT, "lora_packed_backward: the row table must be in device memory (token_rows)");
    if (u && (st = check_u(u, ldu, max_rank_used(segs), "u"))) return st;
    if (!adapters->A_ptrs || !adapters->B_ptrs) return fail(LORA_INVALID_ARGUMENT, "A_ptrs/B_ptrs is NULL");
  }
  const WsLayout L = ws_layout(LORA_OP_BACKWARD, adapters, segments);
  if ((st = check_ws(ws, ws_bytes, L.total))) return st;

  char* wsb = static_cast<char*>(ws);
  float* partials = reinterpret_cast<float*>(wsb + L.partials);
  int32_t* counters = reinterpret_cast<int32_t*>(wsb + L.counters);
  float* dU = reinterpret_cast<float*>(wsb + L.du);
  const int rmax = max_rank_all(adapters);

  // u for dB: the caller's, or recomputed into the workspace
  const float* Uuse = u;
  int64_t lduse = ldu;
  if (!segs.empty() && !u) {
    FwdCall c{};
    c.mode_op = LORA_OP_SHRINK;
    c.X = static_cast<const uint16_t*>(x); c.ldx = ldx;
    c.U = reinterpret_cast<float*>(wsb + L.urec); c.ldu = L.lddu;
    c.Wtab = adapters->A_ptrs; c.v_round = 1;
    if (adapters->A_ptrs_host && adapters->B_ptrs_host) c.Wtab_host = adapters->A_ptrs_host;
    c.K = adapters->h_in; c.N = adapters->h_out;
    c.token_rows = segments->token_rows;
    c.partials = partials; c.counters = counters; c.rmax = rmax;
    if ((st = run_fwd(c, segs, {}, launcher))) return st;
    Uuse = c.U;
    lduse = L.lddu;
  }

  // adapter groups of at most kMaxSlots, in order of first appearance
  std::vector<int> order;
  {
    std::vector<int> seen(N, 0);
    for (const auto& s : segs)
      if (!seen[s.adapter]) { seen[s.adapter] = 1; order.push_back(s.adapter); }
  }
  // Weight gradients of the adapters marked in `member` (adapters without
  // tokens among them get zero gradients in overwrite mode).
  auto run_wgrad = [&](const std::vector<char>& member) -> int {
    // weight gradients: one job per adapter (several chained jobs if it has
    // too many segments)
    struct Job {
      int adapter, rank, accum;
      float scale;
      std::vector<std::pair<int, int>> segs;
      int part = -1;  // >= 0: a token-range part writing partial slot `part`
    };
    std::vector<Job> jobs;
    std::vector<std::vector<std::pair<int, int>>> per(N);
    for (const auto& s : segs)
      if (member[s.adapter]) per[s.adapter].push_back({s.tok0, s.ntok});
    // Load balance ("Technische Samenvatting: PLoRA" (gist.science),
    // "Kernelontwerp": balance over heterogeneous adapters): when the jobs
    // leave at least half of the GPU's resident workgroup slots idle, the
    // adapters with the longest token walks get their token ranges cut into
    // parts that run side by side, each into its own partial slot; a reduce
    // pass adds the parts in slot order, so the result does not depend on
    // scheduling. Parts go one at a time to the adapter whose part is longest,
    // while slots and idle workgroup slots last; the split is kept only if it
    // cuts the longest walk by at least 1.5x (a partial split that leaves an
    // unsplit adapter as long as before only adds traffic).
    std::vector<int> nparts(N, 1);
    {
      const int slots_gpu = 2 * launcher.dev().cus;
      int64_t items = 0;
      std::vector<int> steps(N, 0), it(N, 0);
      for (int a = 0; a < N; ++a) {
        if (adapters->ranks[a] == 0 || per[a].empty()) continue;
        for (auto& p : per[a]) steps[a] += cdiv(p.second, kTileM);
        it[a] = wgrad_items_for_rank(adapters->ranks[a], adapters->h_in, adapters->h_out);
        items += it[a];
      }
      int free_slots = L.wpart_slots;
      if (items > 0 && 2 * items <= slots_gpu && free_slots >= 2) {
        auto part_len = [&](int a) { return cdiv(steps[a], nparts[a]); };
        int crit0 = 0;
        for (int a = 0; a < N; ++a) crit0 = std::max(crit0, steps[a]);
        for (;;) {
          int best = -1;
          for (int a = 0; a < N; ++a)
            if (steps[a] > 0 && (best < 0 || part_len(a) > part_len(best))) best = a;
          if (best < 0) break;
          const int np = nparts[best] + 1;
          const int cost = nparts[best] == 1 ? 2 : 1;  // a split adapter uses a slot per part
          if ((int)per[best].size() > kMaxJobSeg || steps[best] / np < kSplitMinSteps ||
              cost > free_slots || items + it[best] > slots_gpu)
            break;
          nparts[best] = np;
          free_slots -= cost;
          items += it[best];
        }
        int crit1 = 0;
        for (int a = 0; a < N; ++a)
          if (steps[a] > 0) crit1 = std::max(crit1, part_len(a));
        if (2 * crit0 < 3 * crit1) std::fill(nparts.begin(), nparts.end(), 1);
      }
    }
    struct Red { int adapter, slot0, nparts; };
    std::vector<Red> reds;
    int next_slot = 0;
    for (int a = 0; a < N; ++a) {
      if (adapters->ranks[a] == 0 || !member[a]) continue;
      if (per[a].empty()) {
        if (!accumulate) jobs.push_back(Job{a, adapters->ranks[a], 0, adapters->scales[a], {}});
        continue;
      }
      if (nparts[a] > 1) {
        // part p takes 32-token steps [p S / P, (p + 1) S / P) of the adapter's
        // S steps, in segment order; a segment cut inside keeps whole steps
        int S = 0;
        for (auto& p : per[a]) S += cdiv(p.second, kTileM);
        const int P = nparts[a];
        reds.push_back(Red{a, next_slot, P});
        size_t seg = 0;
        int off = 0;  // tokens of per[a][seg] already given out
        for (int p = 0; p < P; ++p) {
          int need = (int)((int64_t)(p + 1) * S / P - (int64_t)p * S / P);
          Job j{a, adapters->ranks[a], 0, adapters->scales[a], {}, next_slot + p};
          while (need > 0 && seg < per[a].size()) {
            const int t0 = per[a][seg].first + off;
            const int left = per[a][seg].second - off;
            const int take = std::min(left, need * kTileM);
            j.segs.push_back({t0, take});
            need -= cdiv(take, kTileM);
            off += take;
            if (off >= per[a][seg].second) { ++seg; off = 0; }
          }
          jobs.push_back(std::move(j));
        }
        next_slot += P;
        continue;
      }
      for (size_t k = 0; k < per[a].size(); k += kMaxJobSeg) {
        Job j{a, adapters->ranks[a], (accumulate || k > 0) ? 1 : 0, adapters->scales[a], {}};
        for (size_t q = k; q < std::min(per[a].size(), k + kMaxJobSeg); ++q) j.segs.push_back(per[a][q]);
        jobs.push_back(std::move(j));
      }
    }
    // heavy jobs first; continuation jobs of one adapter must land in later launches
    std::vector<size_t> idx(jobs.size());
    for (size_t i = 0; i < idx.size(); ++i) idx[i] = i;
    auto tokens_of = [&](const Job& j) {
      int64_t n = 0;
      for (auto& p : j.segs) n += p.second;
      return n;
    };
    std::stable_sort(idx.begin(), idx.end(), [&](size_t p, size_t q) {
      const Job &a = jobs[p], &b = jobs[q];
      if (a.accum != b.accum && a.adapter == b.adapter) return a.accum < b.accum;
      return tokens_of(a) * (int64_t)(a.rank + 16) > tokens_of(b) * (int64_t)(b.rank + 16);
    });
    std::vector<int> done(jobs.size(), 0);
    size_t remaining = jobs.size();
    while (remaining > 0) {
      WgradPlan W;
      std::memset(&W, 0, sizeof(W));
      W.x = static_cast<const uint16_t*>(x); W.ldx = ldx;
      W.dy = static_cast<const uint16_t*>(dy); W.lddy = lddy;
      W.U = Uuse; W.ldu = lduse; W.dU = dU; W.lddu = L.lddu;
      W.dA_tab = dA_ptrs; W.dB_tab = dB_ptrs; W.token_rows = segments->token_rows;
      W.h_in = adapters->h_in; W.h_out = adapters->h_out;
      W.part_base = reinterpret_cast<float*>(wsb + L.wpart);
      W.part_stride = L.wpart_stride;
      int nj = 0, nseg = 0, grid = 0;
      std::vector<int> adapter_in_launch(N, 0);
      for (size_t ii = 0; ii < idx.size(); ++ii) {
        const size_t j = idx[ii];
        if (done[j]) continue;
        const Job& J = jobs[j];
        if (nj >= kMaxJobs || nseg + (int)J.segs.size() > kMaxJobSeg) break;
        if (J.part < 0) {
          // chained jobs of one adapter: one per launch, in order
          if (adapter_in_launch[J.adapter]) continue;
          bool earlier_pending = false;
          for (size_t q = 0; q < jobs.size(); ++q)
            if (!done[q] && q != j && jobs[q].adapter == J.adapter && jobs[q].accum < J.accum) earlier_pending = true;
          if (earlier_pending) continue;
        }
        W.job_item0[nj] = grid;
        W.job_adapter[nj] = J.adapter;
        W.job_seg0[nj] = nseg;
        W.job_nseg[nj] = (int)J.segs.size();
        W.job_nsteps[nj] = 0;
        for (auto& p : J.segs) W.job_nsteps[nj] += cdiv(p.second, kTileM);
        W.job_accum[nj] = J.accum;
        W.job_scale[nj] = J.scale;
        W.job_rank[nj] = J.rank;
        W.job_part[nj] = J.part;
        for (auto& p : J.segs) { W.seg_tok0[nseg] = p.first; W.seg_ntok[nseg] = p.second; ++nseg; }
        grid += wgrad_items_for_rank(J.rank, adapters->h_in, adapters->h_out);
        if (J.part < 0) adapter_in_launch[J.adapter] = 1;
        done[j] = 1;
        --remaining;
        ++nj;
      }
      if (nj == 0) return fail(LORA_DEVICE_ERROR, "internal planner error (no weight-gradient job placed)");
      W.n_jobs = nj;
      W.job_item0[nj] = grid;
      const hipError_t e = launcher.wgrad(W, grid);
      if (e != hipSuccess) return fail(LORA_DEVICE_ERROR, "weight-gradient launch failed: %s", hipGetErrorString(e));
    }
    if (!reds.empty()) {
      WgradReducePlan R;
      std::memset(&R, 0, sizeof(R));
      R.part_base = reinterpret_cast<const float*>(wsb + L.wpart);
      R.part_stride = L.wpart_stride;
      R.dA_tab = dA_ptrs; R.dB_tab = dB_ptrs;
      R.h_in = adapters->h_in; R.h_out = adapters->h_out;
      R.accumulate = accumulate ? 1 : 0;
      int grid = 0;
      for (const Red& r : reds) {
        const int j = R.n_red++;
        R.red_item0[j] = grid;
        R.red_adapter[j] = r.adapter;
        R.red_rank[j] = adapters->ranks[r.adapter];
        R.red_slot0[j] = r.slot0;
        R.red_nparts[j] = r.nparts;
        grid += (int)cdiv64((int64_t)(adapters->h_in + adapters->h_out) * R.red_rank[j], kReduceElems);
      }
      R.red_item0[R.n_red] = grid;
      const hipError_t e = launcher.reduce(R);
      if (e != hipSuccess) return fail(LORA_DEVICE_ERROR, "weight-gradient reduce launch failed: %s", hipGetErrorString(e));
    }
    return LORA_OK;
  };

  // Adapter groups: at most kMaxSlots adapters, and (with a byte budget set)
  // at most that many bytes of dy. Each group runs its du/dx pass and then
  // its weight gradients, so that a group's dy can still be in the
  // Infinity Cache when the weight-gradient pass reads it a second time.
  const int64_t budget = bwd_group_bytes();
  std::vector<int64_t> tok_of(N, 0);
  for (const auto& s : segs) tok_of[s.adapter] += s.ntok;
  std::vector<size_t> gstart{0};
  {
    int64_t bytes = 0;
    for (size_t k = 0; k < order.size(); ++k) {
      const int64_t b = tok_of[order[k]] * (int64_t)adapters->h_out * 2;
      const size_t n = k - gstart.back();
      if (n > 0 && (n >= (size_t)kMaxSlots || (budget > 0 && bytes + b > budget))) {
        gstart.push_back(k);
        bytes = 0;
      }
      bytes += b;
    }
    if (gstart.back() != order.size()) gstart.push_back(order.size());
  }
  std::vector<char> has_tokens(N, 0);
  for (int a : order) has_tokens[a] = 1;
  std::vector<int> slot_of(N, 0);
  for (size_t gi = 0; gi + 1 < gstart.size(); ++gi) {
    const size_t g0 = gstart[gi];
    const int ng = (int)(gstart[gi + 1] - g0);
    std::vector<int> in_group(N, 0);
    TransposePlan T;
    std::memset(&T, 0, sizeof(T));
    T.A_tab = adapters->A_ptrs; T.B_tab = adapters->B_ptrs;
    T.Bt = reinterpret_cast<uint16_t*>(wsb + L.bt);
    T.At = reinterpret_cast<uint16_t*>(wsb + L.at);
    T.bt_slot_elems = L.bt_slot; T.at_slot_elems = L.at_slot;
    T.h_in = adapters->h_in; T.h_out = adapters->h_out;
    T.n_slots = ng;
    int grmax = 0;
    for (int k = 0; k < ng; ++k) {
      const int a = order[g0 + k];
      in_group[a] = 1;
      slot_of[a] = k;
      T.slot_adapter[k] = a;
      T.slot_rank[k] = adapters->ranks[a];
      grmax = std::max(grmax, adapters->ranks[a]);
    }
    T.tb_cols = cdiv(grmax, 64);
    T.tiles_b = cdiv(adapters->h_out, 64) * T.tb_cols;
    T.ta_cols = cdiv(adapters->h_in, 64);
    T.tiles_a = cdiv(round_up(grmax, 8), 64) * T.ta_cols;
    hipError_t e = launcher.transpose(T);
    if (e != hipSuccess) return fail(LORA_DEVICE_ERROR, "transpose launch failed: %s", hipGetErrorString(e));

    std::vector<ActiveSeg> gsegs;
    for (const auto& s : segs)
      if (in_group[s.adapter]) gsegs.push_back(s);
    // du = s B^T dy (kept in the workspace) and dx += A^T du
    FwdCall c{};
    c.mode_op = dx ? LORA_OP_FUSED : LORA_OP_SHRINK;
    c.X = static_cast<const uint16_t*>(dy); c.ldx = lddy;
    c.Y = static_cast<uint16_t*>(dx); c.ldy = lddx;
    c.U = dU; c.ldu = L.lddu; c.write_u = true;
    c.Wslots = T.Bt; c.Vslots = T.At;
    c.w_slot_elems = L.bt_slot; c.v_slot_elems = L.at_slot;
    c.v_round = 8; c.scale_in_shrink = 1;
    c.K = adapters->h_out; c.N = adapters->h_in;
    c.token_rows = segments->token_rows;
    c.partials = partials; c.counters = counters; c.rmax = rmax;
    if ((st = run_fwd(c, gsegs, slot_of, launcher))) return st;
    // the group's weight gradients (the last group also writes the zero
    // gradients of adapters that have no tokens)
    const bool last = gi + 2 == gstart.size();
    std::vector<char> member(N, 0);
    for (int k = 0; k < ng; ++k) member[order[g0 + k]] = 1;
    if (last)
      for (int a2 = 0; a2 < N; ++a2)
        if (!has_tokens[a2]) member[a2] = 1;
    if ((st = run_wgrad(member))) return st;
  }
  if (order.empty()) {
    // no tokens at all: only the zero gradients (overwrite mode)
    std::vector<char> member(N, 1);
    if ((st = run_wgrad(member))) return st;
  }

  return LORA_OK;
}

int lora_packed_backward(const void* x, int64_t ldx, const void* dy, int64_t lddy, const float* u,
                         int64_t ldu, const lora_adapters_t* adapters,
                         const lora_segments_t* segments, void* dx, int64_t lddx,
                         const uint64_t* dA_ptrs, const uint64_t* dB_ptrs, uint32_t flags,
                         void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  HipLauncher launcher(stream);
  return packed_backward_impl(x, ldx, dy, lddy, u, ldu, adapters, segments, dx, lddx, dA_ptrs, dB_ptrs, flags,
                              ws, ws_bytes, launcher);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Batches planned on the device (graph-capturable decode)
// ---------------------------------------------------------------------------
namespace {

struct GraphLayout {
  size_t counters = 0, epoch = 0, partials = 0, tiles = 0, hdr = 0, perm = 0, total = 0;
  int max_tiles = 0;
};

// Workspace of lora_sgmv_fused_graph: hand-off words, the epoch's slots
// (these two at the same offsets for every num_tokens), split-shrink parts
// for the largest tile count the batch can have (each adapter adds at most
// one ragged tile), the tile table, a 256-byte header (tile count at +0) and
// the sorted-position -> row table.
GraphLayout graph_layout(const lora_graph_adapters_t* a, int T) {
  GraphLayout L;
  L.max_tiles = std::max(1, cdiv(T, kTileM) + std::min(a->num_adapters, T));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) / 256 * 256;
    return o;
  };
  L.counters = take(kCounterBytes);
  L.epoch = take((size_t)kEpochSlots * kEpochStride);  // at the same offset for every num_tokens
  const int64_t parts = std::min<int64_t>(kMaxPartials, (int64_t)L.max_tiles * kMaxKs);
  L.partials = take((size_t)parts * kTileM * rpad_for(a->max_rank) * sizeof(float));
  L.tiles = take((size_t)L.max_tiles * sizeof(DevTile));
  L.hdr = take(256);
  L.perm = take((size_t)std::max(T, 1) * sizeof(int32_t));
  L.total = off;
  return L;
}

int check_graph_adapters(const lora_graph_adapters_t* a) {
  if (!a) return fail(LORA_INVALID_ARGUMENT, "adapters is NULL");
  if (a->num_adapters < 1 || a->num_adapters > kMaxGraphAdapters)
    return fail(LORA_INVALID_ARGUMENT, "num_adapters must be in [1, %d]", kMaxGraphAdapters);
  if (a->h_in <= 0 || a->h_out <= 0 || (a->h_in & 7) || (a->h_out & 7))
    return fail(LORA_INVALID_ARGUMENT, "h_in (%d) and h_out (%d) must be positive multiples of 8", a->h_in,
                a->h_out);
  if (a->max_rank < 1) return fail(LORA_INVALID_ARGUMENT, "max_rank must be >= 1");
  if (a->max_rank > LORA_MAX_RANK) return fail(LORA_UNSUPPORTED, "max_rank %d exceeds %d", a->max_rank, LORA_MAX_RANK);
  if (!a->A_ptrs || !a->B_ptrs || !a->ranks || !a->scales)
    return fail(LORA_INVALID_ARGUMENT, "A_ptrs/B_ptrs/ranks/scales device arrays must not be NULL");
  return LORA_OK;
}

int sgmv_fused_graph_impl(const void* x, int64_t ldx, const lora_graph_adapters_t* a, const int32_t* token_ids,
                          int32_t T, void* y, int64_t ldy, void* ws, size_t ws_bytes, Launcher& launcher) {
  int st = check_graph_adapters(a);
  if (st) return st;
  if (T < 0) return fail(LORA_INVALID_ARGUMENT, "num_tokens must be >= 0");
  if (T == 0) return LORA_OK;
  if (!token_ids) return fail(LORA_INVALID_ARGUMENT, "token_ids is NULL");
  if ((st = check_rows(x, ldx, a->h_in, "x", true))) return st;
  if ((st = check_rows(y, ldy, a->h_out, "y", true))) return st;
  // the rows are request rows 0 .. T-1, reached through the in-kernel gather
  lora_segments_t rows{T, 0, nullptr, nullptr, reinterpret_cast<const int32_t*>(1)};
  if ((st = check_gather(&rows, ldx, a->h_in, "x", true))) return st;
  if ((st = check_gather(&rows, ldy, a->h_out, "y", true))) return st;
  if (x == y) return fail(LORA_INVALID_ARGUMENT, "x and y must not overlap");
  const GraphLayout G = graph_layout(a, T);
  if ((st = check_ws(ws, ws_bytes, G.total))) return st;
  char* wsb = static_cast<char*>(ws);
  uint64_t* epoch = reinterpret_cast<uint64_t*>(wsb + G.epoch);
  const bool self_plan = T <= kSelfPlanTokens;
  DevPlanArgs D{};
  D.ids = token_ids;
  D.A_ptrs = a->A_ptrs; D.B_ptrs = a->B_ptrs; D.ranks = a->ranks; D.scales = a->scales;
  D.perm = reinterpret_cast<int32_t*>(wsb + G.perm);
  D.tiles = reinterpret_cast<DevTile*>(wsb + G.tiles);
  D.count = reinterpret_cast<int32_t*>(wsb + G.hdr);
  D.epoch = epoch;
  D.T = T; D.N = a->num_adapters; D.max_rank = a->max_rank; D.max_tiles = G.max_tiles;
  hipError_t e;
  if (!self_plan) {
    e = launcher.dev_plan(D);
    if (e != hipSuccess) return fail(LORA_DEVICE_ERROR, "plan kernel launch failed: %s", hipGetErrorString(e));
  }
  // the fused launch is laid out for the largest tile count; tiles past the
  // count of the batch have no work
  FwdCall c{};
  c.mode_op = LORA_OP_FUSED;
  c.K = a->h_in; c.N = a->h_out;
  FwdPlan P;
  std::memset(&P, 0, sizeof(P));
  P.X = static_cast<const uint16_t*>(x); P.ldx = ldx;
  P.Y = static_cast<uint16_t*>(y); P.ldy = ldy;
  P.partials = reinterpret_cast<float*>(wsb + G.partials);
  P.counters = reinterpret_cast<int32_t*>(wsb + G.counters);
  P.stamps = reinterpret_cast<uint64_t*>(wsb + G.counters + kStampOffset);
  P.dev_epoch = epoch;
  if (self_plan) {
    P.self_ids = token_ids;
    P.self_A = a->A_ptrs; P.self_B = a->B_ptrs; P.self_ranks = a->ranks; P.self_scales = a->scales;
    P.self_T = T; P.self_N = a->num_adapters; P.self_max_rank = a->max_rank;
  } else {
    P.token_rows = D.perm;
    P.dev_tiles = D.tiles; P.dev_count = D.count;
  }
  P.ptrs_in_plan = 1;
  P.K = a->h_in; P.N = a->h_out; P.v_round = 1;
  P.rpad = rpad_for(a->max_rank);
  P.n_seg = 0;
  P.n_tiles = G.max_tiles;
  const DeviceInfo dev = launcher.dev();
  P.spin_ticks = (int)std::min<int64_t>((int64_t)dev.wall_khz * 1000 / 5000, 1 << 30);
  fused_layout(P, c, G.max_tiles, a->max_rank, cdiv(a->h_out, 32), dev);
  if (P.mode == kModeFusedDep && (int64_t)G.max_tiles * P.ks > kMaxPartials)
    return fail(LORA_UNSUPPORTED, "batch too large for the split layout of a device-planned call");
  if ((uint64_t)P.grid >= kEpochCall)
    return fail(LORA_UNSUPPORTED, "grid of %d workgroups too large for a device-planned call", P.grid);
  if (self_plan && P.mode == kModeFusedDep && 4 * G.max_tiles <= dev.cus) {
    // the small-batch split layouts: the workgroups re-lay them out for the
    // tiles the batch has (column chunks per tile; grid and k split kept)
    P.self_relayout = P.xcd_local ? 1 : 2;
    P.self_slots = 2 * dev.cus;
  }
  const int rbmax = a->max_rank <= 32 ? 1 : (a->max_rank <= 64 ? 2 : 4);
  e = launcher.fwd(P, rbmax, nullptr, nullptr, nullptr, 0);
  if (e != hipSuccess) return fail(LORA_DEVICE_ERROR, "kernel launch failed: %s", hipGetErrorString(e));
  return LORA_OK;
}

}  // namespace

extern "C" {

int lora_workspace_size_graph(const lora_graph_adapters_t* adapters, int32_t num_tokens, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(LORA_INVALID_ARGUMENT, "bytes is NULL");
  int st = check_graph_adapters(adapters);
  if (st) return st;
  if (num_tokens < 0) return fail(LORA_INVALID_ARGUMENT, "num_tokens must be >= 0");
  *bytes = graph_layout(adapters, num_tokens).total;
  return LORA_OK;
}

int lora_sgmv_fused_graph(const void* x, int64_t ldx, const lora_graph_adapters_t* adapters,
                          const int32_t* token_ids, int32_t num_tokens, void* y, int64_t ldy, void* ws,
                          size_t ws_bytes, void* stream) {
  g_last_error.clear();
  HipLauncher launcher(stream);
  return sgmv_fused_graph_impl(x, ldx, adapters, token_ids, num_tokens, y, ldy, ws, ws_bytes, launcher);
}

// ---------------------------------------------------------------------------
// Host-only plan inspection (lora_inspect.h)
// ---------------------------------------------------------------------------
namespace {

// Lists the workgroups of every launch instead of launching anything.
struct Recorder final : Launcher {
  DeviceInfo d;
  lora_plan_item_t* items;
  int64_t cap, n = 0;
  int32_t* ranges;
  int64_t rcap, nr = 0;
  int launches = 0;
  int self_tiles = -1;  // launches planned inside themselves: the tiles their batch is taken to have
  void put(const lora_plan_item_t& r) {
    if (n < cap) items[n] = r;
    ++n;
  }
  DeviceInfo dev() override { return d; }
  hipError_t fwd(const FwdPlan& P, int rbmax, const uint64_t*, const uint64_t*, const int32_t*, int) override {
    (void)rbmax;
    if (P.grid <= 0) return hipErrorInvalidConfiguration;
    const int launch = launches++;
    if (P.self_ids || P.dev_tiles) {
      // a device-planned launch: what its workgroups do once the batch has
      // self_tiles tiles (counted by each workgroup, or by the plan kernel)
      const int tiles = std::max(0, self_tiles);
      int n_tiles = P.n_tiles, nc = P.nc, n_a = P.n_items_a, n_b = P.n_items_b, nblk = P.nblk;
      if (self_relayout_needed(P.self_relayout, tiles, P.n_tiles)) {
        nblk = self_relayout(P.self_relayout, tiles, P.ks, cdiv(P.N, 32), P.self_slots, P.grid, nc);
        n_tiles = tiles;
        n_a = tiles * P.ks;
        n_b = tiles * nc;
      }
      for (int b = 0; b < P.grid; ++b) {
        lora_plan_item_t r{};
        r.launch = launch; r.phase = LORA_PHASE_FWD; r.block = b; r.grid = P.grid; r.mode = P.mode;
        r.part = P.ks; r.aux = nc; r.adapter = -1; r.tok0 = -1; r.ntok = -1;
        const FwdItem it = fwd_item_at(P.mode, P.xcd_local, P.xcd_remap, P.grid, n_tiles, P.ks, nc, n_a, n_b, b);
        if (it.g < 0 || it.g >= tiles) {
          r.kind = -1; r.tile = -1;
        } else {
          r.kind = it.kind; r.tile = it.g;
          if (it.kind == kItemShrink) shrink_range(P.K, P.kchunk, it.c, r.lo, r.hi);
          else expand_cols(P.N, nblk, it.c, r.lo, r.hi);
        }
        put(r);
      }
      return hipSuccess;
    }
    for (int b = 0; b < P.grid; ++b) {
      lora_plan_item_t r{};
      r.launch = launch; r.phase = LORA_PHASE_FWD; r.block = b; r.grid = P.grid; r.mode = P.mode;
      r.part = P.ks; r.aux = P.nc;
      const FwdItem it = fwd_item(P, b);
      if (it.g < 0 || it.g >= P.n_tiles) {
        r.kind = -1; r.tile = -1; r.adapter = -1;
        put(r);
        continue;
      }
      int sel = 0;
      for (int i = 1; i < P.n_seg; ++i)
        if (it.g >= P.seg_tile0[i]) sel = i;
      const int tt = it.g - P.seg_tile0[sel];
      r.kind = it.kind; r.tile = it.g;
      r.adapter = P.seg_adapter[sel]; r.proj = P.seg_proj[sel]; r.rank = P.seg_rank[sel];
      r.tok0 = P.seg_tok0[sel] + tt * kTileM;
      r.ntok = std::min(kTileM, P.seg_ntok[sel] - tt * kTileM);
      if (it.kind == kItemShrink) {
        shrink_range(P.K, P.kchunk, it.c, r.lo, r.hi);
      } else {
        const int p = r.proj;
        expand_cols(p == 0 ? P.N : P.proj_N[p], p == 0 ? P.nblk : P.proj_nblk[p], it.c, r.lo, r.hi);
      }
      put(r);
    }
    return hipSuccess;
  }
  hipError_t transpose(const TransposePlan& P) override {
    if (P.n_slots * (P.tiles_b + P.tiles_a) <= 0) return hipErrorInvalidConfiguration;
    const int launch = launches++;
    for (int k = 0; k < P.n_slots; ++k) {
      lora_plan_item_t r{};
      r.launch = launch; r.phase = LORA_PHASE_TRANSPOSE; r.block = -1;
      r.grid = P.n_slots * (P.tiles_b + P.tiles_a); r.kind = 0; r.tile = k;
      r.adapter = P.slot_adapter[k]; r.rank = P.slot_rank[k];
      put(r);
    }
    return hipSuccess;
  }
  hipError_t wgrad(const WgradPlan& P, int grid) override {
    if (grid <= 0) return hipErrorInvalidConfiguration;
    const int launch = launches++;
    std::vector<int64_t> first(P.n_jobs);
    for (int j = 0; j < P.n_jobs; ++j) {
      first[j] = nr;
      for (int q = 0; q < P.job_nseg[j]; ++q) {
        if (nr < rcap) {
          ranges[2 * nr] = P.seg_tok0[P.job_seg0[j] + q];
          ranges[2 * nr + 1] = P.seg_ntok[P.job_seg0[j] + q];
        }
        ++nr;
      }
    }
    for (int b = 0; b < grid; ++b) {
      int j = 0;
      while (j + 1 < P.n_jobs && b >= P.job_item0[j + 1]) ++j;
      const int rank = P.job_rank[j];
      const int cw = wgrad_cw(rank);
      const int nb_db = cdiv(P.h_out, cw);
      const int local = b - P.job_item0[j];
      lora_plan_item_t r{};
      r.launch = launch; r.phase = LORA_PHASE_WGRAD; r.block = b; r.grid = grid;
      r.kind = local < nb_db ? 0 : 1;
      r.tile = j; r.adapter = P.job_adapter[j]; r.rank = rank;
      r.tok0 = (int32_t)first[j]; r.ntok = P.job_nseg[j];
      const int chunk = r.kind == 0 ? local : local - nb_db;
      const int ncols = r.kind == 0 ? P.h_out : P.h_in;
      r.lo = chunk * cw;
      r.hi = std::min(ncols, r.lo + cw);
      r.part = P.job_part[j]; r.aux = P.job_accum[j];
      put(r);
    }
    return hipSuccess;
  }
  hipError_t dev_plan(const DevPlanArgs& a) override {
    lora_plan_item_t r{};
    r.launch = launches++;
    r.phase = LORA_PHASE_PLAN;
    r.block = 0;
    r.grid = 1;
    r.kind = 0;
    r.tile = -1;
    r.adapter = -1;
    r.ntok = a.T;
    r.hi = a.max_tiles;
    put(r);
    return hipSuccess;
  }
  hipError_t reduce(const WgradReducePlan& R) override {
    const int grid = R.red_item0[R.n_red];
    if (grid <= 0) return hipErrorInvalidConfiguration;
    const int launch = launches++;
    for (int b = 0; b < grid; ++b) {
      int j = 0;
      while (j + 1 < R.n_red && b >= R.red_item0[j + 1]) ++j;
      const int64_t n_all = (int64_t)(R.h_in + R.h_out) * R.red_rank[j];
      lora_plan_item_t r{};
      r.launch = launch; r.phase = LORA_PHASE_REDUCE; r.block = b; r.grid = grid; r.tile = j;
      r.adapter = R.red_adapter[j]; r.rank = R.red_rank[j];
      const int64_t e0 = (int64_t)(b - R.red_item0[j]) * kReduceElems;
      r.lo = (int32_t)std::min(e0, n_all);
      r.hi = (int32_t)std::min(e0 + kReduceElems, n_all);
      r.part = R.red_slot0[j]; r.aux = R.red_nparts[j];
      put(r);
    }
    return hipSuccess;
  }
};

}  // namespace

extern "C" int lora_inspect_plan(int op, int32_t num_proj, const lora_adapters_t* const* adapters,
                                 const lora_segments_t* segments, uint32_t options, int32_t cus, int32_t xccs,
                                 lora_plan_item_t* items, int64_t items_cap, int64_t* n_items, int32_t* ranges,
                                 int64_t ranges_cap, int64_t* n_ranges) {
  g_last_error.clear();
  if (!adapters || !n_items || !n_ranges || (items_cap > 0 && !items) || (ranges_cap > 0 && !ranges))
    return fail(LORA_INVALID_ARGUMENT, "NULL argument");
  if (cus < 8 || xccs < 1) return fail(LORA_INVALID_ARGUMENT, "cus must be >= 8 and xccs >= 1");
  Recorder rec;
  rec.d = DeviceInfo{cus, 100000, xccs};
  rec.items = items; rec.cap = items_cap; rec.ranges = ranges; rec.rcap = ranges_cap;
  // stand-in device addresses (16-byte aligned, distinct, never dereferenced)
  char* const base = reinterpret_cast<char*>((uintptr_t)1 << 40);
  void* x = base;
  void* y = base + ((uintptr_t)1 << 36);
  float* u = reinterpret_cast<float*>(base + ((uintptr_t)2 << 36));
  void* ws = base + ((uintptr_t)3 << 36);
  const size_t ws_bytes = (size_t)1 << 35;
  void* dxp = base + ((uintptr_t)4 << 36);
  const uint64_t* tabs = reinterpret_cast<const uint64_t*>(base + ((uintptr_t)5 << 36));
  int st = LORA_OK;
  if (!adapters[0]) return fail(LORA_INVALID_ARGUMENT, "adapters[0] is NULL");
  const lora_adapters_t* a = adapters[0];
  const int64_t ldx = a->h_in, ldy = a->h_out, ldu = LORA_MAX_RANK;
  if (op == LORA_OP_FUSED && num_proj > 1) {
    void* ys[kMaxProj];
    int64_t lds[kMaxProj];
    for (int p = 0; p < std::min<int32_t>(num_proj, kMaxProj); ++p) {
      ys[p] = base + ((uintptr_t)(8 + p) << 36);
      lds[p] = adapters[p] ? adapters[p]->h_out : 8;
    }
    st = sgmv_fused_multi_impl(x, ldx, num_proj, adapters, segments, ys, lds, ws, ws_bytes, rec);
  } else if (num_proj != 1) {
    st = fail(LORA_INVALID_ARGUMENT, "num_proj must be 1 for this op");
  } else if (op == LORA_OP_SHRINK) {
    st = sgmv_shrink_impl(x, ldx, a, segments, u, ldu, ws, ws_bytes, rec);
  } else if (op == LORA_OP_EXPAND) {
    st = sgmv_expand_impl(u, ldu, a, segments, y, ldy, rec);
  } else if (op == LORA_OP_FUSED) {
    st = sgmv_fused_impl(x, ldx, a, segments, y, ldy, (options & LORA_INSPECT_WITH_U) ? u : nullptr, ldu, ws,
                         ws_bytes, rec);
  } else if (op == LORA_OP_BACKWARD) {
    st = packed_backward_impl(x, ldx, y, ldy, (options & LORA_INSPECT_WITH_U) ? u : nullptr, ldu, a, segments,
                              (options & LORA_INSPECT_WITH_DX) ? dxp : nullptr, ldx, tabs, tabs + 1024,
                              (options & LORA_INSPECT_ACCUMULATE) ? LORA_GRAD_ACCUMULATE : 0u, ws, ws_bytes, rec);
  } else {
    st = fail(LORA_INVALID_ARGUMENT, "unknown op %d", op);
  }
  *n_items = rec.n;
  *n_ranges = rec.nr;
  return st;
}

extern "C" int lora_inspect_graph(const lora_graph_adapters_t* adapters, int32_t num_tokens, int32_t tiles,
                                  int32_t cus, int32_t xccs, lora_plan_item_t* items, int64_t items_cap,
                                  int64_t* n_items) {
  g_last_error.clear();
  if (!adapters || !n_items || (items_cap > 0 && !items)) return fail(LORA_INVALID_ARGUMENT, "NULL argument");
  if (cus < 8 || xccs < 1) return fail(LORA_INVALID_ARGUMENT, "cus must be >= 8 and xccs >= 1");
  Recorder rec;
  rec.d = DeviceInfo{cus, 100000, xccs};
  rec.items = items; rec.cap = items_cap; rec.ranges = nullptr; rec.rcap = 0;
  rec.self_tiles = tiles;
  char* const base = reinterpret_cast<char*>((uintptr_t)1 << 40);
  int st = check_graph_adapters(adapters);
  if (!st) {
    const GraphLayout G = graph_layout(adapters, std::max(num_tokens, 0));
    st = sgmv_fused_graph_impl(base, adapters->h_in, adapters,
                               reinterpret_cast<const int32_t*>(base + ((uintptr_t)1 << 36)), num_tokens,
                               base + ((uintptr_t)2 << 36), adapters->h_out, base + ((uintptr_t)3 << 36), G.total,
                               rec);
  }
  *n_items = rec.n;
  return st;
}

}  // extern "C"

int lora::sgmv_fused_from(const void* x, int64_t ldx, const lora_adapters_t* adapters,
                          const lora_segments_t* segments, void* y, int64_t ldy, float* u_save, int64_t ldu,
                          WsSource& src, void* stream) {
  HipLauncher launcher(stream);
  return sgmv_fused_impl(x, ldx, adapters, segments, y, ldy, u_save, ldu, nullptr, 0, launcher, &src);
}
