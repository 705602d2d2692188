// Host side of the C ABI: argument and schema validation (all before any
// HIP call), the prepared-weight handle, schedule selection by rows per
// expert with a memoised descriptor cache, workspace carving, launch
// sequencing on the caller's stream, and optional per-kernel event timing.
#include <hip/hip_runtime.h>

#include <array>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "moe_launch.h"
#include "moe_layout.h"
#include "moe_w4a16.h"

using namespace moe;

// --------------------------------------------------------------------------
// Errors
// --------------------------------------------------------------------------

namespace {

thread_local std::string g_err;

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moe_status_t ok() {
  g_err.clear();
  return MOE_OK;
}

moe_status_t hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// --------------------------------------------------------------------------
// Environment overrides, read once per prepared handle (part of the
// descriptor key, like the tuning overrides the Chord page memoises with
// each descriptor in "Grouped SM90 kernels").
// --------------------------------------------------------------------------

struct EnvOverrides {
  int schedule = 0;   // MOE_W4A16_SCHEDULE: 0 auto, 1 small-M, 2 large-M
  int nt = 0;         // MOE_W4A16_NT: token tiles per weight pass (1, 2, 4)
  int log = 0;        // MOE_W4A16_LOG: print each new schedule
  int no_resident = 0;   // MOE_W4A16_NO_RESIDENT: keep the K-loop form of large-M for short K
  int job_wgs = 0;       // MOE_W4A16_JOB_WGS: cap on the persistent small-M grid (tests: long job walks)
  int ksplit = 0;        // MOE_W4A16_KSPLIT: force the small-M split-K factor (tests)
  int validate = 0;      // MOE_W4A16_VALIDATE: synchronous checks of device-side index data
  int wide = 0;          // MOE_W4A16_WIDE: large-M K loop over 256-row tiles (two blocks of an expert)
  // MOE_W4A16_XCD_DEAL: large-M K loop on blocks, blocks per unit dealt
  // round-robin to the XCDs (0: each XCD one contiguous range of blocks)
  int xcd_deal = 2;
  void read() {
    auto geti = [](const char* k, int dflt = 0) {
      const char* v = std::getenv(k);
      return v ? std::atoi(v) : dflt;
    };
    schedule = geti("MOE_W4A16_SCHEDULE");
    nt = geti("MOE_W4A16_NT");
    log = geti("MOE_W4A16_LOG");
    no_resident = geti("MOE_W4A16_NO_RESIDENT");
    job_wgs = geti("MOE_W4A16_JOB_WGS");
    ksplit = geti("MOE_W4A16_KSPLIT");
    validate = geti("MOE_W4A16_VALIDATE");
    wide = geti("MOE_W4A16_WIDE");
    xcd_deal = geti("MOE_W4A16_XCD_DEAL", 2);
  }
};

// --------------------------------------------------------------------------
// Kernel timing
// --------------------------------------------------------------------------

struct Profiler {
  std::mutex mu;
  bool on = false;
  struct Pending {
    const char* name;
    hipEvent_t a, b;
  };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  std::map<std::string, std::pair<long, double>> totals;

  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    // timing only: without the system-scope fence, recording an event
    // neither writes back nor invalidates the caches, which would change
    // the speed of the launch that follows it
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
  }
  void drain() {   // caller holds mu
    for (auto& p : pending) {
      float ms = 0.f;
      (void)hipEventSynchronize(p.b);
      (void)hipEventElapsedTime(&ms, p.a, p.b);
      auto& t = totals[p.name];
      t.first += 1;
      t.second += ms;
      pool.push_back(p.a);
      pool.push_back(p.b);
    }
    pending.clear();
  }
};

Profiler& prof() {
  static Profiler* p = new Profiler();   // never destroyed: events outlive static teardown
  return *p;
}

template <class F>
hipError_t run(const char* name, hipStream_t s, F&& f) {
  Profiler& P = prof();
  bool on;
  {
    std::lock_guard<std::mutex> g(P.mu);
    on = P.on;
  }
  if (!on) return f();
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> g(P.mu);
    if (P.pending.size() > 4096) P.drain();
    a = P.get();
    b = P.get();
  }
  if (a) (void)hipEventRecord(a, s);
  hipError_t e = f();
  if (b) (void)hipEventRecord(b, s);
  if (a && b) {
    std::lock_guard<std::mutex> g(P.mu);
    P.pending.push_back({name, a, b});
  }
  return e;
}

// --------------------------------------------------------------------------
// Schedules
// --------------------------------------------------------------------------

enum { SCHED_SMALL_M = 1, SCHED_LARGE_M = 2 };

// Rows per expert at which the large-M schedule takes over (Chord page,
// "Indexed kernels", Fig. 2 and "H200 prefill and TP8": about 80 tokens per
// expert is where block_m starts to follow each expert's padded rows).
constexpr int kLargeMRows = 80;

struct Schedule {
  int kind = SCHED_SMALL_M;
  int block = 16;   // routing alignment block (indexed)
  int nt = 1;       // 16-row token tiles per weight pass (small-M)
  int dispatch = 0; // small-M: 0 semi-static grid over experts, 1 persistent static ranges,
                    // 2 persistent job queue, 3 semi-static grid over routing blocks
  int ksplit13 = 1, ksplit2 = 1;   // small-M semi-static: K splits of W13 / W2 (grid-starved calls)
  int rows = 0;     // rows per expert the choice was made for
};

// Workgroups the K-resident large-M form aims for (about four per CU slot
// of the 256 CUs at two workgroups each).
constexpr int kResidentTargetWgs = 2048;

// Grid of the persistent small-M forms: one workgroup per resident slot (4,
// 3 or 2 per CU by token tiles), and enough that no static job range spans
// more than 62 routing blocks (the kernel keeps one entry per block of its
// range in a 64-lane register).
int job_grid(int nsets, int passes, int quads, int nt, const EnvOverrides& env) {
  const int slots = 256 * (nt == 1 ? 4 : (nt == 2 ? 3 : 2));
  const int64_t jobs = (int64_t)nsets * passes * quads;
  int64_t g = jobs < slots ? jobs : slots;
  if (env.job_wgs > 0 && g > env.job_wgs) g = env.job_wgs;
  const int64_t gmin = (nsets + 59) / 60;
  if (g < gmin) g = gmin;
  return (int)g;
}

// Launches one GEMM (mat 13 or 2) with the schedule's kernel, timed under a
// fixed name. Large-M with K of one or two chunks on a routing or contiguous
// row set takes the K-resident form: the token tile stays in LDS while a
// workgroup walks several quads of output row groups.
hipError_t run_gemm(int mat, const Schedule& sc, const GemmParams& p0, int set, int epi, hipStream_t s,
                    const EnvOverrides& env) {
  if (sc.kind == SCHED_LARGE_M) {
    GemmParams p = p0;
    if (!env.no_resident && p.Kc <= 2 && set != SET_MASKED && p.nsets > 0) {
      const int nquads = (p.RG + 3) / 4;
      int wgs = (kResidentTargetWgs + p.nsets - 1) / p.nsets;
      wgs = wgs < 1 ? 1 : (wgs > nquads ? nquads : wgs);
      p.qpw = (nquads + wgs - 1) / wgs;
      p.wg_per_set = (nquads + p.qpw - 1) / p.qpw;
      p.total_wg = p.nsets * p.wg_per_set;
    }
    // K loop over pairs of blocks
    if (env.wide && p.qpw == 0 && set != SET_MASKED && p.Kc % 2 == 0 && src_fits_u32(p, set)) {
      p.total_wg = (p.nsets + 1) / 2 * p.wg_per_set;
      return run(mat == 13 ? "gemm_w13_large_m" : "gemm_w2_large_m", s,
                 [&] { return launch_gemm_wide(p, set, epi, s); });
    }
    // K loop on blocks: units of xcd_deal blocks dealt round-robin to the
    // XCDs, so that runs of equal-cost blocks (one expert's) spread over all
    // of them (measured on the Zipf prefill: units of 2 blocks -4 % against
    // contiguous ranges per XCD, 1 or 4 blocks -3 %)
    if (p.qpw == 0 && set != SET_MASKED && env.xcd_deal > 0) {
      const int G = env.xcd_deal, units = (p.nsets + G - 1) / G;
      p.xcd_deal = G;
      p.total_wg = 8 * ((units + 7) / 8) * G * p.wg_per_set;
    }
    return run(mat == 13 ? "gemm_w13_large_m" : "gemm_w2_large_m", s,
               [&] { return launch_gemm_large_m(p, set, epi, s); });
  }
  GemmParams p = p0;
  if (p.dispatch) p.total_wg = job_grid(p.nsets, p.passes, p.wg_per_set, sc.nt, env);
  return run(mat == 13 ? "gemm_w13_small_m" : "gemm_w2_small_m", s,
             [&] { return launch_gemm_small_m(p, set, epi, sc.nt, s); });
}

// Routing blocks that can hold rows: each holds at least one of the T*topk.
int block_bound(const RoutingLayout& R, int T, int topk) {
  const int64_t flat = (int64_t)T * topk;
  return flat < R.nblocks ? (int)flat : R.nblocks;
}

// Experts that can hold rows: the per-expert small-M grid covers this many
// sets, the kernel mapping set i to the i-th expert with rows when it is
// below E.
int expert_bound(int E, int T, int topk) {
  const int64_t flat = (int64_t)T * topk;
  return flat < E ? (int)flat : E;
}

int nt_for_rows(int rows) {
  if (rows <= 16) return 1;
  if (rows <= 32) return 2;
  return 4;
}

}  // namespace

// The memo key: the whole descriptor a schedule is a function of (mode, the
// two shape ints, and every override field), compared field by field.
struct ScheduleKey {
  std::array<int32_t, 8> v;
  bool operator<(const ScheduleKey& o) const { return v < o.v; }
};

struct moe_weights {
  moe_weight_desc_t desc{};
  PreparedLayout lay;
  char* prepared = nullptr;
  size_t prepared_bytes = 0;
  int device = 0;
  EnvOverrides env;
  std::mutex mu;
  std::map<ScheduleKey, Schedule> cache;
};

namespace {

ScheduleKey key_of(int mode, int a, int b, const moe_tuning_t* o) {
  ScheduleKey k{};
  k.v = {mode, a, b, o != nullptr, o ? o->block_m : 0, o ? o->schedule : 0,
         o ? o->dispatch : 0, o ? o->global_experts : 0};
  return k;
}

// Indexed: rows per expert tok_e = ceil(T*topk / E) picks the schedule (the
// Chord page's tok_e rule: tokens per expert, not total tokens).
// The large-M kernel works on whole K chunks of 128 (both GEMMs).
bool large_m_fits(const moe_weights* h) {
  return h->desc.hidden % kKC == 0 && h->desc.inter % kKC == 0;
}

const char* kind_name(int kind) { return kind == SCHED_LARGE_M ? "large-M" : "small-M"; }

// An explicit large-M request the kernel cannot serve (K not whole chunks,
// or an alignment block other than its 128-row tile).
bool large_m_rejected(const moe_weights* h, const moe_tuning_t* ovr) {
  return ovr && ovr->schedule == SCHED_LARGE_M &&
         (!large_m_fits(h) || (ovr->block_m && ovr->block_m != 128));
}

// Indexed: rows per expert tok_e = ceil(T*topk / E) picks the schedule (the
// Chord page's tok_e rule: tokens per expert, not total tokens). Large-M
// aligns each expert to 128-row blocks, its token tile.
Schedule schedule_indexed(moe_weights* h, int T, int topk, const moe_tuning_t* ovr) {
  const ScheduleKey key = key_of(MOE_MODE_INDEXED, T, topk, ovr);
  std::lock_guard<std::mutex> g(h->mu);
  auto it = h->cache.find(key);
  if (it != h->cache.end()) return it->second;
  Schedule s;
  // rows per expert: over the handle's experts, or with ovr.global_experts
  // (expert parallelism) over the global pool the routing is drawn from
  const int E = ovr && ovr->global_experts > 0 ? ovr->global_experts : h->desc.num_experts;
  const long rows = ((long)T * topk + E - 1) / E;
  s.rows = (int)rows;
  s.kind = rows < kLargeMRows ? SCHED_SMALL_M : SCHED_LARGE_M;
  if (h->env.schedule) s.kind = h->env.schedule;
  if (ovr && ovr->block_m && ovr->block_m != 128) s.kind = SCHED_SMALL_M;
  if (ovr && ovr->schedule) s.kind = ovr->schedule;
  if (!large_m_fits(h)) s.kind = SCHED_SMALL_M;
  s.nt = nt_for_rows((int)rows);
  if (h->env.nt) s.nt = h->env.nt;
  if (ovr && s.kind == SCHED_SMALL_M) s.dispatch = ovr->dispatch;
  // the routing-block forms take one block per weight pass of 16*nt rows
  s.block = s.kind == SCHED_LARGE_M ? 128 : (s.dispatch ? 16 * s.nt : 16);
  if (ovr && ovr->block_m) s.block = ovr->block_m;
  if (s.kind == SCHED_SMALL_M && (s.dispatch == 0 || s.dispatch == 3)) {
    // split K when the grid cannot fill the resident slots: at most
    // min(E, local rows) experts hold rows, each with ceil(RG/4) quads
    const int Eh = h->desc.num_experts;
    const long flat = (long)T * topk;
    const long local = ovr && ovr->global_experts > 0 ? (flat * Eh + ovr->global_experts - 1) / ovr->global_experts
                                                      : flat;
    const long sets = local < Eh ? local : Eh;
    const int slots = 256 * (s.nt == 1 ? 4 : (s.nt == 2 ? 3 : 2));
    auto split_for = [&](const MatLayout& m) {
      const long wgs = sets * ((m.RG + 3) / 4);
      int k = 1;
      if (wgs > 0 && 2 * wgs <= slots) k = (int)((slots + wgs - 1) / wgs);   // under half full
      if (h->env.ksplit > 0) k = h->env.ksplit;
      const int kmax = m.Kc / 8 > 1 ? m.Kc / 8 : 1;   // at least 8 chunks per split
      if (k > 8) k = 8;
      if (k > kmax) k = h->env.ksplit > 0 ? (h->env.ksplit < m.Kc ? h->env.ksplit : m.Kc) : kmax;
      return k < 1 ? 1 : k;
    };
    s.ksplit13 = split_for(h->lay.w13);
    s.ksplit2 = split_for(h->lay.w2);
  }
  if (h->env.log)
    std::fprintf(stderr, "[moe_w4a16] indexed T=%d topk=%d rows/expert=%ld -> %s nt=%d block=%d\n",
                 T, topk, rows, kind_name(s.kind), s.nt, s.block);
  h->cache.emplace(key, s);
  return s;
}

Schedule schedule_masked(moe_weights* h, int max_m, int expected_m) {
  const ScheduleKey key = key_of(MOE_MODE_MASKED, max_m, expected_m, nullptr);
  std::lock_guard<std::mutex> g(h->mu);
  auto it = h->cache.find(key);
  if (it != h->cache.end()) return it->second;
  Schedule s;
  s.rows = expected_m;
  s.kind = expected_m < kLargeMRows ? SCHED_SMALL_M : SCHED_LARGE_M;
  if (h->env.schedule) s.kind = h->env.schedule;
  if (!large_m_fits(h)) s.kind = SCHED_SMALL_M;
  // Small-M: the row budget bounds every expert's rows; cover it in one
  // weight pass when it fits four token tiles.
  s.nt = nt_for_rows(max_m < 64 ? max_m : 64);
  if (h->env.nt) s.nt = h->env.nt;
  if (h->env.log)
    std::fprintf(stderr, "[moe_w4a16] masked max_m=%d expected_m=%d -> %s nt=%d\n", max_m,
                 expected_m, kind_name(s.kind), s.nt);
  h->cache.emplace(key, s);
  return s;
}

// Contiguous: every block is a full 128-row tile, which the large-M kernel
// covers in one weight pass.
Schedule schedule_contiguous(moe_weights* h, int M_pad) {
  const ScheduleKey key = key_of(MOE_MODE_CONTIGUOUS, M_pad, 0, nullptr);
  std::lock_guard<std::mutex> g(h->mu);
  auto it = h->cache.find(key);
  if (it != h->cache.end()) return it->second;
  Schedule s;
  s.rows = 128;
  s.kind = SCHED_LARGE_M;
  if (h->env.schedule) s.kind = h->env.schedule;
  if (!large_m_fits(h)) s.kind = SCHED_SMALL_M;
  s.nt = 2;
  if (h->env.nt) s.nt = h->env.nt;
  h->cache.emplace(key, s);
  return s;
}

moe_status_t check_desc(const moe_weight_desc_t* d) {
  if (!d) return fail(MOE_ERR_INVALID_ARG, "desc is NULL");
  if (d->bits != 4 || d->group_size != 32 || d->zero_point != 8 || d->scale_dtype != MOE_SCALE_BF16 ||
      d->pack_order != MOE_PACK_INT32_LOW_NIBBLE_FIRST_K)
    return fail(MOE_ERR_UNSUPPORTED_SCHEMA,
                "unsupported quantisation schema (bits=%d group=%d zero_point=%d scale=%d pack=%d); "
                "supported: uint4, group 32, zero point 8, BF16 scales, int32 low-nibble-first along K",
                d->bits, d->group_size, d->zero_point, d->scale_dtype, d->pack_order);
  if (d->hidden <= 0 || d->inter <= 0 || d->hidden % 32 || d->inter % 32)
    return fail(MOE_ERR_UNSUPPORTED_SCHEMA, "hidden (%d) and inter (%d) must be positive multiples of 32",
                d->hidden, d->inter);
  if (d->hidden > (1 << 16) || d->inter > (1 << 16))
    return fail(MOE_ERR_INVALID_ARG, "hidden/inter above 65536");
  if (d->num_experts < 1 || d->num_experts > 4096)
    return fail(MOE_ERR_INVALID_ARG, "num_experts %d outside 1..4096", d->num_experts);
  if (d->mode < MOE_MODE_INDEXED || d->mode > MOE_MODE_MASKED)
    return fail(MOE_ERR_INVALID_ARG, "unknown mode %d", d->mode);
  return MOE_OK;
}

const char* mode_name(int m) {
  return m == MOE_MODE_INDEXED ? "indexed" : m == MOE_MODE_CONTIGUOUS ? "contiguous" : "masked";
}

moe_status_t check_handle(const moe_weights_t* h, int mode) {
  if (!h) return fail(MOE_ERR_INVALID_ARG, "weights handle is NULL");
  if (h->desc.mode != mode)
    return fail(MOE_ERR_MODE_MISMATCH, "weights were prepared for the %s layout, not %s",
                mode_name(h->desc.mode), mode_name(mode));
  return MOE_OK;
}

moe_status_t check_topk(const moe_weights_t* h, int T, int topk) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %d < 0", T);
  if (topk < 1 || topk > h->desc.num_experts || topk > 64)
    return fail(MOE_ERR_INVALID_ARG, "topk = %d outside 1..min(E, 64)", topk);
  if ((int64_t)T * topk > (1 << 28)) return fail(MOE_ERR_INVALID_ARG, "T*topk too large");
  return MOE_OK;
}

// Workspace carving: the BF16 intermediate a, the weighted rows w*y of the
// second GEMM as 16-bit integers (one per flat routed row, summed by the
// combine), the contiguous layout's row-validity map, and the indexed
// layout's own routing.
// Features per weighted row in the workspace: H rounded up to whole 64-feature
// blocks (the lane-contiguous order of store_y16 permutes within a block).
size_t yrow_ld(const moe_weights_t* h) { return ((size_t)h->desc.hidden + 63) / 64 * 64; }

struct WsLayout {
  size_t off_a = 0, off_y = 0, off_part = 0, off_queue = 0, off_check = 0, off_valid = 0,
         off_routing = 0, total = 0;
};

WsLayout ws_indexed(const moe_weights_t* h, int T, int topk, int block, const Schedule& sc) {
  RoutingLayout R;
  R.init(h->desc.num_experts, T, topk, block);
  WsLayout w;
  size_t o = 0;
  w.off_a = o;
  o = round_up(o + (size_t)R.cap * h->desc.inter * 2, kAlign);
  w.off_y = o;   // weighted rows: 16-bit integers with their group scales (2 bytes per feature)
  o = round_up(o + (size_t)T * topk * yrow_ld(h) * 2, kAlign);
  // split-K partials: [ksplit][T*topk][N] FP32 per GEMM (one at a time)
  w.off_part = o;
  const size_t p13 = sc.ksplit13 > 1 ? (size_t)sc.ksplit13 * 2 * h->desc.inter : 0;
  const size_t p2 = sc.ksplit2 > 1 ? (size_t)sc.ksplit2 * h->desc.hidden : 0;
  o = round_up(o + (size_t)T * topk * (p13 > p2 ? p13 : p2) * 4, kAlign);
  w.off_queue = o;   // job counters of the persistent small-M dispatch (W13, W2)
  o += kAlign;
  w.off_check = o;   // counters of the validation mode
  o += kAlign;
  w.off_valid = w.off_routing = o;
  o = round_up(o + (size_t)R.total_ints * 4, kAlign);
  w.total = o;
  return w;
}

// flat_rows: T*topk when the second GEMM feeds the combine, else 0.
WsLayout ws_rows(const moe_weights_t* h, int64_t rows, int64_t flat_rows) {
  WsLayout w;
  size_t o = 0;
  w.off_a = o;
  o = round_up(o + (size_t)rows * h->desc.inter * 2, kAlign);
  w.off_y = o;   // weighted rows: 16-bit integers with their group scales (2 bytes per feature)
  o = round_up(o + (size_t)flat_rows * yrow_ld(h) * 2, kAlign);
  w.off_valid = w.off_routing = o;
  o = round_up(o + (size_t)flat_rows * 4, kAlign);
  w.off_check = o;   // counters of the validation mode
  o += kAlign;
  w.total = o;
  return w;
}

void fill_weights(GemmParams& p, const moe_weights_t* h, const MatLayout& m) {
  p.wq = h->prepared + m.off_words;
  p.wsc = h->prepared + m.off_scales;
  p.E = m.E;
  p.RG = m.RG;
  p.Kc = m.Kc;
  p.K = m.K;
  p.N = m.N;
  p.wg_per_set = (m.RG + 3) / 4;
}

moe_status_t set_device(const moe_weights_t* h) {
  if (!h->prepared)
    return fail(MOE_ERR_INVALID_ARG, "handle from moe_plan_create has no prepared weights");
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (cur != h->device) {
    e = hipSetDevice(h->device);
    if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  }
  return MOE_OK;
}

// ---- validation mode (MOE_W4A16_VALIDATE=1, read when weights are prepared)
// The layer kernels drop or clamp bad index data without a sign; this mode
// counts such entries with small kernels, reads the counts back and
// synchronises the stream, and fails the call (INVALID_ARG, or
// ROUTING_MISMATCH for a routing buffer made for another call) before the
// layer is enqueued.

// The first nonzero of n device counters fails the call with its text.
moe_status_t read_checks(hipStream_t s, const int32_t* cnt, int n, const char* const* what) {
  int32_t host[4] = {0, 0, 0, 0};
  hipError_t e = hipMemcpyAsync(host, cnt, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "validation read-back");
  for (int i = 0; i < n; ++i)
    if (host[i]) return fail(MOE_ERR_INVALID_ARG, "validation: %d %s", host[i], what[i]);
  return MOE_OK;
}

// Expert ids in [-1, hi) (-1: the row routes nowhere), and with an expert
// map its entries in [-1, E). cnt: 2 device ints of scratch.
moe_status_t validate_ids(hipStream_t s, int32_t* cnt, const int32_t* ids, int64_t n, int hi,
                          const int32_t* map, int Eg, int E) {
  hipError_t e = launch_zero_i32(cnt, 2, s);
  if (e == hipSuccess) e = launch_count_outside(ids, n, -1, hi, cnt, s);
  if (e == hipSuccess && map) e = launch_count_outside(map, Eg, -1, E, cnt + 1, s);
  if (e != hipSuccess) return hip_fail(e, "validation launch");
  static const char* const what[] = {"topk_ids outside [-1, experts)", "expert_map entries outside [-1, E)"};
  return read_checks(s, cnt, map ? 2 : 1, what);
}

// A routing buffer passed in must come from moe_align / moe_align_ep for
// this (block, E, T, topk); the kernels otherwise compute nothing.
moe_status_t validate_routing(hipStream_t s, const void* routing, int B, int E, int T, int topk) {
  int32_t hdr[kHdrInts];
  hipError_t e = hipMemcpyAsync(hdr, routing, sizeof(hdr), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "validation read-back");
  if (hdr[HDR_MAGIC] != kRoutingMagic)
    return fail(MOE_ERR_ROUTING_MISMATCH, "validation: the routing buffer holds no alignment");
  if (hdr[HDR_BLOCK] != B || hdr[HDR_E] != E || hdr[HDR_T] != T || hdr[HDR_TOPK] != topk)
    return fail(MOE_ERR_ROUTING_MISMATCH,
                "validation: routing made for block %d, E %d, T %d, topk %d; this call: %d, %d, %d, %d",
                hdr[HDR_BLOCK], hdr[HDR_E], hdr[HDR_T], hdr[HDR_TOPK], B, E, T, topk);
  return MOE_OK;
}

}  // namespace

// --------------------------------------------------------------------------
// ABI
// --------------------------------------------------------------------------

extern "C" {

int moe_abi_version(void) { return MOE_W4A16_ABI_VERSION; }

const char* moe_last_error(void) { return g_err.c_str(); }

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED_SCHEMA: return "MOE_ERR_UNSUPPORTED_SCHEMA";
    case MOE_ERR_MODE_MISMATCH: return "MOE_ERR_MODE_MISMATCH";
    case MOE_ERR_OVERRIDE_REJECTED: return "MOE_ERR_OVERRIDE_REJECTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_ROUTING_MISMATCH: return "MOE_ERR_ROUTING_MISMATCH";
    default: return "MOE_ERR_UNKNOWN";
  }
}

size_t moe_prepared_bytes(const moe_weight_desc_t* desc) {
  if (check_desc(desc) != MOE_OK) return 0;
  PreparedLayout L;
  L.init(desc->num_experts, desc->hidden, desc->inter);
  g_err.clear();
  return L.total + kAlign;   // + one status word for the load-time scale check
}

moe_status_t moe_prepare_weights(const moe_weight_desc_t* desc, const int32_t* w13_q,
                                 const uint16_t* w13_s, const int32_t* w2_q, const uint16_t* w2_s,
                                 void* prepared, size_t prepared_bytes, moe_stream_t stream,
                                 moe_weights_t** out) {
  moe_status_t st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!w13_q || !w13_s || !w2_q || !w2_s || !prepared)
    return fail(MOE_ERR_INVALID_ARG, "a weight or prepared pointer is NULL");
  if (!aligned(w13_q, 16) || !aligned(w2_q, 16) || !aligned(w13_s, 2) || !aligned(w2_s, 2))
    return fail(MOE_ERR_INVALID_ARG, "packed words need 16-byte and scales 2-byte alignment");
  if (!aligned(prepared, kAlign)) return fail(MOE_ERR_INVALID_ARG, "prepared buffer not 256-byte aligned");
  PreparedLayout L;
  L.init(desc->num_experts, desc->hidden, desc->inter);
  if (prepared_bytes < L.total + kAlign)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "prepared buffer %zu bytes < %zu", prepared_bytes,
                L.total + kAlign);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)prepared;
  int32_t* flag = (int32_t*)(base + L.total);
  e = run("zero_flag", s, [&] { return launch_zero_i32(flag, 1, s); });
  if (e == hipSuccess)
    e = run("repack_w13", s, [&] { return launch_repack(L.w13, w13_q, w13_s, base, flag, s); });
  if (e == hipSuccess)
    e = run("repack_w2", s, [&] { return launch_repack(L.w2, w2_q, w2_s, base, flag, s); });
  if (e != hipSuccess) return hip_fail(e, "repack launch");
  int32_t bad = 0;
  e = hipMemcpyAsync(&bad, flag, sizeof bad, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "prepare synchronise");
  if (bad)
    return fail(MOE_ERR_UNSUPPORTED_SCHEMA,
                "a scale is NaN, infinite or of magnitude >= 2^117 (outside the supported range)");
  moe_weights* h = new moe_weights();
  h->desc = *desc;
  h->lay = L;
  h->prepared = base;
  h->prepared_bytes = prepared_bytes;
  h->device = dev;
  h->env.read();
  *out = h;
  return ok();
}

void moe_release_weights(moe_weights_t* h) { delete h; }

moe_weights_t* moe_plan_create(const moe_weight_desc_t* desc) {
  if (check_desc(desc) != MOE_OK) return nullptr;
  moe_weights* h = new moe_weights();
  h->desc = *desc;
  h->lay.init(desc->num_experts, desc->hidden, desc->inter);
  h->prepared = nullptr;
  h->device = -1;
  h->env.read();
  g_err.clear();
  return h;
}

int32_t moe_routing_block(const moe_weights_t* h, int32_t T, int32_t topk, const moe_tuning_t* ovr) {
  if (check_handle(h, MOE_MODE_INDEXED) != MOE_OK || check_topk(h, T, topk) != MOE_OK) return 0;
  if (ovr && ovr->block_m && ovr->block_m != 16 && ovr->block_m != 32 && ovr->block_m != 64 &&
      ovr->block_m != 128) {
    fail(MOE_ERR_INVALID_ARG, "block_m %d not in {16, 32, 64, 128}", ovr->block_m);
    return 0;
  }
  if (ovr && (ovr->dispatch < 0 || ovr->dispatch > 3)) {
    fail(MOE_ERR_INVALID_ARG, "dispatch %d not in 0..3", ovr->dispatch);
    return 0;
  }
  if (ovr && ovr->global_experts < 0) {
    fail(MOE_ERR_INVALID_ARG, "global_experts %d < 0", ovr->global_experts);
    return 0;
  }
  if (large_m_rejected(h, ovr)) {
    fail(MOE_ERR_OVERRIDE_REJECTED,
         "large-M needs hidden and inter divisible by 128 and block_m 0 or 128 (got H=%d I=%d block_m=%d)",
         h->desc.hidden, h->desc.inter, ovr->block_m);
    return 0;
  }
  g_err.clear();
  return schedule_indexed(const_cast<moe_weights_t*>(h), T, topk, ovr).block;
}

moe_status_t moe_routing_layout(const moe_weights_t* h, int32_t T, int32_t topk,
                                const moe_tuning_t* ovr, moe_routing_layout_t* out) {
  if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  const int B = moe_routing_block(h, T, topk, ovr);
  if (!B) return h ? (h->desc.mode != MOE_MODE_INDEXED ? MOE_ERR_MODE_MISMATCH : MOE_ERR_INVALID_ARG)
                   : MOE_ERR_INVALID_ARG;
  RoutingLayout R;
  R.init(h->desc.num_experts, T, topk, B);
  out->block = R.block;
  out->cap = R.cap;
  out->nblocks = R.nblocks;
  out->sentinel = R.sentinel;
  out->off_header = R.off_header;
  out->off_counts = R.off_counts;
  out->off_offsets = R.off_offsets;
  out->off_sorted = R.off_sorted;
  out->off_block_expert = R.off_block_expert;
  out->off_slot_of = R.off_slot_of;
  out->off_scratch = R.off_scratch;
  out->total_ints = R.total_ints;
  return ok();
}

size_t moe_routing_bytes(const moe_weights_t* h, int32_t T, int32_t topk, const moe_tuning_t* ovr) {
  moe_routing_layout_t L;
  if (moe_routing_layout(h, T, topk, ovr, &L) != MOE_OK) return 0;
  return (size_t)L.total_ints * 4;
}

static moe_status_t align_impl(const moe_weights_t* h, const int32_t* topk_ids, int32_t T,
                               int32_t topk, const int32_t* map, int32_t Eg,
                               const moe_tuning_t* ovr, void* routing, size_t routing_bytes,
                               moe_stream_t stream) {
  moe_status_t st = check_handle(h, MOE_MODE_INDEXED);
  if (st != MOE_OK) return st;
  if ((st = check_topk(h, T, topk)) != MOE_OK) return st;
  if (!routing || (T > 0 && !topk_ids)) return fail(MOE_ERR_INVALID_ARG, "NULL routing or topk_ids");
  if (!aligned(routing, 4) || (topk_ids && !aligned(topk_ids, 4)))
    return fail(MOE_ERR_INVALID_ARG, "routing / topk_ids not 4-byte aligned");
  const int B = moe_routing_block(h, T, topk, ovr);
  if (!B) return MOE_ERR_INVALID_ARG;
  RoutingLayout R;
  R.init(h->desc.num_experts, T, topk, B);
  if (routing_bytes < (size_t)R.total_ints * 4)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "routing buffer %zu bytes < %zu", routing_bytes,
                (size_t)R.total_ints * 4);
  if ((st = set_device(h)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (h->env.validate && T > 0) {   // counters in the scratch the alignment overwrites next
    int32_t* cnt = (int32_t*)routing + R.off_scratch;
    if ((st = validate_ids(s, cnt, topk_ids, (int64_t)T * topk, map ? Eg : h->desc.num_experts, map, Eg,
                           h->desc.num_experts)) != MOE_OK)
      return st;
  }
  hipError_t e = run("align", s, [&] {
    return launch_align(topk_ids, T, topk, h->desc.num_experts, R, (int32_t*)routing, s, map, Eg);
  });
  if (e != hipSuccess) return hip_fail(e, "align launch");
  return ok();
}

moe_status_t moe_align(const moe_weights_t* h, const int32_t* topk_ids, int32_t T, int32_t topk,
                       const moe_tuning_t* ovr, void* routing, size_t routing_bytes,
                       moe_stream_t stream) {
  return align_impl(h, topk_ids, T, topk, nullptr, 0, ovr, routing, routing_bytes, stream);
}

moe_status_t moe_align_ep(const moe_weights_t* h, const int32_t* topk_ids, int32_t T, int32_t topk,
                          const int32_t* expert_map, int32_t num_global_experts,
                          const moe_tuning_t* ovr, void* routing, size_t routing_bytes,
                          moe_stream_t stream) {
  if (!expert_map || !aligned(expert_map, 4))
    return fail(MOE_ERR_INVALID_ARG, "expert_map NULL or not 4-byte aligned");
  if (num_global_experts < 1 || num_global_experts > (1 << 20))
    return fail(MOE_ERR_INVALID_ARG, "num_global_experts %d outside 1..2^20", num_global_experts);
  return align_impl(h, topk_ids, T, topk, expert_map, num_global_experts, ovr, routing,
                    routing_bytes, stream);
}

moe_status_t moe_permute(const moe_weights_t* h, const uint16_t* x, int32_t T, int32_t topk,
                         const moe_tuning_t* ovr, const void* routing, uint16_t* a_out,
                         int32_t* m_indices, int32_t* row_src, moe_stream_t stream) {
  moe_status_t st = check_handle(h, MOE_MODE_INDEXED);
  if (st != MOE_OK) return st;
  if ((st = check_topk(h, T, topk)) != MOE_OK) return st;
  if (!routing) return fail(MOE_ERR_INVALID_ARG, "routing is NULL");
  if (a_out && T > 0 && !x) return fail(MOE_ERR_INVALID_ARG, "x is NULL");
  if ((a_out && !aligned(a_out, 16)) || (x && !aligned(x, 16)))
    return fail(MOE_ERR_INVALID_ARG, "x / a_out not 16-byte aligned");
  const int B = moe_routing_block(h, T, topk, ovr);
  if (!B) return MOE_ERR_INVALID_ARG;
  RoutingLayout R;
  R.init(h->desc.num_experts, T, topk, B);
  if ((st = set_device(h)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (h->env.validate && (st = validate_routing(s, routing, B, h->desc.num_experts, T, topk)) != MOE_OK)
    return st;
  hipError_t e = run("permute", s, [&] {
    return launch_permute(x, T, topk, h->desc.hidden, R, (const int32_t*)routing, a_out, m_indices,
                          row_src, s);
  });
  if (e != hipSuccess) return hip_fail(e, "permute launch");
  return ok();
}

size_t moe_workspace_bytes(const moe_weights_t* h, int32_t mode, int32_t rows, int32_t topk,
                           int32_t tokens, const moe_tuning_t* ovr) {
  if (check_handle(h, mode) != MOE_OK) return 0;
  if (mode == MOE_MODE_INDEXED) {
    const int B = moe_routing_block(h, rows, topk, ovr);
    if (!B) return 0;
    return ws_indexed(h, rows, topk, B, schedule_indexed(const_cast<moe_weights_t*>(h), rows, topk, ovr))
        .total;
  }
  if (rows < 0 || tokens < 0) {
    fail(MOE_ERR_INVALID_ARG, "negative rows / tokens");
    return 0;
  }
  g_err.clear();
  if (mode == MOE_MODE_MASKED) return ws_rows(h, (int64_t)h->desc.num_experts * rows, 0).total;
  return ws_rows(h, rows, topk > 0 ? (int64_t)tokens * topk : 0).total;
}

moe_status_t moe_w4a16_indexed(const moe_weights_t* hc, const uint16_t* x, int32_t T, int32_t topk,
                               const int32_t* topk_ids, const float* topk_w, const void* routing,
                               uint16_t* out, void* ws, size_t ws_bytes, const moe_tuning_t* ovr,
                               moe_stream_t stream) {
  moe_weights_t* h = const_cast<moe_weights_t*>(hc);
  moe_status_t st = check_handle(h, MOE_MODE_INDEXED);
  if (st != MOE_OK) return st;
  if ((st = check_topk(h, T, topk)) != MOE_OK) return st;
  if (ovr && ovr->schedule && (ovr->schedule < 0 || ovr->schedule > 2))
    return fail(MOE_ERR_INVALID_ARG, "schedule override %d not in 0..2", ovr->schedule);
  const int B = moe_routing_block(h, T, topk, ovr);
  if (!B) return large_m_rejected(h, ovr) ? MOE_ERR_OVERRIDE_REJECTED : MOE_ERR_INVALID_ARG;
  if (T == 0) return ok();
  if (!x || !topk_w || !out || !ws || (!routing && !topk_ids))
    return fail(MOE_ERR_INVALID_ARG, "NULL x / topk_w / out / ws / topk_ids");
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(ws, kAlign) || !aligned(topk_w, 4) ||
      (routing && !aligned(routing, 4)) || (topk_ids && !aligned(topk_ids, 4)))
    return fail(MOE_ERR_INVALID_ARG, "misaligned pointer (x/out 16 B, ws 256 B, others 4 B)");
  const Schedule sc = schedule_indexed(h, T, topk, ovr);
  const WsLayout W = ws_indexed(h, T, topk, B, sc);
  const size_t need = routing ? W.off_routing : W.total;
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu", ws_bytes, need);
  if ((st = set_device(h)) != MOE_OK) return st;

  hipStream_t s = (hipStream_t)stream;
  char* wsb = (char*)ws;
  RoutingLayout R;
  R.init(h->desc.num_experts, T, topk, B);
  if (h->env.validate) {
    st = routing ? validate_routing(s, routing, B, h->desc.num_experts, T, topk)
                 : validate_ids(s, (int32_t*)(wsb + W.off_check), topk_ids, (int64_t)T * topk,
                                h->desc.num_experts, nullptr, 0, h->desc.num_experts);
    if (st != MOE_OK) return st;
  }
  const int32_t* rt = (const int32_t*)routing;
  hipError_t e = hipSuccess;
  if (!rt) {
    int32_t* own = (int32_t*)(wsb + W.off_routing);
    e = run("align", s, [&] { return launch_align(topk_ids, T, topk, h->desc.num_experts, R, own, s); });
    rt = own;
  }
  const int H = h->desc.hidden, I = h->desc.inter, E = h->desc.num_experts;
  uint16_t* a_ws = (uint16_t*)(wsb + W.off_a);
  uint16_t* yq = (uint16_t*)(wsb + W.off_y);
  GemmParams p{};
  p.counts = rt + R.off_counts;
  p.offsets = rt + R.off_offsets;
  p.sorted_ids = rt + R.off_sorted;
  p.routing_hdr = rt;
  p.sentinel = T * topk;
  p.topk = topk;
  p.block = B;
  p.block_expert = rt + R.off_block_expert;
  // semi-static small-M over experts: one row set per expert; large-M and
  // the other small-M forms: one per routing block
  const bool large = sc.kind == SCHED_LARGE_M;
  const bool blocks = large || sc.dispatch;
  p.nsets = blocks ? block_bound(R, T, topk) : expert_bound(E, T, topk);
  const int set = blocks ? SET_ROUTED : SET_INDEXED;
  if (!large && (sc.dispatch == 1 || sc.dispatch == 2)) {
    p.dispatch = sc.dispatch;
    p.passes = (B + 16 * sc.nt - 1) / (16 * sc.nt);
  }
  int32_t* queue = (int32_t*)(wsb + W.off_queue);
  if (e == hipSuccess && p.dispatch == 2)
    e = run("zero_queue", s, [&] { return launch_zero_i32(queue, 2, s); });

  GemmParams p13 = p;
  fill_weights(p13, h, h->lay.w13);
  p13.total_wg = p13.nsets * p13.wg_per_set;
  p13.queue = queue;
  p13.src = x;
  p13.src_ld = H;
  p13.gather = 1;
  p13.a_out = a_ws;
  p13.a_ld = I;
  float* part = (float*)(wsb + W.off_part);
  const int64_t F = (int64_t)T * topk;
  const bool semi = !large && (sc.dispatch == 0 || sc.dispatch == 3);
  const bool split13 = semi && sc.ksplit13 > 1, split2 = semi && sc.ksplit2 > 1;
  if (split13) {   // grid-starved: K split over ksplit13 workgroups, reduced with the SwiGLU
    p13.ksplit = sc.ksplit13;
    p13.total_wg *= sc.ksplit13;
    p13.part = part;
    p13.part_rows = F;
  }
  if (e == hipSuccess)
    e = run_gemm(13, sc, p13, set, split13 ? EPI_PARTIAL : EPI_SWIGLU, s, h->env);
  if (e == hipSuccess && split13)
    e = run("splitk_swiglu", s, [&] {
      return launch_splitk_swiglu(part, sc.ksplit13, F, I, rt + R.off_sorted, R.cap, T * topk, a_ws, I, s);
    });

  GemmParams p2 = p;
  fill_weights(p2, h, h->lay.w2);
  p2.total_wg = p2.nsets * p2.wg_per_set;
  p2.queue = queue + 1;
  p2.src = a_ws;
  p2.src_ld = I;
  p2.yq = yq;
  p2.topk_w = topk_w;
  p2.yrows_ld = (int64_t)yrow_ld(h);
  if (split2) {   // reduced by the combine
    p2.ksplit = sc.ksplit2;
    p2.total_wg *= sc.ksplit2;
    p2.part = part;
    p2.part_rows = F;
  }
  if (e == hipSuccess)
    e = run_gemm(2, sc, p2, set, split2 ? EPI_PARTIAL : EPI_COMBINE, s, h->env);
  if (e == hipSuccess)
    e = run("combine_topk", s, [&] {
      return split2 ? launch_splitk_combine(part, sc.ksplit2, rt + R.off_slot_of, rt, E, B, topk_w, T, topk,
                                            H, out, s)
                    : launch_combine_rows(yq, (int)yrow_ld(h), rt + R.off_slot_of, rt, E, B, T, topk, H,
                                          out, s);
    });
  if (e != hipSuccess) return hip_fail(e, "indexed launch");
  return ok();
}

}  // extern "C"

// --------------------------------------------------------------------------
// The indexed layer without allocation: its workspace (the routing made by
// the internal alignment, the BF16 intermediate and the weighted rows) lives
// in a fixed device array of this library, so a caller that cannot allocate
// device memory (graph capture, a tight serving loop) passes only inputs and
// outputs. Each GPU holds its own copy of the array at its own address; the
// host-side name `scratch` is not that address, so the address is taken once
// per device with hipGetSymbolAddress and only that pointer reaches kernels.
// --------------------------------------------------------------------------

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (h->device, made
// current by set_device), taken on first use.
moe_status_t scratch_ptr(int device, void** out) {
  if (device < 0 || device >= kMaxDevices)
    return fail(MOE_ERR_INVALID_ARG, "device %d outside 0..%d", device, kMaxDevices - 1);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || !aligned(ptr, kAlign))
      return fail(MOE_ERR_HIP, "scratch array at %p: not 256-byte aligned", ptr);
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_w4a16_indexed_noalloc(const moe_weights_t* hc, const uint16_t* x, int32_t T,
                                       int32_t topk, const int32_t* topk_ids, const float* topk_w,
                                       uint16_t* out, const moe_tuning_t* ovr, moe_stream_t stream) {
  moe_weights_t* h = const_cast<moe_weights_t*>(hc);
  moe_status_t st = check_handle(h, MOE_MODE_INDEXED);
  if (st != MOE_OK) return st;
  if ((st = check_topk(h, T, topk)) != MOE_OK) return st;
  if (T == 0) return ok();
  if (!topk_ids) return fail(MOE_ERR_INVALID_ARG, "NULL topk_ids (this entry point aligns internally)");
  const size_t need = moe_workspace_bytes(h, MOE_MODE_INDEXED, T, topk, T, ovr);
  if (!need) return ovr && large_m_rejected(h, ovr) ? MOE_ERR_OVERRIDE_REJECTED : MOE_ERR_INVALID_ARG;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL,
                "this call needs %zu bytes of workspace; the fixed scratch array holds %zu "
                "(use moe_w4a16_indexed with a workspace of its own)",
                need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  if ((st = set_device(h)) != MOE_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_ptr(h->device, &ws)) != MOE_OK) return st;
  return moe_w4a16_indexed(h, x, T, topk, topk_ids, topk_w, nullptr, out, ws,
                           (size_t)MOE_NOALLOC_SCRATCH_BYTES, ovr, stream);
}

// One grouped GEMM of the indexed layout with a BF16 output at routing-slot
// rows (the unfused step sequence): mat 13 (x gathered through the routing,
// output gate | up) or 2 (a rows at their slots).
static moe_status_t indexed_gemm_step(const moe_weights_t* hc, int mat, const uint16_t* src, int32_t T,
                               int32_t topk, const void* routing, uint16_t* out,
                               const moe_tuning_t* ovr, moe_stream_t stream) {
  moe_weights_t* h = const_cast<moe_weights_t*>(hc);
  moe_status_t st = check_handle(h, MOE_MODE_INDEXED);
  if (st != MOE_OK) return st;
  if ((st = check_topk(h, T, topk)) != MOE_OK) return st;
  if (ovr && ovr->schedule && (ovr->schedule < 0 || ovr->schedule > 2))
    return fail(MOE_ERR_INVALID_ARG, "schedule override %d not in 0..2", ovr->schedule);
  const int B = moe_routing_block(h, T, topk, ovr);
  if (!B) return large_m_rejected(h, ovr) ? MOE_ERR_OVERRIDE_REJECTED : MOE_ERR_INVALID_ARG;
  if (T == 0) return ok();
  if (!src || !routing || !out) return fail(MOE_ERR_INVALID_ARG, "NULL input / routing / output");
  if (!aligned(src, 16) || !aligned(out, 16) || !aligned(routing, 4))
    return fail(MOE_ERR_INVALID_ARG, "misaligned pointer (input/output 16 B, routing 4 B)");
  if ((st = set_device(h)) != MOE_OK) return st;
  const Schedule sc = schedule_indexed(h, T, topk, ovr);
  RoutingLayout R;
  R.init(h->desc.num_experts, T, topk, B);
  const int32_t* rt = (const int32_t*)routing;
  const int H = h->desc.hidden, I = h->desc.inter, E = h->desc.num_experts;
  GemmParams p{};
  p.counts = rt + R.off_counts;
  p.offsets = rt + R.off_offsets;
  p.sorted_ids = rt + R.off_sorted;
  p.routing_hdr = rt;
  p.sentinel = T * topk;
  p.topk = topk;
  p.block = B;
  p.block_expert = rt + R.off_block_expert;
  const bool large = sc.kind == SCHED_LARGE_M;
  p.nsets = large ? block_bound(R, T, topk) : expert_bound(E, T, topk);
  const int set = large ? SET_ROUTED : SET_INDEXED;
  fill_weights(p, h, mat == 13 ? h->lay.w13 : h->lay.w2);
  p.total_wg = p.nsets * p.wg_per_set;
  p.src = src;
  p.src_ld = mat == 13 ? H : I;
  p.gather = mat == 13;
  p.out = out;
  p.out_ld = mat == 13 ? 2 * I : H;
  p.gate_up_I = mat == 13 ? I : 0;
  Schedule semi = sc;
  semi.dispatch = 0;   // the persistent forms serve the fused call only
  hipStream_t s = (hipStream_t)stream;
  if (h->env.validate && (st = validate_routing(s, routing, B, E, T, topk)) != MOE_OK) return st;
  const hipError_t e = run_gemm(mat, semi, p, set, EPI_STORE, s, h->env);
  if (e != hipSuccess) return hip_fail(e, mat == 13 ? "gate_up launch" : "down launch");
  return ok();
}

moe_status_t moe_w4a16_gate_up(const moe_weights_t* h, const uint16_t* x, int32_t T, int32_t topk,
                               const void* routing, uint16_t* h_out, const moe_tuning_t* ovr,
                               moe_stream_t stream) {
  return indexed_gemm_step(h, 13, x, T, topk, routing, h_out, ovr, stream);
}

moe_status_t moe_w4a16_down(const moe_weights_t* h, const uint16_t* a, int32_t T, int32_t topk,
                            const void* routing, uint16_t* y_out, const moe_tuning_t* ovr,
                            moe_stream_t stream) {
  return indexed_gemm_step(h, 2, a, T, topk, routing, y_out, ovr, stream);
}

moe_status_t moe_swiglu(const uint16_t* h, int64_t rows, int32_t inter, uint16_t* a,
                        moe_stream_t stream) {
  if (rows < 0 || inter <= 0 || inter % 8)
    return fail(MOE_ERR_INVALID_ARG, "rows %lld / inter %d (a positive multiple of 8)", (long long)rows,
                inter);
  if (rows == 0) return ok();
  if (!h || !a || !aligned(h, 16) || !aligned(a, 16))
    return fail(MOE_ERR_INVALID_ARG, "h / a NULL or not 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = run("swiglu", s, [&] { return launch_swiglu(h, rows, inter, a, s); });
  if (e != hipSuccess) return hip_fail(e, "swiglu launch");
  return ok();
}

moe_status_t moe_w4a16_contiguous(const moe_weights_t* hc, const uint16_t* a, int32_t M_pad,
                                  const int32_t* m_indices, const int32_t* row_src,
                                  const float* topk_w, int32_t T, int32_t topk, uint16_t* out,
                                  void* ws, size_t ws_bytes, const moe_tuning_t* ovr,
                                  moe_stream_t stream) {
  moe_weights_t* h = const_cast<moe_weights_t*>(hc);
  moe_status_t st = check_handle(h, MOE_MODE_CONTIGUOUS);
  if (st != MOE_OK) return st;
  if (ovr)
    return fail(MOE_ERR_OVERRIDE_REJECTED,
                "the contiguous layout chooses its own schedule; tuning overrides are indexed-only");
  if (M_pad < 0 || M_pad % 128)
    return fail(MOE_ERR_INVALID_ARG, "M_pad = %d must be a non-negative multiple of 128", M_pad);
  if (row_src && (st = check_topk(h, T, topk)) != MOE_OK) return st;
  if (M_pad == 0) return ok();
  if (!a || !m_indices || !out || !ws || (row_src && !topk_w))
    return fail(MOE_ERR_INVALID_ARG, "NULL a / m_indices / out / ws / topk_w");
  if (!aligned(a, 16) || !aligned(out, 16) || !aligned(ws, kAlign) || !aligned(m_indices, 4) ||
      (row_src && (!aligned(row_src, 4) || !aligned(topk_w, 4))))
    return fail(MOE_ERR_INVALID_ARG, "misaligned pointer (a/out 16 B, ws 256 B, others 4 B)");
  const WsLayout W = ws_rows(h, M_pad, row_src ? (int64_t)T * topk : 0);
  if (ws_bytes < W.total)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu", ws_bytes, W.total);
  if ((st = set_device(h)) != MOE_OK) return st;
  const Schedule sc = schedule_contiguous(h, M_pad);

  hipStream_t s = (hipStream_t)stream;
  char* wsb = (char*)ws;
  const int H = h->desc.hidden, I = h->desc.inter;
  uint16_t* a_ws = (uint16_t*)(wsb + W.off_a);
  uint16_t* yq = (uint16_t*)(wsb + W.off_y);
  int32_t* valid = (int32_t*)(wsb + W.off_valid);
  hipError_t e = hipSuccess;
  if (h->env.validate) {   // the row-validity map serves as the row_src scratch
    int32_t* cnt = (int32_t*)(wsb + W.off_check);
    e = launch_zero_i32(cnt, 3, s);
    if (e == hipSuccess) e = launch_count_outside(m_indices, M_pad, -1, h->desc.num_experts, cnt, s);
    if (e == hipSuccess) e = launch_count_mixed_blocks(m_indices, M_pad, cnt + 1, s);
    if (e == hipSuccess && row_src)
      e = launch_count_row_src(m_indices, row_src, M_pad, T * topk, valid, cnt + 2, s);
    if (e != hipSuccess) return hip_fail(e, "validation launch");
    static const char* const what[] = {"m_indices outside [-1, E)",
                                       "128-row blocks holding rows of two experts",
                                       "rows whose row_src is out of range, repeated, or not -1 on a pad row"};
    if ((st = read_checks(s, cnt, row_src ? 3 : 2, what)) != MOE_OK) return st;
  }

  GemmParams p{};
  p.m_indices = m_indices;
  p.row_src = row_src;
  p.block_rows = 128;
  p.nsets = M_pad / 128;
  p.sentinel = row_src ? T * topk : 0;
  p.topk = row_src ? topk : 1;

  GemmParams p13 = p;
  fill_weights(p13, h, h->lay.w13);
  p13.total_wg = p13.nsets * p13.wg_per_set;
  p13.src = a;
  p13.src_ld = H;
  p13.a_out = a_ws;
  p13.a_ld = I;
  if (e == hipSuccess)
    e = run_gemm(13, sc, p13, SET_BLOCKS, EPI_SWIGLU, s, h->env);

  GemmParams p2 = p;
  fill_weights(p2, h, h->lay.w2);
  p2.total_wg = p2.nsets * p2.wg_per_set;
  p2.src = a_ws;
  p2.src_ld = I;
  if (row_src) {
    p2.yq = yq;
    p2.topk_w = topk_w;
    p2.yrows_ld = (int64_t)yrow_ld(h);
    if (e == hipSuccess && T > 0)
      e = run("combine_valid", s, [&] {
        return launch_contiguous_valid(m_indices, row_src, M_pad, h->desc.num_experts, T * topk, valid, s);
      });
    if (e == hipSuccess)
      e = run_gemm(2, sc, p2, SET_BLOCKS, EPI_COMBINE, s, h->env);
    if (e == hipSuccess && T > 0)
      e = run("combine_topk", s, [&] {
        return launch_combine_rows(yq, (int)yrow_ld(h), valid, nullptr, h->desc.num_experts, 0, T, topk,
                                   H, out, s);
      });
  } else {
    p2.out = out;
    p2.out_ld = H;
    if (e == hipSuccess)
      e = run_gemm(2, sc, p2, SET_BLOCKS, EPI_STORE, s, h->env);
  }
  if (e != hipSuccess) return hip_fail(e, "contiguous launch");
  return ok();
}

moe_status_t moe_w4a16_masked(const moe_weights_t* hc, const uint16_t* a3, int32_t max_m,
                              const int32_t* masked_m, int32_t expected_m, uint16_t* out, void* ws,
                              size_t ws_bytes, const moe_tuning_t* ovr, moe_stream_t stream) {
  moe_weights_t* h = const_cast<moe_weights_t*>(hc);
  moe_status_t st = check_handle(h, MOE_MODE_MASKED);
  if (st != MOE_OK) return st;
  if (ovr)
    return fail(MOE_ERR_OVERRIDE_REJECTED,
                "the masked layout chooses its own schedule; tuning overrides are indexed-only");
  if (expected_m <= 0) return fail(MOE_ERR_INVALID_ARG, "expected_m = %d must be positive", expected_m);
  if (max_m < 0 || (int64_t)max_m * h->desc.num_experts > (1 << 28))
    return fail(MOE_ERR_INVALID_ARG, "max_m = %d out of range", max_m);
  if (max_m == 0) return ok();
  if (!a3 || !masked_m || !out || !ws) return fail(MOE_ERR_INVALID_ARG, "NULL a3 / masked_m / out / ws");
  if (!aligned(a3, 16) || !aligned(out, 16) || !aligned(ws, kAlign) || !aligned(masked_m, 4))
    return fail(MOE_ERR_INVALID_ARG, "misaligned pointer (a3/out 16 B, ws 256 B, masked_m 4 B)");
  const WsLayout W = ws_rows(h, (int64_t)h->desc.num_experts * max_m, 0);
  if (ws_bytes < W.total)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu", ws_bytes, W.total);
  if ((st = set_device(h)) != MOE_OK) return st;
  const Schedule sc = schedule_masked(h, max_m, expected_m);

  hipStream_t s = (hipStream_t)stream;
  char* wsb = (char*)ws;
  if (h->env.validate) {
    int32_t* cnt = (int32_t*)(wsb + W.off_check);
    hipError_t ev = launch_zero_i32(cnt, 1, s);
    if (ev == hipSuccess) ev = launch_count_outside(masked_m, h->desc.num_experts, 0, max_m + 1, cnt, s);
    if (ev != hipSuccess) return hip_fail(ev, "validation launch");
    static const char* const what[] = {"masked_m entries outside [0, max_m]"};
    if ((st = read_checks(s, cnt, 1, what)) != MOE_OK) return st;
  }
  const int H = h->desc.hidden, I = h->desc.inter, E = h->desc.num_experts;
  uint16_t* a_ws = (uint16_t*)(wsb + W.off_a);
  GemmParams p{};
  p.masked_m = masked_m;
  p.max_m = max_m;
  p.nsets = E;
  p.topk = 1;

  GemmParams p13 = p;
  fill_weights(p13, h, h->lay.w13);
  p13.total_wg = E * p13.wg_per_set;
  p13.src = a3;
  p13.src_ld = H;
  p13.a_out = a_ws;
  p13.a_ld = I;
  hipError_t e = run_gemm(13, sc, p13, SET_MASKED, EPI_SWIGLU, s, h->env);

  GemmParams p2 = p;
  fill_weights(p2, h, h->lay.w2);
  p2.total_wg = E * p2.wg_per_set;
  p2.src = a_ws;
  p2.src_ld = I;
  p2.out = out;
  p2.out_ld = H;
  if (e == hipSuccess)
    e = run_gemm(2, sc, p2, SET_MASKED, EPI_STORE, s, h->env);
  if (e != hipSuccess) return hip_fail(e, "masked launch");
  return ok();
}

moe_status_t moe_dequant_weights(const moe_weights_t* h, int32_t which, int32_t expert,
                                 uint16_t* out, moe_stream_t stream) {
  if (!h) return fail(MOE_ERR_INVALID_ARG, "weights handle is NULL");
  if (which != 13 && which != 2) return fail(MOE_ERR_INVALID_ARG, "which = %d must be 13 or 2", which);
  if (expert < 0 || expert >= h->desc.num_experts)
    return fail(MOE_ERR_INVALID_ARG, "expert %d outside 0..%d", expert, h->desc.num_experts - 1);
  if (!out || !aligned(out, 16)) return fail(MOE_ERR_INVALID_ARG, "out NULL or not 16-byte aligned");
  moe_status_t st = set_device(h);
  if (st != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const MatLayout& m = which == 13 ? h->lay.w13 : h->lay.w2;
  hipError_t e = run("dequant_expert", s, [&] { return launch_dequant_expert(m, h->prepared, expert, out, s); });
  if (e != hipSuccess) return hip_fail(e, "dequant launch");
  return ok();
}

int moe_describe(const moe_weights_t* hc, int32_t mode, int32_t rows, int32_t topk,
                 int32_t expected_m, const moe_tuning_t* ovr, char* buf, size_t n) {
  moe_weights_t* h = const_cast<moe_weights_t*>(hc);
  if (!buf || n == 0 || check_handle(h, mode) != MOE_OK) return -1;
  const int E = h->desc.num_experts;
  const int wg13 = (h->lay.w13.RG + 3) / 4, wg2 = (h->lay.w2.RG + 3) / 4;
  int len = -1;
  if (mode == MOE_MODE_INDEXED) {
    if (check_topk(h, rows, topk) != MOE_OK) return -1;
    if (large_m_rejected(h, ovr)) return -1;
    const Schedule s = schedule_indexed(h, rows, topk, ovr);
    RoutingLayout R;
    R.init(E, rows, topk, s.block);
    const bool persistent = s.kind == SCHED_SMALL_M && (s.dispatch == 1 || s.dispatch == 2);
    const int sets = s.kind == SCHED_LARGE_M || s.dispatch ? block_bound(R, rows, topk)
                                                           : expert_bound(E, rows, topk);
    const int P = (s.block + 16 * s.nt - 1) / (16 * s.nt);
    const int g13 = persistent ? job_grid(sets, P, wg13, s.nt, h->env) : sets * wg13;
    const int g2 = persistent ? job_grid(sets, P, wg2, s.nt, h->env) : sets * wg2;
    static const char* kDispatch[] = {"semi-static", "persistent-static", "persistent-queue",
                                      "semi-static-blocks"};
    len = std::snprintf(buf, n,
                        "layout=indexed T=%d topk=%d rows_per_expert=%d schedule=%s block=%d nt=%d "
                        "grid_w13=%d grid_w2=%d dispatch=%s ksplit=%d/%d",
                        rows, topk, s.rows, kind_name(s.kind), s.block, s.nt, g13 * s.ksplit13,
                        g2 * s.ksplit2, s.kind == SCHED_SMALL_M ? kDispatch[s.dispatch] : "routing-blocks",
                        s.ksplit13, s.ksplit2);
  } else if (mode == MOE_MODE_MASKED) {
    if (expected_m <= 0 || rows < 0) return -1;
    const Schedule s = schedule_masked(h, rows, expected_m);
    len = std::snprintf(buf, n,
                        "layout=masked max_m=%d expected_m=%d schedule=%s nt=%d grid_w13=%d grid_w2=%d",
                        rows, expected_m, kind_name(s.kind), s.nt, E * wg13, E * wg2);
  } else {
    if (rows < 0 || rows % 128) return -1;
    const Schedule s = schedule_contiguous(h, rows);
    len = std::snprintf(buf, n,
                        "layout=contiguous M_pad=%d blocks=%d schedule=%s nt=%d grid_w13=%d grid_w2=%d",
                        rows, rows / 128, kind_name(s.kind), s.nt, (rows / 128) * wg13, (rows / 128) * wg2);
  }
  if (len < 0) return -1;
  return len < (int)n ? len : (int)n - 1;
}

moe_status_t moe_profile_enable(int enable) {
  Profiler& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  P.on = enable != 0;
  return ok();
}

void moe_profile_reset(void) {
  Profiler& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  P.drain();
  P.totals.clear();
}

int moe_profile_read(char* buf, size_t n) {
  if (!buf || n == 0) return -1;
  Profiler& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  P.drain();
  std::string s;
  char line[256];
  for (auto& kv : P.totals) {
    std::snprintf(line, sizeof line, "%s %ld %.6f\n", kv.first.c_str(), kv.second.first, kv.second.second);
    s += line;
  }
  const size_t m = s.size() < n - 1 ? s.size() : n - 1;
  std::memcpy(buf, s.data(), m);
  buf[m] = 0;
  return (int)m;
}

}  // extern "C"
