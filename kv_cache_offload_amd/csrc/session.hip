// session.hip -- host runtime behind the C ABI of include/dsa.h.
//
// The session owns every allocation (exact sizes, made once at create: the
// page "From 1M total to 15+ streams x 1M: the capacity breakthrough of
// GLM-5.3 KV cache offload", section "The ten-way experiment", found that
// long-lived caches carved from a general caching pool held on to far larger
// blocks; here nothing long-lived comes from a pool).  Host mirrors are pinned,
// device-mapped allocations owned by the session and touched once at create.
// After create, append and decode only enqueue kernels on the caller's stream:
// no allocation, no host synchronisation, no per-selection host work (section
// "Decision 3").  The host keeps a mirror of each unit's logical counters
// (L, M, round) -- they depend only on the call sequence, never on data -- for
// validation and grid sizing; the kernels keep their own copy in device memory.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "dsa.h"
#include "dsa_internal.h"

using namespace dsa;

namespace dsa {
thread_local LaunchTimer t_launch_timer;
}  // namespace dsa

// ---- the step scratch of dsa_decode_step_static ---------------------------
// A file-scope device array, so that the no-allocation step needs no hipMalloc.
// Host code never uses its name as an address: the device address of each
// GPU's copy is looked up once per device (hipGetSymbolAddress, at the first
// session create on that device) and kept in g_static_scratch.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 256;
std::mutex g_static_mu;
void* g_static_scratch[kMaxDevices] = {};

struct UnitHost {
  int64_t L = 0, M = 0, round = 0;
  int64_t floor = 0;             // lowest L a rollback may return to (offload)
  int64_t m_done = 0;            // mirror rows known complete
  int64_t m_event = 0;           // mirror rows covered by `ev`
  hipEvent_t ev = nullptr;
  bool ev_pending = false;
};

struct TimedLaunch {
  int kind;
  hipEvent_t a, b;
};

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

}  // namespace

struct dsa_session {
  dsa_config cfg{};
  Geometry g{};
  int device = 0;
  bool failed = false;
  std::string err;
  void* arena = nullptr;
  size_t arena_bytes = 0;
  std::vector<void*> mirrors;              // host pointers into mirror_block (offload)
  std::vector<UnitDev> units;              // host copies of the device descriptors
  std::vector<SeqScratch> scr;
  std::vector<SeqScratch> scr_pf;          // host copy of the prefetch scratch set
  int64_t u_stride = 0;                    // bytes between consecutive units' arena buffers
  int64_t rows_stride = 0;                 // bytes between consecutive units' row stores
  int64_t s_stride = 0, pf_stride = 0;     // bytes between consecutive sequences' scratch (main, prefetch)
  void* mirror_block = nullptr;            // one pinned allocation holding every unit's mirror (offload)
  std::vector<UnitHost> uh;
  int last_layer = -1;
  int last_R = 0;
  int topk_layer = -1;                     // layer of the most recent full decode step
  int topk_R = 0;
  std::vector<int64_t> topk_L;             // per sequence: L at that step
  hipEvent_t sel_ready = nullptr;          // recorded after that step's Top-K (its selection is final)
  int64_t sel_epoch = 0;                   // full decode steps so far
  // An event recorded between two kernels costs the step a few µs (the next
  // kernel starts later), so a step records sel_ready only once the session
  // has prefetched; until then a prefetch orders itself after everything the
  // step's stream had enqueued (sel_stream), the whole step included.
  bool pf_used = false;
  int64_t sel_recorded_epoch = -1;         // the epoch whose sel_ready is recorded
  hipStream_t sel_stream = nullptr;        // the stream of the most recent full decode step
  hipStream_t sel_waited = nullptr;        // the stream that already waits for this epoch's selection
  int64_t sel_waited_epoch = -1;
  std::vector<hipEvent_t> pf_done;         // per layer: recorded after its prefetch round
  std::vector<uint8_t> pf_pending;         // per layer: a prefetch whose event no reuse step has waited for
  std::vector<hipStream_t> pf_stream;
  bool timing = false;
  std::vector<TimedLaunch> timed;
  std::vector<hipEvent_t> free_events;
  int64_t t_counts[DSA_KERNEL_KINDS] = {};
  double t_ms[DSA_KERNEL_KINDS] = {};
  uint32_t* err_host = nullptr;            // device-side check flags: pinned, mapped host memory
  uint32_t* err_dev = nullptr;             // the same block's device address (kernels write it)
  bool inject_hip = false;                 // test hook: the next checked HIP call reports a failure
  void* static_scratch = nullptr;          // this device's copy of the static scratch array
  bool last_static = false;                // the most recent step ran on the static scratch
};

namespace {

dsa_status fail(dsa_session* s, dsa_status st, const std::string& msg) {
  if (s) s->err = msg;
  return st;
}

dsa_status hip_fail(dsa_session* s, hipError_t e, const char* what) {
  s->failed = true;
  s->err = std::string(what) + ": " + hipGetErrorString(e);
  return DSA_E_HIP;
}

// Test hook of dsa_debug_inject: true once, for the next checked HIP call,
// which is then not made.
bool take_injected(dsa_session* s) {
  if (!s->inject_hip) return false;
  s->inject_hip = false;
  return true;
}

dsa_status injected_fail(dsa_session* s, const char* what) {
  s->failed = true;
  s->err = std::string("injected failure of ") + what;
  return DSA_E_HIP;
}

#define HIPCHK(expr, what)                                 \
  do {                                                     \
    if (take_injected(s)) return injected_fail(s, what);   \
    hipError_t e_ = (expr);                                \
    if (e_ != hipSuccess) return hip_fail(s, e_, what);    \
  } while (0)

// Keeps the caller's current device.
struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

// The device-side check flags (kernels set them when a plan is inconsistent;
// see DevErr): read without blocking, so a step's flags are seen by the first
// call made after the step has run.  Any flag fails the session.
bool device_checks_failed(dsa_session* s) {
  if (!s->err_host) return false;
  static const char* const names[kDevErrWords] = {"selection or union index", "hit slot", "victim slot",
                                                  "writeback position", "", "", "", ""};
  std::string kinds;
  for (int k = 0; k < kDevErrWords; ++k)
    if (reinterpret_cast<volatile uint32_t*>(s->err_host)[k]) kinds += (kinds.empty() ? "" : ", ") + std::string(names[k]);
  if (kinds.empty()) return false;
  s->failed = true;
  s->err = "device-side consistency check failed (" + kinds + " out of range); the session's state is no longer trusted";
  return true;
}

dsa_status entry(dsa_session* s) {
  if (!s) return DSA_E_INVALID;
  if (s->failed) return DSA_E_STATE;
  if (device_checks_failed(s)) return DSA_E_STATE;
  s->err.clear();
  return DSA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

dsa_status check_unit(dsa_session* s, int32_t layer, int32_t seq) {
  if (layer < 0 || layer >= s->cfg.n_layers || seq < 0 || seq >= s->cfg.n_seqs)
    return fail(s, DSA_E_INVALID, "layer or sequence out of range");
  return DSA_OK;
}

size_t unit_index(const dsa_session* s, int32_t layer, int32_t seq) {
  return (size_t)layer * s->cfg.n_seqs + seq;
}

// Event bookkeeping for dsa_mirror_rows.
dsa_status note_mirror(dsa_session* s, UnitHost& h, hipStream_t st) {
  if (h.ev_pending && hipEventQuery(h.ev) == hipSuccess) h.m_done = h.m_event;
  HIPCHK(hipEventRecord(h.ev, st), "hipEventRecord");
  h.m_event = h.M;
  h.ev_pending = true;
  return DSA_OK;
}

hipEvent_t take_event(dsa_session* s) {
  if (!s->free_events.empty()) {
    hipEvent_t e = s->free_events.back();
    s->free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs fn (one or more kernel launches).  With timing on, the group's first
// dispatch carries a start event and its last a stop event: the events take the
// dispatches' own timestamps, so the interval is the kernels' execution time.
template <class F>
dsa_status timed_launch(dsa_session* s, int kind, const char* what, F&& fn) {
  hipEvent_t a = nullptr, b = nullptr;
  if (take_injected(s)) return injected_fail(s, what);
  if (s->timing) {
    a = take_event(s);
    b = take_event(s);
    if (!a || !b) return hip_fail(s, hipErrorOutOfMemory, "hipEventCreate");
    t_launch_timer.start = a;
    t_launch_timer.stop = b;
  }
  const hipError_t e = fn();
  const bool launched = t_launch_timer.start == nullptr;   // consumed by a dispatch
  t_launch_timer.start = nullptr;
  t_launch_timer.stop = nullptr;
  HIPCHK(e, what);
  if (s->timing) {
    if (launched) {
      s->timed.push_back({kind, a, b});
    } else {
      s->free_events.push_back(a);
      s->free_events.push_back(b);
    }
  }
  return DSA_OK;
}

// One sequence's step scratch: 256-byte aligned pieces at these offsets of a
// block of `bytes` bytes.  The session's arena holds one block per sequence;
// dsa_decode_step_static lays the same blocks over the static scratch array.
struct ScrOff {
  size_t scores, sel, sel_n, uni, kind, src, map, compact, po, pml, cnt, info, selmask, hitmask, base_u, base_m,
      pdesc, victim, done, hist0, hist1, cand, cand_n, rowdig;
  size_t bytes;
};

ScrOff scratch_layout(const Geometry& g) {
  const int64_t P = g.p_pad, RK = (int64_t)g.r_max * g.top_k, rb = g.row_bytes;
  ScrOff o{};
  size_t cur = 0;
  auto take = [&](size_t bytes) { size_t at = cur; cur += align_up(bytes ? bytes : 1); return at; };
  o.scores = take((size_t)g.r_max * P * 4);
  o.sel = take((size_t)RK * 4);
  o.sel_n = take((size_t)g.r_max * 4);
  o.uni = take((size_t)RK * 4);
  o.kind = take((size_t)RK * 4);
  o.src = take((size_t)RK * 4);
  o.map = take((size_t)RK * 4);
  o.compact = take((size_t)RK * rb);
  o.po = take((size_t)g.r_max * g.nsplit_max * g.heads * g.latent * 2);
  o.pml = take((size_t)g.r_max * g.nsplit_max * g.heads * 4 * 4);
  o.cnt = take(16 * 8);
  o.info = take(kInfoWords * 8);
  o.selmask = take((size_t)P / 32 * 4);
  o.hitmask = take((size_t)P / 32 * 4);
  o.base_u = take((size_t)P / 32 * 4);
  o.base_m = take((size_t)P / 32 * 4);
  o.pdesc = take((size_t)P * 16);
  o.victim = take((size_t)g.s_words * 32 * 8);
  o.done = take((size_t)(1 + g.r_max) * 4);
  o.hist0 = take((size_t)kHistReps * g.r_max * kRadixBins * 4);
  o.hist1 = take((size_t)g.r_max * kRadixBins * 4);
  o.cand = take((size_t)g.r_max * P * 8);
  o.cand_n = take((size_t)g.r_max * g.n_chunks * 4);
  o.rowdig = take((size_t)g.r_max * 16);
  o.bytes = cur;
  return o;
}

SeqScratch scratch_at(uint8_t* base, const ScrOff& o) {
  SeqScratch c{};
  c.scores = reinterpret_cast<float*>(base + o.scores);
  c.sel = reinterpret_cast<int32_t*>(base + o.sel);
  c.sel_n = reinterpret_cast<int32_t*>(base + o.sel_n);
  c.uni = reinterpret_cast<int32_t*>(base + o.uni);
  c.kind = reinterpret_cast<int32_t*>(base + o.kind);
  c.src = reinterpret_cast<int32_t*>(base + o.src);
  c.map = reinterpret_cast<int32_t*>(base + o.map);
  c.compact = base + o.compact;
  c.part_o = reinterpret_cast<uint16_t*>(base + o.po);
  c.part_ml = reinterpret_cast<float*>(base + o.pml);
  c.counters = reinterpret_cast<int64_t*>(base + o.cnt);
  c.info = reinterpret_cast<int64_t*>(base + o.info);
  c.selmask = reinterpret_cast<uint32_t*>(base + o.selmask);
  c.hitmask = reinterpret_cast<uint32_t*>(base + o.hitmask);
  c.base_u = reinterpret_cast<uint32_t*>(base + o.base_u);
  c.base_m = reinterpret_cast<uint32_t*>(base + o.base_m);
  c.pdesc = reinterpret_cast<i32x4*>(base + o.pdesc);
  c.victim = reinterpret_cast<i32x2*>(base + o.victim);
  c.done = reinterpret_cast<uint32_t*>(base + o.done);
  c.hist0 = reinterpret_cast<uint32_t*>(base + o.hist0);
  c.hist1 = reinterpret_cast<uint32_t*>(base + o.hist1);
  c.cand = reinterpret_cast<i32x2*>(base + o.cand);
  c.cand_n = reinterpret_cast<uint32_t*>(base + o.cand_n);
  c.rowdig = reinterpret_cast<int32_t*>(base + o.rowdig);
  return c;
}

dsa_status validate_config(const dsa_config* c, std::string* why) {
  auto bad = [&](dsa_status st, const char* m) { *why = m; return st; };
  if (c->abi_version != DSA_ABI_VERSION) return bad(DSA_E_INVALID, "abi_version mismatch");
  if (c->n_layers < 1 || c->n_seqs < 1 || c->n_seqs > 64) return bad(DSA_E_INVALID, "n_layers >= 1 and 1 <= n_seqs <= 64");
  if (c->max_positions < 1) return bad(DSA_E_INVALID, "max_positions < 1");
  if (c->max_positions > (int64_t)kMaxTopkChunks * kTopkChunk) return bad(DSA_E_UNSUPPORTED, "max_positions > 4,194,304");
  if (c->mode != DSA_KV_OFFLOAD && c->mode != DSA_KV_HBM_RESIDENT) return bad(DSA_E_INVALID, "unknown mode");
  if (c->top_k < 1 || c->max_query_rows < 1 || c->ring_rows < 1) return bad(DSA_E_INVALID, "top_k, max_query_rows, ring_rows >= 1");
  if (c->mode == DSA_KV_OFFLOAD && (c->hot_slots < 1 || c->hot_slots > (1 << 20))) return bad(DSA_E_INVALID, "hot_slots out of range (1..2^20)");
  if (!std::isfinite(c->softmax_scale)) return bad(DSA_E_INVALID, "softmax_scale not finite");
  if (c->index_dim != 128 || c->latent_dim != 512 || c->rope_dim != 64 || c->group != 64)
    return bad(DSA_E_UNSUPPORTED, "kernels implement index_dim 128, latent 512, rope 64, group 64");
  if (c->index_heads != 4 && c->index_heads != 8 && c->index_heads != 16 && c->index_heads != 32)
    return bad(DSA_E_UNSUPPORTED, "index_heads must be 4, 8, 16 or 32");
  if (c->heads != 16 && c->heads != 32 && c->heads != 64 && c->heads != 128)
    return bad(DSA_E_UNSUPPORTED, "heads must be 16, 32, 64 or 128");
  if (c->max_query_rows > 8 || (int64_t)c->max_query_rows * c->index_heads > 256)
    return bad(DSA_E_UNSUPPORTED, "max_query_rows <= 8 and max_query_rows * index_heads <= 256");
  if (c->top_k > 4096 || (int64_t)c->max_query_rows * c->top_k > kMaxUnion)
    return bad(DSA_E_UNSUPPORTED, "top_k <= 4096 and max_query_rows * top_k <= 16384");
  if (c->ring_rows > 4096) return bad(DSA_E_UNSUPPORTED, "ring_rows <= 4096");
  if (c->replacement != DSA_REPL_RING && c->replacement != DSA_REPL_CLOCK) return bad(DSA_E_INVALID, "unknown replacement");
  return DSA_OK;
}

// Device address of the static scratch array on the current device, looked up
// once per device.
hipError_t static_scratch_address(int device, void** out) {
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (!g_static_scratch[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_static_scratch[device] = p;
  }
  *out = g_static_scratch[device];
  return hipSuccess;
}

void free_all(dsa_session* s) {
  for (auto& h : s->uh)
    if (h.ev) (void)hipEventDestroy(h.ev);
  for (auto& t : s->timed) {
    (void)hipEventDestroy(t.a);
    (void)hipEventDestroy(t.b);
  }
  for (auto e : s->free_events) (void)hipEventDestroy(e);
  if (s->sel_ready) (void)hipEventDestroy(s->sel_ready);
  s->sel_ready = nullptr;
  for (auto e : s->pf_done)
    if (e) (void)hipEventDestroy(e);
  s->pf_done.clear();
  if (s->mirror_block) (void)hipHostFree(s->mirror_block);
  s->mirror_block = nullptr;
  if (s->err_host) (void)hipHostFree(s->err_host);
  s->err_host = nullptr;
  s->err_dev = nullptr;
  if (s->arena) (void)hipFree(s->arena);
  s->uh.clear();
  s->timed.clear();
  s->free_events.clear();
  s->mirrors.clear();
  s->arena = nullptr;
}

// Host side of the end of a round of every sequence of `layer`: the round
// count, the rollback bound (the mirror count the round started with), and the
// batch the round wrote back.
dsa_status finish_round(dsa_session* s, int32_t layer, hipStream_t stream) {
  for (int q = 0; q < s->cfg.n_seqs; ++q) {
    UnitHost& h = s->uh[unit_index(s, layer, q)];
    h.round += 1;
    h.floor = h.M;
    if (s->g.mode == DSA_KV_OFFLOAD && h.L - h.M >= s->g.ring_rows) {
      h.M += s->g.ring_rows;
      dsa_status st = note_mirror(s, h, stream);
      if (st != DSA_OK) return st;
    }
  }
  return DSA_OK;
}

// prefetch_set: the round runs on the prefetch scratch set (offload only).
StepArgs step_args(const dsa_session* s, int32_t layer, int R, bool prefetch_set) {
  StepArgs a{};
  a.u0 = s->units[unit_index(s, layer, 0)];
  if (prefetch_set) {
    if (!s->scr_pf.empty()) a.s0 = s->scr_pf[0];
    a.s_stride = s->pf_stride;
  } else {
    a.s0 = s->scr[0];
    a.s_stride = s->s_stride;
  }
  a.u_stride = s->u_stride;
  a.rows_stride = s->rows_stride;
  a.n_seqs = s->cfg.n_seqs;
  a.R = R;
  a.err = s->err_dev;
  a.l_max = 0;
  for (int q = 0; q < s->cfg.n_seqs; ++q) a.l_max = std::max(a.l_max, s->uh[unit_index(s, layer, q)].L);
  return a;
}

// A round of `layer` on the selection of the most recent full decode step,
// which must be src_layer's, with the same rows per sequence and, for every
// sequence, the same row count as src_layer had then.
// A prefetch round of `layer` enqueued on another stream may still write the
// layer's ring batch back to the mirror and update its slot tables: work of the
// same layer enqueued on `stream` (appends, which reuse ring entries; flush,
// warm and rollback, which move M, L and the slots) waits for it first.
dsa_status wait_prefetch(dsa_session* s, int32_t layer, hipStream_t stream) {
  if (s->pf_pending[layer] && s->pf_stream[layer] != stream)
    HIPCHK(hipStreamWaitEvent(stream, s->pf_done[layer], 0), "hipStreamWaitEvent");
  return DSA_OK;
}

dsa_status check_reuse(dsa_session* s, int32_t layer, int32_t src_layer, int32_t R) {
  dsa_status st = entry(s);
  if (st != DSA_OK) return st;
  if (layer < 0 || layer >= s->cfg.n_layers || src_layer < 0 || src_layer >= s->cfg.n_layers)
    return fail(s, DSA_E_INVALID, "layer out of range");
  if (layer == src_layer) return fail(s, DSA_E_INVALID, "a layer cannot reuse its own selection");
  if (R < 1 || R > s->g.r_max) return fail(s, DSA_E_INVALID, "rows_per_seq out of range");
  if (s->topk_layer != src_layer) return fail(s, DSA_E_STATE, "src_layer's step is not the most recent full decode step");
  if (s->topk_R != R) return fail(s, DSA_E_STATE, "rows_per_seq differs from the source step's");
  for (int q = 0; q < s->cfg.n_seqs; ++q)
    if (s->uh[unit_index(s, layer, q)].L != s->topk_L[q])
      return fail(s, DSA_E_STATE, "a sequence's row count differs from the source layer's at its step");
  return DSA_OK;
}

}  // namespace

extern "C" {

dsa_status dsa_session_create(const dsa_config* cfg, dsa_session** out) {
  if (!out) return DSA_E_INVALID;
  *out = nullptr;
  if (!cfg) return DSA_E_INVALID;
  std::string why;
  dsa_status st = validate_config(cfg, &why);
  if (st != DSA_OK) return st;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || cfg->device < 0 || cfg->device >= ndev || cfg->device >= kMaxDevices)
    return DSA_E_INVALID;

  dsa_session* s = new dsa_session();
  s->cfg = *cfg;
  s->device = cfg->device;
  DeviceGuard dg(s->device);

  Geometry& g = s->g;
  g.index_heads = cfg->index_heads;
  g.index_dim = cfg->index_dim;
  g.heads = cfg->heads;
  g.latent = cfg->latent_dim;
  g.rope = cfg->rope_dim;
  g.group = cfg->group;
  g.top_k = cfg->top_k;
  g.hot_slots = cfg->mode == DSA_KV_OFFLOAD ? cfg->hot_slots : 0;
  g.ring_rows = cfg->ring_rows;
  g.ring_cap = cfg->ring_rows + cfg->max_query_rows;
  g.r_max = cfg->max_query_rows;
  g.row_bytes = cfg->latent_dim + 2 * (cfg->latent_dim / cfg->group) + 2 * cfg->rope_dim;
  g.mode = cfg->mode;
  g.clock = cfg->mode == DSA_KV_OFFLOAD && cfg->replacement == DSA_REPL_CLOCK;
  g.max_positions = cfg->max_positions;
  g.p_pad = (cfg->max_positions + kTopkChunk - 1) / kTopkChunk * kTopkChunk;
  g.n_chunks = (int)(g.p_pad / kTopkChunk);
  g.s_words = (g.hot_slots + 31) / 32;
  g.nsplit_max = (cfg->top_k + 63) / 64;
  g.softmax_scale = cfg->softmax_scale;
  g.n_cu = 0;
  if (hipDeviceGetAttribute(&g.n_cu, hipDeviceAttributeMultiprocessorCount, s->device) != hipSuccess || g.n_cu < 1)
    g.n_cu = 1;                                        // (then the plan never runs beside attention alone)

  const int n_units = cfg->n_layers * cfg->n_seqs;
  const int64_t P = g.p_pad, S = g.hot_slots, RK = (int64_t)g.r_max * g.top_k, rb = g.row_bytes;
  const bool off = cfg->mode == DSA_KV_OFFLOAD;

  // ---- arena layout (exact sizes, 256-byte aligned pieces)
  size_t cur = 0;
  auto take = [&](size_t bytes) { size_t at = cur; cur += align_up(bytes ? bytes : 1); return at; };
  struct UnitOff { size_t keys, rows, slots, ring, pos_slot, hot, slot_pos, fill, pin, ref, hand, dyn, totals; };
  std::vector<UnitOff> uo(n_units);
  for (int i = 0; i < n_units; ++i) {
    uo[i].keys = take((size_t)P * g.index_dim * 2);
    uo[i].rows = off ? 0 : take((size_t)P * rb);
    uo[i].slots = off ? take((size_t)S * rb) : 0;
    uo[i].ring = off ? take((size_t)g.ring_cap * rb) : 0;
    uo[i].pos_slot = off ? take((size_t)P * 8) : 0;
    uo[i].hot = off ? take((size_t)P / 32 * 4) : 0;
    uo[i].slot_pos = off ? take((size_t)S * 4) : 0;
    uo[i].fill = off ? take((size_t)S * 4) : 0;
    uo[i].pin = off ? take((size_t)S * 4) : 0;
    uo[i].ref = off ? take((size_t)g.s_words * 4) : 0;
    uo[i].hand = take(4);
    uo[i].dyn = take(32);
    uo[i].totals = take(128);
  }
  const ScrOff lay = scratch_layout(g);
  std::vector<size_t> so(cfg->n_seqs);
  for (int q = 0; q < cfg->n_seqs; ++q) so[q] = take(lay.bytes);
  // the prefetch rounds' scratch: only what the plan, the assign and the fill use
  struct PfOff { size_t cnt, info, uni, kind, src, selmask, hitmask, base_u, base_m, pdesc, victim, done; };
  std::vector<PfOff> pf(off ? cfg->n_seqs : 0);
  for (auto& x : pf) {
    x.cnt = take(16 * 8);
    x.info = take(kInfoWords * 8);
    x.uni = take((size_t)RK * 4);
    x.kind = take((size_t)RK * 4);
    x.src = take((size_t)RK * 4);
    x.selmask = take((size_t)P / 32 * 4);
    x.hitmask = take((size_t)P / 32 * 4);
    x.base_u = take((size_t)P / 32 * 4);
    x.base_m = take((size_t)P / 32 * 4);
    x.pdesc = take((size_t)P * 16);
    x.victim = take((size_t)g.s_words * 32 * 8);
    x.done = take(4);
  }
  s->arena_bytes = cur;

  auto bail = [&](dsa_status code, const char* msg) {
    free_all(s);
    delete s;
    (void)msg;
    return code;
  };
  hipError_t e;
  if ((e = prepare_score_kernels()) != hipSuccess) return bail(DSA_E_HIP, "prepare");
  if ((e = prepare_topk_kernels()) != hipSuccess) return bail(DSA_E_HIP, "prepare");
  if ((e = static_scratch_address(s->device, &s->static_scratch)) != hipSuccess) return bail(DSA_E_HIP, "static scratch");
  if (hipMalloc(&s->arena, s->arena_bytes) != hipSuccess) {
    s->arena = nullptr;
    (void)hipGetLastError();
    return bail(DSA_E_NOMEM, "hipMalloc");
  }
  uint8_t* base = static_cast<uint8_t*>(s->arena);
  if (hipMemset(s->arena, 0, s->arena_bytes) != hipSuccess) return bail(DSA_E_HIP, "hipMemset");
  {
    void* eh = nullptr;
    if (hipHostMalloc(&eh, kDevErrWords * sizeof(uint32_t), hipHostMallocMapped) != hipSuccess || !eh) {
      (void)hipGetLastError();
      return bail(DSA_E_NOMEM, "hipHostMalloc");
    }
    s->err_host = static_cast<uint32_t*>(eh);
    std::memset(s->err_host, 0, kDevErrWords * sizeof(uint32_t));
    void* ed = nullptr;
    if (hipHostGetDevicePointer(&ed, eh, 0) != hipSuccess) return bail(DSA_E_HIP, "hipHostGetDevicePointer");
    s->err_dev = static_cast<uint32_t*>(ed);
  }

  s->mirrors.assign(n_units, nullptr);
  uint8_t* mirror_dev = nullptr;
  if (off) {
    // every unit's mirror in one pinned, device-mapped block, at a stride of P rows
    const size_t bytes = (size_t)n_units * P * rb;
    if (hipHostMalloc(&s->mirror_block, bytes, hipHostMallocMapped) != hipSuccess || !s->mirror_block) {
      s->mirror_block = nullptr;
      (void)hipGetLastError();
      return bail(DSA_E_NOMEM, "hipHostMalloc");
    }
    std::memset(s->mirror_block, 0, bytes);                  // touch every page once, before use
    void* dp = nullptr;
    if (hipHostGetDevicePointer(&dp, s->mirror_block, 0) != hipSuccess) return bail(DSA_E_HIP, "hipHostGetDevicePointer");
    mirror_dev = static_cast<uint8_t*>(dp);
  }
  s->units.resize(n_units);
  s->uh.resize(n_units);
  for (int i = 0; i < n_units; ++i) {
    UnitDev& u = s->units[i];
    u.keys = reinterpret_cast<uint16_t*>(base + uo[i].keys);
    if (off) {
      s->mirrors[i] = static_cast<uint8_t*>(s->mirror_block) + (size_t)i * P * rb;
      u.rows = mirror_dev + (size_t)i * P * rb;
      u.slots = base + uo[i].slots;
      u.ring = base + uo[i].ring;
      u.pos_slot = reinterpret_cast<i32x2*>(base + uo[i].pos_slot);
      u.hot = reinterpret_cast<uint32_t*>(base + uo[i].hot);
      u.slot_pos = reinterpret_cast<int32_t*>(base + uo[i].slot_pos);
      u.fill_round = reinterpret_cast<int32_t*>(base + uo[i].fill);
      u.pin_round = reinterpret_cast<int32_t*>(base + uo[i].pin);
      u.ref = reinterpret_cast<uint32_t*>(base + uo[i].ref);        // zero (arena cleared above)
      if (hipMemset(u.pos_slot, 0xFF, (size_t)P * 8) != hipSuccess ||
          hipMemset(u.slot_pos, 0xFF, (size_t)S * 4) != hipSuccess ||
          hipMemset(u.fill_round, 0xFF, (size_t)S * 4) != hipSuccess ||
          hipMemset(u.pin_round, 0xFF, (size_t)S * 4) != hipSuccess)
        return bail(DSA_E_HIP, "hipMemset");
    } else {
      u.rows = base + uo[i].rows;
    }
    u.hand = reinterpret_cast<int32_t*>(base + uo[i].hand);
    u.dyn = reinterpret_cast<int64_t*>(base + uo[i].dyn);
    u.totals = reinterpret_cast<int64_t*>(base + uo[i].totals);
    if (hipEventCreateWithFlags(&s->uh[i].ev, hipEventDisableTiming) != hipSuccess) return bail(DSA_E_HIP, "event");
  }
  s->scr.resize(cfg->n_seqs);
  for (int q = 0; q < cfg->n_seqs; ++q) {
    SeqScratch& c = s->scr[q];
    c = scratch_at(base + so[q], lay);
    if (hipMemset(c.sel, 0xFF, (size_t)RK * 4) != hipSuccess || hipMemset(c.map, 0xFF, (size_t)RK * 4) != hipSuccess)
      return bail(DSA_E_HIP, "hipMemset");
  }
  std::vector<SeqScratch>& scr_pf = s->scr_pf;
  scr_pf.assign(pf.size(), SeqScratch{});
  for (size_t q = 0; q < pf.size(); ++q) {
    SeqScratch& c = scr_pf[q];                        // fields not listed stay NULL
    c.counters = reinterpret_cast<int64_t*>(base + pf[q].cnt);
    c.info = reinterpret_cast<int64_t*>(base + pf[q].info);
    c.uni = reinterpret_cast<int32_t*>(base + pf[q].uni);
    c.kind = reinterpret_cast<int32_t*>(base + pf[q].kind);
    c.src = reinterpret_cast<int32_t*>(base + pf[q].src);
    c.selmask = reinterpret_cast<uint32_t*>(base + pf[q].selmask);
    c.hitmask = reinterpret_cast<uint32_t*>(base + pf[q].hitmask);
    c.base_u = reinterpret_cast<uint32_t*>(base + pf[q].base_u);
    c.base_m = reinterpret_cast<uint32_t*>(base + pf[q].base_m);
    c.pdesc = reinterpret_cast<i32x4*>(base + pf[q].pdesc);
    c.victim = reinterpret_cast<i32x2*>(base + pf[q].victim);
    c.done = reinterpret_cast<uint32_t*>(base + pf[q].done);
  }
  s->topk_L.assign(cfg->n_seqs, -1);
  // stream-to-stream ordering on this device only: a device-scope release suffices
  const unsigned order_flags = hipEventDisableTiming | hipEventReleaseToDevice;
  if (hipEventCreateWithFlags(&s->sel_ready, order_flags) != hipSuccess) return bail(DSA_E_HIP, "event");
  s->pf_done.assign(cfg->n_layers, nullptr);
  s->pf_pending.assign(cfg->n_layers, 0);
  s->pf_stream.assign(cfg->n_layers, nullptr);
  for (auto& e : s->pf_done)
    if (hipEventCreateWithFlags(&e, order_flags) != hipSuccess) return bail(DSA_E_HIP, "event");
  // Kernels form sequence q's descriptors from sequence 0's and the strides:
  // check that every descriptor is sequence 0's moved by q strides.
  s->u_stride = n_units > 1 ? (int64_t)(uo[1].keys - uo[0].keys) : 0;
  s->rows_stride = off ? (int64_t)P * rb : s->u_stride;
  s->s_stride = cfg->n_seqs > 1 ? (int64_t)(so[1] - so[0]) : 0;
  s->pf_stride = pf.size() > 1 ? (int64_t)(pf[1].cnt - pf[0].cnt) : 0;
  auto strided = [](const void* d0, const void* dq, int64_t q, int64_t stride, size_t bytes) {
    uint64_t a[64], b[64];
    std::memcpy(a, d0, bytes);
    std::memcpy(b, dq, bytes);
    for (size_t i = 0; i < bytes / 8; ++i)
      if ((a[i] == 0) != (b[i] == 0) || (a[i] && b[i] != a[i] + (uint64_t)(q * stride))) return false;
    return true;
  };
  static_assert(sizeof(UnitDev) <= 64 * 8 && sizeof(SeqScratch) <= 64 * 8, "descriptor check buffers");
  const size_t rows_word = offsetof(UnitDev, rows) / 8;
  for (int i = 0; i < n_units; ++i) {
    UnitDev moved = s->units[i];
    const int q = i % cfg->n_seqs, l0 = i - q;                       // unit (layer, 0) is index l0
    uint64_t w[sizeof(UnitDev) / 8];
    std::memcpy(w, &moved, sizeof(w));
    w[rows_word] = w[rows_word] ? w[rows_word] - (uint64_t)(q * s->rows_stride) + (uint64_t)(q * s->u_stride) : 0;
    std::memcpy(&moved, w, sizeof(w));
    if (!strided(&s->units[l0], &moved, q, s->u_stride, sizeof(UnitDev)))
      return bail(DSA_E_UNSUPPORTED, "unit descriptors are not strided");
  }
  for (int q = 0; q < cfg->n_seqs; ++q)
    if (!strided(&s->scr[0], &s->scr[q], q, s->s_stride, sizeof(SeqScratch)) ||
        (!scr_pf.empty() && !strided(&scr_pf[0], &scr_pf[q], q, s->pf_stride, sizeof(SeqScratch))))
      return bail(DSA_E_UNSUPPORTED, "scratch descriptors are not strided");
  if (hipDeviceSynchronize() != hipSuccess) return bail(DSA_E_HIP, "hipDeviceSynchronize");
  *out = s;
  return DSA_OK;
}

dsa_status dsa_session_destroy(dsa_session* s) {
  if (!s) return DSA_OK;
  {
    DeviceGuard dg(s->device);
    (void)hipDeviceSynchronize();
    free_all(s);
  }
  delete s;
  return DSA_OK;
}

extern "C++" {
namespace {

// Shared by both append calls: validation, the ring spill bound, the launch
// (fn(newM) enqueues the kernels) and the host-side row counts.
template <class F>
dsa_status append_common(dsa_session* s, int32_t layer, int32_t seq, int64_t n, const void* index_keys,
                         std::initializer_list<const void*> bufs, hipStream_t stream, F&& fn) {
  dsa_status st = entry(s);
  if (st != DSA_OK) return st;
  if ((st = check_unit(s, layer, seq)) != DSA_OK) return st;
  if (n < 0) return fail(s, DSA_E_INVALID, "n < 0");
  if (n == 0) return DSA_OK;
  if (!index_keys || !aligned(index_keys, 16)) return fail(s, DSA_E_INVALID, "keys must be non-NULL and 16-byte aligned");
  for (const void* b : bufs)
    if (!b || !aligned(b, 16)) return fail(s, DSA_E_INVALID, "row inputs must be non-NULL and 16-byte aligned");
  const size_t ui = unit_index(s, layer, seq);
  UnitHost& h = s->uh[ui];
  if (h.L + n > s->cfg.max_positions) return fail(s, DSA_E_CAPACITY, "append past max_positions");
  DeviceGuard dg(s->device);
  if ((st = wait_prefetch(s, layer, stream)) != DSA_OK) return st;
  int64_t newM = h.M;
  if (s->g.mode == DSA_KV_OFFLOAD)
    while (h.L + n - newM > s->g.ring_cap) newM += s->g.ring_rows;
  if ((st = timed_launch(s, KK_APPEND, "append kernel", [&] { return fn(s->units[ui], h, newM); })) != DSA_OK)
    return st;
  const bool moved = newM != h.M;
  h.L += n;
  h.M = s->g.mode == DSA_KV_OFFLOAD ? newM : h.L;
  if (moved && s->g.mode == DSA_KV_OFFLOAD) return note_mirror(s, h, stream);
  return DSA_OK;
}

}  // namespace
}  // extern "C++"

dsa_status dsa_append_rows(dsa_session* s, int32_t layer, int32_t seq, int64_t n, const void* index_keys,
                           const void* rows, hipStream_t stream) {
  return append_common(s, layer, seq, n, index_keys, {rows}, stream, [&](const UnitDev& u, const UnitHost& h, int64_t newM) {
    return launch_append(s->g, u, h.L, h.M, newM, n, static_cast<const uint16_t*>(index_keys),
                         static_cast<const uint8_t*>(rows), stream);
  });
}

dsa_status dsa_append_latent(dsa_session* s, int32_t layer, int32_t seq, int64_t n, const void* index_keys,
                             const void* latent, const void* rope, hipStream_t stream) {
  return append_common(s, layer, seq, n, index_keys, {latent, rope}, stream,
                       [&](const UnitDev& u, const UnitHost& h, int64_t newM) {
                         return launch_append_latent(s->g, u, h.L, h.M, newM, n, static_cast<const uint16_t*>(index_keys),
                                                     static_cast<const uint16_t*>(latent),
                                                     static_cast<const uint16_t*>(rope), stream);
                       });
}

dsa_status dsa_quantize_rows(dsa_session* s, int64_t n, const void* latent, const void* rope, void* rows,
                             hipStream_t stream) {
  dsa_status st = entry(s);
  if (st != DSA_OK) return st;
  if (n < 0) return fail(s, DSA_E_INVALID, "n < 0");
  if (n == 0) return DSA_OK;
  if (!latent || !rope || !rows || !aligned(latent, 16) || !aligned(rope, 16) || !aligned(rows, 16))
    return fail(s, DSA_E_INVALID, "latent, rope and rows must be non-NULL and 16-byte aligned");
  DeviceGuard dg(s->device);
  HIPCHK(launch_quantize(s->g, n, static_cast<const uint16_t*>(latent), static_cast<const uint16_t*>(rope),
                         static_cast<uint8_t*>(rows), stream),
         "quantize kernel");
  return DSA_OK;
}

dsa_status dsa_flush(dsa_session* s, int32_t layer, int32_t seq, hipStream_t stream) {
  dsa_status st = entry(s);
  if (st != DSA_OK) return st;
  if ((st = check_unit(s, layer, seq)) != DSA_OK) return st;
  UnitHost& h = s->uh[unit_index(s, layer, seq)];
  if (s->g.mode != DSA_KV_OFFLOAD) return DSA_OK;
  DeviceGuard dg(s->device);
  if ((st = wait_prefetch(s, layer, stream)) != DSA_OK) return st;
  if (h.M < h.L) {
    HIPCHK(launch_flush(s->g, s->units[unit_index(s, layer, seq)], h.M, h.L, stream), "flush kernel");
    h.M = h.L;
  }
  return note_mirror(s, h, stream);
}

dsa_status dsa_warm_hot(dsa_session* s, int32_t layer, int32_t seq, hipStream_t stream) {
  dsa_status st = entry(s);
  if (st != DSA_OK) return st;
  if ((st = check_unit(s, layer, seq)) != DSA_OK) return st;
  if (s->g.mode != DSA_KV_OFFLOAD) return DSA_OK;
  UnitHost& h = s->uh[unit_index(s, layer, seq)];
  if (h.M != h.L) return fail(s, DSA_E_STATE, "warm needs a flushed unit (M == L)");
  DeviceGuard dg(s->device);
  if ((st = wait_prefetch(s, layer, stream)) != DSA_OK) return st;
  HIPCHK(launch_warm(s->g, s->units[unit_index(s, layer, seq)], h.L, stream), "warm kernels");
  h.floor = h.L;
  return DSA_OK;
}

dsa_status dsa_rollback_rows(dsa_session* s, int32_t layer, int32_t seq, int64_t n, hipStream_t stream) {
  dsa_status st = entry(s);
  if (st != DSA_OK) return st;
  if ((st = check_unit(s, layer, seq)) != DSA_OK) return st;
  if (n < 0) return fail(s, DSA_E_INVALID, "n < 0");
  if (n == 0) return DSA_OK;
  const size_t ui = unit_index(s, layer, seq);
  UnitHost& h = s->uh[ui];
  if (n > h.L) return fail(s, DSA_E_STATE, "rollback past the first row");
  const int64_t L2 = h.L - n;
  if (s->g.mode == DSA_KV_OFFLOAD && L2 < h.floor)
    return fail(s, DSA_E_STATE, "rollback below the rows the latest round could cache");
  const int64_t M2 = std::min(h.M, L2);
  DeviceGuard dg(s->device);
  if ((st = wait_prefetch(s, layer, stream)) != DSA_OK) return st;
  HIPCHK(launch_rollback(s->units[ui], L2, M2, stream), "rollback kernel");
  h.L = L2;
  h.M = M2;
  h.m_done = std::min(h.m_done, L2);
  h.m_event = std::min(h.m_event, L2);
  return DSA_OK;
}

extern "C++" {
namespace {

// Shared by the decode entry points: validation, then the step's launches on
// the scratch set `a` names, then the host-side round bookkeeping.  With
// app_keys (an append-and-decode step) every sequence of the layer first gains
// R rows, which the score launch writes (its scoring workgroups read the new
// keys from app_keys); the round's assign pass publishes the new L.
dsa_status decode_common(dsa_session* s, int32_t layer, int32_t R, const void* app_keys, const void* app_rows,
                         const void* index_q, const float* index_w, const void* q_latent, const void* q_rope,
                         float* out, hipStream_t stream, bool on_static) {
  dsa_status st = entry(s);
  if (st != DSA_OK) return st;
  if (layer < 0 || layer >= s->cfg.n_layers) return fail(s, DSA_E_INVALID, "layer out of range");
  if (R < 1 || R > s->g.r_max) return fail(s, DSA_E_INVALID, "rows_per_seq out of range");
  if (!index_q || !index_w || !q_latent || !q_rope || !out || !aligned(index_q, 16) || !aligned(q_latent, 16) ||
      !aligned(q_rope, 16) || !aligned(index_w, 4) || !aligned(out, 4))
    return fail(s, DSA_E_INVALID, "step buffers must be non-NULL; bf16 inputs 16-byte aligned");
  const bool app = app_keys != nullptr;
  if (app && (!app_rows || !aligned(app_keys, 16) || !aligned(app_rows, 16)))
    return fail(s, DSA_E_INVALID, "keys and rows to append must be non-NULL and 16-byte aligned");
  const int n_seqs = s->cfg.n_seqs;
  for (int q = 0; q < n_seqs; ++q) {
    const UnitHost& h = s->uh[unit_index(s, layer, q)];
    if (app && h.L + R > s->cfg.max_positions) return fail(s, DSA_E_CAPACITY, "append past max_positions");
    if (!app && h.L < R) return fail(s, DSA_E_STATE, "a sequence holds fewer rows than rows_per_seq");
  }
  const Geometry& g = s->g;
  if (app) {
    DeviceGuard dg(s->device);
    if ((st = wait_prefetch(s, layer, stream)) != DSA_OK) return st;
    // room in the ring for the new rows: its oldest rows to the mirror first, as an append would
    for (int q = 0; q < n_seqs && g.mode == DSA_KV_OFFLOAD; ++q) {
      const size_t ui = unit_index(s, layer, q);
      UnitHost& h = s->uh[ui];
      int64_t newM = h.M;
      while (h.L + R - newM > g.ring_cap) newM += g.ring_rows;
      if (newM == h.M) continue;
      const int64_t to = std::min(newM, h.L);
      HIPCHK(launch_flush(g, s->units[ui], h.M, to, stream), "ring spill kernel");
      h.M = newM;
      if ((st = note_mirror(s, h, stream)) != DSA_OK) return st;
    }
  }
  StepArgs a = step_args(s, layer, R, false);
  if (app) {
    a.add = R;
    a.l_max += R;
  }
  if (on_static) {
    const ScrOff lay = scratch_layout(g);
    const size_t need = lay.bytes * (size_t)n_seqs;
    if (need > kStaticScratchBytes)
      return fail(s, DSA_E_UNSUPPORTED, "the step needs " + std::to_string(need) + " bytes of scratch; the static scratch holds " +
                                            std::to_string(kStaticScratchBytes));
    a.s0 = scratch_at(static_cast<uint8_t*>(s->static_scratch), lay);
    a.s_stride = (int64_t)lay.bytes;
  }
  DeviceGuard dg(s->device);
  const uint16_t* iq = static_cast<const uint16_t*>(index_q);
  const uint16_t* ql = static_cast<const uint16_t*>(q_latent);
  const uint16_t* qr = static_cast<const uint16_t*>(q_rope);
  // a prefetch on another stream may still read the selection this step replaces
  for (int l = 0; l < s->cfg.n_layers; ++l)
    if (s->pf_pending[l] && s->pf_stream[l] != stream)
      HIPCHK(hipStreamWaitEvent(stream, s->pf_done[l], 0), "hipStreamWaitEvent");
  // the static array keeps the previous call's contents: zero what starts at zero
  if (on_static) HIPCHK(launch_clear_step_scratch(g, a, stream), "scratch clear kernel");
  if ((st = timed_launch(s, KK_SCORE, "score kernel", [&] {
         return launch_score(g, a, iq, index_w, static_cast<const uint16_t*>(app_keys),
                             static_cast<const uint8_t*>(app_rows), stream);
       })) != DSA_OK)
    return st;
  if ((st = timed_launch(s, KK_TOPK_PARTIAL, "top-k collect", [&] { return launch_topk_partial(g, a, stream); })) != DSA_OK)
    return st;
  if ((st = timed_launch(s, KK_TOPK_SELECT, "top-k resolve", [&] { return launch_topk_select(g, a, stream); })) != DSA_OK) return st;
  if (!on_static) {
    s->sel_epoch += 1;
    s->sel_stream = stream;
    if (s->pf_used) {
      HIPCHK(hipEventRecord(s->sel_ready, stream), "hipEventRecord");
      s->sel_recorded_epoch = s->sel_epoch;
    }
  }
  if ((st = timed_launch(s, KK_ATTN, "attention", [&] { return launch_attn(g, a, ql, qr, out, stream, 2 - topk_plan_mode(g, a)); })) != DSA_OK) return st;
  if ((st = timed_launch(s, KK_MERGE, "attention merge and assign", [&] { return launch_attn_merge(g, a, out, stream); })) != DSA_OK)
    return st;
  if (app)
    for (int q = 0; q < n_seqs; ++q) {
      UnitHost& h = s->uh[unit_index(s, layer, q)];
      h.L += R;
      if (g.mode != DSA_KV_OFFLOAD) h.M = h.L;
    }
  s->last_layer = layer;
  s->last_R = R;
  s->last_static = on_static;
  if (on_static) {
    s->topk_layer = -1;                  // the selection is not kept: no layer can reuse it
  } else {
    s->topk_layer = layer;
    s->topk_R = R;
    for (int q = 0; q < n_seqs; ++q) s->topk_L[q] = s->uh[unit_index(s, layer, q)].L;
  }
  return finish_round(s, layer, stream);
}

}  // namespace
}  // extern "C++"

dsa_status dsa_decode_step(dsa_session* s, int32_t layer, int32_t rows_per_seq, const void* index_q,
                           const float* index_w, const void* q_latent, const void* q_rope, float* out,
                           hipStream_t stream) {
  return decode_common(s, layer, rows_per_seq, nullptr, nullptr, index_q, index_w, q_latent, q_rope, out, stream,
                       false);
}

dsa_status dsa_append_decode_step(dsa_session* s, int32_t layer, int32_t rows_per_seq, const void* index_keys,
                                  const void* rows, const void* index_q, const float* index_w, const void* q_latent,
                                  const void* q_rope, float* out, hipStream_t stream) {
  if (!index_keys) {
    const dsa_status st = entry(s);
    return st != DSA_OK ? st : fail(s, DSA_E_INVALID, "keys to append must be non-NULL");
  }
  return decode_common(s, layer, rows_per_seq, index_keys, rows, index_q, index_w, q_latent, q_rope, out, stream,
                       false);
}

dsa_status dsa_decode_step_static(dsa_session* s, int32_t layer, int32_t rows_per_seq, const void* index_q,
                                  const float* index_w, const void* q_latent, const void* q_rope, float* out,
                                  hipStream_t stream) {
  return decode_common(s, layer, rows_per_seq, nullptr, nullptr, index_q, index_w, q_latent, q_rope, out, stream,
                       true);
}

dsa_status dsa_decode_step_reuse(dsa_session* s, int32_t layer, int32_t src_layer, int32_t rows_per_seq,
                                 const void* q_latent, const void* q_rope, float* out, hipStream_t stream) {
  dsa_status st = check_reuse(s, layer, src_layer, rows_per_seq);
  if (st != DSA_OK) return st;
  if (!q_latent || !q_rope || !out || !aligned(q_latent, 16) || !aligned(q_rope, 16) || !aligned(out, 4))
    return fail(s, DSA_E_INVALID, "step buffers must be non-NULL; bf16 inputs 16-byte aligned");
  DeviceGuard dg(s->device);
  const StepArgs a = step_args(s, layer, rows_per_seq, false);
  const Geometry& g = s->g;
  const uint16_t* ql = static_cast<const uint16_t*>(q_latent);
  const uint16_t* qr = static_cast<const uint16_t*>(q_rope);
  if (s->pf_pending[layer]) {                          // the layer's prefetch round comes first
    if (s->pf_stream[layer] != stream) HIPCHK(hipStreamWaitEvent(stream, s->pf_done[layer], 0), "hipStreamWaitEvent");
    s->pf_pending[layer] = 0;
  }
  if ((st = timed_launch(s, KK_TOPK_SELECT, "reuse mark", [&] { return launch_reuse_mark(g, a, s->scr[0], s->s_stride, stream); })) != DSA_OK)
    return st;
  if ((st = timed_launch(s, KK_ATTN, "attention", [&] { return launch_attn(g, a, ql, qr, out, stream, 0); })) != DSA_OK) return st;
  if ((st = timed_launch(s, KK_MERGE, "attention merge and assign", [&] { return launch_attn_merge(g, a, out, stream); })) != DSA_OK)
    return st;
  s->last_layer = layer;
  s->last_R = rows_per_seq;
  s->last_static = false;
  return finish_round(s, layer, stream);
}

dsa_status dsa_prefetch_reuse(dsa_session* s, int32_t layer, int32_t src_layer, int32_t rows_per_seq,
                              hipStream_t stream) {
  dsa_status st = check_reuse(s, layer, src_layer, rows_per_seq);
  if (st != DSA_OK) return st;
  if (s->g.mode != DSA_KV_OFFLOAD) return DSA_OK;
  DeviceGuard dg(s->device);
  const StepArgs a = step_args(s, layer, rows_per_seq, true);
  const Geometry& g = s->g;
  s->pf_used = true;
  if (s->sel_recorded_epoch != s->sel_epoch) {         // the step did not record it: everything it enqueued
    HIPCHK(hipEventRecord(s->sel_ready, s->sel_stream), "hipEventRecord");
    s->sel_recorded_epoch = s->sel_epoch;
  }
  if (s->sel_waited != stream || s->sel_waited_epoch != s->sel_epoch) {   // the selection is final
    HIPCHK(hipStreamWaitEvent(stream, s->sel_ready, 0), "hipStreamWaitEvent");
    s->sel_waited = stream;
    s->sel_waited_epoch = s->sel_epoch;
  }
  HIPCHK(launch_reuse_mark(g, a, s->scr[0], s->s_stride, stream), "prefetch mark");
  HIPCHK(launch_gather(g, a, stream, false), "prefetch assign");
  HIPCHK(launch_prefetch_fill(g, a, stream), "prefetch fill");
  HIPCHK(hipEventRecord(s->pf_done[layer], stream), "hipEventRecord");
  s->pf_pending[layer] = 1;
  s->pf_stream[layer] = stream;
  return finish_round(s, layer, stream);
}

dsa_status dsa_unit_state(const dsa_session* s, int32_t layer, int32_t seq, int64_t out[4]) {
  if (!s || !out) return DSA_E_INVALID;
  if (layer < 0 || layer >= s->cfg.n_layers || seq < 0 || seq >= s->cfg.n_seqs) return DSA_E_INVALID;
  const UnitHost& h = s->uh[unit_index(s, layer, seq)];
  out[0] = h.L;
  out[1] = h.M;
  out[2] = h.round;
  out[3] = s->g.row_bytes;
  return DSA_OK;
}

dsa_status dsa_mirror_rows(dsa_session* s, int32_t layer, int32_t seq, int64_t* rows) {
  dsa_status st = entry(s);
  if (st != DSA_OK) return st;
  if ((st = check_unit(s, layer, seq)) != DSA_OK) return st;
  if (!rows) return DSA_E_INVALID;
  UnitHost& h = s->uh[unit_index(s, layer, seq)];
  if (s->g.mode != DSA_KV_OFFLOAD) {
    *rows = 0;
    return DSA_OK;
  }
  if (h.ev_pending) {
    DeviceGuard dg(s->device);
    hipError_t q = hipEventQuery(h.ev);
    if (q == hipSuccess) {
      h.m_done = h.m_event;
      h.ev_pending = false;
    } else if (q != hipErrorNotReady) {
      return hip_fail(s, q, "hipEventQuery");
    }
  }
  *rows = h.m_done;
  return DSA_OK;
}

const char* dsa_last_error(const dsa_session* s) { return s ? s->err.c_str() : "NULL session"; }

dsa_status dsa_debug_size(const dsa_session* s, int32_t layer, int32_t seq, int32_t item, size_t* bytes) {
  if (!s || !bytes) return DSA_E_INVALID;
  if (layer < 0 || layer >= s->cfg.n_layers || seq < 0 || seq >= s->cfg.n_seqs) return DSA_E_INVALID;
  const Geometry& g = s->g;
  const UnitHost& h = s->uh[unit_index(s, layer, seq)];
  const int64_t R = s->last_R, K = g.top_k, S = g.hot_slots, rb = g.row_bytes;
  size_t b = 0;
  switch (item) {
    case DSA_DBG_SCORES: b = (size_t)R * h.L * 4; break;
    case DSA_DBG_SELECTION: b = (size_t)R * K * 4; break;
    case DSA_DBG_SEL_COUNT: b = (size_t)R * 4; break;
    case DSA_DBG_UNION: case DSA_DBG_UNION_KIND: case DSA_DBG_UNION_SRC: b = (size_t)R * K * 4; break;
    case DSA_DBG_MAP: b = (size_t)R * K * 4; break;
    case DSA_DBG_COMPACT: b = (size_t)R * K * rb; break;
    case DSA_DBG_COUNTERS: b = 72; break;
    case DSA_DBG_SLOT_POS: case DSA_DBG_FILL_ROUND: case DSA_DBG_PIN_ROUND: b = (size_t)S * 4; break;
    case DSA_DBG_POS_SLOT: b = g.mode == DSA_KV_OFFLOAD ? (size_t)h.L * 4 : 0; break;
    case DSA_DBG_HAND: b = 4; break;
    case DSA_DBG_SLOT_BYTES: b = (size_t)S * rb; break;
    case DSA_DBG_MIRROR: b = (size_t)(g.mode == DSA_KV_OFFLOAD ? h.M : h.L) * rb; break;
    case DSA_DBG_KEYS: b = (size_t)h.L * g.index_dim * 2; break;
    case DSA_DBG_TOTALS: b = 72; break;
    case DSA_DBG_REF_BITS: b = (size_t)g.s_words * 4; break;
    default: return DSA_E_INVALID;
  }
  *bytes = b;
  return DSA_OK;
}

dsa_status dsa_debug_get(dsa_session* s, int32_t layer, int32_t seq, int32_t item, void* dst, size_t bytes,
                         hipStream_t stream) {
  dsa_status st = entry(s);
  if (st != DSA_OK) return st;
  if ((st = check_unit(s, layer, seq)) != DSA_OK) return st;
  const bool step_item = item <= DSA_DBG_COUNTERS;
  if (step_item && s->last_layer != layer) return fail(s, DSA_E_STATE, "no step of this layer is the most recent");
  if (step_item && s->last_static)
    return fail(s, DSA_E_STATE, "the most recent step ran on the static scratch, whose step items are not kept");
  size_t need = 0;
  if ((st = dsa_debug_size(s, layer, seq, item, &need)) != DSA_OK) return fail(s, st, "unknown item");
  if (!dst || bytes < need) return fail(s, DSA_E_INVALID, "destination too small");
  if (need == 0) return DSA_OK;
  const Geometry& g = s->g;
  const size_t ui = unit_index(s, layer, seq);
  const UnitDev& u = s->units[ui];
  const SeqScratch& c = s->scr[seq];
  const UnitHost& h = s->uh[ui];
  const int64_t R = s->last_R, K = g.top_k;
  DeviceGuard dg(s->device);
  const void* src = nullptr;
  switch (item) {
    case DSA_DBG_SCORES:
      for (int64_t r = 0; r < R; ++r)
        HIPCHK(hipMemcpyAsync(static_cast<uint8_t*>(dst) + r * h.L * 4, c.scores + r * g.p_pad, (size_t)h.L * 4,
                              hipMemcpyDeviceToDevice, stream), "hipMemcpyAsync");
      return DSA_OK;
    case DSA_DBG_SELECTION: src = c.sel; break;
    case DSA_DBG_SEL_COUNT: src = c.sel_n; break;
    case DSA_DBG_UNION: src = c.uni; break;
    case DSA_DBG_UNION_KIND: src = c.kind; break;
    case DSA_DBG_UNION_SRC: src = c.src; break;
    case DSA_DBG_MAP: src = c.map; break;
    case DSA_DBG_COMPACT: src = c.compact; break;
    case DSA_DBG_COUNTERS: src = c.counters; break;
    case DSA_DBG_SLOT_POS: src = u.slot_pos; break;
    case DSA_DBG_FILL_ROUND: src = u.fill_round; break;
    case DSA_DBG_PIN_ROUND: src = u.pin_round; break;
    case DSA_DBG_POS_SLOT:                             // the slot half of each (slot, fill round) pair
      HIPCHK(hipMemcpy2DAsync(dst, 4, u.pos_slot, 8, 4, need / 4, hipMemcpyDeviceToDevice, stream), "hipMemcpy2DAsync");
      return DSA_OK;
    case DSA_DBG_HAND: src = u.hand; break;
    case DSA_DBG_SLOT_BYTES: src = u.slots; break;
    case DSA_DBG_MIRROR: src = g.mode == DSA_KV_OFFLOAD ? s->mirrors[ui] : (const void*)u.rows; break;
    case DSA_DBG_KEYS:                                 // stored in operand order: back to rows
      if (!aligned(dst, 16)) return fail(s, DSA_E_INVALID, "keys destination must be 16-byte aligned");
      HIPCHK(launch_keys_linear(u, h.L, static_cast<uint16_t*>(dst), stream), "keys kernel");
      return DSA_OK;
    case DSA_DBG_TOTALS: src = u.totals; break;
    case DSA_DBG_REF_BITS: src = u.ref; break;
    default: return fail(s, DSA_E_INVALID, "unknown item");
  }
  (void)K;
  HIPCHK(hipMemcpyAsync(dst, src, need, hipMemcpyDefault, stream), "hipMemcpyAsync");
  return DSA_OK;
}

dsa_status dsa_debug_inject(dsa_session* s, int32_t layer, int32_t seq, int32_t what, hipStream_t stream) {
  dsa_status st = entry(s);
  if (st != DSA_OK) return st;
  if ((st = check_unit(s, layer, seq)) != DSA_OK) return st;
  switch (what) {
    case DSA_INJECT_HIP_FAILURE:
      s->inject_hip = true;
      return DSA_OK;
    case DSA_INJECT_BAD_SLOT: {
      if (s->g.mode != DSA_KV_OFFLOAD) return fail(s, DSA_E_UNSUPPORTED, "bad-slot injection needs offload mode");
      DeviceGuard dg(s->device);
      const size_t ui = unit_index(s, layer, seq);
      HIPCHK(launch_inject_bad_slot(s->g, s->units[ui], s->uh[ui].L, stream), "injection kernel");
      return DSA_OK;
    }
    default:
      return fail(s, DSA_E_INVALID, "unknown injection");
  }
}

dsa_status dsa_set_kernel_timing(dsa_session* s, int32_t enable) {
  dsa_status st = entry(s);
  if (st != DSA_OK) return st;
  s->timing = enable > 0;
  if (enable > 0) {
    // pre-create the events of `enable` decode steps, so timed calls create none
    if (enable > (1 << 18)) return fail(s, DSA_E_INVALID, "timing reserve above 262,144 steps");
    DeviceGuard dg(s->device);
    const size_t want = (size_t)enable * DSA_KERNEL_KINDS * 2;
    while (s->free_events.size() < want) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return hip_fail(s, hipErrorOutOfMemory, "hipEventCreate");
      s->free_events.push_back(e);
    }
  }
  return DSA_OK;
}

dsa_status dsa_kernel_times(dsa_session* s, int64_t counts[DSA_KERNEL_KINDS], double total_ms[DSA_KERNEL_KINDS]) {
  dsa_status st = entry(s);
  if (st != DSA_OK) return st;
  if (!counts || !total_ms) return DSA_E_INVALID;
  DeviceGuard dg(s->device);
  for (auto& t : s->timed) {
    HIPCHK(hipEventSynchronize(t.b), "hipEventSynchronize");
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, t.a, t.b), "hipEventElapsedTime");
    s->t_counts[t.kind] += 1;
    s->t_ms[t.kind] += ms;
    s->free_events.push_back(t.a);
    s->free_events.push_back(t.b);
  }
  s->timed.clear();
  for (int k = 0; k < DSA_KERNEL_KINDS; ++k) {
    counts[k] = s->t_counts[k];
    total_ms[k] = s->t_ms[k];
    s->t_counts[k] = 0;
    s->t_ms[k] = 0.0;
  }
  return DSA_OK;
}

}  // extern "C"
