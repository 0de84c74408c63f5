// C-ABI host side: plan, argument validation, workspace carve-up, launches,
// kernel timing.  No entry point allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "mm_internal.hpp"

using namespace mm;

namespace {

constexpr int64_t kAlign = 256;

inline int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

int elem_size(int usecase) { return usecase == MM_A16W16 ? 2 : 1; }   // activation bytes
bool mx_usecase(int usecase) { return usecase == MM_MXFP8 || usecase == MM_MXFP4; }
bool a8w8_usecase(int usecase) { return usecase == MM_A8W8_FP8 || usecase == MM_A8W8_INT8; }
// weight bytes of n elements (e2m1: two per byte)
int64_t weight_bytes(int usecase, int64_t n) { return usecase == MM_MXFP4 ? n / 2 : n * elem_size(usecase); }

// experts with weights (routed + shared) and slots per token (top-k + shared)
int64_t all_experts(const mm_problem& p) { return p.num_experts + p.num_shared_experts; }
int64_t slots_per_token(const mm_problem& p) { return p.num_topk + p.num_shared_experts; }

uint64_t plan_checksum(const mm_plan* p) {
  // FNV-1a over every byte of the plan except the checksum itself
  const uint8_t* b = reinterpret_cast<const uint8_t*>(p);
  const size_t skip0 = offsetof(mm_plan, checksum), skip1 = skip0 + sizeof(p->checksum);
  uint64_t h = 1469598103934665603ull;
  for (size_t i = 0; i < sizeof(mm_plan); ++i) {
    if (i >= skip0 && i < skip1) continue;
    h ^= b[i];
    h *= 1099511628211ull;
  }
  return h ^ 0x6d65676d6f65ull;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Choices the plan makes for the workspace layout, kept in its reserved
// words: [0] the fused kernel's Linear1 reads token rows in place (no pool
// rows gathered), [1] the largest K split of a tail tile (1: none).
bool plan_by_token(const mm_plan& pl) { return pl.reserved[0] != 0; }
int plan_max_split(const mm_plan& pl) { return (int)pl.reserved[1]; }
// [2] the fused kernel's launch: cooperative (1) or ordinary (0)
bool plan_cooperative(const mm_plan& pl) { return pl.reserved[2] != 0; }
// [3] the fused kernel's dependency schedule: on where it applies (1) or off (0)
bool plan_dep(const mm_plan& pl) { return pl.reserved[3] != 0; }
// [4] the fused kernel's 256 x 256 tiles: static round robin (1) or claimed
// from per-XCD counters (0)
bool plan_static_tiles(const mm_plan& pl) { return pl.reserved[4] != 0; }

// ---------------------------------------------------------------- workspace
struct WsLayout {
  int64_t ctl, wave_base, a_stage, contrib, partials, end;                   // 3-call scratch
  int64_t mega_args, counts, offsets, pool_src, route_to_pool, x_pool, x_pool_scale, a_pool, a_pool_scale, x_tok,
      x_tok_scale, dep, fused_end;
};

WsLayout ws_layout(const mm_plan& pl) {
  const mm_problem& p = pl.prob;
  const bool q = p.usecase != MM_A16W16;
  const int64_t P = pl.pool_rows, R = p.num_tokens * slots_per_token(p), Et = all_experts(p);
  WsLayout L{};
  int64_t o = 0;
  auto take = [&](int64_t bytes) { const int64_t at = o; o = align_up(o + bytes, kAlign); return at; };
  L.ctl = take(kCtlWords * 4);
  L.wave_base = take(dispatch_waves(p.num_tokens, (int)slots_per_token(p)) * Et * 4);
  // float32 SwiGLU output, the input of the A8W8 per-row requantisation (MX
  // quantises it in the Linear1 epilogue)
  L.a_stage = a8w8_usecase(p.usecase) ? take(P * p.intermediate_hidden * 4) : -1;
  L.contrib = take(R * p.hidden * (q ? 2 : 4));   // combine slots: bf16 for A8W8, float32 for A16W16
  // partial sums of split tail tiles: one slot per piece in flight
  L.partials = plan_max_split(pl) > 1 ? take((int64_t)kSplitSlots * tile_bm(pl.tile_l1) * tile_bn(pl.tile_l1) * 4) : -1;
  L.end = o;
  L.mega_args = take(sizeof(MegaArgs));
  L.counts = take(Et * 4);
  L.offsets = take((Et + 1) * 4);
  L.pool_src = take(P * 4);
  L.route_to_pool = take(R * 4);
  // pool rows only when the fused Linear1 cannot read the token rows in place
  const bool tok = plan_by_token(pl);
  L.x_pool = tok ? -1 : take(pl.x_pool_bytes);
  L.x_pool_scale = tok || !q ? -1 : take(pl.x_pool_scale_bytes);
  L.a_pool = take(pl.a_pool_bytes);
  L.a_pool_scale = q ? take(pl.a_pool_scale_bytes) : -1;
  // A8W8 / MX codes and scales of the T tokens (the fused kernel's Linear1 reads token rows in place)
  L.x_tok = q && tok ? take(p.num_tokens * p.hidden) : -1;
  L.x_tok_scale = q && tok ? take(mx_usecase(p.usecase) ? p.num_tokens * (p.hidden / 32) : p.num_tokens * 4) : -1;
  // the fused kernel's per-M-block counters (its dependency schedule)
  L.dep = take((2 * (P / pl.block_m) + 16) * 4);
  L.fused_end = o;
  return L;
}

template <typename T>
T* at(void* ws, int64_t off) {
  return off < 0 ? nullptr : reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// ---------------------------------------------------------------- tracing
struct TraceRec {
  int id;
  hipEvent_t a, b;
};
std::mutex g_trace_mu;
bool g_trace_on = false;
std::vector<TraceRec> g_trace;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t get_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launch wrapper: brackets the launch with events when tracing is on.
template <typename F>
mm_status run(int id, hipStream_t s, F&& f) {
  TraceRec rec{id, nullptr, nullptr};
  bool tr = false;
  {
    std::lock_guard<std::mutex> g(g_trace_mu);
    if (g_trace_on) {
      rec.a = get_event();
      rec.b = get_event();
      tr = rec.a && rec.b;
    }
  }
  if (tr && hipEventRecord(rec.a, s) != hipSuccess) return MM_ERR_HIP;
  if (f() != hipSuccess) return MM_ERR_HIP;
  if (tr) {
    if (hipEventRecord(rec.b, s) != hipSuccess) return MM_ERR_HIP;
    std::lock_guard<std::mutex> g(g_trace_mu);
    g_trace.push_back(rec);
  }
  return MM_OK;
}

#define MM_TRY(x)                   \
  do {                              \
    const mm_status st__ = (x);     \
    if (st__ != MM_OK) return st__; \
  } while (0)

mm_status check_plan(const mm_plan* pl) {
  if (!pl) return MM_ERR_INVALID_ARG;
  if (pl->checksum != plan_checksum(pl)) return MM_ERR_INVALID_ARG;
  return MM_OK;
}

// ---------------------------------------------------------------- stages
// Argument blocks of each step; the three-call path launches them as
// separate kernels, mega_moe hands all of them to the fused kernel.
DispatchArgs dispatch_args(const mm_plan& pl, const int32_t* ids, const int8_t* active, const void* x, int32_t* counts,
                           int32_t* offsets, int32_t* pool_src, int32_t* r2p, void* x_pool, void* x_pool_scale,
                           void* ws) {
  const mm_problem& p = pl.prob;
  const WsLayout L = ws_layout(pl);
  DispatchArgs d{};
  d.topk_ids = ids;
  d.active = active;
  d.x = x;
  d.counts = counts;
  d.offsets = offsets;
  d.pool_src = pool_src;
  d.route_to_pool = r2p;
  d.x_pool = x_pool;
  const bool mx = mx_usecase(p.usecase);
  d.x_pool_scale = mx ? nullptr : static_cast<float*>(x_pool_scale);
  d.x_pool_mx = mx ? static_cast<uint8_t*>(x_pool_scale) : nullptr;
  d.wave_base = at<int32_t>(ws, L.wave_base);
  d.err = at<uint32_t>(ws, L.ctl) + 1;
  d.T = p.num_tokens;
  d.H = p.hidden;
  d.P = pl.pool_rows;
  d.E = (int)all_experts(p);
  d.K = (int)slots_per_token(p);
  d.Er = (int)p.num_experts;
  d.Kr = (int)p.num_topk;
  d.block_m = pl.block_m;
  d.usecase = p.usecase;
  return d;
}

// Polls a wait inside a kernel (a fused-kernel grid barrier, a GEMM waiting
// for a partial tile) makes before giving up (about seconds); MM_BARRIER_SPIN
// overrides it, which tests use to exercise the time-out.
uint32_t barrier_spin_limit() {
  if (const char* v = std::getenv("MM_BARRIER_SPIN")) {
    const long n = std::atol(v);
    if (n > 0) return (uint32_t)n;
  }
  return 1u << 21;
}

// Largest K split of a tail tile, chosen by the plan (MM_MAX_SPLIT, read
// when the plan is made, overrides it: 1 turns it off).  Only int8 splits
// by default: its partial sums are exact int32.  With float accumulators a
// split tile rounds differently from an unsplit one, and which M-block of
// its expert (so which tile) a route lands in depends on the order in which
// the dispatch's atomics claim pool rows; unsplit, every route's result
// depends on its own row alone, so the output is the same on every call and
// in both paths.  Split only in the compute regime: measured, splitting the
// last round's tiles makes the 2048 x 4096 layer 2-3% faster and costs the
// 128-token 7168 x 2048 layers 3-5% (the partial sums add traffic to a step
// that is already bound by streaming the weights); neutral in between.
int choose_max_split(const mm_problem& p) {
  if (const char* v = std::getenv("MM_MAX_SPLIT")) {
    const int n = std::atoi(v);
    if (n >= 1 && n <= 8) return n;
  }
  if (p.usecase != MM_A8W8_INT8) return 1;
  const double expected = (double)(p.num_tokens * p.num_topk) / (double)p.num_experts;
  return expected >= 96 ? 8 : 1;
}

// e4m3 Linear1 on exact bf16 MFMA (true) or on the e4m3 MFMA (false).  The
// e4m3 MFMAs round inside their dot products (about 4e-5 of the result's
// RMS, with unit or any block scales, measured against the exact sum); the
// requantisation of the SwiGLU output after Linear1 turns that into code
// changes (0.1-0.2 % of the codes), whose effect on a Y element shrinks like
// 1/sqrt(I): per-row fp8 measured max|dY|/rms 8e-3 at I = 2048 but 7e-2 at
// I = 256, MX 5-17e-2 even at I = 2048 (its per-group scales leave each
// group's largest values in the top binade, where a code step is largest).
// So: per-row fp8 on the e4m3 MFMA for I >= 1024, exact below; MX always
// exact (the MX Linear2 keeps the scaled MX MFMA: nothing is quantised after
// it).  MM_FP8_L1=exact|fast overrides both (tests, tuning).
bool fp8_l1_exact(const mm_plan& pl) {
  if (const char* v = std::getenv("MM_FP8_L1")) {
    if (std::strcmp(v, "exact") == 0) return true;
    if (std::strcmp(v, "fast") == 0) return false;
  }
  if (mx_usecase(pl.prob.usecase)) return true;
  return pl.prob.intermediate_hidden < 1024;
}

// Fused kernel: Linear1 reads the token rows in place through pool_src when
// the token matrix fits one buffer descriptor (< 2^31 bytes); otherwise the
// pool rows are gathered.  MM_L1_BY_TOKEN=0, read when the plan is made,
// forces the gather (a tuning switch).
bool choose_by_token(const mm_problem& p) {
  const char* v = std::getenv("MM_L1_BY_TOKEN");
  if (v && v[0] == '0') return false;
  return p.num_tokens * p.hidden * elem_size(p.usecase) < ((int64_t)1 << 31);
}

// M-blocks per tile group of Linear1 / Linear2 (0: a whole expert);
// MM_GROUP_M1 / MM_GROUP_M2 override (tuning).
int group_m_of(const char* env, int dflt) {
  if (const char* v = std::getenv(env)) {
    const int n = std::atoi(v);
    if (n >= 0 && n <= 1024) return n;
  }
  return dflt;
}

void set_split(GemmArgs& g, const mm_plan& pl, const WsLayout& L, void* ws) {
  g.partials = at<uint32_t>(ws, L.partials);
  g.split_flags = at<uint32_t>(ws, L.ctl) + kSplitFlag0;
  g.max_split = plan_max_split(pl);
  g.spin_limit = barrier_spin_limit();
}

GemmArgs l1_args(const mm_plan& pl, const int32_t* offsets, const int32_t* counts, const void* x_pool,
                 const void* x_pool_scale, const void* w1, const void* w1_scale, void* a_pool, void* a_pool_scale,
                 void* ws) {
  const mm_problem& p = pl.prob;
  const WsLayout L = ws_layout(pl);
  GemmArgs g{};
  g.A = static_cast<const uint8_t*>(x_pool);
  g.B = static_cast<const uint8_t*>(w1);
  g.offsets = offsets;
  g.counts = counts;
  g.P = pl.pool_rows;
  g.E = (int)all_experts(p);
  g.N = (int)(2 * p.intermediate_hidden);
  g.Kdim = (int)p.hidden;
  g.I = (int)p.intermediate_hidden;
  g.H = (int)p.hidden;
  g.K = (int)slots_per_token(p);
  g.Kr = (int)p.num_topk;
  g.gate_up_group = pl.gate_up_group;
  g.clamp = p.clamp_activation ? p.activation_clamp : INFINITY;
  g.routes = p.num_tokens * slots_per_token(p);
  g.err = at<uint32_t>(ws, L.ctl) + 1;
  if (mx_usecase(p.usecase)) {
    g.a_mx = static_cast<const uint8_t*>(x_pool_scale);
    g.a_mx_rows = pl.pool_rows;
    g.b_mx = static_cast<const uint8_t*>(w1_scale);
    g.out_mx = static_cast<uint8_t*>(a_pool_scale);
  } else {
    g.x_scale = static_cast<const float*>(x_pool_scale);
    g.w_scale = static_cast<const float*>(w1_scale);
  }
  g.a_out = a_pool;
  g.a_stage = at<float>(ws, L.a_stage);
  set_split(g, pl, L, ws);
  // pool rows are read once per group of N-blocks: group 8 M-blocks (with 4
  // N-blocks per XCD round) to read each activation stage a quarter as often
  g.group_m = group_m_of("MM_GROUP_M1", 8);
  return g;
}

RequantArgs requant_args(const mm_plan& pl, const GemmArgs& l1, void* a_pool, void* a_pool_scale) {
  RequantArgs r{};
  r.a_stage = l1.a_stage;
  r.offsets = l1.offsets;
  r.counts = l1.counts;
  r.E = l1.E;
  r.a_pool = a_pool;
  r.a_scale = static_cast<float*>(a_pool_scale);
  r.P = pl.pool_rows;
  r.I = l1.I;
  r.usecase = pl.prob.usecase;
  return r;
}

GemmArgs l2_args(const mm_plan& pl, const int32_t* offsets, const int32_t* counts, const int32_t* pool_src,
                 const void* a_pool, const void* a_pool_scale, const void* w2, const void* w2_scale,
                 const float* topk_w, void* ws) {
  const mm_problem& p = pl.prob;
  const WsLayout L = ws_layout(pl);
  GemmArgs g{};
  g.A = static_cast<const uint8_t*>(a_pool);
  g.B = static_cast<const uint8_t*>(w2);
  g.offsets = offsets;
  g.counts = counts;
  g.pool_src = pool_src;
  g.P = pl.pool_rows;
  g.E = (int)all_experts(p);
  g.N = (int)p.hidden;
  g.Kdim = (int)p.intermediate_hidden;
  g.I = (int)p.intermediate_hidden;
  g.H = (int)p.hidden;
  g.K = (int)slots_per_token(p);
  g.Kr = (int)p.num_topk;
  g.routes = p.num_tokens * slots_per_token(p);
  g.err = at<uint32_t>(ws, L.ctl) + 1;
  if (mx_usecase(p.usecase)) {
    g.a_mx = static_cast<const uint8_t*>(a_pool_scale);
    g.a_mx_rows = pl.pool_rows;
    g.b_mx = static_cast<const uint8_t*>(w2_scale);
  } else {
    g.a_scale = static_cast<const float*>(a_pool_scale);
    g.w_scale = static_cast<const float*>(w2_scale);
  }
  g.topk_w = topk_w;
  g.contrib = at<uint8_t>(ws, L.contrib);
  set_split(g, pl, L, ws);
  g.group_m = group_m_of("MM_GROUP_M2", 0);   // measured: grouping slows Linear2 (its weight tiles are re-read per group)
  return g;
}

CombineArgs combine_args(const mm_plan& pl, const void* contrib, const int32_t* r2p, void* y) {
  const mm_problem& p = pl.prob;
  CombineArgs c{};
  c.contrib = contrib;
  c.route_to_pool = r2p;
  c.y = y;
  c.T = p.num_tokens;
  c.H = (int)p.hidden;
  c.K = (int)slots_per_token(p);
  c.y_f32 = p.y_dtype == MM_OUT_F32;
  c.slot_bf16 = p.usecase != MM_A16W16;
  return c;
}

mm_status do_dispatch(const mm_plan& pl, const int32_t* ids, const int8_t* active, const void* x, int32_t* counts,
                      int32_t* offsets, int32_t* pool_src, int32_t* r2p, void* x_pool, void* x_pool_scale, void* ws,
                      hipStream_t s) {
  const DispatchArgs d = dispatch_args(pl, ids, active, x, counts, offsets, pool_src, r2p, x_pool, x_pool_scale, ws);
  uint32_t* ctl = at<uint32_t>(ws, ws_layout(pl).ctl);
  MM_TRY(run(MM_K_ZERO, s, [&] { return launch_zero(counts, d.E, ctl, 0, kCtlWords, s); }));
  MM_TRY(run(MM_K_COUNT, s, [&] { return launch_count(d, s); }));
  MM_TRY(run(MM_K_SCATTER, s, [&] { return launch_scatter(d, s); }));
  MM_TRY(run(MM_K_GATHER, s, [&] { return launch_gather(d, s); }));
  return MM_OK;
}

// The ready flags of split tail tiles start at zero: a GEMM entry point may
// get a workspace no dispatch has cleared, or one where a waiter gave up
// before a late producer set its flag.  Only when tiles can split.
mm_status clear_split_flags(const GemmArgs& g, hipStream_t s) {
  if (g.max_split < 2) return MM_OK;
  uint32_t* ctl = g.split_flags - kSplitFlag0;
  return run(MM_K_ZERO, s, [&] { return launch_zero(nullptr, 0, ctl, kSplitFlag0, kSplitSlots, s); });
}

mm_status do_l1(const mm_plan& pl, const int32_t* offsets, const int32_t* counts, const void* x_pool,
                const void* x_pool_scale, const void* w1, const void* w1_scale, void* a_pool, void* a_pool_scale,
                void* ws, hipStream_t s) {
  const mm_problem& p = pl.prob;
  const GemmArgs g = l1_args(pl, offsets, counts, x_pool, x_pool_scale, w1, w1_scale, a_pool, a_pool_scale, ws);
  const int grid = gemm_grid(pl.tile_l1, pl.pool_rows, g.N, num_cus());
  MM_TRY(clear_split_flags(g, s));
  MM_TRY(run(MM_K_L1, s, [&] { return launch_gemm(0, p.usecase, pl.tile_l1, fp8_l1_exact(pl), g, grid, s); }));
  if (a8w8_usecase(p.usecase)) {
    const RequantArgs r = requant_args(pl, g, a_pool, a_pool_scale);
    MM_TRY(run(MM_K_REQUANT, s, [&] { return launch_requant(r, s); }));
  }
  return MM_OK;
}

mm_status do_l2(const mm_plan& pl, const int32_t* offsets, const int32_t* counts, const int32_t* pool_src,
                const int32_t* r2p, const void* a_pool, const void* a_pool_scale, const void* w2,
                const void* w2_scale, const float* topk_w, void* y, void* ws, hipStream_t s) {
  const mm_problem& p = pl.prob;
  const GemmArgs g = l2_args(pl, offsets, counts, pool_src, a_pool, a_pool_scale, w2, w2_scale, topk_w, ws);
  const int grid = gemm_grid(pl.tile_l2, pl.pool_rows, g.N, num_cus());
  MM_TRY(clear_split_flags(g, s));
  MM_TRY(run(MM_K_L2, s, [&] { return launch_gemm(1, p.usecase, pl.tile_l2, false, g, grid, s); }));
  const CombineArgs c = combine_args(pl, g.contrib, r2p, y);
  MM_TRY(run(MM_K_COMBINE, s, [&] { return launch_combine(c, s); }));
  return MM_OK;
}

bool ok16(const void* p) { return p && aligned(p, 16); }
bool ok4(const void* p) { return p && aligned(p, 4); }

// ---------------------------------------------------------------- static scratch
// The workspace of mega_moe_noalloc: a device array of the library itself,
// one copy per GPU, held until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the
// symbol): its device address comes from hipGetSymbolAddress, once per
// device, with that device current.
constexpr int64_t kScratchBytes = (int64_t)96 << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

mm_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MM_ERR_HIP;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MM_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MM_OK;
}

}  // namespace

extern "C" {

mm_status mm_plan_create(const mm_problem* problem, mm_plan* plan) {
  if (!problem || !plan) return MM_ERR_INVALID_ARG;
  const mm_problem p = *problem;
  if (p.usecase < MM_A16W16 || p.usecase > MM_MXFP4) return MM_ERR_UNSUPPORTED;
  if (p.y_dtype != MM_OUT_BF16 && p.y_dtype != MM_OUT_F32) return MM_ERR_UNSUPPORTED;
  if (p.clamp_activation != 0 && p.clamp_activation != 1) return MM_ERR_INVALID_ARG;
  if (p.clamp_activation && !(p.activation_clamp >= 0.0f)) return MM_ERR_INVALID_ARG;   // negative or NaN
  if (p.num_tokens < 1 || p.num_tokens > (1 << 24)) return MM_ERR_INVALID_ARG;
  if (p.hidden < 256 || p.hidden > 16384 || p.hidden % 256) return MM_ERR_INVALID_ARG;
  if (p.intermediate_hidden < 128 || p.intermediate_hidden > 16384 || p.intermediate_hidden % 128)
    return MM_ERR_INVALID_ARG;
  if (p.num_experts < 1 || p.num_experts > 1024) return MM_ERR_INVALID_ARG;
  if (p.num_topk < 1 || p.num_topk > 64 || p.num_topk > p.num_experts) return MM_ERR_INVALID_ARG;
  if (p.num_shared_experts < 0 || p.num_shared_experts > 1 || p.reserved0 != 0) return MM_ERR_INVALID_ARG;
  if (slots_per_token(p) > 64 || all_experts(p) > (mx_usecase(p.usecase) ? 512 : 1024)) return MM_ERR_INVALID_ARG;
  const int64_t R = p.num_tokens * slots_per_token(p);
  if (R > (int64_t)1 << 30) return MM_ERR_INVALID_ARG;

  mm_plan pl;
  std::memset(&pl, 0, sizeof(pl));
  pl.prob = p;
  // BLOCK_M from the expected rows per expert (small loads -> small blocks).
  // Measured on the 7168 x 2048, 32-expert, top-8 layer: BLOCK_M 64 is 6-9%
  // faster at 16 rows per expert, 128 is 4-5% faster at 32 rows and 16% / 31%
  // faster at 128 / 256 rows (fewer passes over each expert's weights).
  // 256 x 256 from 1024 rows per expert on (measured on the same layer:
  // 3-6% faster at 2048 and 4096 rows; at 1024 rows, with the fused
  // kernel's tiles claimed across XCDs, 3.02 vs 3.13 ms for bf16); not for
  // the MX use cases (their scale copies need eight waves).
  const double expected = (double)R / (double)p.num_experts;
  int tile = expected < 24 ? TILE_M64_N128 : expected < 1024 ? TILE_M128_N256 : TILE_M256_N256;
  // tuning override: MM_FORCE_TILE=<0..2> selects BLOCK_M 64/128/256
  if (const char* f = std::getenv("MM_FORCE_TILE")) {
    const int v = std::atoi(f);
    if (v >= 0 && v < TILE_COUNT) tile = v;
  }
  if (tile == TILE_M256_N256 && mx_usecase(p.usecase)) tile = TILE_M128_N256;
  pl.tile_l1 = tile;
  pl.tile_l2 = tile;
  pl.block_m = tile_bm(tile);
  pl.gate_up_group = 32;
  pl.reserved[0] = choose_by_token(p) ? 1 : 0;
  pl.reserved[1] = choose_max_split(p);
  // MM_COOPERATIVE=1 when the plan is made: launch the fused kernel cooperatively
  if (const char* v = std::getenv("MM_COOPERATIVE")) pl.reserved[2] = std::atoi(v) == 1 ? 1 : 0;
  // MM_DEP=1 when the plan is made: the fused kernel replaces the grid
  // barriers between Linear1, the requantisation and Linear2 by per-M-block
  // counters.  Off by default: measured slower for A8W8 (6.12 vs 5.99 ms at
  // 16K fp8 tokens, 0.372 vs 0.340 ms at 128), no faster for bf16 and MX.
  if (const char* v = std::getenv("MM_DEP")) pl.reserved[3] = std::atoi(v) == 1 ? 1 : 0;
  // MM_STATIC_TILES=1 when the plan is made: no per-XCD tile counters
  if (const char* v = std::getenv("MM_STATIC_TILES")) pl.reserved[4] = std::atoi(v) == 1 ? 1 : 0;
  const int64_t P = align_up(R + all_experts(p) * (pl.block_m - 1), pl.block_m);
  if (P > ((int64_t)1 << 31) - 1) return MM_ERR_INVALID_ARG;
  pl.pool_rows = P;
  const int es = elem_size(p.usecase);
  pl.x_pool_bytes = P * p.hidden * es;
  pl.a_pool_bytes = P * p.intermediate_hidden * es;
  pl.x_pool_scale_bytes = mx_usecase(p.usecase) ? P * (p.hidden / 32) : a8w8_usecase(p.usecase) ? P * 4 : 0;
  pl.a_pool_scale_bytes = mx_usecase(p.usecase) ? P * (p.intermediate_hidden / 32) : a8w8_usecase(p.usecase) ? P * 4 : 0;
  pl.w1_bytes = weight_bytes(p.usecase, all_experts(p) * p.hidden * 2 * p.intermediate_hidden);
  pl.w2_bytes = weight_bytes(p.usecase, all_experts(p) * p.intermediate_hidden * p.hidden);
  const WsLayout L = ws_layout(pl);
  pl.workspace_bytes = L.end;
  pl.fused_workspace_bytes = L.fused_end;
  pl.checksum = plan_checksum(&pl);
  *plan = pl;
  return MM_OK;
}

mm_status mm_prepare_weights(const mm_plan* plan, const void* w1, const void* w2, void* w1_out, void* w2_out,
                             void* stream) {
  MM_TRY(check_plan(plan));
  if (!ok16(w1) || !ok16(w2) || !ok16(w1_out) || !ok16(w2_out)) return MM_ERR_INVALID_ARG;
  const mm_problem& p = plan->prob;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return run(MM_K_PREPARE, s, [&] {
    return launch_prepare(w1, w2, w1_out, w2_out, (int)all_experts(p), (int)p.hidden, (int)p.intermediate_hidden,
                          p.usecase == MM_MXFP4 ? 0 : elem_size(p.usecase), plan->gate_up_group, s);
  });
}

mm_status mm_dispatch_layout(const mm_plan* plan, const int32_t* topk_ids, const int8_t* x_active_mask, const void* x,
                             int32_t* expert_counts, int32_t* expert_offsets, int32_t* pool_src, int32_t* route_to_pool,
                             void* x_pool, void* x_pool_scale, void* workspace, uint64_t workspace_bytes,
                             void* stream) {
  MM_TRY(check_plan(plan));
  const bool q = plan->prob.usecase != MM_A16W16;
  if (!ok4(topk_ids) || !ok16(x) || !ok4(expert_counts) || !ok4(expert_offsets) || !ok4(pool_src) ||
      !ok4(route_to_pool) || !ok16(x_pool) || !ok16(workspace))
    return MM_ERR_INVALID_ARG;
  if (q && !ok4(x_pool_scale)) return MM_ERR_INVALID_ARG;
  if ((int64_t)workspace_bytes < plan->workspace_bytes) return MM_ERR_WORKSPACE;
  return do_dispatch(*plan, topk_ids, x_active_mask, x, expert_counts, expert_offsets, pool_src, route_to_pool, x_pool,
                     q ? x_pool_scale : nullptr, workspace, static_cast<hipStream_t>(stream));
}

mm_status mm_grouped_l1_swiglu(const mm_plan* plan, const int32_t* expert_offsets, const int32_t* expert_counts,
                               const void* x_pool, const void* x_pool_scale, const void* w1, const void* w1_scale,
                               void* a_pool, void* a_pool_scale, void* workspace, uint64_t workspace_bytes,
                               void* stream) {
  MM_TRY(check_plan(plan));
  const bool q = plan->prob.usecase != MM_A16W16;
  if (!ok4(expert_offsets) || !ok4(expert_counts) || !ok16(x_pool) || !ok16(w1) || !ok16(a_pool) ||
      !ok16(workspace))
    return MM_ERR_INVALID_ARG;
  if (q && (!ok4(x_pool_scale) || !ok4(w1_scale) || !ok4(a_pool_scale))) return MM_ERR_INVALID_ARG;
  if ((int64_t)workspace_bytes < plan->workspace_bytes) return MM_ERR_WORKSPACE;
  return do_l1(*plan, expert_offsets, expert_counts, x_pool, x_pool_scale, w1, w1_scale, a_pool, a_pool_scale,
               workspace, static_cast<hipStream_t>(stream));
}

mm_status mm_grouped_l2_combine(const mm_plan* plan, const int32_t* expert_offsets, const int32_t* expert_counts,
                                const int32_t* pool_src, const int32_t* route_to_pool, const void* a_pool,
                                const void* a_pool_scale, const void* w2, const void* w2_scale,
                                const float* topk_weights, void* y, void* workspace, uint64_t workspace_bytes,
                                void* stream) {
  MM_TRY(check_plan(plan));
  const bool q = plan->prob.usecase != MM_A16W16;
  if (!ok4(expert_offsets) || !ok4(expert_counts) || !ok4(pool_src) || !ok4(route_to_pool) || !ok16(a_pool) ||
      !ok16(w2) || !ok4(topk_weights) || !ok16(y) || !ok16(workspace))
    return MM_ERR_INVALID_ARG;
  if (q && (!ok4(a_pool_scale) || !ok4(w2_scale))) return MM_ERR_INVALID_ARG;
  if ((int64_t)workspace_bytes < plan->workspace_bytes) return MM_ERR_WORKSPACE;
  return do_l2(*plan, expert_offsets, expert_counts, pool_src, route_to_pool, a_pool, a_pool_scale, w2, w2_scale,
               topk_weights, y, workspace, static_cast<hipStream_t>(stream));
}

mm_status mega_moe(const mm_plan* plan, const void* x, const int32_t* topk_ids, const float* topk_weights,
                   const int8_t* x_active_mask, const void* w1, const void* w1_scale, const void* w2,
                   const void* w2_scale, void* y, int32_t* expert_token_nums, void* workspace,
                   uint64_t workspace_bytes, void* stream) {
  MM_TRY(check_plan(plan));
  const bool q = plan->prob.usecase != MM_A16W16;
  if (!ok16(x) || !ok4(topk_ids) || !ok4(topk_weights) || !ok16(w1) || !ok16(w2) || !ok16(y) ||
      !ok4(expert_token_nums) || !ok16(workspace))
    return MM_ERR_INVALID_ARG;
  if (q && (!ok4(w1_scale) || !ok4(w2_scale))) return MM_ERR_INVALID_ARG;
  if ((int64_t)workspace_bytes < plan->fused_workspace_bytes) return MM_ERR_WORKSPACE;
  const WsLayout L = ws_layout(*plan);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* counts = at<int32_t>(workspace, L.counts);
  int32_t* offsets = at<int32_t>(workspace, L.offsets);
  int32_t* pool_src = at<int32_t>(workspace, L.pool_src);
  int32_t* r2p = at<int32_t>(workspace, L.route_to_pool);
  void* x_pool = at<uint8_t>(workspace, L.x_pool);
  void* xs = q ? at<uint8_t>(workspace, L.x_pool_scale) : nullptr;
  void* a_pool = at<uint8_t>(workspace, L.a_pool);
  void* as = q ? at<uint8_t>(workspace, L.a_pool_scale) : nullptr;
  const mm_plan& pl = *plan;
  MegaArgs m{};
  m.d = dispatch_args(pl, topk_ids, x_active_mask, x, counts, offsets, pool_src, r2p, x_pool, xs, workspace);
  m.l1 = l1_args(pl, offsets, counts, x_pool, xs, w1, w1_scale, a_pool, as, workspace);
  m.rq = requant_args(pl, m.l1, a_pool, as);
  m.l2 = l2_args(pl, offsets, counts, pool_src, a_pool, as, w2, w2_scale, topk_weights, workspace);
  m.counts_out = expert_token_nums;
  m.cb = combine_args(pl, m.l2.contrib, r2p, y);
  m.ctl = at<uint32_t>(workspace, L.ctl);
  m.nwaves = dispatch_waves(pl.prob.num_tokens, (int)slots_per_token(pl.prob));
  // Linear1 reads the token rows in place (x, or the token codes) through
  // pool_src when the token matrix fits one buffer descriptor
  if (plan_by_token(pl)) {
    m.l1_by_token = 1;
    m.x_tok = q ? at<uint8_t>(workspace, L.x_tok) : nullptr;
    m.x_tok_scale = q ? at<uint8_t>(workspace, L.x_tok_scale) : nullptr;
    m.l1.A = static_cast<const uint8_t*>(q ? m.x_tok : x);
    if (mx_usecase(pl.prob.usecase)) {
      m.l1.a_mx = static_cast<const uint8_t*>(m.x_tok_scale);
      m.l1.a_mx_rows = pl.prob.num_tokens;
    } else {
      m.l1.x_scale = static_cast<const float*>(m.x_tok_scale);
    }
    m.l1.a_route = pool_src;
    m.l1.a_rows = pl.prob.num_tokens;
    // token rows are shared K-fold and stay cached: weight reuse order; with
    // the claimed 256 x 256 tiles, groups of 8 M-blocks (measured: 16K
    // tokens fp8 5.88 vs 5.96 ms, bf16 10.91 vs 10.98 ms; 128 x 256: none)
    m.l1.group_m = group_m_of("MM_GROUP_M1", pl.block_m == 256 ? 8 : 0);
  }
  m.spin_limit = barrier_spin_limit();
  m.dep = at<uint32_t>(workspace, L.dep);
  m.dep_blocks = pl.pool_rows / pl.block_m;
  m.no_dep = plan_dep(pl) ? 0 : 1;
  m.static_tiles = plan_static_tiles(pl) ? 1 : 0;
  MegaArgs* dev_args = at<MegaArgs>(workspace, L.mega_args);
  MM_TRY(run(MM_K_ZERO, s, [&] { return launch_mega_prep(m, dev_args, s); }));
  MM_TRY(run(MM_K_MEGA, s, [&] {
    return launch_mega(pl.prob.usecase, pl.tile_l1, fp8_l1_exact(pl), dev_args, mega_grid(pl.tile_l1, num_cus()),
                       plan_cooperative(pl), s);
  }));
  return MM_OK;
}

mm_status mega_moe_noalloc(const mm_plan* plan, const void* x, const int32_t* topk_ids, const float* topk_weights,
                           const int8_t* x_active_mask, const void* w1, const void* w1_scale, const void* w2,
                           const void* w2_scale, void* y, int32_t* expert_token_nums, void* stream) {
  MM_TRY(check_plan(plan));
  if (plan->fused_workspace_bytes > kScratchBytes) return MM_ERR_WORKSPACE;
  void* ws = nullptr;
  MM_TRY(scratch_of_current_device(&ws));
  return mega_moe(plan, x, topk_ids, topk_weights, x_active_mask, w1, w1_scale, w2, w2_scale, y, expert_token_nums,
                  ws, (uint64_t)kScratchBytes, stream);
}

mm_status mm_read_device_error(const mm_plan* plan, const void* workspace, int32_t* host_out, void* stream) {
  MM_TRY(check_plan(plan));
  if (!workspace) {   // the static scratch of mega_moe_noalloc
    void* ws = nullptr;
    MM_TRY(scratch_of_current_device(&ws));
    workspace = ws;
  }
  if (!ok16(workspace) || !host_out) return MM_ERR_INVALID_ARG;
  const uint8_t* word = static_cast<const uint8_t*>(workspace) + ws_layout(*plan).ctl + 4;
  if (hipMemcpyAsync(host_out, word, 4, hipMemcpyDeviceToHost, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MM_ERR_HIP;
  return MM_OK;
}

mm_status mm_debug_raw_accumulators(const mm_plan* plan, int which, const int32_t* expert_offsets,
                                    const int32_t* expert_counts, const void* act_pool, const void* w_prepared,
                                    int32_t* c_out, void* workspace, uint64_t workspace_bytes, void* stream) {
  MM_TRY(check_plan(plan));
  const mm_problem& p = plan->prob;
  if (p.usecase != MM_A8W8_INT8 && p.usecase != MM_A8W8_FP8) return MM_ERR_UNSUPPORTED;
  if ((which != 1 && which != 2) || !ok4(expert_offsets) || !ok4(expert_counts) || !ok16(act_pool) ||
      !ok16(w_prepared) || !ok4(c_out) || !ok16(workspace))
    return MM_ERR_INVALID_ARG;
  if ((int64_t)workspace_bytes < plan->workspace_bytes) return MM_ERR_WORKSPACE;
  const WsLayout L = ws_layout(*plan);
  GemmArgs g{};
  g.A = static_cast<const uint8_t*>(act_pool);
  g.B = static_cast<const uint8_t*>(w_prepared);
  g.offsets = expert_offsets;
  g.counts = expert_counts;
  g.P = plan->pool_rows;
  g.E = (int)all_experts(p);
  g.I = (int)p.intermediate_hidden;
  g.H = (int)p.hidden;
  g.K = (int)slots_per_token(p);
  g.Kr = (int)p.num_topk;
  g.raw_out = c_out;
  g.err = at<uint32_t>(workspace, L.ctl) + 1;
  set_split(g, *plan, L, workspace);   // tail tiles split along K as in the entry points
  if (which == 1) {
    g.N = (int)(2 * p.intermediate_hidden);
    g.Kdim = (int)p.hidden;
    g.gate_up_group = plan->gate_up_group;
  } else {
    g.N = (int)p.hidden;
    g.Kdim = (int)p.intermediate_hidden;
    g.gate_up_group = 0;
  }
  const int tile = which == 1 ? plan->tile_l1 : plan->tile_l2;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int grid = gemm_grid(tile, plan->pool_rows, g.N, num_cus());
  MM_TRY(clear_split_flags(g, s));
  const bool exact = which == 1 && p.usecase == MM_A8W8_FP8 && fp8_l1_exact(*plan);
  return run(which == 1 ? MM_K_L1 : MM_K_L2, s, [&] { return launch_gemm(2, p.usecase, tile, exact, g, grid, s); });
}

mm_status mm_read_kernel_clock(const mm_plan* plan, const void* workspace, uint64_t* host_out, void* stream) {
  MM_TRY(check_plan(plan));
  if (!ok16(workspace) || !host_out) return MM_ERR_INVALID_ARG;
  const uint8_t* words = static_cast<const uint8_t*>(workspace) + ws_layout(*plan).ctl + kClockWord0 * 4;
  if (hipMemcpyAsync(host_out, words, 32, hipMemcpyDeviceToHost, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MM_ERR_HIP;
  return MM_OK;
}

mm_status mm_debug_fused_layout(const mm_plan* plan, const void* workspace, int32_t* offsets_out,
                                int32_t* pool_src_out, int32_t* route_to_pool_out, void* stream) {
  MM_TRY(check_plan(plan));
  if (!ok4(offsets_out) || !ok4(pool_src_out) || !ok4(route_to_pool_out)) return MM_ERR_INVALID_ARG;
  if (!workspace) {   // the static scratch of mega_moe_noalloc
    void* ws = nullptr;
    MM_TRY(scratch_of_current_device(&ws));
    workspace = ws;
  }
  if (!ok16(workspace)) return MM_ERR_INVALID_ARG;
  const mm_problem& p = plan->prob;
  const WsLayout L = ws_layout(*plan);
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const struct { void* dst; int64_t off, bytes; } parts[3] = {
      {offsets_out, L.offsets, (all_experts(p) + 1) * 4},
      {pool_src_out, L.pool_src, plan->pool_rows * 4},
      {route_to_pool_out, L.route_to_pool, p.num_tokens * slots_per_token(p) * 4}};
  for (const auto& c : parts)
    if (hipMemcpyAsync(c.dst, ws + c.off, (size_t)c.bytes, hipMemcpyDeviceToDevice, s) != hipSuccess) return MM_ERR_HIP;
  return MM_OK;
}

mm_status mm_trace_enable(int on) {
  std::lock_guard<std::mutex> g(g_trace_mu);
  g_trace_on = on != 0;
  return MM_OK;
}

mm_status mm_trace_collect(int32_t* launches, double* total_ms) {
  if (!launches || !total_ms) return MM_ERR_INVALID_ARG;
  std::vector<TraceRec> recs;
  {
    std::lock_guard<std::mutex> g(g_trace_mu);
    recs.swap(g_trace);
  }
  for (int i = 0; i < MM_K_COUNT_IDS; ++i) {
    launches[i] = 0;
    total_ms[i] = 0.0;
  }
  mm_status st = MM_OK;
  for (const TraceRec& r : recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      st = MM_ERR_HIP;
    } else if (r.id >= 0 && r.id < MM_K_COUNT_IDS) {
      launches[r.id] += 1;
      total_ms[r.id] += ms;
    }
  }
  std::lock_guard<std::mutex> g(g_trace_mu);
  for (const TraceRec& r : recs) {
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
  }
  return st;
}

const char* mm_kernel_name(int id) {
  static const char* names[] = {"zero",    "count",   "scatter", "gather", "l1_swiglu",
                                "requant", "l2_gate", "combine", "prepare", "mega"};
  if (id < 0 || id >= MM_K_COUNT_IDS) return "unknown";
  return names[id];
}

const char* mm_status_string(mm_status s) {
  switch (s) {
    case MM_OK: return "ok";
    case MM_ERR_INVALID_ARG: return "invalid argument";
    case MM_ERR_UNSUPPORTED: return "unsupported";
    case MM_ERR_WORKSPACE: return "workspace too small";
    case MM_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

}  // extern "C"
