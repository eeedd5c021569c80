// C ABI of the MoE layer library: argument checks, workspace sizing, the
// order of kernel launches of each call, and the optional kernel timer.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "gemm.h"
#include "kernels.h"

using namespace moe;

// ---------------------------------------------------------------- errors
static thread_local char g_err[512] = "";

namespace moe {
void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

moe_status_t check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

// ---------------------------------------------------------------- timer
namespace {
struct ProfRec {
  std::string name;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_pool;
std::string g_names;
std::vector<std::string> g_select;  // names to record; empty = every kernel

bool selected(const char* name) {
  if (g_select.empty()) return true;
  for (auto& n : g_select)
    if (n == name) return true;
  return false;
}

hipEvent_t pool_get() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

int prof_begin(const char* name, hipStream_t s) {
  if (!g_prof_on) return -1;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!selected(name)) return -1;
  ProfRec r{name, pool_get(), pool_get()};
  if (!r.a || !r.b) return -1;
  (void)hipEventRecord(r.a, s);
  g_recs.push_back(r);
  return (int)g_recs.size() - 1;
}

void prof_end(int tok, hipStream_t s) {
  if (tok < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (tok < (int)g_recs.size()) (void)hipEventRecord(g_recs[tok].b, s);
}
}  // namespace moe

extern "C" moe_status_t moe_prof_enable(int on) {
  g_prof_on = on != 0;
  return MOE_OK;
}

extern "C" moe_status_t moe_prof_select(const char* names) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_select.clear();
  if (!names) return MOE_OK;
  std::string cur;
  for (const char* c = names;; ++c) {
    if (*c == ',' || *c == 0) {
      if (!cur.empty()) g_select.push_back(cur);
      cur.clear();
      if (*c == 0) break;
    } else {
      cur += *c;
    }
  }
  return MOE_OK;
}

extern "C" moe_status_t moe_prof_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_recs) {
    (void)hipEventSynchronize(r.b);
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  return MOE_OK;
}

extern "C" moe_status_t moe_prof_read(const char* name, double* total_ms, int64_t* launches) {
  if (!name || !total_ms || !launches) {
    set_error("moe_prof_read: null argument");
    return MOE_ERR_ARG;
  }
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double tot = 0;
  int64_t n = 0;
  for (auto& r : g_recs) {
    if (r.name != name) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) {
      set_error("moe_prof_read: event wait failed");
      return MOE_ERR_HIP;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      set_error("moe_prof_read: elapsed time failed");
      return MOE_ERR_HIP;
    }
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return MOE_OK;
}

extern "C" const char* moe_prof_names(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_names.clear();
  std::vector<std::string> seen;
  for (auto& r : g_recs) {
    bool dup = false;
    for (auto& s : seen) dup = dup || s == r.name;
    if (dup) continue;
    seen.push_back(r.name);
    if (!g_names.empty()) g_names += ",";
    g_names += r.name;
  }
  return g_names.c_str();
}

// ---------------------------------------------------------------- utility
extern "C" const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_ARG: return "MOE_ERR_ARG";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
    case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
  }
  return "MOE_ERR_UNKNOWN";
}

extern "C" const char* moe_last_error(void) { return g_err; }

extern "C" const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

// ---------------------------------------------------------------- checks
namespace {

#define MOE_TRY(x)                      \
  do {                                  \
    moe_status_t _st = (x);             \
    if (_st != MOE_OK) return _st;      \
  } while (0)

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

struct Dims {
  int T, d, E, k, I, e_lo, e_hi, E_loc, R_cap;
  bool bf16;
  int eb;  // element bytes
  bool balanced;
};

moe_status_t check_shape(const moe_shape_t* s, const char* fn, Dims* o) {
  if (!s) return fail(MOE_ERR_ARG, "%s: shape is NULL", fn);
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return fail(MOE_ERR_DTYPE, "%s: unknown dtype %d", fn, (int)s->dtype);
  if (s->gate != MOE_GATE_SOFTMAX_TOPK && s->gate != MOE_GATE_BALANCED)
    return fail(MOE_ERR_ARG, "%s: unknown gate %d", fn, (int)s->gate);
  if (s->T <= 0 || s->d <= 0 || s->E <= 0 || s->k <= 0 || s->I <= 0)
    return fail(MOE_ERR_SHAPE, "%s: T, d, E, k, I must be positive", fn);
  if (s->k > s->E) return fail(MOE_ERR_ARG, "%s: k=%d > E=%d", fn, s->k, s->E);
  if (s->e_lo < 0 || s->e_hi > s->E || s->e_lo >= s->e_hi)
    return fail(MOE_ERR_ARG, "%s: local experts [%d,%d) not inside [0,%d)", fn, s->e_lo, s->e_hi, s->E);
  const int64_t rows = (int64_t)s->T * s->k;
  if (rows >= ((int64_t)1 << 31)) return fail(MOE_ERR_SHAPE, "%s: T*k overflows int32", fn);
  if (s->R_cap < 0 || s->R_cap > rows) return fail(MOE_ERR_SHAPE, "%s: R_cap=%d outside [0, T*k]", fn, s->R_cap);
  if (s->gate == MOE_GATE_BALANCED && s->E % s->k)
    return fail(MOE_ERR_ARG, "%s: the balanced gate needs k | E", fn);
  if (s->d % 64 || s->I % 64) return fail(MOE_ERR_UNSUPPORTED, "%s: d and I must be multiples of 64", fn);
  if (s->E > 512) return fail(MOE_ERR_UNSUPPORTED, "%s: E > 512", fn);
  if (s->dtype == MOE_BF16 && s->E % 8) return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 needs E %% 8 == 0", fn);
  if (s->k > 32) return fail(MOE_ERR_UNSUPPORTED, "%s: k > 32", fn);
  if ((int64_t)s->R_cap * 2 * s->I >= ((int64_t)1 << 40) || (int64_t)rows * s->d >= ((int64_t)1 << 40))
    return fail(MOE_ERR_SHAPE, "%s: buffers too large", fn);
  o->T = s->T; o->d = s->d; o->E = s->E; o->k = s->k; o->I = s->I;
  o->e_lo = s->e_lo; o->e_hi = s->e_hi; o->E_loc = s->e_hi - s->e_lo;
  o->R_cap = s->R_cap ? s->R_cap : (int)rows;
  o->bf16 = s->dtype == MOE_BF16;
  o->eb = o->bf16 ? 2 : 4;
  o->balanced = s->gate == MOE_GATE_BALANCED;
  return MOE_OK;
}

// Every listed pointer must be non-NULL and 16-byte aligned.
moe_status_t need(const char* fn, std::initializer_list<std::pair<const char*, const void*>> ptrs) {
  for (auto& p : ptrs) {
    if (!p.second) return fail(MOE_ERR_ARG, "%s: %s is NULL", fn, p.first);
    if ((uintptr_t)p.second & 15) return fail(MOE_ERR_UNSUPPORTED, "%s: %s is not 16-byte aligned", fn, p.first);
  }
  return MOE_OK;
}

// Optional pointers: NULL allowed, else 16-byte aligned.
moe_status_t opt(const char* fn, std::initializer_list<std::pair<const char*, const void*>> ptrs) {
  for (auto& p : ptrs)
    if (p.second && ((uintptr_t)p.second & 15))
      return fail(MOE_ERR_UNSUPPORTED, "%s: %s is not 16-byte aligned", fn, p.first);
  return MOE_OK;
}

// Tile tables of the row-grouped GEMMs: one for 256-row and one for 128-row
// tiles, each (1 + 2 * (R_cap / BM + E_loc)) int32.
int64_t one_table_bytes(const Dims& D, int bm) {
  return round_up((1 + 2 * ((int64_t)D.R_cap / bm + D.E_loc)) * 4, 256);
}
int64_t kcost_bytes(const Dims& D) { return round_up((int64_t)(D.E_loc + 1) * 4, 256); }
int64_t tok_bytes(const Dims& D) { return round_up((int64_t)D.R_cap * 4, 256); }
// moe_combine_ffn_bwd_gather (bf16): the gate gradient's shares from the
// dSwiGLU GEMM, fp32 [R_cap][I / 32].
int64_t gate_part_bytes(const Dims& D) { return round_up((int64_t)D.R_cap * (D.I / 32) * 4, 256); }
int64_t tile_table_bytes(const Dims& D) {
  return one_table_bytes(D, 256) + one_table_bytes(D, 128) + kcost_bytes(D) + tok_bytes(D);
}
int max_m_tiles(const Dims& D, int bm) { return D.R_cap / bm + D.E_loc; }

// Builds the tile tables a call needs, once each, in its workspace.
// With perm (the gathered calls) also the token row of every routed row.
struct TileTables {
  const Dims& D;
  int32_t* base;
  const int32_t* off;
  hipStream_t s;
  const int32_t* perm = nullptr;
  const CombinePrep* cmb = nullptr;  // the fused combine's preparation, in the same launch
  bool built = false;
  int32_t* t256() const { return base; }
  int32_t* t128() const { return base + one_table_bytes(D, 256) / 4; }
  int32_t* kcost() const { return t128() + one_table_bytes(D, 128) / 4; }
  int32_t* tok() const { return kcost() + kcost_bytes(D) / 4; }
  moe_status_t ensure() {  // all tables in one launch, on first use
    if (!built) {
      MOE_TRY(launch_tile_tables(off, D.E_loc, t256(), t128(), kcost(), s, perm, D.k, tok(),
                                 D.R_cap, cmb));
      built = true;
    }
    return MOE_OK;
  }
  // A rows of a gather role: the token table (bf16 kernels) or perm with k (fp32)
  moe_status_t rows(GemmParams* p) {
    if (D.bf16) {
      MOE_TRY(ensure());
      p->a_rows = tok();
      p->a_rows_div = 1;
    } else {
      p->a_rows = perm;
      p->a_rows_div = D.k;
    }
    return MOE_OK;
  }
  moe_status_t get(GemmRole role, const int32_t** out) {
    MOE_TRY(ensure());
    *out = tile_bm(role_tile(role)) == 256 ? t256() : t128();
    return MOE_OK;
  }
};

// Router-backward workspace: the bf16 copy of dL (bf16 layers), per-workgroup
// column sums of dL, and the split-K partials of x^T dL (bf16 layers).
struct RouteBwdWs {
  int64_t dl16 = 0, dbp = 0, dwp = 0, total = 0;
  int nblk = 0, nsplit = 0, k_chunk = 0;
  explicit RouteBwdWs(const Dims& D) {
    nblk = (int)ceil_div(D.T, ROUTE_BWD_TOKENS);
    if (D.bf16) {
      // about 512 token rows per split, at most 16 splits, whole 64-row K slices
      nsplit = (int)std::min<int64_t>(16, std::max<int64_t>(1, ceil_div(D.T, 512)));
      k_chunk = (int)round_up(ceil_div(D.T, nsplit), 64);
      nsplit = (int)ceil_div(D.T, k_chunk);
    }
    const int64_t a = D.bf16 ? round_up((int64_t)D.T * D.E * 2, 256) : 0;
    const int64_t b = round_up((int64_t)nblk * D.E * 4, 256);
    const int64_t c = D.bf16 ? round_up((int64_t)nsplit * D.d * D.E * 4, 256) : 0;
    dl16 = 0;
    dbp = a;
    dwp = a + b;
    total = a + b + c;
  }
};

// The few-token router's partial logits (softmax top-k gate, T small enough),
// then the small-batch FFN's workspace.
bool small_router_used(const Dims& D) { return !D.balanced && D.T <= SMALL_ROUTE_MAX_T; }
int64_t small_routed_ws_bytes(const Dims& D) {
  return (small_router_used(D) ? small_router_ws_bytes(D.T, D.d, D.E) : 0) +
         round_up(small_ffn_ws_bytes(D.T, D.d, D.k, D.I, D.e_lo, D.e_hi, D.eb), 256);
}

// The fused combine's workspace after the tile tables: kept slots per token
// [T] and the arrival counters [T][d/64].
int64_t fused_kept_bytes(const Dims& D) { return round_up((int64_t)D.T * 4, 256); }
int64_t fused_cnt_bytes(const Dims& D) { return round_up((int64_t)D.T * (D.d / 64) * 4, 256); }

int64_t ws_bytes(const Dims& D, int op) {
  switch (op) {
    case MOE_OP_SMALL_ROUTED_FWD:
      return small_routed_ws_bytes(D);
    case MOE_OP_ROUTE_PERMUTE:
      return D.balanced ? 0 : round_up(permute_ws_bytes(D.T, D.E_loc), 256);
    case MOE_OP_FFN_FWD_FUSED:
      return D.bf16 ? tile_table_bytes(D) + fused_kept_bytes(D) + fused_cnt_bytes(D) : 0;
    case MOE_OP_PERMUTE: return round_up(permute_ws_bytes(D.T, D.E_loc), 256);
    case MOE_OP_FFN_FWD: return D.bf16 ? tile_table_bytes(D) : 0;
    case MOE_OP_FFN_BWD:
      return round_up((int64_t)D.R_cap * 2 * D.I * D.eb, 256) +
             (D.bf16 ? tile_table_bytes(D) + gate_part_bytes(D) : 0);
    case MOE_OP_SMALL_FWD: return small_ffn_ws_bytes(D.T, D.d, D.k, D.I, D.e_lo, D.e_hi, D.eb);
    case MOE_OP_AUX_LOSS: return D.balanced ? 0 : aux_loss_ws_bytes(D.T, D.E);
    case MOE_OP_CHECK_ROUTING: return round_up((int64_t)D.E_loc * 4, 256);
    case MOE_OP_ROUTE_BWD: {
      if (D.balanced) return 0;
      const RouteBwdWs r(D);
      return r.total;
    }
    default: return 0;
  }
}

moe_status_t check_ws(const char* fn, const Dims& D, int op, const void* ws, size_t bytes) {
  int64_t want = ws_bytes(D, op);
  if (want == 0) return MOE_OK;
  if (!ws || (int64_t)bytes < want)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %lld bytes needed, %zu given", fn, (long long)want, bytes);
  if ((uintptr_t)ws & 255) return fail(MOE_ERR_UNSUPPORTED, "%s: workspace must be 256-byte aligned", fn);
  return MOE_OK;
}

hipStream_t S(moe_stream_t s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" moe_status_t moe_workspace_size(const moe_shape_t* shape, int op, size_t* bytes) {
  Dims D;
  if (!bytes) return fail(MOE_ERR_ARG, "moe_workspace_size: bytes is NULL");
  MOE_TRY(check_shape(shape, "moe_workspace_size", &D));
  if (op < MOE_OP_ROUTE || op > MOE_OP_CHECK_ROUTING)
    return fail(MOE_ERR_ARG, "moe_workspace_size: unknown op %d", op);
  *bytes = (size_t)ws_bytes(D, op);
  return MOE_OK;
}

// ---------------------------------------------------------------- forward
extern "C" moe_status_t moe_route(const moe_shape_t* shape, const void* x, const void* w_router,
                                  const float* bias, float* logits, int32_t* topk_idx, float* topk_w,
                                  moe_stream_t stream) {
  const char* fn = "moe_route";
  Dims D;
  MOE_TRY(check_shape(shape, fn, &D));
  MOE_TRY(need(fn, {{"topk_idx", topk_idx}, {"topk_w", topk_w}}));
  if (D.balanced) return launch_balanced_gate(D.T, D.E, D.k, topk_idx, topk_w, S(stream));
  MOE_TRY(need(fn, {{"x", x}, {"w_router", w_router}, {"logits", logits}}));
  MOE_TRY(opt(fn, {{"bias", bias}}));
  if (few_token_logits_fit(D.T, D.E, D.eb)) {
    MOE_TRY(launch_few_token_logits(x, w_router, bias, D.T, D.d, D.E, D.eb, logits, S(stream)));
    return launch_topk_softmax(logits, D.T, D.E, D.k, topk_idx, topk_w, S(stream));
  }
  GemmParams p{};
  p.A = x; p.lda = D.d;
  p.B0 = w_router; p.ldb = D.E;
  p.M = D.T; p.N = D.E; p.K = D.d;
  p.m_tiles = (int)ceil_div(D.T, 64); p.n_tiles = (int)ceil_div(D.E, 64);
  p.groups = 1;
  p.C0 = logits; p.ldc = D.E; p.bias = bias;
  MOE_TRY(launch_gemm(D.bf16, R_ROUTE_LOGITS, p, p.m_tiles, S(stream)));
  return launch_topk_softmax(logits, D.T, D.E, D.k, topk_idx, topk_w, S(stream));
}

extern "C" moe_status_t moe_permute(const moe_shape_t* shape, const int32_t* topk_idx, const void* x,
                                    int32_t* group_offsets, int32_t* perm, int32_t* inv, void* xp,
                                    void* ws, size_t ws_bytes_, moe_stream_t stream) {
  const char* fn = "moe_permute";
  Dims D;
  MOE_TRY(check_shape(shape, fn, &D));
  MOE_TRY(need(fn, {{"topk_idx", topk_idx}, {"group_offsets", group_offsets}, {"perm", perm},
                    {"inv", inv}}));
  if (xp) MOE_TRY(need(fn, {{"x", x}, {"xp", xp}}));
  MOE_TRY(check_ws(fn, D, MOE_OP_PERMUTE, ws, ws_bytes_));
  return launch_permute(topk_idx, x, D.T, D.d, D.k, D.e_lo, D.e_hi, D.R_cap, D.eb, group_offsets,
                        perm, inv, xp, ws, S(stream));
}

extern "C" moe_status_t moe_route_permute(const moe_shape_t* shape, const void* x,
                                          const void* w_router, const float* bias, float* logits,
                                          int32_t* topk_idx, float* topk_w,
                                          int32_t* group_offsets, int32_t* perm, int32_t* inv,
                                          void* xp, void* ws, size_t ws_bytes_,
                                          moe_stream_t stream) {
  const char* fn = "moe_route_permute";
  Dims D;
  MOE_TRY(check_shape(shape, fn, &D));
  MOE_TRY(need(fn, {{"topk_idx", topk_idx}, {"topk_w", topk_w}, {"group_offsets", group_offsets},
                    {"perm", perm}, {"inv", inv}}));
  if (xp) MOE_TRY(need(fn, {{"x", x}, {"xp", xp}}));
  if (!D.balanced) {  // the router, then the sort
    MOE_TRY(need(fn, {{"x", x}, {"w_router", w_router}, {"logits", logits}}));
    MOE_TRY(opt(fn, {{"bias", bias}}));
    MOE_TRY(check_ws(fn, D, MOE_OP_ROUTE_PERMUTE, ws, ws_bytes_));
    MOE_TRY(moe_route(shape, x, w_router, bias, logits, topk_idx, topk_w, stream));
    return launch_permute(topk_idx, x, D.T, D.d, D.k, D.e_lo, D.e_hi, D.R_cap, D.eb,
                          group_offsets, perm, inv, xp, ws, S(stream));
  }
  MOE_TRY(launch_balanced_route_permute(D.T, D.E, D.k, D.e_lo, D.e_hi, D.R_cap, topk_idx, topk_w,
                                        group_offsets, perm, inv, S(stream)));
  if (xp) return launch_permute_gather(x, inv, D.T, D.d, D.k, D.eb, xp, S(stream));
  return MOE_OK;
}

extern "C" moe_status_t moe_check_routing(const moe_shape_t* shape, const int32_t* topk_idx,
                                          const int32_t* group_offsets, int32_t* flags, void* ws,
                                          size_t ws_bytes_, moe_stream_t stream) {
  const char* fn = "moe_check_routing";
  Dims D;
  MOE_TRY(check_shape(shape, fn, &D));
  MOE_TRY(need(fn, {{"topk_idx", topk_idx}, {"flags", flags}}));
  if (group_offsets) MOE_TRY(check_ws(fn, D, MOE_OP_CHECK_ROUTING, ws, ws_bytes_));
  return launch_check_routing(topk_idx, D.T, D.k, D.E, D.e_lo, D.e_hi, D.R_cap, group_offsets,
                              static_cast<int32_t*>(ws), flags, S(stream));
}

namespace {

// The gathered forms read row p of Xp as row perm[p] / k of x; their A byte
// offsets are 32-bit.
moe_status_t check_gather(const char* fn, const Dims& D) {
  if ((int64_t)D.T * D.d * D.eb >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "%s: x of %lld bytes; the gathered form needs < 2^31", fn,
                (long long)D.T * D.d * D.eb);
  return MOE_OK;
}

// The fused combine's arguments (moe_grouped_ffn_fwd_fused).
struct FusedCombine {
  const int32_t* inv;
  const float* topk_w;
  void* y;
};

// Forward FFN over Xp rows: xp itself, or (gather) x read through perm; with
// fc, the combine runs in the down projection's epilogue (bf16) or right after
// it (fp32).
moe_status_t ffn_fwd(const char* fn, bool gather, const moe_shape_t* shape, const void* a_src,
                     const int32_t* perm, const int32_t* group_offsets, const void* w_gate,
                     const void* w_up, const void* w_down, void* h_save, void* a_save, void* yp,
                     void* ws, size_t ws_bytes_, moe_stream_t stream,
                     const FusedCombine* fc = nullptr) {
  Dims D;
  MOE_TRY(check_shape(shape, fn, &D));
  if (fc) {
    MOE_TRY(need(fn, {{"inv", fc->inv}, {"topk_w", fc->topk_w}, {"y", fc->y}}));
    if ((int64_t)D.R_cap * D.d * D.eb >= ((int64_t)1 << 31))
      return fail(MOE_ERR_UNSUPPORTED, "%s: yp of %lld bytes; the fused combine needs < 2^31", fn,
                  (long long)D.R_cap * D.d * D.eb);
  }
  MOE_TRY(need(fn, {{gather ? "x" : "xp", a_src}, {"group_offsets", group_offsets},
                    {"w_gate", w_gate}, {"w_up", w_up}, {"w_down", w_down}, {"a_save", a_save}, {"yp", yp}}));
  if (!gather) perm = nullptr;
  if (gather) {
    MOE_TRY(need(fn, {{"perm", perm}}));
    MOE_TRY(check_gather(fn, D));
  }
  MOE_TRY(opt(fn, {{"h_save", h_save}}));
  MOE_TRY(check_ws(fn, D, fc ? MOE_OP_FFN_FWD_FUSED : MOE_OP_FFN_FWD, ws, ws_bytes_));
  TileTables tt{D, static_cast<int32_t*>(ws), group_offsets, S(stream), perm};
  CombinePrep prep{};
  const bool fuse = fc && D.bf16;
  if (fuse) {
    char* base = static_cast<char*>(ws) + tile_table_bytes(D);
    prep.inv = fc->inv;
    prep.T = D.T;
    prep.k = D.k;
    prep.kept = reinterpret_cast<int32_t*>(base);
    prep.cnt = reinterpret_cast<int32_t*>(base + fused_kept_bytes(D));
    prep.ncb = D.d / 64;
    prep.y = fc->y;
    prep.y_row_bytes = D.d * D.eb;
    tt.cmb = &prep;
  }
  // fp32: the row count; bf16: the most M tiles the tile table can hold
  auto rows_or_tiles = [&](GemmRole r) { return D.bf16 ? max_m_tiles(D, tile_bm(role_tile(r))) : D.R_cap; };

  const GemmRole gu = perm ? R_GATEUP_FWD_GATHER : R_GATEUP_FWD;
  GemmParams g{};
  g.A = a_src; g.lda = D.d;
  if (perm) MOE_TRY(tt.rows(&g));
  g.B0 = w_gate; g.B1 = w_up; g.ldb = D.I; g.b_estride = (int64_t)D.d * D.I;
  g.N = D.I; g.K = D.d;
  g.off = group_offsets; g.groups = D.E_loc;
  g.n_tiles = (int)ceil_div(D.I, tile_bn(role_tile(gu)) / 2);
  g.C0 = h_save; g.C2 = a_save; g.I = D.I;
  if (D.bf16) MOE_TRY(tt.get(gu, &g.tiles));
  MOE_TRY(launch_gemm(D.bf16, gu, g, rows_or_tiles(gu), S(stream)));

  const GemmRole dr = fuse ? R_DOWN_FWD_COMBINE : R_DOWN_FWD;
  GemmParams p{};
  p.A = a_save; p.lda = D.I;
  p.B0 = w_down; p.ldb = D.d; p.b_estride = (int64_t)D.I * D.d;
  p.N = D.d; p.K = D.I;
  p.off = group_offsets; p.groups = D.E_loc;
  p.n_tiles = (int)ceil_div(D.d, tile_bn(role_tile(dr)));
  p.C0 = yp; p.ldc = D.d;
  if (D.bf16) MOE_TRY(tt.get(dr, &p.tiles));
  if (fuse) {
    MOE_TRY(tt.ensure());  // built above with the gate/up GEMM's table; here for clarity
    p.cmb_tok = tt.tok();
    p.cmb_inv = fc->inv;
    p.cmb_w = fc->topk_w;
    p.cmb_kept = prep.kept;
    p.cmb_cnt = prep.cnt;
    p.cmb_y = fc->y;
    p.cmb_k = D.k;
  }
  MOE_TRY(launch_gemm(D.bf16, dr, p, rows_or_tiles(dr), S(stream)));
  if (fc && !fuse)  // fp32 layers: the combine kernel after the GEMM
    return launch_gather_sum(yp, fc->inv, fc->topk_w, D.T, D.d, D.k, D.eb, fc->y, S(stream),
                             "combine");
  return MOE_OK;
}

}  // namespace

extern "C" moe_status_t moe_grouped_ffn_fwd(const moe_shape_t* shape, const void* xp,
                                            const int32_t* group_offsets, const void* w_gate,
                                            const void* w_up, const void* w_down, void* h_save,
                                            void* a_save, void* yp, void* ws, size_t ws_bytes_,
                                            moe_stream_t stream) {
  return ffn_fwd("moe_grouped_ffn_fwd", false, shape, xp, nullptr, group_offsets, w_gate, w_up,
                 w_down, h_save, a_save, yp, ws, ws_bytes_, stream);
}

extern "C" moe_status_t moe_grouped_ffn_fwd_gather(const moe_shape_t* shape, const void* x,
                                                   const int32_t* perm,
                                                   const int32_t* group_offsets,
                                                   const void* w_gate, const void* w_up,
                                                   const void* w_down, void* h_save, void* a_save,
                                                   void* yp, void* ws, size_t ws_bytes_,
                                                   moe_stream_t stream) {
  return ffn_fwd("moe_grouped_ffn_fwd_gather", true, shape, x, perm, group_offsets, w_gate, w_up,
                 w_down, h_save, a_save, yp, ws, ws_bytes_, stream);
}

// ---------------------------------------------------------------- no allocation
// The gathered FFN forward for callers that cannot allocate (code under
// HIP-graph capture, serving loops, harnesses that forbid allocation): its
// tile tables and token table live in this file-scope device array instead
// of a caller workspace.  Each device holds its own copy until the process
// ends; host code reaches it only through the address hipGetSymbolAddress
// returns for the current device (the array's name on the host is a
// host-side stand-in, not a device address).
constexpr int64_t MOE_NOALLOC_SCRATCH_BYTES = (int64_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MOE_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[MOE_MAX_DEVICES] = {};

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
moe_status_t noalloc_scratch(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= MOE_MAX_DEVICES)
    return fail(MOE_ERR_UNSUPPORTED, "%s: device %d beyond the %d this library tracks", fn, dev,
                MOE_MAX_DEVICES);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(MOE_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}
}  // namespace

extern "C" moe_status_t moe_grouped_ffn_fwd_gather_noalloc(
    const moe_shape_t* shape, const void* x, const int32_t* perm, const int32_t* group_offsets,
    const void* w_gate, const void* w_up, const void* w_down, void* h_save, void* a_save, void* yp,
    moe_stream_t stream) {
  const char* fn = "moe_grouped_ffn_fwd_gather_noalloc";
  Dims D;
  MOE_TRY(check_shape(shape, fn, &D));
  const int64_t want = ws_bytes(D, MOE_OP_FFN_FWD);
  if (want > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_UNSUPPORTED,
                "%s: this shape needs %lld bytes of scratch; the static scratch holds %lld "
                "(use moe_grouped_ffn_fwd_gather with a workspace)",
                fn, (long long)want, (long long)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  MOE_TRY(noalloc_scratch(fn, &ws));
  return ffn_fwd(fn, true, shape, x, perm, group_offsets, w_gate, w_up, w_down, h_save, a_save, yp,
                 ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" moe_status_t moe_grouped_ffn_fwd_fused(const moe_shape_t* shape, const void* x,
                                                  const int32_t* perm, const int32_t* inv,
                                                  const float* topk_w,
                                                  const int32_t* group_offsets,
                                                  const void* w_gate, const void* w_up,
                                                  const void* w_down, void* h_save, void* a_save,
                                                  void* yp, void* y, void* ws, size_t ws_bytes_,
                                                  moe_stream_t stream) {
  const FusedCombine fc{inv, topk_w, y};
  return ffn_fwd("moe_grouped_ffn_fwd_fused", true, shape, x, perm, group_offsets, w_gate, w_up,
                 w_down, h_save, a_save, yp, ws, ws_bytes_, stream, &fc);
}

namespace {
// Shapes the small-batch FFN takes.
moe_status_t check_small(const char* fn, const Dims& D) {
  if ((int64_t)D.T * D.k > SMALL_MAX_PAIRS)
    return fail(MOE_ERR_UNSUPPORTED, "%s: T*k = %lld > %lld (use the grouped FFN)", fn,
                (long long)D.T * D.k, (long long)SMALL_MAX_PAIRS);
  if (D.d > SMALL_MAX_WIDTH || D.I > SMALL_MAX_WIDTH)
    return fail(MOE_ERR_UNSUPPORTED, "%s: d and I must be <= %d", fn, SMALL_MAX_WIDTH);
  if (D.R_cap != D.T * D.k)
    return fail(MOE_ERR_UNSUPPORTED, "%s: no row capacity (R_cap must be 0 or T*k)", fn);
  return MOE_OK;
}
}  // namespace

extern "C" moe_status_t moe_ffn_small_fwd(const moe_shape_t* shape, const void* x,
                                          const int32_t* topk_idx, const float* topk_w,
                                          const void* w_gate, const void* w_up,
                                          const void* w_down, void* y, void* ws,
                                          size_t ws_bytes_, moe_stream_t stream) {
  const char* fn = "moe_ffn_small_fwd";
  Dims D;
  MOE_TRY(check_shape(shape, fn, &D));
  MOE_TRY(need(fn, {{"x", x}, {"topk_idx", topk_idx}, {"topk_w", topk_w}, {"w_gate", w_gate},
                    {"w_up", w_up}, {"w_down", w_down}, {"y", y}}));
  MOE_TRY(check_small(fn, D));
  MOE_TRY(check_ws(fn, D, MOE_OP_SMALL_FWD, ws, ws_bytes_));
  return launch_small_ffn(x, topk_idx, topk_w, w_gate, w_up, w_down, D.T, D.d, D.k, D.I, D.e_lo,
                          D.e_hi, D.eb, y, ws, S(stream));
}

extern "C" moe_status_t moe_small_fwd(const moe_shape_t* shape, const void* x,
                                      const void* w_router, const float* bias, float* logits,
                                      int32_t* topk_idx, float* topk_w, const void* w_gate,
                                      const void* w_up, const void* w_down, void* y, void* ws,
                                      size_t ws_bytes_, moe_stream_t stream) {
  const char* fn = "moe_small_fwd";
  Dims D;
  MOE_TRY(check_shape(shape, fn, &D));
  MOE_TRY(need(fn, {{"x", x}, {"topk_idx", topk_idx}, {"topk_w", topk_w}, {"w_gate", w_gate},
                    {"w_up", w_up}, {"w_down", w_down}, {"y", y}}));
  if (!D.balanced) {
    MOE_TRY(need(fn, {{"w_router", w_router}, {"logits", logits}}));
    MOE_TRY(opt(fn, {{"bias", bias}}));
  }
  MOE_TRY(check_small(fn, D));
  MOE_TRY(check_ws(fn, D, MOE_OP_SMALL_ROUTED_FWD, ws, ws_bytes_));
  char* wsb = static_cast<char*>(ws);
  hipStream_t s = S(stream);
  int64_t ffn_at = 0;
  if (D.balanced) {
    MOE_TRY(launch_balanced_gate(D.T, D.E, D.k, topk_idx, topk_w, s));
  } else if (small_router_used(D)) {
    float* rpart = reinterpret_cast<float*>(wsb);
    const int nsplit = D.d / SMALL_ROUTE_KC;
    ffn_at = small_router_ws_bytes(D.T, D.d, D.E);
    if ((int64_t)D.T * D.E <= SMALL_FUSED_ROUTE_MAX_TE &&
        (int64_t)D.T * D.E * nsplit <= SMALL_FUSED_ROUTE_MAX) {
      // the top-k runs inside the FFN's first kernel: one launch less
      MOE_TRY(launch_small_router_part(x, w_router, D.T, D.d, D.E, D.eb, rpart, s));
      const SmallRoute r{rpart, bias, nsplit, D.E, logits, topk_idx, topk_w};
      return launch_small_ffn(x, topk_idx, topk_w, w_gate, w_up, w_down, D.T, D.d, D.k, D.I,
                              D.e_lo, D.e_hi, D.eb, y, wsb + ffn_at, s, &r);
    }
    if (few_token_logits_fit(D.T, D.E, D.eb)) {  // moe_route's few-token logits and top-k
      MOE_TRY(launch_few_token_logits(x, w_router, bias, D.T, D.d, D.E, D.eb, logits, s));
      MOE_TRY(launch_topk_softmax(logits, D.T, D.E, D.k, topk_idx, topk_w, s));
    } else {
      MOE_TRY(launch_small_router(x, w_router, bias, D.T, D.d, D.E, D.k, D.eb, logits, topk_idx,
                                  topk_w, rpart, s));
    }
  } else {
    MOE_TRY(moe_route(shape, x, w_router, bias, logits, topk_idx, topk_w, stream));
  }
  return launch_small_ffn(x, topk_idx, topk_w, w_gate, w_up, w_down, D.T, D.d, D.k, D.I, D.e_lo,
                          D.e_hi, D.eb, y, wsb + ffn_at, s);
}

extern "C" moe_status_t moe_combine(const moe_shape_t* shape, const void* yp, const int32_t* inv,
                                    const float* topk_w, void* y, moe_stream_t stream) {
  const char* fn = "moe_combine";
  Dims D;
  MOE_TRY(check_shape(shape, fn, &D));
  MOE_TRY(need(fn, {{"yp", yp}, {"inv", inv}, {"topk_w", topk_w}, {"y", y}}));
  return launch_gather_sum(yp, inv, topk_w, D.T, D.d, D.k, D.eb, y, S(stream), "combine");
}

// ---------------------------------------------------------------- backward
extern "C" moe_status_t moe_combine_bwd(const moe_shape_t* shape, const void* dy, const void* yp,
                                        const int32_t* inv, const float* topk_w, void* dyp,
                                        float* dtopk_w, moe_stream_t stream) {
  const char* fn = "moe_combine_bwd";
  Dims D;
  MOE_TRY(check_shape(shape, fn, &D));
  MOE_TRY(need(fn, {{"dy", dy}, {"yp", yp}, {"inv", inv}, {"topk_w", topk_w}, {"dyp", dyp},
                    {"dtopk_w", dtopk_w}}));
  return launch_combine_bwd(dy, yp, inv, topk_w, D.T, D.d, D.k, D.eb, dyp, dtopk_w, S(stream));
}

namespace {

// The combine backward run inside the gathered FFN backward
// (moe_combine_ffn_bwd_gather): after the tile-table launch, so that dyp is
// written only when a kernel reads it; where it is not, the kernels form the
// rows g * dY[t] of dYp from dY through the token table.
struct DyForm {
  const void* dy;
  const void* yp;
  const int32_t* inv;
  const float* topk_w;
  float* dtopk_w;
};

// Backward FFN over Xp rows: xp itself, or (gather) x read through perm.
moe_status_t ffn_bwd(const char* fn, bool gather, const moe_shape_t* shape, const void* xp,
                     const int32_t* perm, const int32_t* group_offsets, const void* w_gate,
                     const void* w_up, const void* w_down, const void* h_save,
                     const void* a_save, const void* dyp, void* dxp, void* dw_gate, void* dw_up,
                     void* dw_down, void* ws, size_t ws_bytes_, moe_stream_t stream,
                     const DyForm* dyf = nullptr) {
  Dims D;
  MOE_TRY(check_shape(shape, fn, &D));
  if (!gather) perm = nullptr;
  if (gather) {
    MOE_TRY(need(fn, {{"perm", perm}}));
    MOE_TRY(check_gather(fn, D));
  }
  if (dyf)
    MOE_TRY(need(fn, {{"dy", dyf->dy}, {"yp", dyf->yp}, {"inv", dyf->inv},
                      {"topk_w", dyf->topk_w}, {"dtopk_w", dyf->dtopk_w}}));
  MOE_TRY(need(fn, {{gather ? "x" : "xp", xp}, {"group_offsets", group_offsets},
                    {"w_gate", w_gate}, {"w_up", w_up}, {"w_down", w_down}, {"h_save", h_save}, {"a_save", a_save},
                    {"dyp", dyp}, {"dxp", dxp}, {"dw_gate", dw_gate}, {"dw_up", dw_up},
                    {"dw_down", dw_down}}));
  MOE_TRY(check_ws(fn, D, MOE_OP_FFN_BWD, ws, ws_bytes_));
  char* wsb = static_cast<char*>(ws);
  void* dH = wsb;
  hipStream_t s = S(stream);
  TileTables tt{D, reinterpret_cast<int32_t*>(wsb + round_up((int64_t)D.R_cap * 2 * D.I * D.eb, 256)),
                group_offsets, s, perm};
  auto rows_or_tiles = [&](GemmRole r) { return D.bf16 ? max_m_tiles(D, tile_bm(role_tile(r))) : D.R_cap; };

  // Order: the weight gradient of the down projection and the dSwiGLU GEMM
  // read dYp while it is fresh in the memory-side cache, the gate/up weight
  // gradient reads dH right after it is written, and dXp is written last, so
  // that the permute backward that follows reads it back from that cache.
  if (D.bf16) MOE_TRY(tt.ensure());
  // the bf16 kernels on g * dY[t] (dy_k); the fp32 path reads dYp throughout
  const bool dy_k = dyf && D.bf16;
  // the gate gradient's shares (dy_k, while no expert has more than STRIP_K rows)
  float* dg_part = reinterpret_cast<float*>(
      wsb + round_up((int64_t)D.R_cap * 2 * D.I * D.eb, 256) + (D.bf16 ? tile_table_bytes(D) : 0));
  if (dyf) {
    // a6 (dYp and the gate gradient) only when the weight gradients' tile
    // kernels have work (kcost[groups] > 0: some expert has more than STRIP_K
    // rows), and always in fp32; else the dSwiGLU GEMM yields the gate
    // gradient and no kernel reads dYp
    MOE_TRY(launch_combine_bwd(dyf->dy, dyf->yp, dyf->inv, dyf->topk_w, D.T, D.d, D.k, D.eb,
                               const_cast<void*>(dyp), dyf->dtopk_w, s,
                               dy_k ? tt.kcost() + D.E_loc : nullptr));
  }
  {  // a8: dWd[e] = A_e^T dYp_e
    GemmParams p{};
    p.A = a_save; p.lda = D.I;
    p.B0 = dyp; p.ldb = D.d;
    p.M = D.I; p.N = D.d;
    p.off = group_offsets; p.groups = D.E_loc;
    const TileCfg t = role_tile(R_DOWN_WGRAD);
    p.m_tiles = (int)ceil_div(D.I, tile_bm(t)); p.n_tiles = (int)ceil_div(D.d, tile_bn(t));
    p.C0 = dw_down; p.ldc = D.d; p.c_estride = (int64_t)D.I * D.d;
    if (D.bf16) p.kcost = tt.kcost();
    if (dy_k) {  // the strip kernel reads g * dY[t]; the tile kernel dYp
      p.B0 = dyf->dy;
      MOE_TRY(tt.rows(&p));
      p.row_gate = dyf->topk_w;
      p.row_slot = perm;
      MOE_TRY(launch_down_wgrad_dy(p, dyp, p.m_tiles, s));
    } else {
      MOE_TRY(launch_gemm(D.bf16, R_DOWN_WGRAD, p, p.m_tiles, s));
    }
  }
  {  // a7: dA = dYp Wd^T with the dSwiGLU epilogue -> dH = [dHg | dHu]
    const GemmRole r = dy_k ? R_DOWN_DGRAD_GATHER : R_DOWN_DGRAD;
    GemmParams p{};
    p.A = dyp; p.lda = D.d;
    if (dy_k) {  // dA = g * (dY[t] Wd^T), or dYp Wd^T where dYp was written
      p.A = dyf->dy;
      MOE_TRY(tt.rows(&p));
      p.row_gate = dyf->topk_w;
      p.row_slot = perm;
      p.a_alt = dyp;
      p.kcost = tt.kcost();
      p.dg_part = dg_part;
      p.dg_stride = D.I / 32;
    }
    p.B0 = w_down; p.ldb = D.d; p.b_estride = (int64_t)D.I * D.d;
    p.N = D.I; p.K = D.d;
    p.off = group_offsets; p.groups = D.E_loc;
    p.n_tiles = (int)ceil_div(D.I, tile_bn(role_tile(r, D.I)));
    p.C0 = dH; p.aux = h_save; p.I = D.I;
    if (D.bf16) MOE_TRY(tt.get(r, &p.tiles));
    MOE_TRY(launch_gemm(D.bf16, r, p, rows_or_tiles(r), s));
    if (dy_k)  // dG[t,j] = <dY[t], Yp[p]> = sum of the row's shares (when a6 did not run)
      MOE_TRY(launch_gate_grad_sum(dyf->inv, dg_part, D.I / 32, D.T * D.k, tt.kcost() + D.E_loc,
                                   dyf->dtopk_w, s));
  }
  {  // a10: [dWg | dWu][e] = Xp_e^T [dHg | dHu]_e
    const GemmRole gw = perm ? R_GATEUP_WGRAD_GATHER : R_GATEUP_WGRAD;
    GemmParams p{};
    p.A = xp; p.lda = D.d;
    if (perm) MOE_TRY(tt.rows(&p));
    p.B0 = dH; p.ldb = 2 * (int64_t)D.I;
    p.M = D.d; p.N = 2 * D.I;
    p.off = group_offsets; p.groups = D.E_loc;
    const TileCfg t = role_tile(gw);
    p.m_tiles = (int)ceil_div(D.d, tile_bm(t)); p.n_tiles = (int)ceil_div(2 * D.I, tile_bn(t));
    p.C0 = dw_gate; p.C1 = dw_up; p.n_split = D.I; p.ldc = D.I;
    p.c_estride = (int64_t)D.d * D.I;
    if (D.bf16) p.kcost = tt.kcost();
    MOE_TRY(launch_gemm(D.bf16, gw, p, p.m_tiles, s));
  }
  {  // a9: dXp = dHg Wg^T + dHu Wu^T (one K loop over [dHg | dHu])
    GemmParams p{};
    p.A = dH; p.lda = 2 * (int64_t)D.I;
    p.B0 = w_gate; p.B1 = w_up; p.ldb = D.I; p.b_estride = (int64_t)D.d * D.I;
    p.k_split = D.I;
    p.N = D.d; p.K = 2 * D.I;
    p.off = group_offsets; p.groups = D.E_loc;
    p.n_tiles = (int)ceil_div(D.d, tile_bn(role_tile(R_GATEUP_DGRAD)));
    p.C0 = dxp; p.ldc = D.d;
    if (D.bf16) MOE_TRY(tt.get(R_GATEUP_DGRAD, &p.tiles));
    MOE_TRY(launch_gemm(D.bf16, R_GATEUP_DGRAD, p, rows_or_tiles(R_GATEUP_DGRAD), s));
  }
  return MOE_OK;
}

}  // namespace

extern "C" moe_status_t moe_grouped_ffn_bwd(const moe_shape_t* shape, const void* xp,
                                            const int32_t* group_offsets, const void* w_gate,
                                            const void* w_up, const void* w_down,
                                            const void* h_save, const void* a_save,
                                            const void* dyp, void* dxp, void* dw_gate,
                                            void* dw_up, void* dw_down, void* ws,
                                            size_t ws_bytes_, moe_stream_t stream) {
  return ffn_bwd("moe_grouped_ffn_bwd", false, shape, xp, nullptr, group_offsets, w_gate, w_up,
                 w_down, h_save, a_save, dyp, dxp, dw_gate, dw_up, dw_down, ws, ws_bytes_, stream);
}

extern "C" moe_status_t moe_grouped_ffn_bwd_gather(const moe_shape_t* shape, const void* x,
                                                   const int32_t* perm,
                                                   const int32_t* group_offsets,
                                                   const void* w_gate, const void* w_up,
                                                   const void* w_down, const void* h_save,
                                                   const void* a_save, const void* dyp, void* dxp,
                                                   void* dw_gate, void* dw_up, void* dw_down,
                                                   void* ws, size_t ws_bytes_,
                                                   moe_stream_t stream) {
  return ffn_bwd("moe_grouped_ffn_bwd_gather", true, shape, x, perm, group_offsets, w_gate, w_up,
                 w_down, h_save, a_save, dyp, dxp, dw_gate, dw_up, dw_down, ws, ws_bytes_, stream);
}

extern "C" moe_status_t moe_combine_ffn_bwd_gather(
    const moe_shape_t* shape, const void* x, const int32_t* perm, const int32_t* inv,
    const int32_t* group_offsets, const float* topk_w, const void* w_gate, const void* w_up,
    const void* w_down, const void* h_save, const void* a_save, const void* yp, const void* dy,
    void* dyp, float* dtopk_w, void* dxp, void* dw_gate, void* dw_up, void* dw_down, void* ws,
    size_t ws_bytes_, moe_stream_t stream) {
  const DyForm dyf{dy, yp, inv, topk_w, dtopk_w};
  return ffn_bwd("moe_combine_ffn_bwd_gather", true, shape, x, perm, group_offsets, w_gate, w_up,
                 w_down, h_save, a_save, dyp, dxp, dw_gate, dw_up, dw_down, ws, ws_bytes_, stream,
                 &dyf);
}

extern "C" moe_status_t moe_permute_bwd(const moe_shape_t* shape, const void* dxp, const int32_t* inv,
                                        void* dx, moe_stream_t stream) {
  const char* fn = "moe_permute_bwd";
  Dims D;
  MOE_TRY(check_shape(shape, fn, &D));
  MOE_TRY(need(fn, {{"dxp", dxp}, {"inv", inv}, {"dx", dx}}));
  return launch_gather_sum(dxp, inv, nullptr, D.T, D.d, D.k, D.eb, dx, S(stream), "permute_bwd");
}

namespace {
moe_status_t route_bwd(const char* fn, const moe_shape_t* shape, const void* x, const void* w_router,
                       const int32_t* topk_idx, const float* topk_w, const float* dtopk_w,
                       const float* logits, const float* aux_w, float* dlogits, void* dw_router,
                       float* dbias, void* dx, void* ws, size_t ws_bytes_, moe_stream_t stream) {
  Dims D;
  MOE_TRY(check_shape(shape, fn, &D));
  hipStream_t s = S(stream);
  if (aux_w) {
    if (D.balanced) return fail(MOE_ERR_ARG, "%s: the balanced gate has no router probabilities", fn);
    MOE_TRY(need(fn, {{"logits", logits}}));
  }
  if (D.balanced) {
    MOE_TRY(opt(fn, {{"dlogits", dlogits}, {"dw_router", dw_router}, {"dbias", dbias}}));
    return launch_fill_zero(dlogits, (int64_t)D.T * D.E * 4, dw_router, (int64_t)D.d * D.E * D.eb,
                            dbias, (int64_t)D.E * 4, s);
  }
  MOE_TRY(need(fn, {{"x", x}, {"w_router", w_router}, {"topk_idx", topk_idx}, {"topk_w", topk_w},
                    {"dtopk_w", dtopk_w}, {"dlogits", dlogits}, {"dw_router", dw_router}, {"dx", dx}}));
  MOE_TRY(opt(fn, {{"dbias", dbias}}));
  MOE_TRY(check_ws(fn, D, MOE_OP_ROUTE_BWD, ws, ws_bytes_));
  const RouteBwdWs rw(D);
  char* wsb = static_cast<char*>(ws);
  bf16_t* dl16 = D.bf16 ? reinterpret_cast<bf16_t*>(wsb + rw.dl16) : nullptr;
  float* db_part = reinterpret_cast<float*>(wsb + rw.dbp);
  float* dw_part = D.bf16 ? reinterpret_cast<float*>(wsb + rw.dwp) : nullptr;
  MOE_TRY(launch_route_bwd_dl(topk_idx, topk_w, dtopk_w, D.T, D.E, D.k, dlogits, dl16, db_part,
                              aux_w ? logits : nullptr, aux_w, s));
  const void* dl = D.bf16 ? static_cast<const void*>(dl16) : static_cast<const void*>(dlogits);
  {  // dWr = x^T dL: bf16 layers as fp32 partials over nsplit K (token) ranges
    GemmParams p{};
    p.A = x; p.lda = D.d;
    p.B0 = dl; p.ldb = D.E;
    p.M = D.d; p.N = D.E; p.K = D.T;
    p.off = nullptr;
    p.groups = D.bf16 ? rw.nsplit : 1;
    p.k_chunk = D.bf16 ? rw.k_chunk : 0;
    p.m_tiles = (int)ceil_div(D.d, 64); p.n_tiles = (int)ceil_div(D.E, 64);
    p.C0 = D.bf16 ? static_cast<void*>(dw_part) : dw_router; p.ldc = D.E;
    p.c_estride = (int64_t)D.d * D.E;
    MOE_TRY(launch_gemm(D.bf16, R_ROUTE_DW, p, p.m_tiles, s));
  }
  // fixed-order sums: the split partials into dWr (bf16), the column sums into db
  MOE_TRY(launch_route_bwd_reduce(dw_part, D.bf16 ? rw.nsplit : 0, (int64_t)D.d * D.E,
                                  static_cast<bf16_t*>(dw_router), db_part, rw.nblk, D.E, dbias, s));
  {  // dX += dL Wr^T
    GemmParams p{};
    p.A = dl; p.lda = D.E;
    p.B0 = w_router; p.ldb = D.E;
    p.M = D.T; p.N = D.d; p.K = D.E;
    const TileCfg tc = role_tile(R_ROUTE_DX);
    p.m_tiles = (int)ceil_div(D.T, tile_bm(tc)); p.n_tiles = (int)ceil_div(D.d, tile_bn(tc));
    p.groups = 1;
    p.C0 = dx; p.ldc = D.d;
    MOE_TRY(launch_gemm(D.bf16, R_ROUTE_DX, p, p.m_tiles, s));
  }
  return MOE_OK;
}
}  // namespace

extern "C" moe_status_t moe_route_bwd(const moe_shape_t* shape, const void* x, const void* w_router,
                                      const int32_t* topk_idx, const float* topk_w,
                                      const float* dtopk_w, float* dlogits, void* dw_router,
                                      float* dbias, void* dx, void* ws, size_t ws_bytes_,
                                      moe_stream_t stream) {
  return route_bwd("moe_route_bwd", shape, x, w_router, topk_idx, topk_w, dtopk_w, nullptr, nullptr,
                   dlogits, dw_router, dbias, dx, ws, ws_bytes_, stream);
}

extern "C" moe_status_t moe_route_bwd_aux(const moe_shape_t* shape, const void* x,
                                          const void* w_router, const int32_t* topk_idx,
                                          const float* topk_w, const float* dtopk_w,
                                          const float* logits, const float* aux_w, float* dlogits,
                                          void* dw_router, float* dbias, void* dx, void* ws,
                                          size_t ws_bytes_, moe_stream_t stream) {
  const char* fn = "moe_route_bwd_aux";
  MOE_TRY(need(fn, {{"aux_w", aux_w}}));
  return route_bwd(fn, shape, x, w_router, topk_idx, topk_w, dtopk_w, logits, aux_w, dlogits,
                   dw_router, dbias, dx, ws, ws_bytes_, stream);
}

extern "C" moe_status_t moe_aux_loss(const moe_shape_t* shape, const float* logits,
                                     const int32_t* topk_idx, float alpha, float* loss,
                                     float* aux_w, void* ws, size_t ws_bytes_,
                                     moe_stream_t stream) {
  const char* fn = "moe_aux_loss";
  Dims D;
  MOE_TRY(check_shape(shape, fn, &D));
  if (D.balanced) return fail(MOE_ERR_ARG, "%s: the balanced gate has no router probabilities", fn);
  if (!std::isfinite(alpha)) return fail(MOE_ERR_ARG, "%s: alpha must be finite", fn);
  MOE_TRY(need(fn, {{"logits", logits}, {"topk_idx", topk_idx}, {"loss", loss}, {"aux_w", aux_w}}));
  MOE_TRY(check_ws(fn, D, MOE_OP_AUX_LOSS, ws, ws_bytes_));
  return launch_aux_loss(logits, topk_idx, D.T, D.E, D.k, alpha, loss, aux_w, ws, S(stream));
}
