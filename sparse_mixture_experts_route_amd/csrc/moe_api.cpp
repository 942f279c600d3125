// C-ABI entry points of libmoe_mi355x.so: host-side argument checks,
// workspace carving and launch sequencing.  Nothing here synchronises with
// the host or allocates device memory; every launch goes to the caller's
// stream in order.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <mutex>
#include <stdint.h>
#include <string.h>

#include <vector>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(const moe_shape* s) {
  if (!s) return MOE_EINVAL;
  if (s->T < 0 || s->H <= 0 || s->E <= 0 || s->I <= 0 || s->Is < 0) return MOE_EINVAL;
  if (s->k <= 0 || s->k > s->E) return MOE_EINVAL;
  if (s->E > 256 || s->k > 64) return MOE_EUNSUPPORTED;
  if (s->dtype != MOE_DTYPE_FP32 && s->dtype != MOE_DTYPE_BF16) return MOE_EUNSUPPORTED;
  if (s->score < MOE_SCORE_SOFTMAX || s->score > MOE_SCORE_SQRTSOFTPLUS) return MOE_EUNSUPPORTED;
  if (s->H % 8 || s->I % 8 || s->Is % 8) return MOE_EUNSUPPORTED;
  if (s->T * s->k >= (int64_t)1 << 31) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

inline size_t esize(const moe_shape* s) { return s->dtype == MOE_DTYPE_BF16 ? 2 : 4; }

struct Carve {
  char* base;
  size_t used = 0;
  explicit Carve(void* b) : base((char*)b) {}
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    used += align_up(bytes);
    return p;
  }
};

moe::GemmProblem gp();

// The shared expert's down projection (M = T rows, one group).
moe::GemmProblem shared_down_problem(const moe_shape* s) {
  moe::GemmProblem q = gp();
  q.sched = moe::SCHED_GROUP_M;
  q.epi = moe::EPI_STORE_F32;
  q.lda = s->Is;
  q.ldb = s->Is;
  q.ldc = s->H;
  q.G = 1;
  q.M = s->T;
  q.N = s->H;
  q.K = s->Is;
  return q;
}

// The shared expert's gate_up projection + SwiGLU (M = T rows, one group).
moe::GemmProblem shared_gate_up_problem(const moe_shape* s) {
  moe::GemmProblem q = gp();
  q.sched = moe::SCHED_GROUP_M;
  q.epi = moe::EPI_SWIGLU;
  q.lda = s->H;
  q.ldb = s->H;
  q.ldc = s->Is;
  q.ld_aux = 2 * s->Is;
  q.G = 1;
  q.M = s->T;
  q.N = 2 * s->Is;
  q.K = s->H;
  q.n_half = s->Is;
  return q;
}

// The routed gate_up projection + SwiGLU over the expert segments (A rows
// through perm) and the routed down projection: the shape-dependent fields.
moe::GemmProblem routed_gate_up_problem(const moe_shape* s) {
  moe::GemmProblem q = gp();
  q.sched = moe::SCHED_GROUP_M;
  q.epi = moe::EPI_SWIGLU;
  q.lda = s->H;
  q.a_div = (int)s->k;
  q.ldb = s->H;
  q.strideB = 2 * s->I * s->H;
  q.ldc = s->I;
  q.ld_aux = 2 * s->I;
  q.G = (int)s->E;
  q.M = s->T * s->k;
  q.N = 2 * s->I;
  q.K = s->H;
  q.n_half = s->I;
  q.rows_bound = s->T * s->k;
  return q;
}

moe::GemmProblem routed_down_problem(const moe_shape* s) {
  moe::GemmProblem q = gp();
  q.sched = moe::SCHED_GROUP_M;
  q.epi = moe::EPI_STORE_F32;
  q.lda = s->I;
  q.ldb = s->I;
  q.strideB = s->H * s->I;
  q.ldc = s->H;
  q.G = (int)s->E;
  q.M = s->T * s->k;
  q.N = s->H;
  q.K = s->I;
  q.rows_bound = s->T * s->k;
  return q;
}

// Split bf16 activation of an inference forward (no saved activations) in a
// bf16 layer whose expert GEMMs are weight streams: the SwiGLU epilogue
// writes h as its bf16 rounding plus the bf16 rounding of the remainder, and
// the down projection multiplies both, so its operand carries about 16
// significant bits instead of 8 at no cost a weight stream would notice.
// Per pair of GEMMs: the routed experts' and the shared expert's.
bool split_routed(const moe_shape* s) {
  const int bf = s->dtype == MOE_DTYPE_BF16;
  // as launched: E segments (device offsets) and the gate_up rows read through perm
  const int32_t* dev = (const int32_t*)16;
  moe::GemmProblem gu = routed_gate_up_problem(s), dn = routed_down_problem(s);
  gu.offsets = dn.offsets = dev;
  gu.a_idx = dev;
  return bf && s->T > 0 && moe::gemm_split_operand_ok(gu, bf) && moe::gemm_split_operand_ok(dn, bf);
}
bool split_shared(const moe_shape* s) {
  const int bf = s->dtype == MOE_DTYPE_BF16;
  return bf && s->Is && s->T > 0 && moe::gemm_split_operand_ok(shared_gate_up_problem(s), bf) &&
         moe::gemm_split_operand_ok(shared_down_problem(s), bf);
}

// Workspace layout of the forward (inference): h [P,I] and s_h [T,Is] in the
// layer dtype, y [P,H] and S [T,H] (binary16 in a bf16 layer, else fp32), and
// the fp32 K-split partials of the shared expert's GEMMs when they split
// (one region: the two run one after the other on the stream).  With
// `split_ok` (moe_ffn_forward without saved activations) also the lo parts
// h_lo [P,I] and s_h_lo [T,Is] where the split activation applies.
size_t fwd_layout(const moe_shape* s, const moe_saved* saved, void* ws, void** h, void** y, void** sh, void** sy,
                  void** split = nullptr, bool split_ok = false, void** h_lo = nullptr, void** sh_lo = nullptr) {
  const size_t b = esize(s);
  const int64_t P = s->T * s->k;
  Carve c(ws);
  void* ph = (saved && saved->h) ? saved->h : c.take((size_t)P * s->I * b);
  const bool no_save = !saved || (!saved->h && !saved->s_h);
  void* phl = (split_ok && no_save && split_routed(s)) ? c.take((size_t)P * s->I * b) : nullptr;
  const size_t yb = s->dtype == MOE_DTYPE_BF16 ? 2 : 4;  // y, s_y: binary16 for a bf16 layer
  void* py = (saved && saved->y) ? saved->y : c.take((size_t)P * s->H * yb);
  void* psh = nullptr;
  void* pshl = nullptr;
  void* psy = nullptr;
  void* psp = nullptr;
  if (s->Is) {
    psh = (saved && saved->s_h) ? saved->s_h : c.take((size_t)s->T * s->Is * b);
    if (split_ok && no_save && split_shared(s)) pshl = c.take((size_t)s->T * s->Is * b);
    psy = (saved && saved->s_y) ? saved->s_y : c.take((size_t)s->T * s->H * yb);
    const int bf = s->dtype == MOE_DTYPE_BF16;
    const size_t spb = std::max(moe::gemm_split_ws_bytes(shared_down_problem(s), bf),
                                moe::gemm_split_ws_bytes(shared_gate_up_problem(s), bf));
    if (spb) psp = c.take(spb);
  }
  if (split) *split = psp;
  if (h_lo) *h_lo = phl;
  if (sh_lo) *sh_lo = pshl;
  if (h) *h = ph;
  if (y) *y = py;
  if (sh) *sh = psh;
  if (sy) *sy = psy;
  return c.used;
}

struct BwdWs {
  void* xs;     // gathered x rows when the caller passes no x_sorted [P,H] (dtype)
  void* dy;     // [P,H] dtype: weighted dout rows, operand of the dh GEMM and dw_down
  void* dgu;    // [P,2I] dtype: (dg | du), operand of the dx GEMM and dw_gate_up
  void* dxs;    // [P,H] per-row data gradient before the sum over slots (binary16 / fp32 layer: fp32)
  void* ds;     // [T,H] dtype: gated dout for the shared expert
  void* dsgu;   // [T,2Is] dtype
  void* dxsh;   // [T,H] shared-expert data gradient (binary16 / fp32 layer: fp32)
  float* dw;    // [T,k]
  float* dz;    // [T]
  float* dl;    // [T,E]
  void* red;    // row-reduction partials
};

size_t bwd_layout(const moe_shape* s, bool need_xs, bool need_dl, void* ws, BwdWs* o) {
  const size_t b = esize(s);
  const int64_t P = s->T * s->k;
  Carve c(ws);
  BwdWs w;
  w.xs = need_xs ? c.take((size_t)P * s->H * b) : nullptr;
  w.dy = c.take((size_t)P * s->H * b);
  w.dgu = c.take((size_t)P * 2 * s->I * b);
  const size_t gb = s->dtype == MOE_DTYPE_BF16 ? 2 : 4;  // dxs, dxsh: binary16 in a bf16 layer
  w.dxs = c.take((size_t)P * s->H * gb);
  w.ds = s->Is ? c.take((size_t)s->T * s->H * b) : nullptr;
  w.dsgu = s->Is ? c.take((size_t)s->T * 2 * s->Is * b) : nullptr;
  w.dxsh = s->Is ? c.take((size_t)s->T * s->H * gb) : nullptr;
  w.dw = (float*)c.take((size_t)P * 4);
  w.dz = (float*)c.take((size_t)s->T * 4);
  w.dl = need_dl ? (float*)c.take((size_t)s->T * s->E * 4) : nullptr;
  const size_t r1 = moe::rowreduce_ws_bytes(s->T, s->E + 1, s->H);  // + the shared-gate column
  w.red = c.take(r1);
  if (o) *o = w;
  return c.used;
}

// ---- stage timing: events recorded on the caller's stream at stage ends
struct Profile {
  bool active = false;
  int max_calls = 0;
  int used = 0;
  int kinds[2] = {0, 0};        // forward, backward calls recorded
  std::vector<hipEvent_t> ev;   // [max_calls][MOE_N_STAGES + 1]; event 0 = call start
  std::vector<int> stage_of;    // stage ended by event i of a slot
  std::vector<int> nmarks;      // events recorded per slot
};
Profile g_prof;

struct Marks {
  int slot = -1;
  hipStream_t stream = nullptr;
  void end(int stage) {
    if (slot < 0) return;
    const int i = g_prof.nmarks[slot]++;
    g_prof.stage_of[(size_t)slot * (MOE_N_STAGES + 1) + i] = stage;
    hipEventRecord(g_prof.ev[(size_t)slot * (MOE_N_STAGES + 1) + i], stream);
  }
};

Marks prof_begin(int kind, hipStream_t stream) {
  Marks m;
  if (!g_prof.active || g_prof.used >= g_prof.max_calls) return m;
  m.slot = g_prof.used++;
  m.stream = stream;
  g_prof.kinds[kind]++;
  g_prof.nmarks[m.slot] = 0;
  m.end(-1);  // start event
  return m;
}

moe::GemmProblem gp() {
  moe::GemmProblem q;
  memset(&q, 0, sizeof(q));
  q.a_kmajor = 1;
  q.b_kmajor = 1;
  q.a_div = 1;
  return q;
}

// A per-device side stream (default priority) with a fork and a join event,
// created on first use and kept for the life of the process; `mu` orders the
// fork / join sequences of concurrent callers.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};
SideStream* side_stream() {
  static SideStream slots[64];
  static std::mutex init_mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(init_mu);
  SideStream& ss = slots[dev];
  if (!ss.s) {
    hipStream_t st = nullptr;
    hipEvent_t f = nullptr, jn = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&jn, hipEventDisableTiming) != hipSuccess) {
      if (f) hipEventDestroy(f);
      hipStreamDestroy(st);
      return nullptr;
    }
    ss.fork = f;
    ss.join = jn;
    ss.s = st;
  }
  return &ss;
}

// The shared expert's GEMMs of the forward on `sstr`: gate_up + SwiGLU
// into sh (its lo part into sh_lo, the fp32 pre-activations into s_gu when
// non-null), then the down projection into sy (binary16 when y_f16, else
// fp32).  Stages 2 and 3 of the profile.
int launch_shared_expert(const moe_shape* s, const moe_weights* w, const void* x, void* s_gu, void* sh, void* sy,
                         void* split, int bf, int y_f16, hipStream_t sstr, Marks& pm, void* sh_lo) {
  moe::GemmProblem q = shared_gate_up_problem(s);
  q.A = x;
  q.B = w->ws_gate_up;
  q.C = sh;
  q.C_lo = sh_lo;
  q.aux = s_gu;
  q.split_ws = split;
  if (moe::launch_gemm(q, bf, sstr)) return MOE_ELAUNCH;
  pm.end(2);
  q = shared_down_problem(s);
  q.c_f16 = y_f16;
  q.A = sh;
  q.A_lo = sh_lo;
  q.B = w->ws_down;
  q.C = sy;
  q.split_ws = split;
  if (moe::launch_gemm(q, bf, sstr)) return MOE_ELAUNCH;
  pm.end(3);
  return MOE_OK;
}

// The routed experts' GEMMs of the forward on `str`: gate_up + SwiGLU over
// the expert segments (h, its lo part into h_lo, the fp32 pre-activations
// into gu when non-null), then the down projection into the rows y
// (binary16 when y_f16, else fp32).  Stages 0 and 1 of the profile.
int launch_routed_experts(const moe_shape* s, const moe_weights* w, const void* x, const void* x_sorted,
                          const int32_t* offsets, const int32_t* perm, void* gu, void* h, void* y, int bf,
                          int y_f16, hipStream_t str, Marks& pm, void* h_lo) {
  moe::GemmProblem gu_q = routed_gate_up_problem(s);
  gu_q.A = x_sorted ? x_sorted : x;
  gu_q.a_idx = x_sorted ? nullptr : perm;
  gu_q.a_div = x_sorted ? 1 : (int)s->k;
  gu_q.B = w->w_gate_up;
  gu_q.C = h;
  gu_q.C_lo = h_lo;
  gu_q.aux = gu;
  gu_q.offsets = offsets;
  if (moe::launch_gemm(gu_q, bf, str)) return MOE_ELAUNCH;
  pm.end(0);
  moe::GemmProblem dn_q = routed_down_problem(s);
  dn_q.c_f16 = y_f16;
  dn_q.A = h;
  dn_q.A_lo = h_lo;
  dn_q.B = w->w_down;
  dn_q.C = y;
  dn_q.offsets = offsets;
  if (moe::launch_gemm(dn_q, bf, str)) return MOE_ELAUNCH;
  pm.end(1);
  return MOE_OK;
}

// Whether the routed GEMMs of a layer of this shape are weight streams (the
// streaming kernel: decode-sized batches), as launched with device offsets.
bool routed_streams(const moe_shape* s, int bf) {
  moe::GemmProblem gu_q = routed_gate_up_problem(s);
  gu_q.offsets = (const int32_t*)16;
  return moe::gemm_uses_stream(gu_q, bf);
}

// Expert GEMMs of the forward: the routed experts' (launch_routed_experts)
// and, when Is > 0, the shared expert's (launch_shared_expert, reading
// x_shared when given, else x).  Stages 0..3 of the profile.  When the
// routed GEMMs are weight streams (decode-sized layers) and no stage profile
// is being taken, the shared expert's GEMMs run on the side stream, forked
// from and joined back into `str` by events, so their launches and tails
// overlap the routed stream.
int run_experts(const moe_shape* s, const moe_weights* w, const void* x, const void* x_sorted,
                const int32_t* offsets, const int32_t* perm, void* gu, void* h, void* y, void* s_gu, void* sh,
                void* sy, void* split, int bf, int y_f16, hipStream_t str, Marks& pm,
                const void* x_shared = nullptr, void* h_lo = nullptr, void* sh_lo = nullptr,
                bool side_ok = true) {
  const int64_t Is = s->Is;
  const void* xs = x_shared ? x_shared : x;
  auto routed = [&]() {
    return launch_routed_experts(s, w, x, x_sorted, offsets, perm, gu, h, y, bf, y_f16, str, pm, h_lo);
  };
  SideStream* ss = (side_ok && Is && pm.slot < 0 && bf && routed_streams(s, bf)) ? side_stream() : nullptr;
  if (!ss) {
    const int st = routed();
    return (st || !Is) ? st : launch_shared_expert(s, w, xs, s_gu, sh, sy, split, bf, y_f16, str, pm, sh_lo);
  }
  std::lock_guard<std::mutex> lock(ss->mu);
  if (hipEventRecord(ss->fork, str) != hipSuccess || hipStreamWaitEvent(ss->s, ss->fork, 0) != hipSuccess)
    return MOE_ELAUNCH;
  const int st_shared = launch_shared_expert(s, w, xs, s_gu, sh, sy, split, bf, y_f16, ss->s, pm, sh_lo);
  const int st_routed = routed();
  // join even after a failed launch, so `str` never runs ahead of work queued on the side stream
  if (hipEventRecord(ss->join, ss->s) != hipSuccess || hipStreamWaitEvent(str, ss->join, 0) != hipSuccess)
    return MOE_ELAUNCH;
  return st_shared ? st_shared : st_routed;
}

// Checks shared by the two forward entry points.
int check_forward(const moe_shape* s, const moe_weights* w, const void* x, const void* x_sorted,
                  const int32_t* offsets, const int32_t* perm, const moe_saved* saved) {
  int st = check_shape(s);
  if (st) return st;
  if (s->T == 0) return MOE_OK;  // no tokens: nothing is read or written
  if (!w || !w->w_gate_up || !w->w_down || !x || !offsets) return MOE_EINVAL;
  if (!x_sorted && !perm) return MOE_EINVAL;
  if (s->Is && (!w->ws_gate_up || !w->ws_down)) return MOE_EINVAL;
  const void* ptrs[] = {x, x_sorted, w->w_gate_up, w->w_down, w->ws_gate_up, w->ws_down};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MOE_EINVAL;
  (void)saved;
  return MOE_OK;
}

// moe_route, with the per-tile expert loads written to tile_counts when it
// is set (moe_route_dispatch).
int route_impl(const moe_shape* s, const void* x, const void* w_router, const void* w_shared_gate,
               const float* sel_bias, float* logits, float* weights, int64_t* ids, float* gate,
               float* score_sums, void* ws, size_t ws_bytes, int flags, void* stream, int32_t* tile_counts,
               int32_t* d_counts = nullptr, int32_t* d_offsets = nullptr, int32_t* d_perm = nullptr,
               int32_t* d_pos = nullptr, int* dispatched = nullptr) {
  int st = check_shape(s);
  if (st) return st;
  if (s->T == 0) {  // nothing to route; the [T]-sized pointers may be NULL
    if (!score_sums) return MOE_OK;
    if (!ws || ws_bytes < moe::route_ws_bytes(0, s->H, s->E, s->dtype == MOE_DTYPE_BF16) || !aligned16(ws))
      return MOE_EWORKSPACE;
  }
  const bool logits_in = (flags & MOE_ROUTE_LOGITS_IN) != 0;
  if (s->T > 0 && (!weights || !ids)) return MOE_EINVAL;
  if (s->T == 0) {
    // score sums of no tokens: zeros (written by the reduction over no tiles)
  } else if (logits_in) {
    if (!logits || gate) return MOE_EINVAL;
  } else {
    if (!x || !w_router) return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(w_router) || (w_shared_gate && !aligned16(w_shared_gate))) return MOE_EINVAL;
  }
  if (gate && !w_shared_gate) return MOE_EINVAL;
  if (score_sums || ws) {
    if (!ws || ws_bytes < moe::route_ws_bytes(s->T, s->H, s->E, s->dtype == MOE_DTYPE_BF16) || !aligned16(ws))
      return MOE_EWORKSPACE;
  }
  if (s->T == 0 && !score_sums) return MOE_OK;  // with score_sums: zero sums are written
  moe::RouteLaunch p{};
  p.tile_counts = tile_counts;
  p.d_counts = d_counts;
  p.d_offsets = d_offsets;
  p.d_perm = d_perm;
  p.d_pos = d_pos;
  p.dispatched = dispatched;
  p.x = x;
  p.w_router = w_router;
  p.w_gate = logits_in ? nullptr : (gate ? w_shared_gate : nullptr);
  p.bias = sel_bias;
  p.logits = logits;
  p.weights = weights;
  p.ids = ids;
  p.gate = gate;
  p.score_sums = score_sums;
  p.ws = ws;
  p.ws_bytes = ws ? ws_bytes : 0;
  p.T = s->T;
  p.H = s->H;
  p.E = s->E;
  p.k = s->k;
  p.score = s->score;
  p.renorm = s->renorm;
  p.logits_in = logits_in ? 1 : 0;
  p.bf16 = s->dtype == MOE_DTYPE_BF16;
  return moe::launch_route(p, (hipStream_t)stream) ? MOE_ELAUNCH : MOE_OK;
}

// Scratch of moe_route_dispatch: the router's (score sums, split reduction),
// then the per-tile expert loads for tiles of at least 16 tokens.
size_t route_dispatch_ws_bytes(const moe_shape* s) {
  const int bf = s->dtype == MOE_DTYPE_BF16;
  const int64_t tiles = (s->T + 15) / 16;
  return align_up(moe::route_ws_bytes(s->T, s->H, s->E, bf)) + align_up((size_t)(tiles > 0 ? tiles : 1) * s->E * 4);
}

}  // namespace

extern "C" {

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape, dtype or option";
    case MOE_EWORKSPACE: return "workspace missing or too small";
    case MOE_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

size_t moe_workspace_bytes(const moe_shape* s, int op) {
  if (check_shape(s) != MOE_OK) return 0;
  switch (op) {
    case MOE_OP_DISPATCH: return moe::dispatch_ws_bytes(s->T * s->k, s->E);
    case MOE_OP_FFN_FORWARD: return fwd_layout(s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, true);
    case MOE_OP_FFN_BACKWARD: return bwd_layout(s, true, true, nullptr, nullptr);
    case MOE_OP_ROUTE: return moe::route_ws_bytes(s->T, s->H, s->E, s->dtype == MOE_DTYPE_BF16);
    case MOE_OP_ROUTE_DISPATCH: return route_dispatch_ws_bytes(s);
    case MOE_OP_LAYER_FORWARD:
      return align_up(route_dispatch_ws_bytes(s)) +
             fwd_layout(s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, true);
    case MOE_OP_BLOCK:
      return align_up((size_t)s->T * s->H * esize(s)) +
             fwd_layout(s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    case MOE_OP_FFN_PARTIAL: {
      moe_saved lay;
      memset(&lay, 0, sizeof(lay));
      lay.y = lay.s_y = (void*)16;  // the caller's outputs: not in the workspace
      return fwd_layout(s, &lay, nullptr, nullptr, nullptr, nullptr, nullptr);
    }
    default: return 0;
  }
}

int moe_route(const moe_shape* s, const void* x, const void* w_router, const void* w_shared_gate,
              const float* sel_bias, float* logits, float* weights, int64_t* ids, float* gate,
              float* score_sums, void* ws, size_t ws_bytes, int flags, void* stream) {
  return route_impl(s, x, w_router, w_shared_gate, sel_bias, logits, weights, ids, gate, score_sums, ws, ws_bytes,
                    flags, stream, nullptr);
}

int moe_route_dispatch(const moe_shape* s, const void* x, const void* w_router, const void* w_shared_gate,
                       const float* sel_bias, float* logits, float* weights, int64_t* ids, float* gate,
                       float* score_sums, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos, void* ws,
                       size_t ws_bytes, int flags, void* stream) {
  int st = check_shape(s);
  if (st) return st;
  if (!counts || !offsets) return MOE_EINVAL;
  if (s->T > 0 && (!ids || !weights || !perm || !pos)) return MOE_EINVAL;
  const int bf = s->dtype == MOE_DTYPE_BF16;
  const size_t rws = align_up(moe::route_ws_bytes(s->T, s->H, s->E, bf));
  if (!ws || ws_bytes < route_dispatch_ws_bytes(s) || !aligned16(ws)) return MOE_EWORKSPACE;
  int32_t* tc = (int32_t*)((char*)ws + rws);
  int dispatched = 0;
  st = route_impl(s, x, w_router, w_shared_gate, sel_bias, logits, weights, ids, gate, score_sums, ws, rws, flags,
                  stream, s->T > 0 ? tc : nullptr, counts, offsets, perm, pos, &dispatched);
  if (st) return st;
  if (dispatched) return MOE_OK;  // a one-tile batch: the router's workgroup sorted it
  const bool logits_in = (flags & MOE_ROUTE_LOGITS_IN) != 0;
  const int64_t ncols = s->E + ((!logits_in && gate) ? 1 : 0);
  const int tm = moe::route_tile_tokens(s->T, s->H, ncols, bf, logits_in ? 1 : 0);
  return moe::launch_dispatch_tiles(ids, s->T, s->k, s->E, tm, tc, counts, offsets, perm, pos, (hipStream_t)stream)
             ? MOE_ELAUNCH
             : MOE_OK;
}

int moe_dispatch(const moe_shape* s, const int64_t* ids, const void* x, int32_t* counts, int32_t* offsets,
                 int32_t* perm, int32_t* pos, void* x_sorted, void* ws, size_t ws_bytes, void* stream) {
  int st = check_shape(s);
  if (st) return st;
  if (!counts || !offsets) return MOE_EINVAL;
  if (s->T > 0 && (!ids || !perm || !pos)) return MOE_EINVAL;
  if (s->T > 0 && x_sorted && (!x || !aligned16(x) || !aligned16(x_sorted))) return MOE_EINVAL;
  if (!ws || ws_bytes < moe::dispatch_ws_bytes(s->T * s->k, s->E) || !aligned16(ws)) return MOE_EWORKSPACE;
  hipStream_t str = (hipStream_t)stream;
  if (moe::launch_dispatch(ids, s->T, s->k, s->E, counts, offsets, perm, pos, ws, str)) return MOE_ELAUNCH;
  if (x_sorted && s->T > 0) {
    if (moe::launch_gather(x, s->T, s->k, s->H * (int64_t)esize(s), pos, x_sorted, str)) return MOE_ELAUNCH;
  }
  return MOE_OK;
}

}  // extern "C"

namespace {

// moe_ffn_forward with a choice of the side stream (the no-allocation entry
// point runs everything on the caller's stream: creating the side stream
// would create a stream and two events).
int ffn_forward(const moe_shape* s, const moe_weights* w, const void* x, const void* x_sorted,
                const int32_t* offsets, const int32_t* perm, const int32_t* pos, const float* weights,
                const float* gate, void* out, const moe_saved* saved, void* ws, size_t ws_bytes, void* stream,
                bool side_ok) {
  int st = check_forward(s, w, x, x_sorted, offsets, perm, saved);
  if (st) return st;
  if (s->T == 0) return MOE_OK;
  if (!pos || !weights || !out || !aligned16(out)) return MOE_EINVAL;
  if (s->Is && s->shared_gated && !gate) return MOE_EINVAL;
  if (saved && (!saved->gu || !saved->h || !saved->y)) return MOE_EINVAL;
  if (saved && s->Is && (!saved->s_gu || !saved->s_h || !saved->s_y)) return MOE_EINVAL;
  const size_t need = fwd_layout(s, saved, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, true);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return MOE_EWORKSPACE;
  void *h, *y, *sh, *sy, *split, *h_lo, *sh_lo;
  fwd_layout(s, saved, ws, &h, &y, &sh, &sy, &split, true, &h_lo, &sh_lo);
  const int bf = s->dtype == MOE_DTYPE_BF16;
  hipStream_t str = (hipStream_t)stream;
  Marks pm = prof_begin(0, str);
  st = run_experts(s, w, x, x_sorted, offsets, perm, saved ? saved->gu : nullptr, h, y,
                   saved ? saved->s_gu : nullptr, sh, sy, split, bf, bf, str, pm, nullptr, h_lo, sh_lo, side_ok);
  if (st) return st;
  if (moe::launch_combine(y, bf, pos, weights, s->Is ? sy : nullptr,
                          (s->Is && s->shared_gated) ? gate : nullptr, out, s->T, s->k, s->H, bf, str))
    return MOE_ELAUNCH;
  pm.end(4);
  return MOE_OK;
}

// Device scratch of moe_ffn_forward_noalloc, for callers that cannot
// allocate: one copy per GPU the library runs on, held until the process
// ends.  Host code never uses this name as an address: the device address
// comes from hipGetSymbolAddress, once per device (noalloc_scratch).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

// The device address of `scratch` on the current device (looked up on the
// first call made with that device current), or null on error.
void* noalloc_scratch() {
  static std::mutex mu;
  static void* ptr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

}  // namespace

extern "C" {

int moe_ffn_forward(const moe_shape* s, const moe_weights* w, const void* x, const void* x_sorted,
                    const int32_t* offsets, const int32_t* perm, const int32_t* pos, const float* weights,
                    const float* gate, void* out, const moe_saved* saved, void* ws, size_t ws_bytes,
                    void* stream) {
  return ffn_forward(s, w, x, x_sorted, offsets, perm, pos, weights, gate, out, saved, ws, ws_bytes, stream, true);
}

int moe_layer_forward(const moe_shape* s, const moe_weights* w, const void* x, const void* w_router,
                      const void* w_shared_gate, const float* sel_bias, float* weights, int64_t* ids, float* gate,
                      int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos, void* out, void* ws,
                      size_t ws_bytes, void* stream) {
  int st = check_shape(s);
  if (st) return st;
  const size_t rdb = align_up(route_dispatch_ws_bytes(s));
  const size_t fb = fwd_layout(s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, true);
  if (!ws || ws_bytes < rdb + fb || !aligned16(ws)) return MOE_EWORKSPACE;
  void* fws = (char*)ws + rdb;
  hipStream_t str = (hipStream_t)stream;
  const int bf = s->dtype == MOE_DTYPE_BF16;
  // every argument of both halves checked before the first launch
  if (!counts || !offsets) return MOE_EINVAL;
  if (s->T > 0) {
    st = check_forward(s, w, x, nullptr, offsets, perm, nullptr);
    if (st) return st;
    if (!w_router || !aligned16(w_router) || !weights || !ids || !pos || !out || !aligned16(out)) return MOE_EINVAL;
    if (s->Is && s->shared_gated && (!gate || !w_shared_gate || !aligned16(w_shared_gate))) return MOE_EINVAL;
    if (gate && (!w_shared_gate || !aligned16(w_shared_gate))) return MOE_EINVAL;
  }
  // decode-sized layers with a shared expert (routed GEMMs that are weight
  // streams, at most 8 rows an expert on average): the shared expert's GEMMs
  // need only x, so they go to the side stream before the routing, whose
  // small kernels leave HBM idle, and overlap it and the routed weight
  // streams (Qwen2-MoE shape, T = 16 / 64: 0.195 -> 0.193 ms, 0.263 -> 0.255
  // ms; at T = 256, 17 rows an expert, it measured no faster)
  SideStream* ss = (s->T > 0 && s->Is && bf && !g_prof.active && s->T * s->k <= 8 * s->E && routed_streams(s, bf))
                       ? side_stream()
                       : nullptr;
  if (!ss) {
    st = moe_route_dispatch(s, x, w_router, w_shared_gate, sel_bias, nullptr, weights, ids, gate, nullptr, counts,
                            offsets, perm, pos, ws, rdb, 0, stream);
    if (st) return st;
    return ffn_forward(s, w, x, nullptr, offsets, perm, pos, weights, gate, out, nullptr, fws, fb, stream, true);
  }
  void *h, *y, *sh, *sy, *split, *h_lo, *sh_lo;
  fwd_layout(s, nullptr, fws, &h, &y, &sh, &sy, &split, true, &h_lo, &sh_lo);
  Marks pm;  // no stage profile on this path
  std::lock_guard<std::mutex> lock(ss->mu);
  if (hipEventRecord(ss->fork, str) != hipSuccess || hipStreamWaitEvent(ss->s, ss->fork, 0) != hipSuccess)
    return MOE_ELAUNCH;
  const int st_shared = launch_shared_expert(s, w, x, nullptr, sh, sy, split, bf, bf, ss->s, pm, sh_lo);
  int st_routed = moe_route_dispatch(s, x, w_router, w_shared_gate, sel_bias, nullptr, weights, ids, gate, nullptr,
                                     counts, offsets, perm, pos, ws, rdb, 0, stream);
  if (!st_routed)
    st_routed = launch_routed_experts(s, w, x, nullptr, offsets, perm, nullptr, h, y, bf, bf, str, pm, h_lo);
  // join even after a failed launch, so `str` never runs ahead of work queued on the side stream
  if (hipEventRecord(ss->join, ss->s) != hipSuccess || hipStreamWaitEvent(str, ss->join, 0) != hipSuccess)
    return MOE_ELAUNCH;
  if (st_shared || st_routed) return st_shared ? st_shared : st_routed;
  return moe::launch_combine(y, bf, pos, weights, sy, s->shared_gated ? gate : nullptr, out, s->T, s->k, s->H, bf,
                             str)
             ? MOE_ELAUNCH
             : MOE_OK;
}

int moe_ffn_forward_noalloc(const moe_shape* s, const moe_weights* w, const void* x, const void* x_sorted,
                            const int32_t* offsets, const int32_t* perm, const int32_t* pos, const float* weights,
                            const float* gate, void* out, void* stream) {
  const int st = check_shape(s);
  if (st) return st;
  if (fwd_layout(s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, true) > kNoAllocScratchBytes)
    return MOE_EWORKSPACE;
  if (s->T == 0) return ffn_forward(s, w, x, x_sorted, offsets, perm, pos, weights, gate, out, nullptr, nullptr, 0,
                                    stream, false);
  void* ws = noalloc_scratch();
  if (!ws) return MOE_ELAUNCH;
  return ffn_forward(s, w, x, x_sorted, offsets, perm, pos, weights, gate, out, nullptr, ws, kNoAllocScratchBytes,
                     stream, false);
}

int moe_ffn_forward_partial(const moe_shape* s, const moe_weights* w, const void* x, const void* x_sorted,
                            const int32_t* offsets, const int32_t* perm, float* y_part, float* s_part,
                            const moe_saved* saved, void* ws, size_t ws_bytes, void* stream) {
  int st = check_forward(s, w, x, x_sorted, offsets, perm, saved);
  if (st) return st;
  if (s->T == 0) return MOE_OK;
  if (!y_part || !aligned16(y_part) || (s->Is && (!s_part || !aligned16(s_part)))) return MOE_EINVAL;
  // activations go to saved (when given) or the workspace; y and s_y are the
  // caller's partial outputs
  moe_saved lay;
  memset(&lay, 0, sizeof(lay));
  if (saved) lay = *saved;
  lay.y = y_part;
  lay.s_y = s->Is ? s_part : nullptr;
  const size_t need = fwd_layout(s, &lay, nullptr, nullptr, nullptr, nullptr, nullptr);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return MOE_EWORKSPACE;
  if (s->T == 0) return MOE_OK;
  void *h, *y, *sh, *sy, *split;
  fwd_layout(s, &lay, ws, &h, &y, &sh, &sy, &split);
  hipStream_t str = (hipStream_t)stream;
  Marks pm = prof_begin(0, str);
  return run_experts(s, w, x, x_sorted, offsets, perm, lay.gu, h, y, lay.s_gu, sh, sy, split,
                     s->dtype == MOE_DTYPE_BF16, 0, str, pm);
}

int moe_combine(const moe_shape* s, const float* y, const int32_t* pos, const float* weights, const float* gate,
                const float* s_y, void* out, void* stream) {
  int st = check_shape(s);
  if (st) return st;
  if (s->T == 0) return MOE_OK;
  if (!y || !pos || !weights || !out || !aligned16(y) || !aligned16(out)) return MOE_EINVAL;
  if (s_y && !aligned16(s_y)) return MOE_EINVAL;
  if (gate && !s_y) return MOE_EINVAL;
  if (s->T == 0) return MOE_OK;
  return moe::launch_combine(y, 0, pos, weights, s_y, gate, out, s->T, s->k, s->H, s->dtype == MOE_DTYPE_BF16,
                             (hipStream_t)stream)
             ? MOE_ELAUNCH
             : MOE_OK;
}

int moe_parallel_block_forward(const moe_shape* s, const moe_weights* w, const moe_block_norms* nrm,
                               const void* residual, const void* x_dense, const int32_t* offsets,
                               const int32_t* perm, const int32_t* pos, const float* weights, void* out, void* ws,
                               size_t ws_bytes, void* stream) {
  int st = check_forward(s, w, residual, nullptr, offsets, perm, nullptr);
  if (st) return st;
  if (s->T == 0) return MOE_OK;
  if (!nrm || !nrm->g_pre_moe || !nrm->g_post_dense || !nrm->g_post_moe || !nrm->g_post) return MOE_EINVAL;
  if (!x_dense || !pos || !weights || !out || !aligned16(x_dense) || !aligned16(out)) return MOE_EINVAL;
  if (s->Is <= 0 || s->shared_gated) return MOE_EINVAL;
  const void* gs[] = {nrm->g_pre_moe, nrm->g_post_dense, nrm->g_post_moe, nrm->g_post};
  for (const void* q : gs)
    if (!aligned16(q)) return MOE_EINVAL;
  if (s->k > 8 || s->H > 8192) return MOE_EUNSUPPORTED;
  const size_t xb = align_up((size_t)s->T * s->H * esize(s));
  const size_t need = xb + fwd_layout(s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
  if (!ws || ws_bytes < need || !aligned16(ws)) return MOE_EWORKSPACE;
  if (s->T == 0) return MOE_OK;
  void* x_moe = ws;
  void *h, *y, *sh, *sy, *split;
  fwd_layout(s, nullptr, (char*)ws + xb, &h, &y, &sh, &sy, &split);
  const int bf = s->dtype == MOE_DTYPE_BF16;
  hipStream_t str = (hipStream_t)stream;
  // the experts read the normalised residual; the dense MLP (shared-expert
  // GEMMs) reads x_dense
  if (moe::launch_rmsnorm(residual, nrm->g_pre_moe, nrm->eps, x_moe, s->T, s->H, bf, str)) return MOE_ELAUNCH;
  Marks pm = prof_begin(0, str);
  st = run_experts(s, w, x_moe, nullptr, offsets, perm, nullptr, h, y, nullptr, sh, sy, split, bf, bf, str, pm,
                   x_dense);
  if (st) return st;
  if (moe::launch_block_out(y, bf, pos, weights, sy, residual, nrm->g_post_dense, nrm->g_post_moe, nrm->g_post,
                            nrm->eps, nrm->layer_scalar, out, s->T, s->k, s->H, bf, str))
    return MOE_ELAUNCH;
  pm.end(4);
  return MOE_OK;
}

int moe_ffn_backward(const moe_shape* s, const moe_weights* w, const void* x, const void* w_router,
                     const float* logits, const int64_t* ids, const float* weights, const float* gate,
                     const int32_t* offsets, const int32_t* perm, const int32_t* pos, const void* x_sorted,
                     const moe_saved* saved, const void* dout, const float* aux_coef, const moe_grads* g,
                     void* ws, size_t ws_bytes, void* stream) {
  int st = check_shape(s);
  if (st) return st;
  if (s->k > 8) return MOE_EUNSUPPORTED;
  if (s->T == 0) {  // no tokens: every weight gradient is zero; nothing else is read or written
    if (!g || !g->dw_router || !g->dw_gate_up || !g->dw_down) return MOE_EINVAL;
    if (s->Is && (!g->dws_gate_up || !g->dws_down || (s->shared_gated && !g->dw_shared_gate))) return MOE_EINVAL;
    hipStream_t str = (hipStream_t)stream;
    const int64_t E = s->E, H = s->H, I = s->I, Is = s->Is;
    int bad = moe::launch_zero_f32(g->dw_router, E * H, str) | moe::launch_zero_f32(g->dw_gate_up, E * 2 * I * H, str) |
              moe::launch_zero_f32(g->dw_down, E * H * I, str);
    if (Is) {
      bad |= moe::launch_zero_f32(g->dws_gate_up, 2 * Is * H, str) | moe::launch_zero_f32(g->dws_down, H * Is, str);
      if (s->shared_gated) bad |= moe::launch_zero_f32(g->dw_shared_gate, H, str);
    }
    return bad ? MOE_ELAUNCH : MOE_OK;
  }
  if (!w || !w->w_gate_up || !w->w_down || !x || !w_router || !logits || !ids || !weights || !offsets || !perm ||
      !pos || !saved || !dout || !g)
    return MOE_EINVAL;
  if (!saved->gu || !saved->h || !saved->y) return MOE_EINVAL;
  if (!g->dx || !g->dw_router || !g->dw_gate_up || !g->dw_down) return MOE_EINVAL;
  if (s->Is) {
    if (!w->ws_gate_up || !w->ws_down || !saved->s_gu || !saved->s_h || !saved->s_y) return MOE_EINVAL;
    if (!g->dws_gate_up || !g->dws_down) return MOE_EINVAL;
    if (s->shared_gated && (!gate || !w->w_shared_gate || !g->dw_shared_gate)) return MOE_EINVAL;
  }
  const void* ptrs[] = {x, x_sorted, dout, w->w_gate_up, w->w_down, w->ws_gate_up, w->ws_down, saved->gu,
                        saved->h, saved->y, saved->s_gu, saved->s_h, saved->s_y, g->dx};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MOE_EINVAL;
  const bool need_xs = x_sorted == nullptr;
  const bool need_dl = g->dlogits == nullptr;
  const size_t need = bwd_layout(s, need_xs, need_dl, nullptr, nullptr);
  if (!ws || ws_bytes < need || !aligned16(ws)) return MOE_EWORKSPACE;
  if (s->T == 0) return MOE_OK;
  BwdWs b;
  bwd_layout(s, need_xs, need_dl, ws, &b);
  float* dl = need_dl ? b.dl : g->dlogits;
  const int bf = s->dtype == MOE_DTYPE_BF16;
  hipStream_t str = (hipStream_t)stream;
  const int64_t T = s->T, P = s->T * s->k, H = s->H, I = s->I, Is = s->Is, E = s->E;
  const size_t eb = esize(s);
  const void* xs = x_sorted;
  if (need_xs) {
    if (moe::launch_gather(x, T, s->k, H * (int64_t)eb, pos, b.xs, str)) return MOE_ELAUNCH;
    xs = b.xs;
  }
  const bool gated = Is && s->shared_gated;
  Marks pm = prof_begin(1, str);
  // dy, dweights, shared dS and gate-logit gradient
  if (moe::launch_combine_bwd(dout, saved->y, bf, pos, weights, Is ? saved->s_y : nullptr,
                              gated ? gate : nullptr, b.dy,
                              b.dw, b.ds, gated ? b.dz : nullptr, T, s->k, H, bf, str))
    return MOE_ELAUNCH;
  pm.end(5);
  void* dxs = b.dxs;
  // the routed expert GEMMs (stages 6-9)
  auto routed_bwd = [&]() -> int {
    // dh = dy . w_down[e], SwiGLU backward -> dgu
    moe::GemmProblem q = gp();
    q.sched = moe::SCHED_GROUP_M;
    q.epi = moe::EPI_DSWIGLU;
    q.A = b.dy;
    q.lda = H;
    // B(n = i, k = h) = w_down[e][h][i]: N-contiguous, read as stored
    q.B = w->w_down;
    q.b_kmajor = 0;
    q.ldb = I;
    q.strideB = H * I;
    q.aux = saved->gu;
    q.aux_out = b.dgu;
    q.ld_aux = 2 * I;
    q.offsets = offsets;
    q.G = (int)E;
    q.M = P;
    q.N = I;
    q.K = H;
    q.n_half = I;
    q.rows_bound = P;
    if (moe::launch_gemm(q, bf, str)) return MOE_ELAUNCH;
    pm.end(6);
    // dw_down[e] = dy_e^T h_e
    q = gp();
    q.sched = moe::SCHED_GROUP_K;
    q.epi = moe::EPI_STORE_F32;
    q.A = b.dy;
    q.a_kmajor = 0;
    q.lda = H;
    q.B = saved->h;
    q.b_kmajor = 0;
    q.ldb = I;
    q.C = g->dw_down;
    q.ldc = I;
    q.strideC = H * I;
    q.offsets = offsets;
    q.G = (int)E;
    q.M = H;
    q.N = I;
    q.K = P;
    if (moe::launch_gemm(q, bf, str)) return MOE_ELAUNCH;
    pm.end(7);
    // dw_gate_up[e] = dgu_e^T x_e
    q = gp();
    q.sched = moe::SCHED_GROUP_K;
    q.epi = moe::EPI_STORE_F32;
    q.A = b.dgu;
    q.a_kmajor = 0;
    q.lda = 2 * I;
    q.B = xs;
    q.b_kmajor = 0;
    q.ldb = H;
    q.C = g->dw_gate_up;
    q.ldc = H;
    q.strideC = 2 * I * H;
    q.offsets = offsets;
    q.G = (int)E;
    q.M = 2 * I;
    q.N = H;
    q.K = P;
    if (moe::launch_gemm(q, bf, str)) return MOE_ELAUNCH;
    pm.end(8);
    // dx_sorted = dgu . w_gate_up[e]  (binary16 in a bf16 layer, else fp32)
    q = gp();
    q.sched = moe::SCHED_GROUP_M;
    q.epi = moe::EPI_STORE_F32;
    q.A = b.dgu;
    q.lda = 2 * I;
    // B(n = h, k = i2) = w_gate_up[e][i2][h]: N-contiguous, read as stored
    q.B = w->w_gate_up;
    q.b_kmajor = 0;
    q.ldb = H;
    q.strideB = 2 * I * H;
    q.C = dxs;
    q.c_f16 = bf;
    q.ldc = H;
    q.offsets = offsets;
    q.G = (int)E;
    q.M = P;
    q.N = H;
    q.K = 2 * I;
    q.rows_bound = P;
    if (moe::launch_gemm(q, bf, str)) return MOE_ELAUNCH;
    pm.end(9);
    return MOE_OK;
  };
  // the shared expert's backward (stage 10): dsh -> dsgu, dws_down,
  // dws_gate_up, dxsh, on stream sstr
  void* dxsh = Is ? b.dxsh : nullptr;
  auto shared_bwd = [&](hipStream_t sstr) -> int {
    moe::GemmProblem q;
    // shared expert: dsh = dS . ws_down -> dsgu
    q = gp();
    q.sched = moe::SCHED_GROUP_M;
    q.epi = moe::EPI_DSWIGLU;
    q.A = b.ds;
    q.lda = H;
    q.B = w->ws_down;
    q.b_kmajor = 0;
    q.ldb = Is;
    q.aux = saved->s_gu;
    q.aux_out = b.dsgu;
    q.ld_aux = 2 * Is;
    q.G = 1;
    q.M = T;
    q.N = Is;
    q.K = H;
    q.n_half = Is;
    if (moe::launch_gemm(q, bf, sstr)) return MOE_ELAUNCH;
    q = gp();
    q.sched = moe::SCHED_GROUP_K;
    q.epi = moe::EPI_STORE_F32;
    q.A = b.ds;
    q.a_kmajor = 0;
    q.lda = H;
    q.B = saved->s_h;
    q.b_kmajor = 0;
    q.ldb = Is;
    q.C = g->dws_down;
    q.ldc = Is;
    q.G = 1;
    q.M = H;
    q.N = Is;
    q.K = T;
    if (moe::launch_gemm(q, bf, sstr)) return MOE_ELAUNCH;
    q = gp();
    q.sched = moe::SCHED_GROUP_K;
    q.epi = moe::EPI_STORE_F32;
    q.A = b.dsgu;
    q.a_kmajor = 0;
    q.lda = 2 * Is;
    q.B = x;
    q.b_kmajor = 0;
    q.ldb = H;
    q.C = g->dws_gate_up;
    q.ldc = H;
    q.G = 1;
    q.M = 2 * Is;
    q.N = H;
    q.K = T;
    if (moe::launch_gemm(q, bf, sstr)) return MOE_ELAUNCH;
    q = gp();
    q.sched = moe::SCHED_GROUP_M;
    q.epi = moe::EPI_STORE_F32;
    q.A = b.dsgu;
    q.lda = 2 * Is;
    q.B = w->ws_gate_up;
    q.b_kmajor = 0;
    q.ldb = H;
    q.C = dxsh;
    q.c_f16 = bf;
    q.ldc = H;
    q.G = 1;
    q.M = T;
    q.N = H;
    q.K = 2 * Is;
    if (moe::launch_gemm(q, bf, sstr)) return MOE_ELAUNCH;
    pm.end(10);
    return MOE_OK;
  };
  // router: dlogits, dw_router = dlogits^T x (stage 11)
  auto router_part = [&]() -> int {
    if (moe::launch_router_bwd(logits, ids, weights, b.dw, aux_coef, dl, T, E, s->k, s->score, s->renorm, str))
      return MOE_ELAUNCH;
    // dw_shared_gate = dz^T x rides along as one more column when gated
    if (moe::launch_rowreduce(dl, gated ? b.dz : nullptr, x, g->dw_router, gated ? g->dw_shared_gate : nullptr, T, E,
                              H, bf, b.red, str))
      return MOE_ELAUNCH;
    pm.end(11);
    return MOE_OK;
  };
  // The shared expert's backward needs only combine_bwd's outputs: without a
  // stage profile it runs on the side stream beside the routed backward (its
  // weight gradients, 176 and 352 tiles of K = T at the Qwen2-MoE training
  // shape, leave CUs idle in their last round that the routed GEMMs fill),
  // joined back before the dx sum, which reads dxsh.
  SideStream* ss = (Is && pm.slot < 0) ? side_stream() : nullptr;
  if (ss) {
    std::lock_guard<std::mutex> lock(ss->mu);
    if (hipEventRecord(ss->fork, str) != hipSuccess || hipStreamWaitEvent(ss->s, ss->fork, 0) != hipSuccess)
      return MOE_ELAUNCH;
    const int st_shared = shared_bwd(ss->s);
    int st_routed = routed_bwd();
    if (!st_routed) st_routed = router_part();
    // join even after a failed launch, so `str` never runs ahead of work queued on the side stream
    if (hipEventRecord(ss->join, ss->s) != hipSuccess || hipStreamWaitEvent(str, ss->join, 0) != hipSuccess)
      return MOE_ELAUNCH;
    if (st_shared || st_routed) return st_shared ? st_shared : st_routed;
  } else {
    int st = routed_bwd();
    if (!st && Is) st = shared_bwd(str);
    if (!st) st = router_part();
    if (st) return st;
  }
  if (moe::launch_dx_sum(dxs, pos, dxsh, dl, w_router, gated ? b.dz : nullptr, gated ? w->w_shared_gate : nullptr,
                         g->dx, T, s->k, E, H, bf, str))
    return MOE_ELAUNCH;
  pm.end(12);
  return MOE_OK;
}

int moe_score_f32(int score, const float* l, float* s, int64_t n, void* stream) {
  if (n < 0 || (n > 0 && (!l || !s))) return MOE_EINVAL;
  if (score < MOE_SCORE_SOFTMAX || score > MOE_SCORE_SQRTSOFTPLUS) return MOE_EUNSUPPORTED;
  return moe::launch_score(score, l, s, n, (hipStream_t)stream) ? MOE_ELAUNCH : MOE_OK;
}

int moe_bandwidth_probe(int kind, const void* src, void* dst, int64_t bytes, int wgs, void* stream) {
  if (kind < 0 || kind > 2 || bytes < 0) return MOE_EINVAL;
  if ((kind != 1 && (!src || !aligned16(src))) || !dst || !aligned16(dst)) return MOE_EINVAL;
  if (wgs <= 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return MOE_ELAUNCH;
    wgs = 8 * std::max(1, cus);
  }
  return moe::launch_probe(kind, src, dst, bytes, wgs, (hipStream_t)stream) ? MOE_ELAUNCH : MOE_OK;
}

int moe_profile_begin(int max_calls) {
  if (max_calls <= 0 || max_calls > 100000 || g_prof.active) return MOE_EINVAL;
  g_prof = Profile();
  g_prof.max_calls = max_calls;
  const size_t n = (size_t)max_calls * (MOE_N_STAGES + 1);
  g_prof.ev.resize(n);
  g_prof.stage_of.assign(n, -1);
  g_prof.nmarks.assign(max_calls, 0);
  for (size_t i = 0; i < n; ++i)
    if (hipEventCreate(&g_prof.ev[i]) != hipSuccess) return MOE_ELAUNCH;
  g_prof.active = true;
  return MOE_OK;
}

int moe_profile_end(float* stage_ms, int n_stages, int* n_calls) {
  if (!g_prof.active || !stage_ms || n_stages < 0) return MOE_EINVAL;
  int st = MOE_OK;
  for (int s = 0; s < n_stages; ++s) stage_ms[s] = 0.0f;
  for (int slot = 0; slot < g_prof.used; ++slot) {
    hipEvent_t* ev = &g_prof.ev[(size_t)slot * (MOE_N_STAGES + 1)];
    const int* so = &g_prof.stage_of[(size_t)slot * (MOE_N_STAGES + 1)];
    const int n = g_prof.nmarks[slot];
    if (n > 0 && hipEventSynchronize(ev[n - 1]) != hipSuccess) st = MOE_ELAUNCH;
    for (int i = 1; i < n; ++i) {
      float ms = 0.0f;
      if (hipEventElapsedTime(&ms, ev[i - 1], ev[i]) != hipSuccess) st = MOE_ELAUNCH;
      if (so[i] >= 0 && so[i] < n_stages) stage_ms[so[i]] += ms;
    }
  }
  if (n_calls) {
    n_calls[0] = g_prof.kinds[0];
    n_calls[1] = g_prof.kinds[1];
  }
  for (hipEvent_t e : g_prof.ev) hipEventDestroy(e);
  g_prof = Profile();
  return st;
}

int moe_aux_loss(const moe_shape* s, const float* score_sums, const int32_t* counts, float alpha, float* loss,
                 float* coef, void* stream) {
  int st = check_shape(s);
  if (st) return st;
  if (!score_sums || !counts || (!loss && !coef)) return MOE_EINVAL;
  if (s->T == 0) return MOE_EINVAL;
  return moe::launch_aux_loss(score_sums, counts, s->T, s->k, s->E, alpha, loss, coef, (hipStream_t)stream)
             ? MOE_ELAUNCH
             : MOE_OK;
}

int moe_balance_counts(const moe_shape* s, const int64_t* ids, int32_t* counts, float* bias, float rate,
                       void* stream) {
  int st = check_shape(s);
  if (st) return st;
  if (!counts) return MOE_EINVAL;
  if (ids == nullptr && bias == nullptr) return MOE_EINVAL;
  return moe::launch_balance(ids, counts, bias, rate, s->T, s->k, s->E, (hipStream_t)stream) ? MOE_ELAUNCH : MOE_OK;
}

}  // extern "C"
