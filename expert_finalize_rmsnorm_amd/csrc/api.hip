// api.hip -- the C ABI of libmoetail (declared in include/moetail.h).
//
// b == 0 returns at once, before any other check ([tail] BoundTail.run
// returns for zero rows before it checks the arguments).  Otherwise every
// entry point checks all of its arguments first and enqueues nothing when
// one is refused ([tail] _check_tail_args refuses a call before anything
// launches).
#include "moetail.h"

#include <atomic>
#include <mutex>

#include "kernels.h"

// The allocation-free entry point's scratch (moetail_decode_tail_noalloc):
// a file-scope device array, one copy per GPU, held until the process ends.
// In host code `scratch` is only a stand-in for the symbol: its device
// address on each GPU comes from hipGetSymbolAddress, looked up once per
// device with that device current and kept in scratch_ptr; kernels get that
// address, never the host name.
constexpr size_t kScratchBytes = MOETAIL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

using namespace moetail;

constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxScratchDevices];  // device address of `scratch` per device

// The scratch of the device that runs `stream` (the current device for the
// null stream).  The first call on a device looks the address up with that
// device current, then restores the caller's device.
int scratch_for(hipStream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return MOETAIL_EHIP;
  hipDevice_t dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return MOETAIL_EHIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return MOETAIL_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return MOETAIL_EHIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return MOETAIL_EHIP;
    if (e != hipSuccess || p == nullptr) return MOETAIL_EHIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return MOETAIL_OK;
}

}  // namespace

namespace {

using namespace moetail;

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }
bool a16(const void* p) { return p != nullptr && aligned(p, 16); }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int check_norm_args(const void* w, int w_dtype, const uint16_t* gamma, float eps, int K, int P,
                    int tp, int b, bool uses_gamma = true) {
  if (b < 0 || K <= 0 || P <= 0 || tp <= 0) return MOETAIL_EINVAL;
  if (w_dtype != MOETAIL_F32 && w_dtype != MOETAIL_BF16) return MOETAIL_EINVAL;
  if (!(eps >= 0.0f) || eps == __builtin_inff()) return MOETAIL_EINVAL;  // rejects NaN too
  if (w == nullptr || !aligned(w, w_dtype == MOETAIL_F32 ? 4 : 2)) return MOETAIL_EINVAL;
  if (uses_gamma ? !a16(gamma) : (gamma && !aligned(gamma, 16))) return MOETAIL_EINVAL;
  if (P % 8 || P > MOETAIL_MAX_WIDTH || K > MOETAIL_MAX_ROUTES || tp > MOETAIL_MAX_TP ||
      b > MOETAIL_MAX_TOKENS)
    return MOETAIL_EUNSUPPORTED;
  return MOETAIL_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOETAIL_OK : MOETAIL_EHIP; }

bool layout_ok(int w_layout) {
  return w_layout == MOETAIL_W_ROWS || w_layout == MOETAIL_W_TILED;
}

// Projection kinds of moetail_set_projection_tuning, and the overrides set
// through it (all zeros: the library's own plan).  Read under plan_mutex.
ProjTuning tunings[3];
std::mutex plan_mutex;

// The expert-TP workspace: the one-pass kernel's token generations [b]
// (zero before the first use) and its tagged 512-column block totals
// [b][16 or 32][ceil(P/512)] (64-bit words); then, for more than
// kTpOnePassMaxRanks ranks (or tp unknown, 0), the two-pass path's
// rank-summed route rows [b][K][P] BF16 and their sum-of-squares block
// totals [b][K][ceil(P/512)] FP32.
size_t tp_gen_bytes(int b) { return round_up(sizeof(unsigned) * (size_t)b, 256); }
size_t tp_slot_bytes(int b, int K, int P) {
  const int kslots = K <= 16 ? 16 : 32;  // the kernel's route capacity: every slot is written
  return round_up(sizeof(uint64_t) * (size_t)b * kslots * ((P + 511) / 512), 256);
}
size_t tp_rows_bytes(int b, int K, int P) { return round_up(sizeof(uint16_t) * (size_t)b * K * P, 256); }
size_t tp_workspace(int b, int K, int P, int tp) {
  size_t n = tp_gen_bytes(b) + tp_slot_bytes(b, K, P);
  if (tp <= 0 || tp > kTpOnePassMaxRanks)
    n += tp_rows_bytes(b, K, P) +
         round_up(sizeof(float) * (size_t)b * K * ((P + 511) / 512), 256);  // 512-column blocks
  return n;
}

// The one-pass expert-TP kernel's wait limit for a block total (100 MHz
// ticks; 20 ms; < 0: no wait, a wave forms the totals that are not there).
std::atomic<long long> tp_wait_ticks{2000000};

struct UpprojLayout {
  ProjPlan plan;
  size_t y_bytes, part_bytes;
};
UpprojLayout upproj_layout(int b, int L, int N) {
  UpprojLayout l;
  l.plan = plan_projection(b, N, L, false, tunings[MOETAIL_PROJ_UPPROJ]);
  l.y_bytes = round_up(sizeof(uint16_t) * (size_t)b * L, 256);
  l.part_bytes = round_up(proj_partial_bytes(l.plan, b, N, false), 256);
  return l;
}

struct SharedLayout {
  ProjPlan gate_up, down;
  size_t h_bytes, part_bytes;
};
SharedLayout shared_layout(int b, int H, int I) {
  SharedLayout l;
  l.gate_up = plan_projection(b, 2 * I, H, true, tunings[MOETAIL_PROJ_GATEUP]);
  l.down = plan_projection(b, H, I, false, tunings[MOETAIL_PROJ_DOWN]);
  l.h_bytes = round_up(sizeof(uint16_t) * (size_t)b * I, 256);
  const size_t g = proj_partial_bytes(l.gate_up, b, 2 * I, true);
  const size_t d = proj_partial_bytes(l.down, b, H, false);
  l.part_bytes = round_up(g > d ? g : d, 256);
  return l;
}

struct TailLayout {
  ProjPlan gate_up, down, up;
  GroupPlan group;
  size_t counter_bytes, h_bytes, y_bytes, down_part_bytes, part_bytes;
};
// The gate/up, down and up projections keep the plans of their own entry
// points (so the sums are the same bits); down and up always go through
// partials, since rs is formed before out.  The workspace starts with the
// output-tile counters of the launches that form their own sums (one per
// tile of h, then of out), always at offset 0 whatever else the caller
// passes: they are zero between calls.
TailLayout tail_layout(int b, int L, int H, int I) {
  TailLayout l;
  l.gate_up = plan_projection(b, 2 * I, H, true, tunings[MOETAIL_PROJ_GATEUP]);
  l.down = plan_projection(b, H, I, false, tunings[MOETAIL_PROJ_DOWN]);
  l.up = plan_projection(b, H, L, false, tunings[MOETAIL_PROJ_UPPROJ]);
  l.group = (l.down.splits && l.up.splits) ? plan_group(b, l.down, H, l.up, H) : GroupPlan{};
  l.counter_bytes = round_up(sizeof(unsigned) * (size_t)(I / 16 + H / 16), 256);
  l.h_bytes = round_up(sizeof(uint16_t) * (size_t)b * I, 256);
  l.y_bytes = round_up(sizeof(uint16_t) * (size_t)b * L, 256);
  const size_t g = proj_partial_bytes(l.gate_up, b, 2 * I, true);
  l.down_part_bytes = round_up(proj_partial_bytes(l.down, b, H, true), 256);
  const size_t du = l.down_part_bytes + proj_partial_bytes(l.up, b, H, true);
  l.part_bytes = round_up(g > du ? g : du, 256);
  return l;
}
// (Without a grouped plan the down and up projections run as two launches.)
bool tail_ok(const TailLayout& l) { return l.gate_up.splits && l.down.splits && l.up.splits; }

// Plans are searched once per (operation, sizes, CU count, overrides) and
// kept: the entry points look theirs up instead of searching on every call
// (the [tail] BoundTail.run picks a kernel compiled once per set of
// constants).  A fixed table of the last kPlanSlots shapes, guarded by
// plan_mutex; a change of overrides empties it.
constexpr int kPlanSlots = 64;
struct PlanSlot {
  bool used;
  int op, b, d0, d1, d2, cu;
  UpprojLayout up;
  SharedLayout sh;
  TailLayout tail;
  ProjPlan proj;
};
PlanSlot plan_slots[kPlanSlots];
int plan_next = 0;
std::atomic<uint64_t> plan_searches{0}, plan_hits{0};

// The layouts of one operation's call (the member for `op` is filled).
PlanSlot plans_for(int op, int b, int d0, int d1, int d2) {
  const int cu = device_cu_count();
  std::lock_guard<std::mutex> lock(plan_mutex);
  for (const PlanSlot& e : plan_slots)
    if (e.used && e.op == op && e.b == b && e.d0 == d0 && e.d1 == d1 && e.d2 == d2 && e.cu == cu) {
      plan_hits.fetch_add(1, std::memory_order_relaxed);
      return e;
    }
  plan_searches.fetch_add(1, std::memory_order_relaxed);
  PlanSlot e{};
  e.used = true;
  e.op = op, e.b = b, e.d0 = d0, e.d1 = d1, e.d2 = d2, e.cu = cu;
  if (op == MOETAIL_OP_COMBINE_NORM_UPPROJ) e.up = upproj_layout(b, d0, d1);
  if (op == MOETAIL_OP_SHARED_EXPERT) e.sh = shared_layout(b, d0, d1);
  if (op == MOETAIL_OP_TAIL) e.tail = tail_layout(b, d0, d1, d2);
  // (the stage's plan in the composite calls: partials always for gate/up)
  if (op == MOETAIL_OP_PROJECTION)
    e.proj = plan_projection(b, d0, d1, d2 == MOETAIL_PROJ_GATEUP, tunings[d2]);
  plan_slots[plan_next] = e;
  plan_next = (plan_next + 1) % kPlanSlots;
  return e;
}
UpprojLayout upproj_plan(int b, int L, int N) {
  return plans_for(MOETAIL_OP_COMBINE_NORM_UPPROJ, b, L, N, 0).up;
}
SharedLayout shared_plan(int b, int H, int I) {
  return plans_for(MOETAIL_OP_SHARED_EXPERT, b, H, I, 0).sh;
}
// moetail_gate_up: the shared expert's gate/up plan (the same sums); the
// h tiles' counters at offset 0, then the partials.
struct GateUpLayout {
  ProjPlan plan;
  size_t counter_bytes, part_bytes;
};
GateUpLayout gate_up_plan(int b, int H, int I) {
  GateUpLayout l;
  l.plan = shared_plan(b, H, I).gate_up;
  l.counter_bytes = round_up(sizeof(unsigned) * (size_t)(I / 16), 256);
  l.part_bytes = round_up(proj_partial_bytes(l.plan, b, 2 * I, true), 256);
  return l;
}
TailLayout tail_plan(int b, int L, int H, int I) {
  return plans_for(MOETAIL_OP_TAIL, b, L, H, I).tail;
}
// The projection's plan and its partial bytes (0: it writes none, or no
// plan fits).
ProjPlan projection_plan(int kind, int b, int N, int K, size_t* bytes) {
  const ProjPlan p = plans_for(MOETAIL_OP_PROJECTION, b, N, K, kind).proj;
  *bytes = p.splits ? round_up(proj_partial_bytes(p, b, N, kind == MOETAIL_PROJ_GATEUP), 256) : 0;
  return p;
}
bool projection_dims_ok(int kind, int b, int N, int K) {
  return kind >= MOETAIL_PROJ_UPPROJ && kind <= MOETAIL_PROJ_DOWN && b > 0 &&
         b <= MOETAIL_MAX_GEMM_TOKENS && N > 0 && N % (kind == MOETAIL_PROJ_GATEUP ? 32 : 16) == 0 &&
         K > 0 && K % 32 == 0 && K <= MOETAIL_MAX_GEMM_K;
}

}  // namespace

extern "C" {

int moetail_finalize(const uint16_t* rows, int64_t rows_per_rank, const int32_t* permuted_idx,
                     const void* route_w, int route_w_dtype, const uint16_t* gamma,
                     float gain_center, float eps, int weight_before_norm, int b, int K, int P,
                     int tp, uint16_t* partials, uint16_t* out, hipStream_t stream) {
  if (b == 0) return MOETAIL_OK;
  if (weight_before_norm < MOETAIL_NORM_GAIN_AFTER || weight_before_norm > MOETAIL_NO_NORM)
    return MOETAIL_EINVAL;
  int st = check_norm_args(route_w, route_w_dtype, gamma, eps, K, P, tp, b,
                           weight_before_norm != MOETAIL_NO_NORM);
  if (st) return st;
  if (!a16(rows) || rows_per_rank <= 0 || permuted_idx == nullptr || !aligned(permuted_idx, 4))
    return MOETAIL_EINVAL;
  if (partials == nullptr && out == nullptr) return MOETAIL_EINVAL;
  if ((partials && !a16(partials)) || (out && !a16(out))) return MOETAIL_EINVAL;
  if (!__builtin_isfinite(gain_center)) return MOETAIL_EINVAL;
  EpArgs a{rows, rows_per_rank, permuted_idx, route_w, route_w_dtype == MOETAIL_BF16, gamma,
           gain_center, eps, weight_before_norm, b, K, P, tp, partials, out};
  return hip_status(launch_ep_finalize(a, stream));
}

int moetail_tp_finalize(const uint16_t* kpartials, int64_t num_rows, const int32_t* permuted_idx,
                        const void* route_w, int route_w_dtype, const uint16_t* gamma,
                        float gain_center, float eps, int weight_before_norm, int b, int K, int P,
                        int tp, uint16_t* out, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (b == 0) return MOETAIL_OK;
  if (weight_before_norm != 0 && weight_before_norm != 1) return MOETAIL_EINVAL;
  int st = check_norm_args(route_w, route_w_dtype, gamma, eps, K, P, tp, b);
  if (st) return st;
  if (!a16(kpartials) || num_rows <= 0 || permuted_idx == nullptr || !aligned(permuted_idx, 4) ||
      !a16(out) || !__builtin_isfinite(gain_center))
    return MOETAIL_EINVAL;
  const size_t need = tp_workspace(b, K, P, tp);
  if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < need)
    return MOETAIL_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  char* rows = ws + tp_gen_bytes(b) + tp_slot_bytes(b, K, P);
  TpArgs a{kpartials, num_rows, permuted_idx, route_w, route_w_dtype == MOETAIL_BF16, gamma,
           gain_center, eps, weight_before_norm != 0, b, K, P, tp, out,
           reinterpret_cast<unsigned*>(ws), reinterpret_cast<uint64_t*>(ws + tp_gen_bytes(b)),
           tp_wait_ticks.load(std::memory_order_relaxed), reinterpret_cast<uint16_t*>(rows),
           reinterpret_cast<float*>(rows + tp_rows_bytes(b, K, P))};
  return hip_status(launch_tp_finalize(a, stream));
}

int moetail_combine_norm_upproj(const uint16_t* latent_partials, int tp, const uint16_t* gamma,
                                float eps, const uint16_t* w_up, int N, const uint16_t* rs, int b,
                                int L, uint16_t* normed, uint16_t* out, int w_layout,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (b == 0) return MOETAIL_OK;
  if (b < 0 || tp <= 0 || N <= 0 || L <= 0 || !layout_ok(w_layout)) return MOETAIL_EINVAL;
  if (!(eps >= 0.0f) || eps == __builtin_inff()) return MOETAIL_EINVAL;
  if (!a16(latent_partials) || !a16(gamma) || !a16(w_up) || !a16(out)) return MOETAIL_EINVAL;
  if ((rs && !a16(rs)) || (normed && !a16(normed))) return MOETAIL_EINVAL;
  if (L % 32 || L > MOETAIL_MAX_WIDTH || N % 64 || tp > MOETAIL_MAX_TP ||
      b > MOETAIL_MAX_GEMM_TOKENS)
    return MOETAIL_EUNSUPPORTED;
  const UpprojLayout lay = upproj_plan(b, L, N);
  if (lay.plan.splits == 0) return MOETAIL_EUNSUPPORTED;
  const size_t need = (normed ? 0 : lay.y_bytes) + lay.part_bytes;
  if (need && (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < need))
    return MOETAIL_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  uint16_t* y = normed ? normed : reinterpret_cast<uint16_t*>(ws);
  float* part = lay.part_bytes ? reinterpret_cast<float*>(ws + (normed ? 0 : lay.y_bytes)) : nullptr;
  hipError_t e = launch_latent_norm(latent_partials, tp, b, L, gamma, eps, y, stream);
  if (e == hipSuccess) e = launch_linear(w_up, w_layout, N, L, y, b, rs, out, lay.plan, part, stream);
  return hip_status(e);
}

int moetail_projection_partials(int kind, const uint16_t* w0, const uint16_t* w1, int N, int K,
                                const uint16_t* x, int b, int w_layout, float* partials,
                                size_t partial_bytes, hipStream_t stream) {
  if (kind < MOETAIL_PROJ_UPPROJ || kind > MOETAIL_PROJ_DOWN) return MOETAIL_EINVAL;
  if (b == 0) return MOETAIL_OK;
  if (b < 0 || N <= 0 || K <= 0 || !layout_ok(w_layout)) return MOETAIL_EINVAL;
  if (!a16(w0) || !a16(x) || partials == nullptr || !aligned(partials, 256)) return MOETAIL_EINVAL;
  if (kind == MOETAIL_PROJ_GATEUP ? !a16(w1) : w1 != nullptr) return MOETAIL_EINVAL;
  if (!projection_dims_ok(kind, b, N, K)) return MOETAIL_EUNSUPPORTED;
  size_t need = 0;
  const ProjPlan plan = projection_plan(kind, b, N, K, &need);
  if (need == 0) return MOETAIL_EUNSUPPORTED;
  if (partial_bytes < need) return MOETAIL_EWORKSPACE;
  const int n0 = kind == MOETAIL_PROJ_GATEUP ? N / 2 : N;
  return hip_status(launch_projection_partials(w0, w1, n0, N, K, x, b,
                                               w_layout == MOETAIL_W_TILED, plan, partials,
                                               stream));
}

int moetail_shared_expert(const uint16_t* x, int b, int H, const uint16_t* w_gate,
                          const uint16_t* w_upw, int I, const uint16_t* w_down, uint16_t* h,
                          uint16_t* rs, int w_layout, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  if (b == 0) return MOETAIL_OK;
  if (b < 0 || H <= 0 || I <= 0 || !layout_ok(w_layout)) return MOETAIL_EINVAL;
  if (!a16(x) || !a16(w_gate) || !a16(w_upw) || !a16(w_down) || !a16(rs)) return MOETAIL_EINVAL;
  if (h && !a16(h)) return MOETAIL_EINVAL;
  if (H % 64 || I % 64 || H > MOETAIL_MAX_GEMM_K || I > MOETAIL_MAX_GEMM_K ||
      b > MOETAIL_MAX_GEMM_TOKENS)
    return MOETAIL_EUNSUPPORTED;
  const SharedLayout lay = shared_plan(b, H, I);
  if (lay.gate_up.splits == 0 || lay.down.splits == 0) return MOETAIL_EUNSUPPORTED;
  const size_t need = (h ? 0 : lay.h_bytes) + lay.part_bytes;
  if (need && (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < need))
    return MOETAIL_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  uint16_t* hb = h ? h : reinterpret_cast<uint16_t*>(ws);
  float* part = lay.part_bytes ? reinterpret_cast<float*>(ws + (h ? 0 : lay.h_bytes)) : nullptr;
  hipError_t e =
      launch_gate_up(w_gate, w_upw, w_layout, I, H, x, b, hb, lay.gate_up, part, stream);
  if (e == hipSuccess)
    e = launch_linear(w_down, w_layout, H, I, hb, b, nullptr, rs, lay.down, part, stream);
  return hip_status(e);
}

int moetail_tail(const uint16_t* latent_partials, int tp, const uint16_t* gamma, float eps,
                 const uint16_t* w_up, int L, const uint16_t* x, const uint16_t* w_gate,
                 const uint16_t* w_upw, const uint16_t* w_down, int H, int I, int b,
                 uint16_t* out, uint16_t* rs, uint16_t* normed, uint16_t* h, int w_layout,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (b == 0) return MOETAIL_OK;
  if (b < 0 || tp <= 0 || L <= 0 || H <= 0 || I <= 0 || !layout_ok(w_layout))
    return MOETAIL_EINVAL;
  if (!(eps >= 0.0f) || eps == __builtin_inff()) return MOETAIL_EINVAL;
  if (!a16(latent_partials) || !a16(gamma) || !a16(w_up) || !a16(x) || !a16(w_gate) ||
      !a16(w_upw) || !a16(w_down) || !a16(out))
    return MOETAIL_EINVAL;
  if ((rs && !a16(rs)) || (normed && !a16(normed)) || (h && !a16(h))) return MOETAIL_EINVAL;
  if (L % 32 || L > MOETAIL_MAX_WIDTH || H % 64 || I % 64 || H > MOETAIL_MAX_GEMM_K ||
      I > MOETAIL_MAX_GEMM_K || tp > MOETAIL_MAX_TP || b > MOETAIL_MAX_GEMM_TOKENS)
    return MOETAIL_EUNSUPPORTED;
  const TailLayout lay = tail_plan(b, L, H, I);
  if (!tail_ok(lay)) return MOETAIL_EUNSUPPORTED;
  const size_t need =
      lay.counter_bytes + (h ? 0 : lay.h_bytes) + (normed ? 0 : lay.y_bytes) + lay.part_bytes;
  if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < need)
    return MOETAIL_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  unsigned* counters = reinterpret_cast<unsigned*>(ws);
  ws += lay.counter_bytes;
  uint16_t* hb = h;
  if (!hb) {
    hb = reinterpret_cast<uint16_t*>(ws);
    ws += lay.h_bytes;
  }
  uint16_t* yb = normed;
  if (!yb) {
    yb = reinterpret_cast<uint16_t*>(ws);
    ws += lay.y_bytes;
  }
  TailArgs a{x, w_gate, w_upw, w_down, H, I, latent_partials, tp, gamma, eps, w_up, L, b, hb, yb,
             rs, out, reinterpret_cast<float*>(ws), lay.down_part_bytes, w_layout, counters};
  return hip_status(launch_tail(a, lay.gate_up, lay.down, lay.up, lay.group, stream));
}

int moetail_gate_up(const uint16_t* x, int b, int H, const uint16_t* w_gate,
                    const uint16_t* w_upw, int I, uint16_t* h,
                    const uint16_t* latent_partials, int tp, const uint16_t* gamma, float eps,
                    int L, uint16_t* normed, int w_layout, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  if (b == 0) return MOETAIL_OK;
  if (b < 0 || H <= 0 || I <= 0 || !layout_ok(w_layout)) return MOETAIL_EINVAL;
  if (!a16(x) || !a16(w_gate) || !a16(w_upw) || !a16(h)) return MOETAIL_EINVAL;
  if (H % 64 || I % 64 || H > MOETAIL_MAX_GEMM_K || I > MOETAIL_MAX_GEMM_K ||
      b > MOETAIL_MAX_GEMM_TOKENS)
    return MOETAIL_EUNSUPPORTED;
  if (latent_partials) {
    if (tp <= 0 || L <= 0 || !(eps >= 0.0f) || eps == __builtin_inff()) return MOETAIL_EINVAL;
    if (!a16(latent_partials) || !a16(gamma) || !a16(normed)) return MOETAIL_EINVAL;
    if (L % 32 || L > MOETAIL_MAX_WIDTH || tp > MOETAIL_MAX_TP) return MOETAIL_EUNSUPPORTED;
  }
  const GateUpLayout lay = gate_up_plan(b, H, I);
  if (lay.plan.splits == 0) return MOETAIL_EUNSUPPORTED;
  const size_t need = lay.counter_bytes + lay.part_bytes;
  if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < need)
    return MOETAIL_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  return hip_status(launch_gate_up_h(w_gate, w_upw, w_layout == MOETAIL_W_TILED, I, H, x, b, h,
                                     lay.plan, reinterpret_cast<float*>(ws + lay.counter_bytes),
                                     reinterpret_cast<unsigned*>(ws), latent_partials, tp, gamma,
                                     eps, L, normed, stream));
}

int moetail_pack_weights(const uint16_t* w, int64_t n, int k, uint16_t* packed,
                         hipStream_t stream) {
  if (n == 0) return MOETAIL_OK;
  if (n < 0 || k <= 0 || !a16(w) || !a16(packed)) return MOETAIL_EINVAL;
  if (n % 16 || k % 32) return MOETAIL_EUNSUPPORTED;
  const uintptr_t bytes = (uintptr_t)n * (uintptr_t)k * sizeof(uint16_t);
  const uintptr_t wi = reinterpret_cast<uintptr_t>(w), pi = reinterpret_cast<uintptr_t>(packed);
  if (wi < pi + bytes && pi < wi + bytes) return MOETAIL_EINVAL;  // overlapping
  return hip_status(launch_pack_weights(w, n, k, packed, stream));
}

}  // extern "C"

namespace {

// moetail_decode_tail with its workspace; the allocation-free variant passes
// this device's static scratch.
int decode_tail_impl(const uint16_t* rows, int64_t rows_per_rank, const int32_t* permuted_idx,
                     const void* route_w, int route_w_dtype, const uint16_t* fin_gamma,
                     float gain_center, float fin_eps, int weight_before_norm, int K,
                     uint16_t* latent_partials, int tp, const uint16_t* gamma, float eps,
                     const uint16_t* w_up, int L, const uint16_t* x, const uint16_t* w_gate,
                     const uint16_t* w_upw, const uint16_t* w_down, int H, int I, int b,
                     uint16_t* out, uint16_t* rs, uint16_t* normed, uint16_t* h, int w_layout,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  // the finalize's checks (P = L) ...
  if (weight_before_norm < MOETAIL_NORM_GAIN_AFTER || weight_before_norm > MOETAIL_NO_NORM)
    return MOETAIL_EINVAL;
  int st = check_norm_args(route_w, route_w_dtype, fin_gamma, fin_eps, K, L, tp, b,
                           weight_before_norm != MOETAIL_NO_NORM);
  if (st) return st;
  if (!a16(rows) || rows_per_rank <= 0 || permuted_idx == nullptr || !aligned(permuted_idx, 4) ||
      !a16(latent_partials) || !__builtin_isfinite(gain_center))
    return MOETAIL_EINVAL;
  // ... and the tail's
  if (b < 0 || H <= 0 || I <= 0 || !layout_ok(w_layout)) return MOETAIL_EINVAL;
  if (!(eps >= 0.0f) || eps == __builtin_inff()) return MOETAIL_EINVAL;
  if (!a16(gamma) || !a16(w_up) || !a16(x) || !a16(w_gate) || !a16(w_upw) || !a16(w_down) ||
      !a16(out))
    return MOETAIL_EINVAL;
  if ((rs && !a16(rs)) || (normed && !a16(normed)) || (h && !a16(h))) return MOETAIL_EINVAL;
  if (L % 32 || H % 64 || I % 64 || H > MOETAIL_MAX_GEMM_K || I > MOETAIL_MAX_GEMM_K ||
      b > MOETAIL_MAX_GEMM_TOKENS)
    return MOETAIL_EUNSUPPORTED;
  const TailLayout lay = tail_plan(b, L, H, I);
  if (!tail_ok(lay)) return MOETAIL_EUNSUPPORTED;
  const size_t need =
      lay.counter_bytes + (h ? 0 : lay.h_bytes) + (normed ? 0 : lay.y_bytes) + lay.part_bytes;
  if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < need)
    return MOETAIL_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  unsigned* counters = reinterpret_cast<unsigned*>(ws);
  ws += lay.counter_bytes;
  uint16_t* hb = h;
  if (!hb) {
    hb = reinterpret_cast<uint16_t*>(ws);
    ws += lay.h_bytes;
  }
  uint16_t* yb = normed;
  if (!yb) {
    yb = reinterpret_cast<uint16_t*>(ws);
    ws += lay.y_bytes;
  }
  TailArgs a{x, w_gate, w_upw, w_down, H, I, latent_partials, tp, gamma, eps, w_up, L, b, hb, yb,
             rs, out, reinterpret_cast<float*>(ws), lay.down_part_bytes, w_layout, counters};
  EpArgs ep{rows, rows_per_rank, permuted_idx, route_w, route_w_dtype == MOETAIL_BF16, fin_gamma,
            gain_center, fin_eps, weight_before_norm, b, K, L, tp, latent_partials, nullptr};
  hipError_t e = launch_ep_finalize(ep, stream);
  if (e == hipSuccess) e = launch_tail(a, lay.gate_up, lay.down, lay.up, lay.group, stream);
  return hip_status(e);
}

}  // namespace

extern "C" {

int moetail_decode_tail(const uint16_t* rows, int64_t rows_per_rank, const int32_t* permuted_idx,
                        const void* route_w, int route_w_dtype, const uint16_t* fin_gamma,
                        float gain_center, float fin_eps, int weight_before_norm, int K,
                        uint16_t* latent_partials, int tp, const uint16_t* gamma, float eps,
                        const uint16_t* w_up, int L, const uint16_t* x, const uint16_t* w_gate,
                        const uint16_t* w_upw, const uint16_t* w_down, int H, int I, int b,
                        uint16_t* out, uint16_t* rs, uint16_t* normed, uint16_t* h,
                        int w_layout, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (b == 0) return MOETAIL_OK;
  return decode_tail_impl(rows, rows_per_rank, permuted_idx, route_w, route_w_dtype, fin_gamma,
                          gain_center, fin_eps, weight_before_norm, K, latent_partials, tp, gamma,
                          eps, w_up, L, x, w_gate, w_upw, w_down, H, I, b, out, rs, normed, h,
                          w_layout, workspace, workspace_bytes, stream);
}

int moetail_decode_tail_noalloc(const uint16_t* rows, int64_t rows_per_rank,
                                const int32_t* permuted_idx, const void* route_w,
                                int route_w_dtype, const uint16_t* fin_gamma, float gain_center,
                                float fin_eps, int weight_before_norm, int K,
                                uint16_t* latent_partials, int tp, const uint16_t* gamma,
                                float eps, const uint16_t* w_up, int L, const uint16_t* x,
                                const uint16_t* w_gate, const uint16_t* w_upw,
                                const uint16_t* w_down, int H, int I, int b, uint16_t* out,
                                uint16_t* rs, uint16_t* normed, uint16_t* h, int w_layout,
                                hipStream_t stream) {
  if (b == 0) return MOETAIL_OK;
  void* ws = nullptr;
  const int st = scratch_for(stream, &ws);
  if (st) return st;
  return decode_tail_impl(rows, rows_per_rank, permuted_idx, route_w, route_w_dtype, fin_gamma,
                          gain_center, fin_eps, weight_before_norm, K, latent_partials, tp, gamma,
                          eps, w_up, L, x, w_gate, w_upw, w_down, H, I, b, out, rs, normed, h,
                          w_layout, ws, kScratchBytes, stream);
}

size_t moetail_workspace_bytes(int op, int b, int dim0, int dim1, int dim2) {
  if (op == MOETAIL_OP_TP_FINALIZE) {
    if (b <= 0 || b > MOETAIL_MAX_TOKENS || dim0 <= 0 || dim0 > MOETAIL_MAX_ROUTES || dim1 <= 0 ||
        dim1 % 8 || dim1 > MOETAIL_MAX_WIDTH)
      return 0;
    if (dim2 < 0 || dim2 > MOETAIL_MAX_TP) return 0;
    return tp_workspace(b, dim0, dim1, dim2);
  }
  if (b <= 0 || b > MOETAIL_MAX_GEMM_TOKENS) return 0;
  switch (op) {
    case MOETAIL_OP_COMBINE_NORM_UPPROJ: {
      if (dim0 <= 0 || dim1 <= 0 || dim0 % 32 || dim1 % 64 || dim0 > MOETAIL_MAX_WIDTH) return 0;
      (void)dim2;
      const UpprojLayout l = upproj_plan(b, dim0, dim1);
      return l.plan.splits ? l.y_bytes + l.part_bytes : 0;
    }
    case MOETAIL_OP_TAIL: {
      if (dim0 <= 0 || dim1 <= 0 || dim2 <= 0 || dim0 % 32 || dim0 > MOETAIL_MAX_WIDTH ||
          dim1 % 64 || dim2 % 64 || dim1 > MOETAIL_MAX_GEMM_K || dim2 > MOETAIL_MAX_GEMM_K)
        return 0;
      const TailLayout l = tail_plan(b, dim0, dim1, dim2);
      return tail_ok(l) ? l.counter_bytes + l.h_bytes + l.y_bytes + l.part_bytes : 0;
    }
    case MOETAIL_OP_GATE_UP: {
      if (dim0 <= 0 || dim1 <= 0 || dim0 % 64 || dim1 % 64 || dim0 > MOETAIL_MAX_GEMM_K ||
          dim1 > MOETAIL_MAX_GEMM_K)
        return 0;
      const GateUpLayout l = gate_up_plan(b, dim0, dim1);
      return l.plan.splits ? l.counter_bytes + l.part_bytes : 0;
    }
    case MOETAIL_OP_PROJECTION: {
      if (!projection_dims_ok(dim2, b, dim0, dim1)) return 0;
      size_t bytes = 0;
      projection_plan(dim2, b, dim0, dim1, &bytes);
      return bytes;
    }
    case MOETAIL_OP_SHARED_EXPERT: {
      if (dim0 <= 0 || dim1 <= 0 || dim0 % 64 || dim1 % 64 || dim0 > MOETAIL_MAX_GEMM_K ||
          dim1 > MOETAIL_MAX_GEMM_K)
        return 0;
      const SharedLayout l = shared_plan(b, dim0, dim1);
      return l.gate_up.splits && l.down.splits ? l.h_bytes + l.part_bytes : 0;
    }
    default:
      return 0;
  }
}

int moetail_set_projection_tuning(int kind, int splits, int waves, int blocks, int tiles_per_unit,
                                  int prefetch, int passes) {
  if (kind < MOETAIL_PROJ_UPPROJ || kind > MOETAIL_PROJ_DOWN) return MOETAIL_EINVAL;
  if (splits < 0 || waves < 0 || blocks < 0 || tiles_per_unit < 0 || prefetch < 0 || passes < 0)
    return MOETAIL_EINVAL;
  std::lock_guard<std::mutex> lock(plan_mutex);
  tunings[kind] = ProjTuning{splits, waves, blocks, tiles_per_unit, prefetch, passes};
  for (PlanSlot& e : plan_slots) e.used = false;  // plans made under the old overrides
  return MOETAIL_OK;
}

void moetail_set_tp_wait_limit(int64_t ticks) {
  tp_wait_ticks.store(ticks, std::memory_order_relaxed);
}

void moetail_plan_cache_stats(uint64_t* searches, uint64_t* hits) {
  if (searches) *searches = plan_searches.load(std::memory_order_relaxed);
  if (hits) *hits = plan_hits.load(std::memory_order_relaxed);
}

const char* moetail_status_string(int status) {
  switch (status) {
    case MOETAIL_OK: return "ok";
    case MOETAIL_EINVAL: return "invalid argument (null pointer, shape, dtype or alignment)";
    case MOETAIL_EUNSUPPORTED: return "unsupported size (outside the library's limits)";
    case MOETAIL_EWORKSPACE: return "workspace missing or too small";
    case MOETAIL_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
