// C ABI of the GBLA library: argument validation, workspace carving and the
// launch sequence of the forward and backward passes (see include/gbla.h).
#include "gbla.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>

#include "internal.h"

using namespace gbla;

namespace {

// ---------------------------------------------------------------- workspace plan
struct Carver {
  size_t off = 0;
  template <typename P> P* take(char* base, size_t bytes) {
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off += (bytes + 255) & ~size_t(255);
    return p;
  }
};

struct Dims {
  int N, T, d, H, dh, D, E, NP, Kp, slots, nsplit, conv_rb;
  bool softmax;  // softmax key gate: the gate array holds logits, saved ends with the logit maxima
  bool gated;    // gated RMSNorm output (Eq. (7)): a fourth projection segment R
  float eps;     // its RMSNorm epsilon
  size_t esz;    // bytes per activation element
};

Dims dims_of(const gbla_problem* p) {
  Dims m;
  m.N = p->num_seqs; m.T = p->total_tokens; m.d = p->d_model; m.H = p->num_heads; m.dh = p->head_dim;
  m.gated = p->output_gate == GBLA_OUTPUT_GATED_RMSNORM;
  m.eps = p->norm_eps;
  m.D = m.H * m.dh; m.E = m.dh * m.dh + m.dh; m.NP = proj_cols(m.dh, m.gated); m.Kp = grad_cols(m.H, m.dh, m.gated);
  m.slots = max_chunks(m.T, m.N);
  const int dt = p->dtype == GBLA_DTYPE_BF16 ? BF16 : F32;
  m.nsplit = dw_splits(dt, m.d, m.Kp, m.T);
  m.conv_rb = dx_token_tiles(p->dtype == GBLA_DTYPE_BF16 ? BF16 : F32, m.T, m.d);
  m.esz = p->dtype == GBLA_DTYPE_BF16 ? 2 : 4;
  m.softmax = p->gate == GBLA_GATE_SOFTMAX;
  return m;
}

// activations kept from the forward for the backward (ra: the gated output's R),
// with the batch's chunk table, which the backward then need not rebuild
struct Act {
  int* nchunks; int* chunk_off; Chunk* tab;
  void* xt; void* qa; void* ka; void* va; float* ga; void* ra;
};

Act carve_act(const Dims& m, Carver& c, char* base) {
  Act a;
  const size_t TD = (size_t)m.T * m.D * m.esz;
  a.nchunks = c.take<int>(base, sizeof(int));
  a.chunk_off = c.take<int>(base, sizeof(int) * (m.N + 1));
  a.tab = c.take<Chunk>(base, sizeof(Chunk) * m.slots);
  a.xt = c.take<char>(base, (size_t)m.T * m.d * m.esz);
  a.qa = c.take<char>(base, TD);
  a.ka = c.take<char>(base, TD);
  a.va = c.take<char>(base, TD);
  a.ga = c.take<float>(base, sizeof(float) * (size_t)m.T * m.H);
  a.ra = m.gated ? c.take<char>(base, TD) : nullptr;
  return a;
}

size_t act_bytes(const Dims& m) {
  Carver c;
  carve_act(m, c, nullptr);
  return c.off;
}

struct FwdWs {
  void* wp; float* partial; float* mpart; Act act;
};
struct BwdWs {
  void* wp; void* wt; float* partial; float* dsz; float* dbg_part;
  float* dgam_part; void* G; void* edge; float* dw_part; float* dconv_part; Act act;
};

// The workspace of gbla_forward always has room for the activations, so it
// suffices whether or not the caller passes an activation cache; the
// allocation-free forward reserves that region only when no cache is passed
// (act_region). The activations are the last region, so the two sizes differ
// by exactly act_bytes(m).
size_t plan_fwd(const Dims& m, char* base, FwdWs* w, bool act_region = true) {
  Carver c;
  FwdWs t;
  t.wp = c.take<char>(base, (size_t)m.H * m.NP * m.d * m.esz);
  t.partial = c.take<float>(base, sizeof(float) * (size_t)m.slots * m.H * m.E);
  t.mpart = m.softmax ? c.take<float>(base, sizeof(float) * (size_t)m.slots * m.H) : nullptr;
  t.act = act_region ? carve_act(m, c, base) : Act{};
  if (w) *w = t;
  return c.off;
}

size_t plan_bwd(const Dims& m, char* base, BwdWs* w) {
  Carver c;
  BwdWs t;
  t.wp = c.take<char>(base, (size_t)m.H * m.NP * m.d * m.esz);
  t.wt = c.take<char>(base, (size_t)wt_rows(m.d) * m.Kp * m.esz);
  t.partial = c.take<float>(base, sizeof(float) * (size_t)m.slots * m.H * m.E);
  t.dsz = c.take<float>(base, sizeof(float) * (size_t)m.N * m.H * m.E);
  t.dbg_part = c.take<float>(base, sizeof(float) * (size_t)m.slots * m.H);
  t.dgam_part = m.gated ? c.take<float>(base, sizeof(float) * (size_t)m.slots * m.H * m.dh) : nullptr;
  t.G = c.take<char>(base, (size_t)m.T * m.Kp * m.esz);
  t.edge = c.take<char>(base, m.esz * (size_t)std::max(1, m.conv_rb) * 6 * m.d);
  t.dw_part = c.take<float>(base, sizeof(float) * (size_t)m.nsplit * m.d * m.Kp);
  t.dconv_part = c.take<float>(base, sizeof(float) * (size_t)std::max(1, m.conv_rb) * m.d * 4);
  t.act = carve_act(m, c, base);
  if (w) *w = t;
  return c.off;
}

gbla_status check_problem(const gbla_problem* p) {
  if (!p) return GBLA_ERR_NULL_ARG;
  if (p->dtype != GBLA_DTYPE_F32 && p->dtype != GBLA_DTYPE_BF16) return GBLA_ERR_UNSUPPORTED;
  if (p->head_dim != 32 && p->head_dim != 64) return GBLA_ERR_UNSUPPORTED;
  if ((p->gate != GBLA_GATE_SIGMOID && p->gate != GBLA_GATE_SOFTMAX) || p->conv_width != 4)
    return GBLA_ERR_UNSUPPORTED;
  if (p->output_gate != GBLA_OUTPUT_PLAIN && p->output_gate != GBLA_OUTPUT_GATED_RMSNORM) return GBLA_ERR_UNSUPPORTED;
  if (p->output_gate == GBLA_OUTPUT_GATED_RMSNORM && !(std::isfinite(p->norm_eps) && p->norm_eps >= 0.f))
    return GBLA_ERR_BAD_SHAPE;
  if (p->num_seqs < 1 || p->total_tokens < 0 || p->num_heads < 1 || p->d_model < 8 || p->d_model % 8 != 0)
    return GBLA_ERR_BAD_SHAPE;
  const long long T = p->total_tokens;
  const long long widest =
      std::max<long long>(p->d_model, grad_cols(p->num_heads, p->head_dim, p->output_gate != GBLA_OUTPUT_PLAIN));
  // widest < 2^21: a chunk's rows of the widest array fit the kernels' 32-bit buffer offsets
  if (T * widest >= (1LL << 31) || widest >= (1LL << 21) ||
      (long long)p->num_heads * p->head_dim * 4 + 64 >= (1LL << 24) ||
      (long long)p->num_seqs >= (1LL << 24) ||
      (long long)wt_rows(p->d_model) * grad_cols(p->num_heads, p->head_dim, p->output_gate != GBLA_OUTPUT_PLAIN) >=
          (1LL << 31))
    return GBLA_ERR_BAD_SHAPE;
  return GBLA_OK;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

// argument checks of the forward entry points (everything but the workspace)
gbla_status check_forward_args(const gbla_problem* p, const void* x, const int32_t* cu_seqlens, const void* conv_w,
                               const void* w_q, const void* w_k, const void* w_v, const void* w_g, const float* b_g,
                               const void* w_r, const float* gamma, const void* y, const float* saved,
                               const void* act) {
  gbla_status st = check_problem(p);
  if (st != GBLA_OK) return st;
  if (!cu_seqlens || !conv_w || !w_q || !w_k || !w_v || !w_g || !b_g || !saved) return GBLA_ERR_NULL_ARG;
  if (p->total_tokens > 0 && (!x || !y)) return GBLA_ERR_NULL_ARG;
  const bool gated = p->output_gate == GBLA_OUTPUT_GATED_RMSNORM;
  if (gated != (w_r != nullptr) || (!gated && gamma)) return GBLA_ERR_NULL_ARG;
  for (const void* a : {x, conv_w, w_q, w_k, w_v, w_g, w_r, y, (const void*)saved, act})
    if (!aligned(a, 16)) return GBLA_ERR_MISALIGNED;
  if (!aligned(b_g, 4) || !aligned(gamma, 4) || !aligned(cu_seqlens, 4)) return GBLA_ERR_MISALIGNED;
  return GBLA_OK;
}

// the forward's launch sequence on a carved workspace w (w.act: the activations)
gbla_status enqueue_forward(const gbla_problem* p, const Dims& m, const void* x, const int32_t* cu_seqlens,
                            const void* conv_w, const void* w_q, const void* w_k, const void* w_v, const void* w_g,
                            const float* b_g, const void* w_r, const float* gamma, void* y, float* saved,
                            const FwdWs& w, hipStream_t s) {
  const int dt = p->dtype == GBLA_DTYPE_BF16 ? BF16 : F32;
  const Act& A = w.act;
  (void)hipGetLastError();
  const ProjPackArgs pack{w_q, w_k, w_v, w_r, m.d, m.H, m.dh, w.wp};
  { StageScope ps(ST_CONV_FWD, s);  // with the projection's weight packing and the chunk table
    launch_conv_fwd(dt, x, cu_seqlens, m.N, m.T, m.d, m.H, conv_w, w_g, b_g, m.softmax, A.xt, A.ga, s, &pack,
                    Sched{cu_seqlens, m.N, m.T, kChunk, m.slots, A.nchunks, A.chunk_off, A.tab}); }
  { StageScope ps(ST_PROJ_FWD, s);
    launch_proj(dt, m.dh, A.xt, w.wp, m.T, m.d, m.H, A.qa, A.ka, A.va, s, true, A.ra); }
  { StageScope ps(ST_STATE_PARTIAL, s);
    launch_state_partial(dt, m.dh, A.ka, A.va, A.ga, A.nchunks, A.tab, m.slots, m.H, w.partial, w.mpart, s); }
  { StageScope ps(ST_COMBINE_STATE, s);  // softmax gate: the logit maxima follow the N*H states
    launch_combine(w.partial, A.nchunks, A.chunk_off, m.N, m.H, m.E, saved, s, w.mpart,
                   m.softmax ? saved + (size_t)m.N * m.H * m.E : nullptr); }
  { StageScope ps(ST_READOUT, s);
    launch_readout(dt, m.dh, A.qa, saved, A.nchunks, A.tab, m.slots, m.H, y, s, A.ra, gamma, m.eps); }
  return hipGetLastError() == hipSuccess ? GBLA_OK : GBLA_ERR_HIP;
}

// ---------------------------------------------------------------- static scratch
// The allocation-free forward carves its workspace from this array. Every GPU
// the library runs on holds its own copy, at its own address, until the process
// ends. The array's name is a host-side stand-in in host code: its device
// address is obtained once per device with hipGetSymbolAddress (with that
// device current) and only that address is ever handed to kernels.
__device__ __align__(256) char scratch[GBLA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<char*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// device address of the current device's scratch array (null on failure)
char* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  char* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!ptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    ptr = static_cast<char*>(addr);
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace

extern "C" {

const char* gbla_status_string(int status) {
  switch (status) {
    case GBLA_OK: return "GBLA_OK";
    case GBLA_ERR_NULL_ARG: return "GBLA_ERR_NULL_ARG: a required pointer is NULL";
    case GBLA_ERR_BAD_SHAPE: return "GBLA_ERR_BAD_SHAPE: sizes out of the supported range";
    case GBLA_ERR_UNSUPPORTED: return "GBLA_ERR_UNSUPPORTED: dtype, head_dim, gate or conv width not supported";
    case GBLA_ERR_MISALIGNED: return "GBLA_ERR_MISALIGNED: pointer alignment violated";
    case GBLA_ERR_WORKSPACE_TOO_SMALL: return "GBLA_ERR_WORKSPACE_TOO_SMALL: workspace below the size query";
    case GBLA_ERR_HIP: return "GBLA_ERR_HIP: a HIP launch failed";
    case GBLA_ERR_SCRATCH_LIMIT:
      return "GBLA_ERR_SCRATCH_LIMIT: the problem needs more than the allocation-free entry point's static scratch";
    default: return "unknown gbla_status";
  }
}

int gbla_version(void) { return 5; }

gbla_status gbla_saved_size(const gbla_problem* p, size_t* bytes) {
  if (!bytes) return GBLA_ERR_NULL_ARG;
  const gbla_status st = check_problem(p);
  if (st != GBLA_OK) return st;
  const size_t NH = (size_t)p->num_seqs * p->num_heads;
  *bytes = sizeof(float) * NH * (p->head_dim * p->head_dim + p->head_dim + (p->gate == GBLA_GATE_SOFTMAX ? 1 : 0));
  return GBLA_OK;
}

gbla_status gbla_workspace_size(const gbla_problem* p, int backward, size_t* bytes) {
  if (!bytes) return GBLA_ERR_NULL_ARG;
  const gbla_status st = check_problem(p);
  if (st != GBLA_OK) return st;
  const Dims m = dims_of(p);
  *bytes = backward ? plan_bwd(m, nullptr, nullptr) : plan_fwd(m, nullptr, nullptr);
  return GBLA_OK;
}

gbla_status gbla_activation_size(const gbla_problem* p, size_t* bytes) {
  if (!bytes) return GBLA_ERR_NULL_ARG;
  const gbla_status st = check_problem(p);
  if (st != GBLA_OK) return st;
  *bytes = act_bytes(dims_of(p));
  return GBLA_OK;
}

gbla_status gbla_forward(const gbla_problem* p, const void* x, const int32_t* cu_seqlens, const void* conv_w,
                         const void* w_q, const void* w_k, const void* w_v, const void* w_g, const float* b_g,
                         const void* w_r, const float* gamma, void* y, float* saved, void* act, void* workspace,
                         size_t workspace_bytes, void* stream) {
  gbla_status st = check_forward_args(p, x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, w_r, gamma, y, saved, act);
  if (st != GBLA_OK) return st;
  if (!workspace) return GBLA_ERR_NULL_ARG;
  if (!aligned(workspace, 16)) return GBLA_ERR_MISALIGNED;
  const Dims m = dims_of(p);
  FwdWs w;
  if (workspace_bytes < plan_fwd(m, static_cast<char*>(workspace), &w)) return GBLA_ERR_WORKSPACE_TOO_SMALL;
  if (act) {
    Carver c;
    w.act = carve_act(m, c, static_cast<char*>(act));
  }
  return enqueue_forward(p, m, x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, w_r, gamma, y, saved, w,
                         static_cast<hipStream_t>(stream));
}

gbla_status gbla_forward_noalloc(const gbla_problem* p, const void* x, const int32_t* cu_seqlens, const void* conv_w,
                                 const void* w_q, const void* w_k, const void* w_v, const void* w_g, const float* b_g,
                                 const void* w_r, const float* gamma, void* y, float* saved, void* act,
                                 void* stream) {
  gbla_status st = check_forward_args(p, x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, w_r, gamma, y, saved, act);
  if (st != GBLA_OK) return st;
  const Dims m = dims_of(p);
  // without a cache the activations live in the scratch too
  if (plan_fwd(m, nullptr, nullptr, act == nullptr) > (size_t)GBLA_STATIC_SCRATCH_BYTES) return GBLA_ERR_SCRATCH_LIMIT;
  char* base = scratch_for_current_device();
  if (!base) return GBLA_ERR_HIP;
  FwdWs w;
  plan_fwd(m, base, &w, act == nullptr);
  if (act) {
    Carver c;
    w.act = carve_act(m, c, static_cast<char*>(act));
  }
  return enqueue_forward(p, m, x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, w_r, gamma, y, saved, w,
                         static_cast<hipStream_t>(stream));
}

gbla_status gbla_backward(const gbla_problem* p, const void* x, const int32_t* cu_seqlens, const void* conv_w,
                          const void* w_q, const void* w_k, const void* w_v, const void* w_g, const float* b_g,
                          const void* w_r, const float* gamma, const float* saved, const void* act, const void* dy,
                          void* dx, float* dconv_w, float* dw_q, float* dw_k, float* dw_v, float* dw_g, float* db_g,
                          float* dw_r, float* dgamma, void* workspace, size_t workspace_bytes, void* stream) {
  gbla_status st = check_problem(p);
  if (st != GBLA_OK) return st;
  if (!cu_seqlens || !conv_w || !w_q || !w_k || !w_v || !w_g || !b_g || !saved || !dconv_w || !dw_q || !dw_k ||
      !dw_v || !dw_g || !db_g || !workspace)
    return GBLA_ERR_NULL_ARG;
  if (p->total_tokens > 0 && (!x || !dy || !dx)) return GBLA_ERR_NULL_ARG;
  const bool gated = p->output_gate == GBLA_OUTPUT_GATED_RMSNORM;
  if (gated != (w_r != nullptr) || gated != (dw_r != nullptr) || (gamma != nullptr) != (dgamma != nullptr) ||
      (!gated && gamma))
    return GBLA_ERR_NULL_ARG;
  for (const void* a : {x, conv_w, w_q, w_k, w_v, w_g, w_r, (const void*)saved, act, dy, (const void*)dx,
                        (const void*)dw_q, (const void*)dw_k, (const void*)dw_v, (const void*)dw_g, (const void*)dw_r,
                        (const void*)workspace})
    if (!aligned(a, 16)) return GBLA_ERR_MISALIGNED;
  if (!aligned(b_g, 4) || !aligned(db_g, 4) || !aligned(dconv_w, 4) || !aligned(cu_seqlens, 4) ||
      !aligned(gamma, 4) || !aligned(dgamma, 4))
    return GBLA_ERR_MISALIGNED;
  const Dims m = dims_of(p);
  BwdWs w;
  if (workspace_bytes < plan_bwd(m, static_cast<char*>(workspace), &w)) return GBLA_ERR_WORKSPACE_TOO_SMALL;
  if (act) {
    Carver c;
    w.act = carve_act(m, c, static_cast<char*>(const_cast<void*>(act)));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int dt = p->dtype == GBLA_DTYPE_BF16 ? BF16 : F32;
  const Act& A = w.act;

  (void)hipGetLastError();
  // with an activation cache the chunk table is the forward's; without one,
  // the recomputation's conv launch builds it in the workspace
  if (!act) {  // recompute x~, g, phi(q), phi(k), v into the workspace
    const ProjPackArgs pack{w_q, w_k, w_v, w_r, m.d, m.H, m.dh, w.wp};
    { StageScope ps(ST_CONV_RECOMPUTE, s);  // with the projection's weight packing and the chunk table
      launch_conv_fwd(dt, x, cu_seqlens, m.N, m.T, m.d, m.H, conv_w, w_g, b_g, m.softmax, A.xt, A.ga, s, &pack,
                      Sched{cu_seqlens, m.N, m.T, kChunk, m.slots, A.nchunks, A.chunk_off, A.tab}); }
    { StageScope ps(ST_PROJ_RECOMPUTE, s);
      launch_proj(dt, m.dh, A.xt, w.wp, m.T, m.d, m.H, A.qa, A.ka, A.va, s, true, A.ra); }
  }
  { StageScope ps(ST_BWD_DSTATE, s);
    launch_bwd_dstate(dt, m.dh, A.qa, dy, saved, A.nchunks, A.tab, m.slots, m.H, m.Kp, w.partial, w.G, s, A.ra,
                      gamma, m.eps, gamma ? w.dgam_part : nullptr); }
  { StageScope ps(ST_COMBINE_DSTATE, s);  // with the packing of the dX~ GEMM's weights
    const WtPackArgs pack{w_q, w_k, w_v, w_r, w_g, m.d, m.H, m.dh, m.Kp, w.wt};
    launch_combine(w.partial, A.nchunks, A.chunk_off, m.N, m.H, m.E, w.dsz, s, nullptr, nullptr, &pack, dt); }
  { StageScope ps(ST_BWD_TOKEN, s);
    launch_bwd_token(dt, m.dh, A.ka, A.va, A.ga, w.dsz, A.nchunks, A.tab, m.slots, m.H, m.Kp, m.gated ? 4 : 3, w.G,
                     w.dbg_part,
                     m.softmax ? saved + (size_t)m.N * m.H * m.E : nullptr, s); }
  if (m.T > 0) {  // dX~ = G Wt^T with the conv's vector-Jacobian product in its epilogue
    StageScope ps(ST_GEMM_DX, s);
    launch_gemm_dx_conv(dt, w.G, w.wt, m.T, m.d, m.Kp, grad_cols_read(m.H, m.dh, m.gated), x, cu_seqlens, m.N,
                        conv_w, dx, w.dconv_part, w.edge, s);
  }
  { StageScope ps(ST_GEMM_DW, s); launch_gemm_dw(dt, A.xt, w.G, m.T, m.d, m.Kp, m.nsplit, w.dw_part, s); }
  {
    StageScope ps(ST_FINALIZE, s);
    BwdFinalize f{};
    f.dw_part = w.dw_part; f.nsplit = m.nsplit; f.d = m.d; f.H = m.H; f.dh = m.dh; f.Kp = m.Kp;
    f.dw_blocks = bwd_finalize_dw_blocks(m.d, m.Kp);
    f.dw_q = dw_q; f.dw_k = dw_k; f.dw_v = dw_v; f.dw_r = dw_r; f.dw_g = dw_g;
    f.dconv_part = w.dconv_part; f.conv_rb = m.conv_rb; f.dconv_w = dconv_w;
    f.nchunks = A.nchunks; f.dbg_part = w.dbg_part; f.db_g = db_g;
    f.dgam_part = gamma ? w.dgam_part : nullptr; f.dgamma = gamma ? dgamma : nullptr;
    f.dt = dt; f.tile_rows = dx_token_tile_rows(dt, m.T, m.d); f.nseq = m.N;
    f.edge = m.T > 0 ? w.edge : nullptr; f.conv_w = conv_w; f.cu = cu_seqlens; f.dx = dx;
    launch_bwd_finalize(f, s);
  }
  return hipGetLastError() == hipSuccess ? GBLA_OK : GBLA_ERR_HIP;
}

}  // extern "C"
