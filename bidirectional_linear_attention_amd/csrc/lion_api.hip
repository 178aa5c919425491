// C ABI of the LION-s layer: argument validation, workspace carving and the
// launch sequence of the forward and backward passes (see include/lion.h).
#include "lion.h"

#include <algorithm>

#include "internal.h"
#include "lion_internal.h"

using namespace gbla;

namespace {

struct Carver {
  size_t off = 0;
  template <typename P> P* take(char* base, size_t bytes) {
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off += (bytes + 255) & ~size_t(255);
    return p;
  }
};

struct LDims {
  int N, T, d, H, dh, D, E, Kp, slots, nsplit;
  size_t esz;
};

LDims dims_of(const lion_problem* p) {
  LDims m;
  m.N = p->num_seqs; m.T = p->total_tokens; m.d = p->d_model; m.H = p->num_heads; m.dh = p->head_dim;
  m.D = m.H * m.dh; m.E = m.dh * m.dh + m.dh; m.Kp = grad_cols(m.H, m.dh);
  m.slots = max_chunks(m.T, m.N, kLionChunk);
  const int dt = p->dtype == GBLA_DTYPE_BF16 ? BF16 : F32;
  m.nsplit = dw_splits(dt, m.d, m.Kp, m.T);
  m.esz = p->dtype == GBLA_DTYPE_BF16 ? 2 : 4;
  return m;
}

// activations kept from the forward for the backward
struct LAct { void* q; void* k; void* v; float* logl; float* rsum; float* st; float* lam; };

LAct carve_act(const LDims& m, Carver& c, char* base) {
  LAct a;
  const size_t TD = (size_t)m.T * m.D * m.esz, TH = sizeof(float) * (size_t)m.T * m.H;
  a.q = c.take<char>(base, TD);
  a.k = c.take<char>(base, TD);
  a.v = c.take<char>(base, TD);
  a.logl = c.take<float>(base, TH);
  a.rsum = c.take<float>(base, TH);
  a.st = c.take<float>(base, sizeof(float) * (size_t)m.slots * m.H * 2 * m.E);
  a.lam = c.take<float>(base, sizeof(float) * (size_t)m.slots * m.H);
  return a;
}

size_t act_bytes(const LDims& m) {
  Carver c;
  carve_act(m, c, nullptr);
  return c.off;
}

struct LFwdWs { int* nchunks; int* chunk_off; Chunk* tab; void* wp; LAct act; };
struct LBwdWs {
  int* nchunks; int* chunk_off; Chunk* tab; void* wt; float* hst; void* hrows; float* dA_loc; float* dA_tot;
  float* db_part; void* G; float* dw_part;
};

size_t plan_fwd(const LDims& m, char* base, LFwdWs* w) {
  Carver c;
  LFwdWs t;
  t.nchunks = c.take<int>(base, sizeof(int));
  t.chunk_off = c.take<int>(base, sizeof(int) * (m.N + 1));
  t.tab = c.take<Chunk>(base, sizeof(Chunk) * m.slots);
  t.wp = c.take<char>(base, (size_t)m.H * proj_cols(m.dh) * m.d * m.esz);
  t.act = carve_act(m, c, base);
  if (w) *w = t;
  return c.off;
}

size_t plan_bwd(const LDims& m, char* base, LBwdWs* w) {
  Carver c;
  LBwdWs t;
  t.nchunks = c.take<int>(base, sizeof(int));
  t.chunk_off = c.take<int>(base, sizeof(int) * (m.N + 1));
  t.tab = c.take<Chunk>(base, sizeof(Chunk) * m.slots);
  t.wt = c.take<char>(base, (size_t)wt_rows(m.d) * m.Kp * m.esz);
  t.hst = c.take<float>(base, sizeof(float) * (size_t)m.slots * m.H * 2 * m.E);
  t.hrows = c.take<char>(base, (size_t)m.slots * m.H * 2 * m.dh * m.dh * m.esz);
  t.dA_loc = c.take<float>(base, sizeof(float) * (size_t)m.T * m.H);
  t.dA_tot = c.take<float>(base, sizeof(float) * (size_t)m.slots * m.H);
  t.db_part = c.take<float>(base, sizeof(float) * (size_t)m.slots * m.H);
  t.G = c.take<char>(base, (size_t)m.T * m.Kp * m.esz);
  t.dw_part = c.take<float>(base, sizeof(float) * (size_t)m.nsplit * m.d * m.Kp);
  if (w) *w = t;
  return c.off;
}

gbla_status check_problem(const lion_problem* p) {
  if (!p) return GBLA_ERR_NULL_ARG;
  if (p->dtype != GBLA_DTYPE_F32 && p->dtype != GBLA_DTYPE_BF16) return GBLA_ERR_UNSUPPORTED;
  if (p->head_dim != 32 && p->head_dim != 64) return GBLA_ERR_UNSUPPORTED;
  if (p->chunk != kLionChunk) return GBLA_ERR_UNSUPPORTED;
  if (p->decay != LION_DECAY_SELECTIVE && p->decay != LION_DECAY_FIXED && p->decay != LION_DECAY_NONE)
    return GBLA_ERR_UNSUPPORTED;
  if (p->num_seqs < 1 || p->total_tokens < 0 || p->num_heads < 1 || p->d_model < 8 || p->d_model % 8 != 0)
    return GBLA_ERR_BAD_SHAPE;
  const long long T = p->total_tokens;
  const long long widest = std::max<long long>(p->d_model, grad_cols(p->num_heads, p->head_dim));
  // widest < 2^21: a run of rows of the widest array fits the kernels' 32-bit buffer offsets
  if (T * widest >= (1LL << 31) || widest >= (1LL << 21) ||
      (long long)p->num_heads * p->head_dim * 4 + 64 >= (1LL << 24) ||
      (long long)p->num_seqs >= (1LL << 24) ||
      (long long)wt_rows(p->d_model) * grad_cols(p->num_heads, p->head_dim) >= (1LL << 31))
    return GBLA_ERR_BAD_SHAPE;
  const long long slots = (T + kLionChunk - 1) / kLionChunk + p->num_seqs;
  const long long E = (long long)p->head_dim * p->head_dim + p->head_dim;
  if (slots * p->num_heads * 2 * E >= (1LL << 40)) return GBLA_ERR_BAD_SHAPE;
  return GBLA_OK;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

}  // namespace

extern "C" {

gbla_status lion_workspace_size(const lion_problem* p, int backward, size_t* bytes) {
  if (!bytes) return GBLA_ERR_NULL_ARG;
  const gbla_status st = check_problem(p);
  if (st != GBLA_OK) return st;
  const LDims m = dims_of(p);
  *bytes = backward ? plan_bwd(m, nullptr, nullptr) : plan_fwd(m, nullptr, nullptr);
  return GBLA_OK;
}

gbla_status lion_activation_size(const lion_problem* p, size_t* bytes) {
  if (!bytes) return GBLA_ERR_NULL_ARG;
  const gbla_status st = check_problem(p);
  if (st != GBLA_OK) return st;
  *bytes = act_bytes(dims_of(p));
  return GBLA_OK;
}

gbla_status lion_forward(const lion_problem* p, const void* x, const int32_t* cu_seqlens, const void* w_q,
                         const void* w_k, const void* w_v, const void* w_lam, const float* b_lam, void* y, void* act,
                         void* workspace, size_t workspace_bytes, void* stream) {
  gbla_status st = check_problem(p);
  if (st != GBLA_OK) return st;
  const bool sel = p->decay == LION_DECAY_SELECTIVE, fixed = p->decay == LION_DECAY_FIXED;
  if (!cu_seqlens || !w_q || !w_k || !w_v || !workspace || (sel && !w_lam) || ((sel || fixed) && !b_lam))
    return GBLA_ERR_NULL_ARG;
  if (p->total_tokens > 0 && (!x || !y)) return GBLA_ERR_NULL_ARG;
  for (const void* a : {x, w_q, w_k, w_v, w_lam, (const void*)y, (const void*)act, (const void*)workspace})
    if (!aligned(a, 16)) return GBLA_ERR_MISALIGNED;
  if (!aligned(b_lam, 4) || !aligned(cu_seqlens, 4)) return GBLA_ERR_MISALIGNED;
  const LDims m = dims_of(p);
  LFwdWs w;
  if (workspace_bytes < plan_fwd(m, static_cast<char*>(workspace), &w)) return GBLA_ERR_WORKSPACE_TOO_SMALL;
  if (act) {
    Carver c;
    w.act = carve_act(m, c, static_cast<char*>(act));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int dt = p->dtype == GBLA_DTYPE_BF16 ? BF16 : F32;
  const LAct& A = w.act;

  (void)hipGetLastError();
  { StageScope ps(ST_PACK_PROJ, s);  // and the chunk table
    launch_pack_proj(dt, w_q, w_k, w_v, nullptr, m.d, m.H, m.dh, w.wp,
                     Sched{cu_seqlens, m.N, m.T, kLionChunk, m.slots, w.nchunks, w.chunk_off, w.tab}, s); }
  { StageScope ps(ST_LION_LOG_DECAY, s);
    if (sel) launch_log_decay(dt, x, cu_seqlens, m.N, m.T, m.d, m.H, w_lam, b_lam, A.logl, s);
    else launch_const_log_decay(m.T, m.H, fixed ? b_lam : nullptr, A.logl, s); }
  { StageScope ps(ST_LION_PROJ, s); launch_proj(dt, m.dh, x, w.wp, m.T, m.d, m.H, A.q, A.k, A.v, s, false); }
  { StageScope ps(ST_LION_CHUNK_STATE, s);
    launch_lion_chunk_state(dt, m.dh, 0, A.k, A.v, nullptr, nullptr, A.logl, w.nchunks, w.tab, m.slots, m.H, A.st,
                            A.lam, s); }
  { StageScope ps(ST_LION_SCAN, s);
    launch_lion_scan(A.st, A.lam, w.nchunks, w.chunk_off, m.N, m.H, m.E, dt, nullptr, m.dh, s); }
  { StageScope ps(ST_LION_READOUT, s);
    launch_lion_readout(dt, m.dh, A.q, A.k, A.v, A.logl, A.st, w.nchunks, w.tab, m.slots, m.H, y, A.rsum, s); }
  return hipGetLastError() == hipSuccess ? GBLA_OK : GBLA_ERR_HIP;
}

gbla_status lion_backward(const lion_problem* p, const void* x, const int32_t* cu_seqlens, const void* w_q,
                          const void* w_k, const void* w_v, const void* w_lam, const float* b_lam, const void* act,
                          const void* y, const void* dy, void* dx, float* dw_q, float* dw_k, float* dw_v,
                          float* dw_lam, float* db_lam, void* workspace, size_t workspace_bytes, void* stream) {
  gbla_status st = check_problem(p);
  if (st != GBLA_OK) return st;
  const bool sel = p->decay == LION_DECAY_SELECTIVE, fixed = p->decay == LION_DECAY_FIXED;
  if (!cu_seqlens || !w_q || !w_k || !w_v || !act || !dw_q || !dw_k || !dw_v || !workspace ||
      (sel && (!w_lam || !dw_lam)) || ((sel || fixed) && (!b_lam || !db_lam)))
    return GBLA_ERR_NULL_ARG;
  if (p->total_tokens > 0 && (!x || !y || !dy || !dx)) return GBLA_ERR_NULL_ARG;
  for (const void* a : {x, w_q, w_k, w_v, w_lam, act, y, dy, (const void*)dx, (const void*)dw_q, (const void*)dw_k,
                        (const void*)dw_v, (const void*)dw_lam, (const void*)workspace})
    if (!aligned(a, 16)) return GBLA_ERR_MISALIGNED;
  if (!aligned(b_lam, 4) || !aligned(db_lam, 4) || !aligned(cu_seqlens, 4)) return GBLA_ERR_MISALIGNED;
  const LDims m = dims_of(p);
  LBwdWs w;
  if (workspace_bytes < plan_bwd(m, static_cast<char*>(workspace), &w)) return GBLA_ERR_WORKSPACE_TOO_SMALL;
  Carver c;
  const LAct A = carve_act(m, c, static_cast<char*>(const_cast<void*>(act)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int dt = p->dtype == GBLA_DTYPE_BF16 ? BF16 : F32;

  (void)hipGetLastError();
  { StageScope ps(ST_PACK_WT, s);  // and the chunk table
    launch_pack_wt(dt, w_q, w_k, w_v, nullptr, sel ? w_lam : nullptr, m.d, m.H, m.dh, m.Kp, w.wt,
                   Sched{cu_seqlens, m.N, m.T, kLionChunk, m.slots, w.nchunks, w.chunk_off, w.tab}, s); }
  { StageScope ps(ST_LION_BWD_STATE, s);
    launch_lion_chunk_state(dt, m.dh, 1, A.q, dy, y, A.rsum, A.logl, w.nchunks, w.tab, m.slots, m.H, w.hst, nullptr,
                            s); }
  { StageScope ps(ST_LION_BWD_SCAN, s);  // HF, HB: the dh x dh part leaves as the row image
    launch_lion_scan(w.hst, A.lam, w.nchunks, w.chunk_off, m.N, m.H, m.E, dt, w.hrows, m.dh, s); }
  { StageScope ps(ST_LION_BWD_TOKEN, s);
    launch_lion_bwd_token(dt, m.dh, A.q, A.k, A.v, A.logl, y, dy, A.rsum, A.st, w.hst, w.hrows, w.nchunks, w.tab,
                          m.slots, m.H, m.Kp, w.G, w.dA_loc, w.dA_tot, s); }
  { StageScope ps(ST_LION_DA, s);
    launch_lion_da(A.logl, w.dA_loc, w.dA_tot, w.nchunks, w.tab, m.slots, m.H, m.D, m.Kp, dt, sel, w.G, w.db_part,
                   s); }
  if (sel || fixed) {
    StageScope ps(ST_LION_DB_REDUCE, s);
    launch_sum_parts(w.db_part, m.H, 0, w.nchunks, db_lam, s);
  }
  if (m.T > 0) {
    StageScope ps(ST_GEMM_DX, s);
    launch_gemm_dx(dt, w.G, w.wt, m.T, m.d, m.Kp, grad_cols_read(m.H, m.dh), dx, s);
  }
  { StageScope ps(ST_GEMM_DW, s); launch_gemm_dw(dt, x, w.G, m.T, m.d, m.Kp, m.nsplit, w.dw_part, s); }
  { StageScope ps(ST_DW_REDUCE, s);
    launch_dw_reduce(w.dw_part, m.nsplit, m.d, m.H, m.dh, m.Kp, dw_q, dw_k, dw_v, nullptr, sel ? dw_lam : nullptr,
                     s); }
  return hipGetLastError() == hipSuccess ? GBLA_OK : GBLA_ERR_HIP;
}

}  // extern "C"
