// Host-side launchers shared between the kernel translation units and the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace gbla {

enum DType { F32 = 0, BF16 = 1 };

// stages timed by the optional profiling window (gbla_profile_begin/end)
enum StageId {
  ST_PACK_PROJ, ST_CONV_FWD, ST_PROJ_FWD, ST_STATE_PARTIAL, ST_COMBINE_STATE, ST_READOUT,
  ST_PACK_WT, ST_CONV_RECOMPUTE, ST_PROJ_RECOMPUTE, ST_BWD_DSTATE, ST_COMBINE_DSTATE, ST_BWD_TOKEN,
  ST_DBG_REDUCE, ST_GEMM_DX, ST_CONV_BWD, ST_GEMM_DW, ST_DW_REDUCE, ST_DCONV_REDUCE,
  ST_LION_LOG_DECAY, ST_LION_PROJ, ST_LION_CHUNK_STATE, ST_LION_SCAN, ST_LION_READOUT,
  ST_LION_BWD_STATE, ST_LION_BWD_SCAN, ST_LION_BWD_TOKEN, ST_LION_DA, ST_LION_DB_REDUCE, ST_FINALIZE,
  kNumStages
};

// brackets the launches of one stage with events while a profiling window is
// open; without one it costs a single atomic load
class StageScope {
 public:
  StageScope(int stage_id, hipStream_t s);
  ~StageScope();
  StageScope(const StageScope&) = delete;
  StageScope& operator=(const StageScope&) = delete;

 private:
  int rec_;
  uint64_t gen_;
  hipStream_t s_;
};

// tokens per chunk of the split-L reductions and per-token attention kernels
constexpr int kChunk = 256;

// upper bound on the number of chunks of `chunk` tokens for T tokens in N sequences
inline int max_chunks(int T, int N, int chunk = kChunk) { return (T + chunk - 1) / chunk + N; }

// rows of the packed per-head projection weights: Q, K and V features, and with
// the gated RMSNorm output also R (the gate pre-activation x~ W_R)
inline int proj_cols(int dh, bool out_gate = false) { return (out_gate ? 4 : 3) * dh; }

// columns of the gradient matrix [dQ | dK | dV | (dR) | ds | 0-pad], padded to 64
// rows of the packed dX~ weight operand: d rounded up to whole 32-row groups
// (its row order is tile_row_perm within each group; rows past d are zero)
__host__ __device__ inline int wt_rows(int d) { return (d + 31) / 32 * 32; }
inline int grad_cols(int H, int dh, bool out_gate = false) {
  return (((out_gate ? 4 : 3) * H * dh + H) + 63) / 64 * 64;
}
// columns of G the dX~ GEMM reads (its k extent): the used columns rounded up
// to 8; only the padding columns below this bound are written (as zeros)
inline int grad_cols_read(int H, int dh, bool out_gate = false) {
  return (((out_gate ? 4 : 3) * H * dh + H) + 7) / 8 * 8;
}

// ---- forward / shared
// The chunk table (runs of <= chunk tokens inside each sequence, from cu) is
// built by one extra block of a weight-packing launch, the first launch of each
// pass (cu null: no table).
struct Sched {
  const int32_t* cu;
  int N, T, chunk, max_slots;
  int* nchunks;
  int* chunk_off;
  Chunk* tab;
};

// The chunk of a (chunk, head) block: the count and the entry are loaded
// together rather than one after the other (slot < max_slots, the table's
// size, so the entry load stays inside the table even past the count).
__device__ __forceinline__ bool block_chunk(const int* __restrict__ nchunks, const Chunk* __restrict__ tab, int slot,
                                            Chunk& ch) {
  const int nc = *nchunks;
  ch = tab[slot];
  return slot < nc;
}

// ---- the chunk table (run by one block of NT threads)
// Sequences are taken NT at a time: thread b reads its offsets once, the chunk
// counts are prefix-summed with wave shuffles plus one pass over the wave
// totals, and the table entries of the batch are then written by all threads
// in parallel (entry s finds its sequence by binary search over the batch's
// offsets in LDS). Malformed offsets schedule nothing, so no kernel reads
// outside [0, T).
template <int NT>
__device__ inline void schedule_block(const Sched& sc) {
  static_assert(NT % 64 == 0, "whole waves");
  __shared__ int off[NT + 1];
  __shared__ int wsum[NT / 64];
  const int32_t* cu = sc.cu;
  const int N = sc.N, chunk = sc.chunk, max_slots = sc.max_slots;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int bad = 0;
  if (tid == 0) bad = (cu[0] != 0) || (cu[N] != sc.T);
  for (int b = tid; b < N; b += NT)
    if (cu[b + 1] < cu[b]) bad = 1;
  if (__syncthreads_or(bad)) {
    for (int b = tid; b <= N; b += NT) sc.chunk_off[b] = 0;
    if (tid == 0) *sc.nchunks = 0;
    return;
  }
  int carry = 0;
  for (int b0 = 0; b0 < N; b0 += NT) {
    const int b = b0 + tid, nb = min(NT, N - b0);
    const int s0 = b < N ? cu[b] : 0, s1 = b < N ? cu[b + 1] : 0;
    const int n = b < N ? (s1 - s0 + chunk - 1) / chunk : 0;
    int inc = n;  // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, 64);
      if (lane >= o) inc += v;
    }
    if (lane == 63) wsum[wv] = inc;
    __syncthreads();
    int wbase = 0;
    for (int k = 0; k < wv; ++k) wbase += wsum[k];
    const int excl = wbase + inc - n;  // within the batch
    off[tid] = excl;
    if (tid == NT - 1) off[NT] = excl + n;
    if (b < N) sc.chunk_off[b] = min(carry + excl, max_slots);
    __syncthreads();
    const int total = off[nb];
    for (int e = tid; e < total && carry + e < max_slots; e += NT) {
      int lo = 0, hi = nb - 1;  // last sequence i with off[i] <= e
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= e) lo = mid; else hi = mid - 1;
      }
      const int c = e - off[lo];
      const int st = cu[b0 + lo] + c * chunk;
      Chunk ch;
      ch.seq = b0 + lo;
      ch.start = st;
      ch.end = min(st + chunk, cu[b0 + lo + 1]);
      ch.pad = 0;
      sc.tab[carry + e] = ch;
    }
    carry += total;
    __syncthreads();
  }
  if (tid == 0) {
    sc.chunk_off[N] = min(carry, max_slots);
    *sc.nchunks = min(carry, max_slots);
  }
}

// wt[p][n] = [W_Q[c,:] | W_K[c,:] | W_V[c,:] | (W_R[c,:]) | w_g[:,c] | 0] for
// channel c = tile_row_perm(p) (zero rows for c >= d; wt_rows(d) rows in all).
// Thread = 8 consecutive columns n (16-byte loads and stores in the weight
// column blocks, which start at multiples of 32; element-wise in the gate and
// padding columns); `blocks` blocks stride over the array.
struct WtPackArgs {
  const void* w_q; const void* w_k; const void* w_v; const void* w_r; const void* w_g;  // w_r, w_g may be null
  int d, H, dh, Kp;
  void* wt;
};
template <typename T>
struct WtPack {
  const T* w_q; const T* w_k; const T* w_v; const T* w_r; const T* w_g;
  int d, H, dh, Kp;
  T* wt;
  int blocks;  // 0: no packing in this launch
};
inline int wt_pack_blocks(int d, int Kp) {
  const long total = (long)wt_rows(d) * Kp / 8;
  return (int)(total < 4096L * 256 ? (total + 255) / 256 : 4096);
}
template <typename T>
WtPack<T> wt_pack_of(const WtPackArgs& a) {
  return WtPack<T>{(const T*)a.w_q, (const T*)a.w_k, (const T*)a.w_v, (const T*)a.w_r, (const T*)a.w_g,
                   a.d, a.H, a.dh, a.Kp, (T*)a.wt, wt_pack_blocks(a.d, a.Kp)};
}
template <typename T>
__device__ __forceinline__ void pack_wt_range(const WtPack<T>& pk, int blk) {
  const int d = pk.d, D = pk.H * pk.dh, GD = (pk.w_r ? 4 : 3) * D;  // first gate column
  const int per_row = pk.Kp / 8, total = wt_rows(d) * per_row;  // < 2^31 (checked on the host)
  for (int e8 = blk * 256 + (int)threadIdx.x; e8 < total; e8 += pk.blocks * 256) {
    const int p = e8 / per_row, n = 8 * (e8 - p * per_row);
    const size_t e = (size_t)p * pk.Kp + n;
    const int c = tile_row_perm(p);
    Frag8<T> v = frag_zero<T>();
    if (c < d) {
      if (n < GD) {
        const int seg = n / D;
        const T* src = seg == 0 ? pk.w_q : (seg == 1 ? pk.w_k : (seg == 2 ? pk.w_v : pk.w_r));
        v = frag_load(src + (long)c * D + n - seg * D);
      } else if (pk.w_g) {  // no w_g: zero rows
        float f[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) f[u] = n + u < GD + pk.H ? to_f<T>(pk.w_g[(long)(n + u - GD) * d + c]) : 0.f;
        v = frag_from<T>(f);
      }
    }
    frag_store(pk.wt + e, v);
  }
}

// w_r non-null: a fourth per-head segment (the gated RMSNorm output's W_R)
void launch_pack_proj(int dt, const void* w_q, const void* w_k, const void* w_v, const void* w_r, int d, int H,
                      int dh, void* wp, const Sched& sc, hipStream_t s);
// the operands of the projection's weight packing (w_r null: three segments)
struct ProjPackArgs {
  const void* w_q; const void* w_k; const void* w_v; const void* w_r;
  int d, H, dh;
  void* wp;
};
// g gets sigmoid(x~ w_g + b_g), or the logit itself for the softmax key gate.
// pack non-null: the same launch also packs the projection weights; sc.cu
// non-null: it also builds the chunk table.
void launch_conv_fwd(int dt, const void* x, const int32_t* cu, int N, int T, int d, int H, const void* conv_w,
                     const void* w_g, const float* b_g, bool softmax_gate, void* xt, float* g, hipStream_t s,
                     const ProjPackArgs* pack = nullptr, const Sched& sc = Sched{});
// r_out non-null: wp holds four segments per head and the fourth (linear) goes to r_out
void launch_proj(int dt, int dh, const void* xt, const void* wp, int T, int d, int H, void* q_out, void* k_out,
                 void* v_out, hipStream_t s, bool phi = true, void* r_out = nullptr);
void launch_log_decay(int dt, const void* x, const int32_t* cu, int N, int T, int d, int H, const void* w_lam,
                      const float* b_lam, float* logl, hipStream_t s);
// log lambda of every token for a decay that does not depend on the token:
// log sigmoid(b_lam[h]) (b_lam non-null) or 0 (b_lam null)
void launch_const_log_decay(int T, int H, const float* b_lam, float* logl, hipStream_t s);
// mpart non-null: softmax key gate (ga holds logits; chunk maxima go to mpart)
void launch_state_partial(int dt, int dh, const void* ka, const void* va, const float* ga, const int* nchunks,
                          const Chunk* tab, int max_slots, int H, float* partial, float* mpart, hipStream_t s);
// mpart non-null: rescale the partials to the sequence's largest chunk maximum (written to mout)
// pack non-null: the same launch also packs the dX~ weights (dtype dt)
void launch_combine(const float* partial, const int* nchunks, const int* chunk_off, int N, int H, int elems,
                    float* out, hipStream_t s, const float* mpart = nullptr, float* mout = nullptr,
                    const WtPackArgs* pack = nullptr, int dt = F32);
// out[e] = sum over the first P parts, P = (*P_dev) * p_mul if P_dev else P_host
void launch_sum_parts(const float* in, int E, int P_host, const int* P_dev, float* out, hipStream_t s,
                      int p_mul = 1);
// ra non-null: gated RMSNorm output, y = gamma (.) O / sqrt(mean(O^2) + eps) (.) SiLU(r)
// per head (gamma null: no scale)
void launch_readout(int dt, int dh, const void* qa, const float* saved, const int* nchunks, const Chunk* tab,
                    int max_slots, int H, void* y, hipStream_t s, const void* ra = nullptr,
                    const float* gamma = nullptr, float eps = 0.f);

// ---- backward
// w_g may be null (its rows of Wt are zero); w_r non-null: the R segment
// follows V ([W_Q | W_K | W_V | W_R | w_g^T])
void launch_pack_wt(int dt, const void* w_q, const void* w_k, const void* w_v, const void* w_r, const void* w_g,
                    int d, int H, int dh, int Kp, void* wt, const Sched& sc, hipStream_t s);


// ra non-null: gated RMSNorm output; dy is then the gradient of the gated
// output, dR goes to G's R columns and per-(chunk, head) partials of dgamma
// to dgam_part (gamma non-null)
void launch_bwd_dstate(int dt, int dh, const void* qa, const void* dy, const float* saved, const int* nchunks,
                       const Chunk* tab, int max_slots, int H, int Kp, float* partial, void* G, hipStream_t s,
                       const void* ra = nullptr, const float* gamma = nullptr, float eps = 0.f,
                       float* dgam_part = nullptr);
// gmax non-null: softmax key gate (ga holds logits; the gate is exp(s - gmax[seq][h]))
// G's gate column of head h is nseg * H * dh + h (nseg = 4 with the R segment)
void launch_bwd_token(int dt, int dh, const void* ka, const void* va, const float* ga, const float* dsz,
                      const int* nchunks, const Chunk* tab, int max_slots, int H, int Kp, int nseg, void* G,
                      float* dbg_part, const float* gmax, hipStream_t s);
// dx = G Wt^T (no conv: LION)
void launch_gemm_dx(int dt, const void* G, const void* wt, int T, int d, int Kp, int Kr, void* dxt, hipStream_t s);
// dX~ = G Wt^T with the causal conv's VJP in the epilogue (GBLA): dx (but the
// last three tokens of each token tile other than the last, left to
// k_bwd_finalize), per-token-tile dconv_w partials [dx_token_tiles][d][4] and
// the tiles' edge rows [dx_token_tiles][6][d]
void launch_gemm_dx_conv(int dt, const void* G, const void* wt, int T, int d, int Kp, int Kr, const void* x,
                         const int32_t* cu, int N, const void* conv_w, void* dx, float* dconv_part, void* edge,
                         hipStream_t s);
int dx_token_tiles(int dt, int T, int d);
int dx_token_tile_rows(int dt, int T, int d);
int dw_tiles(int dt, int d, int Kp);
int dw_splits(int dt, int d, int Kp, int T);
void launch_gemm_dw(int dt, const void* xt, const void* G, int T, int d, int Kp, int nsplit, float* part,
                    hipStream_t s);
// dw_g may be null (its columns are not written); dw_r non-null: G has the R segment
// the backward's closing sums (dW split-K partials, dconv_w row blocks, db_g and
// dgamma chunk partials) in one launch
// With edge non-null (the conv VJP fused into the dX~ GEMM) it also forms dx of
// the last three tokens of every token tile but the last (conv_rb tiles of
// tile_rows tokens).
struct BwdFinalize {
  const float* dw_part; int nsplit, d, H, dh, Kp, dw_blocks;
  float *dw_q, *dw_k, *dw_v, *dw_r, *dw_g;
  const float* dconv_part; int conv_rb; float* dconv_w;
  const int* nchunks; const float* dbg_part; float* db_g;
  const float* dgam_part; float* dgamma;
  int dt, tile_rows, nseq;
  const void* edge; const void* conv_w; const int32_t* cu; void* dx;
};
int bwd_finalize_dw_blocks(int d, int Kp);
void launch_bwd_finalize(const BwdFinalize& f, hipStream_t s);
void launch_dw_reduce(const float* part, int nsplit, int d, int H, int dh, int Kp, float* dw_q, float* dw_k,
                      float* dw_v, float* dw_r, float* dw_g, hipStream_t s);

}  // namespace gbla
