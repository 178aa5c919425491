// GBLA forward kernels for gfx950.
//
// The layer ("Gated Bidirectional Linear Attention for Generative Retrieval",
// core method, Eqs. (4)-(6)) per packed sequence b and head h:
//   x~ = causal depthwise Conv1d_4(x)             (Eq. (4), restarted per sequence)
//   q, k, v = x~ W_Q^h, x~ W_K^h, x~ W_V^h        (Eq. (4))
//   g = sigmoid(x~ w_g^h + b_g^h)                 (key gate, Eq. (5))
//   S = sum_j g_j phi(k_j) v_j^T,  z = sum_j g_j phi(k_j),  phi = elu + 1
//   y_i = phi(q_i)^T S / phi(q_i)^T z             (Eqs. (5)/(6) in the state-first order of Eq. (3))
//
// Kernels (all on the caller's stream, no host synchronisation):
//   k_conv_fwd      causal conv -> x~, and the gates g = sigmoid(x~ w_g + b_g) of every head;
//                   its extra blocks pack the per-head weights [H][3*dh][d] (Q, K, V
//                   columns, k contiguous; pack_proj_block) and build the chunk table of
//                   <= kChunk-token runs inside each sequence from cu_seqlens (schedule_block)
//   k_pack_proj     the same packing (and table) as a launch of its own (LION-s)
//   k_proj          projection GEMM x~ [W_Q|W_K|W_V]^h (pipelined MFMA) with phi epilogue
//   k_state_partial split-L partial [S | z] per (chunk, head), MFMA over the token axis
//   k_combine       fixed-order sum of the partials of each (sequence, head)
//   k_readout       y = phi(Q) [S | z] (MFMA), divide
#include <algorithm>
#include <atomic>

#include "gemm.h"
#include "internal.h"

namespace gbla {

// ============================================================== weight packing
// wp[h][p][c] (k = c contiguous) holds column f = tile_row_perm(p) of the head's
// [W_Q | W_K | W_V (| W_R)] block (f < dh: W_Q[:, h*dh + f], then W_K, W_V, W_R).
// The row order within each 32-row group is what lets the projection epilogue
// store 8 consecutive features per lane (see k_proj).
// Block = one 32-row group of one head x 64 channels c, transposed through
// LDS: 16-byte loads of 8 consecutive features of one weight row, 16-byte
// stores of 8 consecutive channels of one packed row. d % 8 == 0. The blocks
// run on their own (k_pack_proj, whose last block builds the chunk table when
// given a schedule) or as the leading blocks of the conv launch.
template <typename T>
struct ProjPack {
  const T* w_q; const T* w_k; const T* w_v; const T* w_r;  // w_r null: three segments per head
  int d, H, dh;
  T* wp;
  int blocks;  // proj_pack_blocks(); 0: no packing in this launch
};
inline int proj_pack_blocks(int d, int H, int dh, bool four) { return H * (proj_cols(dh, four) / 32) * ((d + 63) / 64); }

template <typename T>
__device__ __forceinline__ void pack_proj_block(const ProjPack<T>& pk, int blk) {
  __shared__ float tile[32][65];
  const int d = pk.d, dh = pk.dh;
  const int NP = (pk.w_r ? 4 : 3) * dh, D = pk.H * dh, G = NP / 32;
  const int cb = blk % ((d + 63) / 64), rest = blk / ((d + 63) / 64);
  const int g = rest % G, h = rest / G;
  const int c0 = 64 * cb, f0 = 32 * g, seg = f0 / dh;
  const T* src = seg == 0 ? pk.w_q : (seg == 1 ? pk.w_k : (seg == 2 ? pk.w_v : pk.w_r));
  const int t = threadIdx.x;
  {
    const int c = t >> 2, fc = 8 * (t & 3);
    if (c0 + c < d) {
      const Frag8<T> v = frag_load(src + (size_t)(c0 + c) * D + h * dh + (f0 % dh) + fc);
#pragma unroll
      for (int j = 0; j < 8; ++j) tile[fc + j][c] = frag_get(v, j);
    }
  }
  __syncthreads();
  const int pr = t >> 3, cc = 8 * (t & 7);
  if (c0 + cc < d) {
    const int f = tile_row_perm(pr);  // pr < 32: the feature within the group
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = tile[f][cc + j];
    frag_store(pk.wp + ((size_t)h * NP + f0 + pr) * d + c0 + cc, frag_from<T>(v));
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_pack_proj(ProjPack<T> pk, Sched sc) {
  if (sc.cu && (int)blockIdx.x == pk.blocks) {
    schedule_block<256>(sc);
    return;
  }
  pack_proj_block(pk, blockIdx.x);
}

template <typename T>
ProjPack<T> proj_pack_of(const ProjPackArgs& a) {
  return ProjPack<T>{(const T*)a.w_q, (const T*)a.w_k, (const T*)a.w_v, (const T*)a.w_r, a.d, a.H, a.dh, (T*)a.wp,
                     proj_pack_blocks(a.d, a.H, a.dh, a.w_r != nullptr)};
}

void launch_pack_proj(int dt, const void* w_q, const void* w_k, const void* w_v, const void* w_r, int d, int H,
                      int dh, void* wp, const Sched& sc, hipStream_t s) {
  const ProjPackArgs a{w_q, w_k, w_v, w_r, d, H, dh, wp};
  const int grid = proj_pack_blocks(d, H, dh, w_r != nullptr) + (sc.cu ? 1 : 0);
  if (dt == BF16) hipLaunchKernelGGL(k_pack_proj<bf16>, dim3(grid), dim3(256), 0, s, proj_pack_of<bf16>(a), sc);
  else hipLaunchKernelGGL(k_pack_proj<float>, dim3(grid), dim3(256), 0, s, proj_pack_of<float>(a), sc);
}

// ============================================================== causal conv + gate
// A wave owns RUN consecutive token rows (4 RUN per block); lane l owns channel
// groups c = 8 * (l + 64 m). The rows stream through two register batches of
// 4 (the next batch loads while the current one is computed and stored), and
// the three previous rows slide in registers; the row walk is unrolled. The
// gate logits s_h = x~ . w_g^h are reduced over the wave with a reduce-scatter
// butterfly (butterfly8): 8 head partials per lane become one head total per 8
// lanes in 4 + 2 lane-half swaps and 4 DPP adds.
// RUN = 32 rows per wave; with fewer than 2048 such waves (T < 65 536), 8 rows,
// so that a small batch still puts several waves on every SIMD
constexpr int kConvRowsPerWave = 32, kConvRowsPerWaveSmall = 8;
constexpr int kConvBatchRows = 4;
inline int conv_rows_per_wave(int T) {
  return (T + kConvRowsPerWave - 1) / kConvRowsPerWave >= 2048 ? kConvRowsPerWave : kConvRowsPerWaveSmall;
}

// sum of the 8 products of two fragments (bf16: four packed dot2 instructions)
template <typename T> __device__ __forceinline__ float gate_dot8(const Frag8<T>& a, const Frag8<T>& b);
template <> __device__ __forceinline__ float gate_dot8<float>(const Frag8<float>& a, const Frag8<float>& b) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += frag_get(a, j) * frag_get(b, j);
  return s;
}
typedef __bf16 gate_bf16x2 __attribute__((ext_vector_type(2)));
template <> __device__ __forceinline__ float gate_dot8<bf16>(const Frag8<bf16>& a, const Frag8<bf16>& b) {
  const uint32_t av[4] = {a.v.x, a.v.y, a.v.z, a.v.w}, bv[4] = {b.v.x, b.v.y, b.v.z, b.v.w};
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(gate_bf16x2, av[j]), __builtin_bit_cast(gate_bf16x2, bv[j]),
                                        s, false);
  return s;
}

// Reduce-scatter of 8 per-lane values over the wave: lane l ends with the
// wave total of value (l >> 3). Halving steps exchange the half a lane does not
// keep: lanes 32-63 keep values 4-7 (v_permlane32_swap), then the odd 16-lane
// rows keep the upper pair (v_permlane16_swap), then lanes with bit 3 set keep
// the odd value (a rotate by 8 within the row); a mirror and two quad
// permutations sum the 8 lanes of each group. All register-to-register.
__device__ __forceinline__ float butterfly8(float (&v)[8], int lane) {
  float u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // lanes 0-31: v[i] of both halves; lanes 32-63: v[4 + i]
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[4 + i]), false, false);
    u[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  float q[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // even 16-lane rows: u[i] of the row pair; odd rows: u[2 + i]
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(u[i]), __float_as_uint(u[2 + i]), false, false);
    q[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const bool b3 = lane & 8;
  float x = (b3 ? q[1] : q[0]) + dpp_f<kDppRowRor8>(b3 ? q[0] : q[1]);  // partner: lane ^ 8
  x += dpp_f<kDppHalfMirror>(x);  // lane i of an 8-lane group + lane 7 - i
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  return x;  // total of value (lane >> 3)
}

// log(sigmoid(z)) = -softplus(-z), stable for any z
__device__ __forceinline__ float log_sigmoidf_(float z) { return fminf(z, 0.f) - log1pf(__expf(-fabsf(z))); }

// CONV = true: GBLA, x~ = causal conv(x) is stored; CONV = false: LION-s, x~ = x
// (nothing stored). With z = x~ w_g + b_g, g_out gets sigmoid(z) (gmode 0, the
// sigmoid key gate), z itself (gmode 1, the logit of the softmax key gate) or
// log sigmoid(z) (gmode 2, the LION-s log decay).
// The conv's blocks may be followed by the projection's weight-packing blocks
// (pk.blocks of them) and then one block that builds the chunk table (sc.cu
// non-null): the projection needs the packed weights and the per-chunk kernels
// the table, and neither needs the conv, so they ride along instead of taking a
// launch of their own. They come last so that the conv's blocks are spread
// evenly over the compute units first.
enum GateMode { kGateSigmoid = 0, kGateLogit = 1, kGateLogSigmoid = 2 };
template <typename T, bool CONV, int RUN>
__global__ __launch_bounds__(256) void k_conv_fwd(const T* __restrict__ x, const int32_t* __restrict__ cu, int nseq,
                                                  int T_, int d, int H, const T* __restrict__ conv_w,
                                                  const T* __restrict__ w_g, const float* __restrict__ b_g,
                                                  int gmode, T* __restrict__ xt, float* __restrict__ g_out,
                                                  ProjPack<T> pk, Sched sc) {
  constexpr int B = kConvBatchRows, NB = RUN / B;
  static_assert(RUN % B == 0 && RUN <= 32, "whole batches; 2 bits per row position in 64");
  const int nconv = (int)gridDim.x - pk.blocks - (sc.cu ? 1 : 0);
  if ((int)blockIdx.x >= nconv) {
    if ((int)blockIdx.x - nconv < pk.blocks) pack_proj_block(pk, blockIdx.x - nconv);
    else schedule_block<256>(sc);
    return;
  }
  __shared__ float sacc[4][RUN][8];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t_begin = (blockIdx.x * 4 + w) * RUN;  // wave-uniform
  const int t_end = min(t_begin + RUN, T_);
  const int ngroups = d / 8;
  // position of each row of the run in its sequence, capped at 3 (2 bits per
  // row), looked up before any row load is in flight: the lookup's loads are
  // wave-uniform, and a wait for them then holds up nothing else
  unsigned long long posbits = 0;
  if (CONV && t_begin < t_end) {
    SeqCursor cur(cu, nseq, t_begin, T_);
    for (int i = 0; i < RUN && t_begin + i < t_end; ++i)
      posbits |= (unsigned long long)min(cur.pos(t_begin + i), 3) << (2 * i);
  }
  // x rows max(t_begin - 3, 0) .. t_end - 1 and the run's x~ rows through buffer
  // range checks: rows past the run read as zeros and their stores are dropped,
  // so no branch surrounds a row load or store and each batch's wait leaves the
  // next batch's loads in flight
  const int x0r = max(t_begin - 3, 0), nx = max(t_end - x0r, 0), nrun = max(t_end - t_begin, 0);
  const RowBuf<T> xb(x + (size_t)x0r * d, nx, d, d);
  const RowBuf<T> xtb(CONV ? xt + (size_t)t_begin * d : x, CONV ? nrun : 0, d, d);
  for (int hg = 0; hg < H; hg += 8) {
    for (int g8 = lane; g8 < ((ngroups + 63) / 64) * 64; g8 += 64) {
      const bool okc = g8 < ngroups;
      const int c = g8 * 8;
      const int cx = okc ? c : (nx + 3) * d, cs = okc ? c : nrun * d;  // out of range for lanes past d
      // every load is issued before any is used: the weights, the three rows
      // before the run (zeros before row 0; sequence starts are cut by the
      // positions) and the first two row batches
      Frag8<T> cwf[4], wgf[8];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        cwf[m] = CONV && okc ? frag_load(conv_w + (size_t)c * 4 + 8 * m) : frag_zero<T>();
#pragma unroll
      for (int hh = 0; hh < 8; ++hh)
        wgf[hh] = okc && hg + hh < H ? frag_load(w_g + (size_t)(hg + hh) * d + c) : frag_zero<T>();
      const int r0 = t_begin - x0r;  // the run's first row in xb
      Frag8<T> xm1 = frag_zero<T>(), xm2 = frag_zero<T>(), xm3 = frag_zero<T>();
      if (CONV) {  // rows before row 0 are read at row nx, past the range (zeros)
        xm1 = xb.load(r0 >= 1 ? r0 - 1 : nx, cx);
        xm2 = xb.load(r0 >= 2 ? r0 - 2 : nx, cx);
        xm3 = xb.load(r0 >= 3 ? r0 - 3 : nx, cx);
      }
      // rows stream through two register batches: one is computed while the next loads
      Frag8<T> xr[2][B];
      auto fetch = [&](int bi) {
#pragma unroll
        for (int i = 0; i < B; ++i) xr[bi % 2][i] = xb.load(r0 + B * bi + i, cx);
      };
      fetch(0);
      if (NB > 1) fetch(1);
      __builtin_amdgcn_sched_barrier(0);  // the conversions below stay behind the loads
      float wv[8][4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) wv[(8 * m + e) >> 2][(8 * m + e) & 3] = frag_get(cwf[m], e);
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) {
#pragma unroll
        for (int i = 0; i < B; ++i) {
          const int u = B * bi + i;  // row of the run
          const int pos = (int)(posbits >> (2 * u)) & 3;
          const Frag8<T> x0 = xr[bi % 2][i];
          float o[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            float a = CONV ? wv[j][3] * frag_get(x0, j) : frag_get(x0, j);
            if (CONV && pos >= 1) a += wv[j][2] * frag_get(xm1, j);
            if (CONV && pos >= 2) a += wv[j][1] * frag_get(xm2, j);
            if (CONV && pos >= 3) a += wv[j][0] * frag_get(xm3, j);
            o[j] = a;
          }
          const Frag8<T> of = frag_from<T>(o);
          if (CONV && hg == 0) xtb.store(u, cs, of);
          float sp[8];
#pragma unroll
          for (int hh = 0; hh < 8; ++hh) sp[hh] = gate_dot8<T>(of, wgf[hh]);  // the rounded x~ that Q, K, V see
          const float tot = butterfly8(sp, lane);
          if ((lane & 7) == 0) {
            float& acc = sacc[w][u][lane >> 3];
            acc = g8 < 64 ? tot : acc + tot;
          }
          xm3 = xm2;
          xm2 = xm1;
          xm1 = x0;
        }
        if (bi + 2 < NB) fetch(bi + 2);
      }
    }
    __syncthreads();
    // sacc[w][row][hh] now holds the full logits of heads hg..hg+7 for this wave's rows
    for (int e = lane; e < RUN * 8; e += 64) {
      const int row = e >> 3, hh = e & 7;
      const int t = t_begin + row, h = hg + hh;
      if (t < t_end && h < H) {
        const float z = sacc[w][row][hh] + b_g[h];
        g_out[(size_t)t * H + h] =
            gmode == kGateSigmoid ? sigmoidf_(z) : (gmode == kGateLogit ? z : log_sigmoidf_(z));
      }
    }
    __syncthreads();
  }
}

void launch_conv_fwd(int dt, const void* x, const int32_t* cu, int N, int T, int d, int H, const void* conv_w,
                     const void* w_g, const float* b_g, bool softmax_gate, void* xt, float* g, hipStream_t s,
                     const ProjPackArgs* pack, const Sched& sc) {
  const int gmode = softmax_gate ? kGateLogit : kGateSigmoid;
  const int run = conv_rows_per_wave(T);
  const int pre = (pack ? proj_pack_blocks(pack->d, pack->H, pack->dh, pack->w_r != nullptr) : 0) + (sc.cu ? 1 : 0);
  const int grid = (T + 4 * run - 1) / (4 * run) + pre;
  if (grid == 0) return;
#define GBLA_CF(TT, RR)                                                                                     \
  hipLaunchKernelGGL((k_conv_fwd<TT, true, RR>), dim3(grid), dim3(256), 0, s, (const TT*)x, cu, N, T, d, H, \
                     (const TT*)conv_w, (const TT*)w_g, b_g, gmode, (TT*)xt, g,                             \
                     pack ? proj_pack_of<TT>(*pack) : ProjPack<TT>{}, sc)
  if (dt == BF16) {
    if (run == kConvRowsPerWave) GBLA_CF(bf16, kConvRowsPerWave); else GBLA_CF(bf16, kConvRowsPerWaveSmall);
  } else {
    if (run == kConvRowsPerWave) GBLA_CF(float, kConvRowsPerWave); else GBLA_CF(float, kConvRowsPerWaveSmall);
  }
#undef GBLA_CF
}

void launch_log_decay(int dt, const void* x, const int32_t* cu, int N, int T, int d, int H, const void* w_lam,
                      const float* b_lam, float* logl, hipStream_t s) {
  if (T == 0) return;
  const int run = conv_rows_per_wave(T);
  const dim3 grid((T + 4 * run - 1) / (4 * run));
  // no conv in this mode: the conv-tap pointer is never dereferenced
#define GBLA_LD(TT, RR)                                                                                  \
  hipLaunchKernelGGL((k_conv_fwd<TT, false, RR>), grid, dim3(256), 0, s, (const TT*)x, cu, N, T, d, H, \
                     (const TT*)w_lam, (const TT*)w_lam, b_lam, (int)kGateLogSigmoid, (TT*)nullptr, logl,   \
                     ProjPack<TT>{}, Sched{})
  if (dt == BF16) {
    if (run == kConvRowsPerWave) GBLA_LD(bf16, kConvRowsPerWave); else GBLA_LD(bf16, kConvRowsPerWaveSmall);
  } else {
    if (run == kConvRowsPerWave) GBLA_LD(float, kConvRowsPerWave); else GBLA_LD(float, kConvRowsPerWaveSmall);
  }
#undef GBLA_LD
}

__global__ __launch_bounds__(256) void k_const_log_decay(int T_, int H, const float* __restrict__ b_lam,
                                                         float* __restrict__ logl) {
  const long total = (long)T_ * H;
  for (long e = blockIdx.x * 256L + threadIdx.x; e < total; e += (long)gridDim.x * 256L)
    logl[e] = b_lam ? log_sigmoidf_(b_lam[e % H]) : 0.f;
}

void launch_const_log_decay(int T, int H, const float* b_lam, float* logl, hipStream_t s) {
  const long total = (long)T * H;
  if (total == 0) return;
  const int grid = (int)std::min<long>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(k_const_log_decay, dim3(grid), dim3(256), 0, s, T, H, b_lam, logl);
}

// ============================================================== projection GEMM
// Block = the [Q | K | V] rows (3 dh each; with the gated RMSNorm output
// [Q | K | V | R], 4 dh) of HPB consecutive heads x BN tokens, computed in the
// transposed orientation: A = the packed weight panel (rows = features, the
// per-head panels are contiguous, so HPB heads are one operand), B = the x~
// tile (rows = tokens). A lane's C tiles then hold features of a single token,
// and with the panel's row order (tile_row_perm) the tiles 2i and 2i+1 of a
// lane hold 8 consecutive features, which leave as one 16-byte (bf16) store
// straight from registers: no LDS staging and no barrier in the epilogue.
// bf16 runs the direct-to-LDS main loop, float the register-staged one; the
// four-segment panel (with R) runs 256 x 256 tiles of 16 waves of 64 x 64.
// Epilogue: phi on Q and K, identity on V and R.
template <typename T, int DH, int NSEG> struct ProjCfg;
template <> struct ProjCfg<bf16, 64, 3> {
  using S = DlShape<192, 128, 64, 2, 4, 2>; static constexpr bool DL = true; static constexpr int HPB = 1;
};
template <> struct ProjCfg<bf16, 32, 3> {
  using S = DlShape<192, 128, 64, 2, 4, 2>; static constexpr bool DL = true; static constexpr int HPB = 2;
};
template <> struct ProjCfg<bf16, 64, 4> {
  using S = DlShape<256, 256, 64, 4, 4, 2>; static constexpr bool DL = true; static constexpr int HPB = 1;
};
template <> struct ProjCfg<bf16, 32, 4> {
  using S = DlShape<256, 256, 64, 4, 4, 2>; static constexpr bool DL = true; static constexpr int HPB = 2;
};
template <> struct ProjCfg<float, 64, 3> {
  using S = GemmShape<float, 192, 32, 32, 2, 2>; static constexpr bool DL = false; static constexpr int HPB = 1;
};
template <> struct ProjCfg<float, 32, 3> {
  using S = GemmShape<float, 96, 64, 32, 1, 4>; static constexpr bool DL = false; static constexpr int HPB = 1;
};
template <> struct ProjCfg<float, 64, 4> {
  using S = GemmShape<float, 256, 32, 32, 2, 2>; static constexpr bool DL = false; static constexpr int HPB = 1;
};
template <> struct ProjCfg<float, 32, 4> {
  using S = GemmShape<float, 128, 64, 32, 1, 4>; static constexpr bool DL = false; static constexpr int HPB = 1;
};

// pipeline depth of a main-loop shape (register-staged shapes have none)
template <class S, class = void> struct NS_OF { static constexpr int n = 2; };
template <class S> struct NS_OF<S, decltype(void(S::NS))> { static constexpr int n = S::NS; };

// PHI = true: phi = elu + 1 on Q and K (GBLA); false: raw projections (LION)
template <typename T, int DH, bool PHI, int NSEG>
__global__ __launch_bounds__((ProjCfg<T, DH, NSEG>::S::NTHREADS), 2) void k_proj(
    const T* __restrict__ xt, const T* __restrict__ wp, int T_, int d, int H, T* __restrict__ q_out,
    T* __restrict__ k_out, T* __restrict__ v_out, T* __restrict__ r_out) {
  using Cfg = ProjCfg<T, DH, NSEG>;
  using S = typename Cfg::S;
  constexpr bool DL = Cfg::DL;
  constexpr int HPB = Cfg::HPB;
  constexpr int NP = NSEG * DH;  // weight rows per head
  static_assert(S::BM == HPB * NP, "a block covers whole heads");
  static_assert(S::WTM % 32 == 0 && NP % 32 == 0, "a wave's features are whole 32-row groups of one head");
  __shared__ __align__(16) T smem[DL ? S::STAGE : 2 * S::STAGE];
  __shared__ __align__(16) T smem1[DL ? S::STAGE : 8];
  __shared__ __align__(16) T smem2[DL && NS_OF<S>::n > 2 ? S::STAGE : 8];
  const int mtiles = (T_ + S::BN - 1) / S::BN, hgroups = (H + HPB - 1) / HPB;
  const int lid = xcd_logical_block(blockIdx.x, mtiles * hgroups);
  if (lid >= mtiles * hgroups) return;
  const int mt = lid / hgroups, h0 = (lid - mt * hgroups) * HPB;
  const int m0 = mt * S::BN;
  const int nf = min(HPB, H - h0) * NP;  // valid weight rows (a last odd head)
  f32x4 acc[S::FM][S::FN];
  if constexpr (DL)
    gemm_nt_dl<S>(wp + (size_t)h0 * NP * d, d, nf, xt + (size_t)m0 * d, d, min(S::BN, T_ - m0), d, smem, smem1,
                  smem2, smem2, acc);
  else
    gemm_nt_mainloop<T, S>(wp + (size_t)h0 * NP * d, d, nf, xt + (size_t)m0 * d, d, min(S::BN, T_ - m0), d,
                           smem, acc);
  // epilogue: lane (grp, col) holds, in tiles 2 i2 and 2 i2 + 1, features
  // 8 grp .. 8 grp + 7 of the wave's 32-row group i2 for token col of tile j
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 15, grp = lane >> 4;
  const int wm = w / S::WGN, wn = w % S::WGN;
  const int D = H * DH;
#pragma unroll
  for (int i2 = 0; i2 < S::FM / 2; ++i2) {
    const int n = wm * S::WTM + 32 * i2 + 8 * grp;  // block-relative feature of the lane's first element
    const int h = h0 + n / NP, nn = n % NP, kind = nn / DH;
    const bool lin = !PHI || kind >= 2;  // v and r columns (and everything without phi) stay linear
    T* out = kind == 0 ? q_out : (kind == 1 ? k_out : (kind == 2 ? v_out : r_out));
    const size_t fo = (size_t)h * DH + (nn % DH);
#pragma unroll
    for (int j = 0; j < S::FN; ++j) {
      const int t = m0 + wn * S::WTN + 16 * j + col;
      float v[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = lin ? acc[2 * i2][j][r] : phi_elu1(acc[2 * i2][j][r]);
        v[4 + r] = lin ? acc[2 * i2 + 1][j][r] : phi_elu1(acc[2 * i2 + 1][j][r]);
      }
      if (t < T_ && h < H) frag_store(out + (size_t)t * D + fo, frag_from<T>(v));
    }
  }
}

// Persistent form for bf16: one block of 16 waves per CU walks 256 x 256 tiles
// (256 rows of the packed panel of all heads x 256 tokens) with the k-chunk
// pipeline running on from tile to tile (gemm_nt_dl_persistent). The tiles of
// an XCD are consecutive logical ids, and consecutive ids share a token tile,
// so the x~ tile is read from HBM once and its other row tiles hit the XCD's L2.
// The epilogue stores through buffer stores (16 per wave per tile), which drop
// rows past the last head and tokens past T. (The tiles' outputs push x~ tiles
// out of the XCD's L2 before every row tile of them has read them: x~ is read
// 2.3 times from beyond the L2. Non-temporal stores cut that to 1.3 but made
// the kernel slower, 513 -> 590 us on a 267k-token batch: the half-line stores
// of a wave then reach memory uncombined.)
template <int DH, bool PHI, int NSEG>
__global__ __launch_bounds__(512, 1) void k_proj_persistent(const bf16* __restrict__ xt, const bf16* __restrict__ wp,
                                                             int T_, int d, int H, bf16* __restrict__ q_out,
                                                             bf16* __restrict__ k_out, bf16* __restrict__ v_out,
                                                             bf16* __restrict__ r_out) {
  using S = DlShape<256, 256, 64, 2, 4, 2>;
  constexpr int NP = NSEG * DH;
  static_assert(S::WTM % 32 == 0 && NP % 32 == 0 && DH % 32 == 0, "32-row groups of one segment of one head");
  __shared__ __align__(16) bf16 st0[S::STAGE];
  __shared__ __align__(16) bf16 st1[S::STAGE];
  const int R = H * NP, FT = (R + S::BM - 1) / S::BM, MT = (T_ + S::BN - 1) / S::BN, n = MT * FT;
  const int D = H * DH;
  auto coords = [&](int i, int& m0, int& f0) -> bool {
    const int v = blockIdx.x + i * gridDim.x;  // gridDim.x % 8 == 0: the same XCD for every i
    if (v >= xcd_grid(n)) return false;
    const int l = xcd_logical_block(v, n);
    if (l >= n) return false;
    const int mt = l / FT;
    m0 = mt * S::BN;
    f0 = (l - mt * FT) * S::BM;
    return true;
  };
  auto item = [&](int i, DlItem& it) -> bool {
    int m0, f0;
    if (!coords(i, m0, f0)) return false;
    it.A = wp + (size_t)f0 * d;
    it.ma = min(S::BM, R - f0);
    it.B = xt + (size_t)m0 * d;
    it.nb = min(S::BN, T_ - m0);
    return true;
  };
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w / S::WGN, wn = w % S::WGN;
  // lane (grp, col) holds, in tiles 2 i2 and 2 i2 + 1, features 8 grp .. 8 grp + 7
  // of the wave's 32-row group i2 for token col of tile j
  auto epi = [&](int i, f32x4(&acc)[S::FM][S::FN]) {
    int m0 = 0, f0 = 0;
    coords(i, m0, f0);
    const int rows = min(S::BN, T_ - m0);
#pragma unroll
    for (int i2 = 0; i2 < S::FM / 2; ++i2) {
      const int row = f0 + wm * S::WTM + 32 * i2;  // wave-uniform
      const int h = row / NP, nn = row % NP, kind = nn / DH;
      const bool lin = !PHI || kind >= 2;
      bf16* out = kind == 0 ? q_out : (kind == 1 ? k_out : (kind == 2 ? v_out : r_out));
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(out + (size_t)m0 * D), 0, h < H ? rows * D * 2 : 0, kBufferRsrcWord3);
      const int fo = h * DH + nn % DH + 8 * grp;
#pragma unroll
      for (int j = 0; j < S::FN; ++j) {
        const int t = wn * S::WTN + 16 * j + col;
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = lin ? acc[2 * i2][j][r] : phi_elu1(acc[2 * i2][j][r]);
          v[4 + r] = lin ? acc[2 * i2 + 1][j][r] : phi_elu1(acc[2 * i2 + 1][j][r]);
        }
        const uint4 u = frag_from<bf16>(v).v;
        const u32x4 uv = {u.x, u.y, u.z, u.w};
        __builtin_amdgcn_raw_buffer_store_b128(uv, ro, (t * D + fo) * 2, 0, 0);
      }
    }
  };
  gemm_nt_dl_persistent<S, S::FM / 2 * S::FN>(d, d, d, item, epi, st0, st1);
}

// compute units of the current device (cached per device)
static int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// tiles of the persistent projection (256 tokens x 256 panel rows)
static int proj_persistent_tiles(int T_, int rows) { return ((T_ + 255) / 256) * ((rows + 255) / 256); }

template <int DH, bool PHI, int NSEG>
static void proj_persistent(const void* xt, const void* wp, int T_, int d, int H, void* q, void* k, void* v, void* r,
                            hipStream_t s) {
  const int n = proj_persistent_tiles(T_, H * NSEG * DH);
  if (n == 0) return;
  const int grid = std::min(xcd_grid(n), std::max(8, device_cu_count() / 8 * 8));
  hipLaunchKernelGGL((k_proj_persistent<DH, PHI, NSEG>), dim3(grid), dim3(512), 0, s, (const bf16*)xt,
                     (const bf16*)wp, T_, d, H, (bf16*)q, (bf16*)k, (bf16*)v, (bf16*)r);
}

template <typename T, int DH, bool PHI, int NSEG>
static void proj_t(const void* xt, const void* wp, int T_, int d, int H, void* q, void* k, void* v, void* r,
                   hipStream_t s) {
  using S = typename ProjCfg<T, DH, NSEG>::S;
  constexpr int HPB = ProjCfg<T, DH, NSEG>::HPB;
  const int n = ((T_ + S::BN - 1) / S::BN) * ((H + HPB - 1) / HPB);
  if (n == 0) return;
  hipLaunchKernelGGL((k_proj<T, DH, PHI, NSEG>), dim3(xcd_grid(n)), dim3(S::NTHREADS), 0, s, (const T*)xt,
                     (const T*)wp, T_, d, H, (T*)q, (T*)k, (T*)v, (T*)r);
}

void launch_proj(int dt, int dh, const void* xt, const void* wp, int T, int d, int H, void* q_out, void* k_out,
                 void* v_out, hipStream_t s, bool phi, void* r_out) {
#define GBLA_PJ(TT, DD)                                                                \
  (r_out ? proj_t<TT, DD, true, 4>(xt, wp, T, d, H, q_out, k_out, v_out, r_out, s)      \
         : (phi ? proj_t<TT, DD, true, 3>(xt, wp, T, d, H, q_out, k_out, v_out, r_out, s) \
                : proj_t<TT, DD, false, 3>(xt, wp, T, d, H, q_out, k_out, v_out, r_out, s)))
  // the persistent form needs d % 128 == 0 (whole pairs of 64-deep chunks) and
  // pays off from about three tiles per compute unit (with fewer, the last
  // round leaves compute units idle; 192 x 128 tiles balance better there)
  const int rows = H * (r_out ? 4 : 3) * dh;
  if (dt == BF16 && d % 128 == 0 && proj_persistent_tiles(T, rows) >= 3 * device_cu_count()) {
#define GBLA_PP(DD)                                                                                \
  (r_out ? proj_persistent<DD, true, 4>(xt, wp, T, d, H, q_out, k_out, v_out, r_out, s)            \
         : (phi ? proj_persistent<DD, true, 3>(xt, wp, T, d, H, q_out, k_out, v_out, r_out, s)     \
                : proj_persistent<DD, false, 3>(xt, wp, T, d, H, q_out, k_out, v_out, r_out, s)))
    if (dh == 64) GBLA_PP(64); else GBLA_PP(32);
#undef GBLA_PP
    return;
  }
  if (dt == BF16) { if (dh == 64) GBLA_PJ(bf16, 64); else GBLA_PJ(bf16, 32); }
  else            { if (dh == 64) GBLA_PJ(float, 64); else GBLA_PJ(float, 32); }
#undef GBLA_PJ
}

// ============================================================== split-L state reduction
// Block = one chunk (<= kChunk tokens of one sequence) x one head. Tiles of 64
// tokens of k~ = g phi(k) and [v | 1] are staged in LDS in token-major order
// exactly as loaded (16-byte vectors); the MFMA operands, which need 8
// consecutive tokens per feature, are read with the transposing LDS read. The
// appended ones column makes the last output column the normaliser z. Each wave
// owns whole 16x16 output tiles, so no cross-wave reduction is needed.
// With the softmax key gate, ga holds the logits s: the chunk's largest logit m
// goes to mpart and the partial uses exp(s - m) (every exponent <= 0); the
// combine rescales the partials to the sequence's largest logit.
template <typename T, int DH, bool SOFTMAX>
__global__ __launch_bounds__(256) void k_state_partial(const T* __restrict__ ka, const T* __restrict__ va,
                                                       const float* __restrict__ ga, const int* __restrict__ nchunks,
                                                       const Chunk* __restrict__ tab, int max_slots, int H,
                                                       float* __restrict__ partial, float* __restrict__ mpart) {
  constexpr int FB = DH / 16, NB = FB + 1;     // key-feature blocks; value blocks + ones block
  constexpr int TILES_S = FB * NB, TPW = (TILES_S + 3) / 4;
  constexpr int ST = 64;                       // tokens per staged tile
  // bf16 pitches of 40 (d_h = 64) or 24 dwords: with the 16-row groups of
  // frag_kmajor_4g, the transposing reads of 40-dword rows are free of bank conflicts
  constexpr bool B16 = sizeof(T) == 2;
  constexpr int LDK = DH + (B16 ? 16 : 4), LDV = 16 * NB + (B16 ? 0 : 4);
  constexpr int E = DH * DH + DH;
  __shared__ __align__(16) T ks[ST * LDK];
  __shared__ __align__(16) T vs[ST * LDV];
  const int lid = xcd_logical_block(blockIdx.x, max_slots * H);
  if (lid >= max_slots * H) return;
  const int slot = lid / H, h = lid - slot * H;
  Chunk ch;
  if (!block_chunk(nchunks, tab, slot, ch)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int D = H * DH;
  for (int e = tid; e < ST * 16; e += 256) {  // ones column (z) and zero padding of the last block
    const int r = e >> 4, c = e & 15;
    vs[r * LDV + DH + c] = from_f<T>(c == 0 ? 1.f : 0.f);
  }
  f32x4 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = zero4();

  // The tile walk is unrolled (a chunk has at most kChunk / ST tiles); SETS
  // tiles are in flight, each in a register set of its own, and rows past the
  // chunk read as zeros through buffer range checks (no branch around a load,
  // so each tile's wait leaves the later tiles' loads in flight).
  constexpr int V8 = DH / 8;  // 8-feature vectors per token row
  constexpr int NV = ST * V8 / 256, TILES = kChunk / ST, SETS = 2;
  static_assert(ST * V8 % 256 == 0 && kChunk % ST == 0, "whole vectors per thread, whole tiles per chunk");
  const int n = ch.end - ch.start;
  const size_t o0 = (size_t)ch.start * D + h * DH;
  const RowBuf<T> kb(ka + o0, n, D, DH), vb(va + o0, n, D, DH);
  const RowScalar gb(ga + (size_t)ch.start * H + h, n, H);
  Frag8<T> pk[SETS][NV], pv[SETS][NV];
  float pg[SETS][NV];
  auto fetch = [&](int i) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int it = tid + 256 * v, r = ST * i + it / V8, c = (it % V8) * 8;
      pg[i % SETS][v] = gb.load(r);  // the gate, or the softmax gate's logit
      pk[i % SETS][v] = kb.load(r, c);
      pv[i % SETS][v] = vb.load(r, c);
    }
  };
#pragma unroll
  for (int i = 0; i < SETS; ++i) fetch(i);
  float gmax = 0.f;  // softmax gate: largest logit of the chunk (reduced while the first tiles load)
  if constexpr (SOFTMAX) {
    __shared__ float wmax[4];
    float m = -INFINITY;
    for (int t = ch.start + tid; t < ch.end; t += 256) m = fmaxf(m, ga[(size_t)t * H + h]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if (lane == 0) wmax[w] = m;
    __syncthreads();
    gmax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    if (tid == 0) mpart[(size_t)slot * H + h] = gmax;
  }
#pragma unroll
  for (int i = 0; i < TILES; ++i) {
    if (ST * i >= n) break;  // uniform (barriers inside)
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int it = tid + 256 * v, r = it / V8, c = (it % V8) * 8;
      const float pgv = pg[i % SETS][v];
      const float g = SOFTMAX ? (ST * i + r < n ? __expf(pgv - gmax) : 0.f) : pgv;
      float kt[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) kt[j] = g * frag_get(pk[i % SETS][v], j);  // rounded once, used by S and z alike
      frag_store(ks + r * LDK + c, frag_from<T>(kt));
      frag_store(vs + r * LDV + c, pv[i % SETS][v]);
    }
    __syncthreads();
    if (i + SETS < TILES) fetch(i + SETS);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tile = w + 4 * u;
      if (tile < TILES_S) {
        const int ib = tile / NB, nb = tile - ib * NB;
#pragma unroll
        for (int k0 = 0; k0 < ST; k0 += 32) {
          const Frag8<T> a = frag_kmajor_4g<T>(ks, LDK, k0, 16 * ib, lane);
          const Frag8<T> b = frag_kmajor_4g<T>(vs, LDV, k0, 16 * nb, lane);
          mma8(acc[u], a, b);
        }
      }
    }
    __syncthreads();
  }
  float* out = partial + ((size_t)slot * H + h) * E;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tile = w + 4 * u;
    if (tile < TILES_S) {
      const int ib = tile / NB, nb = tile - ib * NB;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ib + 4 * grp + r;
        if (nb < FB) out[i * DH + 16 * nb + col] = acc[u][r];
        else if (col == 0) out[DH * DH + i] = acc[u][r];
      }
    }
  }
}

void launch_state_partial(int dt, int dh, const void* ka, const void* va, const float* ga, const int* nchunks,
                          const Chunk* tab, int max_slots, int H, float* partial, float* mpart, hipStream_t s) {
  const dim3 grid(xcd_grid(max_slots * H));
#define GBLA_SP(TT, DD)                                                                                  \
  do {                                                                                                   \
    if (mpart)                                                                                           \
      hipLaunchKernelGGL((k_state_partial<TT, DD, true>), grid, dim3(256), 0, s, (const TT*)ka,          \
                         (const TT*)va, ga, nchunks, tab, max_slots, H, partial, mpart);                 \
    else                                                                                                 \
      hipLaunchKernelGGL((k_state_partial<TT, DD, false>), grid, dim3(256), 0, s, (const TT*)ka,         \
                         (const TT*)va, ga, nchunks, tab, max_slots, H, partial, mpart);                 \
  } while (0)
  if (dt == BF16) { if (dh == 64) GBLA_SP(bf16, 64); else GBLA_SP(bf16, 32); }
  else            { if (dh == 64) GBLA_SP(float, 64); else GBLA_SP(float, 32); }
#undef GBLA_SP
}

// ============================================================== combine
// out[b][h][e] = sum of partial[c][h][e] over the chunks c of sequence b. A
// block covers 256 elements (64 float4) of one (sequence, head); its four
// waves take every fourth chunk and the four sums are added in a fixed order
// (deterministic). E % 4 == 0. With chunk maxima mpart (softmax key gate),
// partial c is scaled by exp(mpart[c] - M), M the largest of the sequence's
// chunk maxima, which goes to mout[b][h] (0 for an empty sequence).
// The launch may end with pk.blocks blocks that pack the dX~ weights (the
// combine of dS leaves most compute units idle).
template <typename T>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ partial, const int* __restrict__ nchunks,
                                                 const int* __restrict__ chunk_off, int H, int E,
                                                 const float* __restrict__ mpart, float* __restrict__ out,
                                                 float* __restrict__ mout, WtPack<T> pk) {
  const int ncomb = (int)gridDim.x - pk.blocks;
  if ((int)blockIdx.x >= ncomb) {
    pack_wt_range(pk, blockIdx.x - ncomb);
    return;
  }
  __shared__ float4 red[4][64];
  const int blk = blockIdx.x;
  const int eblocks = (E + 255) / 256;
  const int bh = blk / eblocks, b = bh / H, h = bh - b * H;
  const int lane = threadIdx.x & 63, ph = threadIdx.x >> 6;
  const int e = (blk - bh * eblocks) * 256 + 4 * lane;
  const int nc = *nchunks;
  const int c0 = min(chunk_off[b], nc), c1 = min(chunk_off[b + 1], nc);
  float M = 0.f;
  if (mpart) {  // every wave reduces the same maximum, its lanes striding over the chunks
    M = -INFINITY;
    for (int c = c0 + lane; c < c1; c += 64) M = fmaxf(M, mpart[(size_t)c * H + h]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    if (c0 == c1) M = 0.f;
    if (mout && blk == bh * eblocks && threadIdx.x == 0) mout[(size_t)b * H + h] = M;
  }
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (e < E)
    for (int c = c0 + ph; c < c1; c += 4) {
      const float4 p = *reinterpret_cast<const float4*>(partial + ((size_t)c * H + h) * E + e);
      const float f = mpart ? __expf(mpart[(size_t)c * H + h] - M) : 1.f;
      s.x += f * p.x; s.y += f * p.y; s.z += f * p.z; s.w += f * p.w;
    }
  red[ph][lane] = s;
  __syncthreads();
  if (ph == 0 && e < E) {
    const float4 a = red[0][lane], b1 = red[1][lane], c2 = red[2][lane], d3 = red[3][lane];
    float4 r;
    r.x = (a.x + b1.x) + (c2.x + d3.x);
    r.y = (a.y + b1.y) + (c2.y + d3.y);
    r.z = (a.z + b1.z) + (c2.z + d3.z);
    r.w = (a.w + b1.w) + (c2.w + d3.w);
    *reinterpret_cast<float4*>(out + ((size_t)b * H + h) * E + e) = r;
  }
}

void launch_combine(const float* partial, const int* nchunks, const int* chunk_off, int N, int H, int elems,
                    float* out, hipStream_t s, const float* mpart, float* mout, const WtPackArgs* pack, int dt) {
  const int grid = ((elems + 255) / 256) * N * H;
  if (pack && dt == BF16)
    hipLaunchKernelGGL(k_combine<bf16>, dim3(grid + wt_pack_blocks(pack->d, pack->Kp)), dim3(256), 0, s, partial,
                       nchunks, chunk_off, H, elems, mpart, out, mout, wt_pack_of<bf16>(*pack));
  else
    hipLaunchKernelGGL(k_combine<float>, dim3(grid + (pack ? wt_pack_blocks(pack->d, pack->Kp) : 0)), dim3(256), 0,
                       s, partial, nchunks, chunk_off, H, elems, mpart, out, mout,
                       pack ? wt_pack_of<float>(*pack) : WtPack<float>{});
}

// out[e] = sum over p < P of in[p * E + e], P = *P_dev * p_mul if given else P_host.
// A block covers EB elements with 256 / EB phases; each thread keeps eight
// independent partial sums so its loads stay in flight. Fixed summation order.
template <int EB>
__global__ __launch_bounds__(256) void k_sum_parts(const float* __restrict__ in, int E, int P_host,
                                                   const int* __restrict__ P_dev, int p_mul, float* __restrict__ out) {
  sum_parts_block<EB>(in, E, P_dev ? *P_dev * p_mul : P_host, out, blockIdx.x);
}

void launch_sum_parts(const float* in, int E, int P_host, const int* P_dev, float* out, hipStream_t s,
                      int p_mul) {
  if (E <= 0) return;
#define GBLA_SUMP(EB) hipLaunchKernelGGL(k_sum_parts<EB>, dim3((E + EB - 1) / EB), dim3(256), 0, s, in, E, P_host, \
                                         P_dev, p_mul, out)
  // the widest blocks that still make about 256 of them; p_mul > 1 sums a long
  // list of parts (one per chunk and head), which wants many threads per element
  if (p_mul == 1 && E >= 64 * 256) GBLA_SUMP(64);
  else if (p_mul == 1 && E >= 16 * 256) GBLA_SUMP(16);
  else GBLA_SUMP(4);
#undef GBLA_SUMP
}

// ============================================================== readout
// Stages [S | z] of the chunk's sequence in LDS as the B operand (column n of
// S, column dh = z), split into a high and a low bfloat16 part for bf16 so the
// state keeps ~16 mantissa bits; A = phi(q) rows straight from HBM.
// GATED: the gated RMSNorm output of Eq. (7) in the epilogue; a token's d_h
// outputs sit in the 16 lanes of one row group (FB per lane), so its mean
// square is a 4-step butterfly; the R tile is staged beside phi(q).
template <typename T> struct SplitState { static constexpr int parts = 2; };
template <> struct SplitState<float> { static constexpr int parts = 1; };

template <typename T, int DH, bool GATED>
__global__ __launch_bounds__(256) void k_readout(const T* __restrict__ qa, const float* __restrict__ saved,
                                                 const int* __restrict__ nchunks, const Chunk* __restrict__ tab,
                                                 int max_slots, int H, T* __restrict__ y, const T* __restrict__ ra,
                                                 const float* __restrict__ gamma, float eps) {
  constexpr int FB = DH / 16;
  constexpr int NR = DH + 16;
  // 40-dword rows for bf16 (d_h = 64): the 16-byte operand reads of 16
  // consecutive rows hit distinct banks (at 36 dwords, 61% of the kernel's LDS
  // cycles were bank conflicts)
  constexpr int LD = sizeof(T) == 2 ? DH + 16 : DH + 4;
  constexpr int P = SplitState<T>::parts;
  constexpr int E = DH * DH + DH;
  constexpr int ST = 64, V8 = DH / 8;
  __shared__ __align__(16) T Bs[P * NR * LD];
  __shared__ __align__(16) T qs[ST * LD];  // phi(q) tile, then y
  __shared__ __align__(16) T rs[GATED ? ST * LD : 8];  // R tile (gated output)
  const int lid = xcd_logical_block(blockIdx.x, max_slots * H);
  if (lid >= max_slots * H) return;
  const int slot = lid / H, h = lid - slot * H;
  Chunk ch;
  if (!block_chunk(nchunks, tab, slot, ch)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int D = H * DH;
  const float* st = saved + ((size_t)ch.seq * H + h) * E;
  const int r0 = 16 * w;
  float gam[FB];  // RMSNorm scale of the lane's features 16 nt + col
#pragma unroll
  for (int nt = 0; nt < FB; ++nt) gam[nt] = GATED && gamma ? gamma[16 * nt + col] : 1.f;

  // A chunk has at most kChunk / ST tiles: the tile walk is unrolled, and the
  // first SETS tiles' loads are issued at the start (while the state is
  // staged), each into a register set of its own; tile i + SETS reuses tile i's
  // set once tile i is in LDS. Rows past the chunk read as zeros and their
  // stores are dropped (buffer range checks), so no branch surrounds a memory
  // operation and each tile's wait leaves the later tiles' loads in flight.
  constexpr int NV = ST * V8 / 256, TILES = kChunk / ST;
  constexpr int SETS = sizeof(T) == 2 && !(GATED && DH == 64) ? TILES : 2;  // within the register budget
  static_assert(ST * V8 % 256 == 0 && kChunk % ST == 0, "whole vectors per thread, whole tiles per chunk");
  const int n = ch.end - ch.start;
  const size_t o0 = (size_t)ch.start * D + h * DH;
  const RowBuf<T> qb(qa + o0, n, D, DH), yb(y + o0, n, D, DH), rb(GATED ? ra + o0 : qa + o0, n, D, DH);
  Frag8<T> pf[SETS][NV], pr[SETS][NV];
  auto fetch = [&](int i) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int it = tid + 256 * v, r = it / V8, c = (it % V8) * 8;
      pf[i % SETS][v] = qb.load(ST * i + r, c);
      if constexpr (GATED) pr[i % SETS][v] = rb.load(ST * i + r, c);
    }
  };
#pragma unroll
  for (int i = 0; i < SETS; ++i) fetch(i);
  stage_state<T, DH, NR>(Bs, nullptr, LD, st, st + DH * DH, tid);
#pragma unroll
  for (int i = 0; i < TILES; ++i) {
    if (ST * i >= n) break;  // uniform (barriers inside)
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int it = tid + 256 * v;
      frag_store(qs + (it / V8) * LD + (it % V8) * 8, pf[i % SETS][v]);
      if constexpr (GATED) frag_store(rs + (it / V8) * LD + (it % V8) * 8, pr[i % SETS][v]);
    }
    __syncthreads();
    if (i + SETS < TILES) fetch(i + SETS);
    const int tb = ch.start + ST * i;
    Frag8<T> a[DH / 32];
#pragma unroll
    for (int s = 0; s < DH / 32; ++s) a[s] = frag_load(qs + (r0 + col) * LD + 32 * s + 8 * grp);
    f32x4 acc[FB + 1];
#pragma unroll
    for (int nt = 0; nt <= FB; ++nt) {
      acc[nt] = zero4();
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int s = 0; s < DH / 32; ++s)
          mma8(acc[nt], a[s], frag_load(Bs + p * NR * LD + (16 * nt + col) * LD + 32 * s + 8 * grp));
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = r0 + 4 * grp + r;
      const bool ok = tb + row < ch.end;
      const float den = col0_bcast(acc[FB][r]);
      const float inv = ok ? fast_rcp(den) : 0.f;
      if constexpr (GATED) {
        // y = gamma (.) O / sqrt(mean(O^2) + eps) (.) SiLU(r)
        float o[FB], ss = 0.f;
#pragma unroll
        for (int nt = 0; nt < FB; ++nt) {
          o[nt] = acc[nt][r] * inv;
          ss += o[nt] * o[nt];
        }
        ss = row16_sum(ss);
        const float rinv = ok ? fast_rsqrt(ss * (1.f / DH) + eps) : 0.f;
#pragma unroll
        for (int nt = 0; nt < FB; ++nt) {
          const float rv = to_f<T>(rs[row * LD + 16 * nt + col]);
          qs[row * LD + 16 * nt + col] = from_f<T>(gam[nt] * o[nt] * rinv * rv * sigmoidf_(rv));
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < FB; ++nt) qs[row * LD + 16 * nt + col] = from_f<T>(acc[nt][r] * inv);
      }
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int it = tid + 256 * v, r = it / V8, c = (it % V8) * 8;
      yb.store(ST * i + r, c, frag_load(qs + r * LD + c));  // rows past the chunk are dropped
    }
    __syncthreads();
  }
}

void launch_readout(int dt, int dh, const void* qa, const float* saved, const int* nchunks, const Chunk* tab,
                    int max_slots, int H, void* y, hipStream_t s, const void* ra, const float* gamma, float eps) {
  const dim3 grid(xcd_grid(max_slots * H));
#define GBLA_RO(TT, DD)                                                                                        \
  do {                                                                                                         \
    if (ra)                                                                                                    \
      hipLaunchKernelGGL((k_readout<TT, DD, true>), grid, dim3(256), 0, s, (const TT*)qa, saved, nchunks, tab, \
                         max_slots, H, (TT*)y, (const TT*)ra, gamma, eps);                                     \
    else                                                                                                       \
      hipLaunchKernelGGL((k_readout<TT, DD, false>), grid, dim3(256), 0, s, (const TT*)qa, saved, nchunks,     \
                         tab, max_slots, H, (TT*)y, (const TT*)ra, gamma, eps);                                \
  } while (0)
  if (dt == BF16) { if (dh == 64) GBLA_RO(bf16, 64); else GBLA_RO(bf16, 32); }
  else            { if (dh == 64) GBLA_RO(float, 64); else GBLA_RO(float, 32); }
#undef GBLA_RO
}

}  // namespace gbla
