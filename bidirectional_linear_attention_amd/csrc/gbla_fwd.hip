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
//   k_schedule      chunk table of <= kChunk-token runs inside each sequence, from cu_seqlens
//   k_pack_proj     per-head packed weights [H][3*dh+16][d]: Q, K, V columns then the gate row
//   k_proj          fused conv + projection GEMM (MFMA) + phi + gate epilogue
//   k_state_partial split-L partial [S | z] per (chunk, head), MFMA over the token axis
//   k_combine       fixed-order sum of the partials of each (sequence, head)
//   k_readout       y = phi(Q) [S | z] (MFMA), divide
#include "internal.h"

namespace gbla {

// ============================================================== schedule
__global__ __launch_bounds__(1024) void k_schedule(const int32_t* __restrict__ cu, int N, int T, int max_slots,
                                                   int* __restrict__ nchunks, int* __restrict__ chunk_off,
                                                   Chunk* __restrict__ tab) {
  __shared__ int scan[1024];
  __shared__ int bad;
  const int tid = threadIdx.x;
  if (tid == 0) bad = (cu[0] != 0) || (cu[N] != T);
  __syncthreads();
  for (int b = tid; b < N; b += 1024)
    if (cu[b + 1] < cu[b]) bad = 1;
  __syncthreads();
  if (bad) {  // malformed offsets: schedule nothing, so no kernel reads outside [0, T)
    for (int b = tid; b <= N; b += 1024) chunk_off[b] = 0;
    if (tid == 0) *nchunks = 0;
    return;
  }
  int carry = 0;
  for (int b0 = 0; b0 < N; b0 += 1024) {
    const int b = b0 + tid;
    int n = 0;
    if (b < N) n = (cu[b + 1] - cu[b] + kChunk - 1) / kChunk;
    scan[tid] = n;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int excl = carry + scan[tid] - n;
    if (b < N) {
      chunk_off[b] = excl;
      const int s = cu[b], e = cu[b + 1];
      for (int c = 0; c < n && excl + c < max_slots; ++c) {
        Chunk ch;
        ch.seq = b;
        ch.start = s + c * kChunk;
        ch.end = min(s + (c + 1) * kChunk, e);
        ch.pad = 0;
        tab[excl + c] = ch;
      }
    }
    carry += scan[1023];
    __syncthreads();
  }
  if (tid == 0) {
    chunk_off[N] = min(carry, max_slots);
    *nchunks = min(carry, max_slots);
  }
}

void launch_schedule(const int32_t* cu, int N, int T, int max_slots, int* nchunks, int* chunk_off, Chunk* tab,
                     hipStream_t s) {
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(1024), 0, s, cu, N, T, max_slots, nchunks, chunk_off, tab);
}

// ============================================================== weight packing
template <typename T>
__global__ void k_pack_proj(const T* __restrict__ w_q, const T* __restrict__ w_k, const T* __restrict__ w_v,
                            const T* __restrict__ w_g, int d, int H, int dh, T* __restrict__ wp) {
  const int NP = 3 * dh + 16, D = H * dh;
  const long total = (long)H * NP * d;
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < total; e += (long)gridDim.x * blockDim.x) {
    const int c = (int)(e % d);
    const int n = (int)((e / d) % NP);
    const int h = (int)(e / ((long)d * NP));
    T v = from_f<T>(0.f);
    if (n < dh) v = w_q[(long)c * D + h * dh + n];
    else if (n < 2 * dh) v = w_k[(long)c * D + h * dh + n - dh];
    else if (n < 3 * dh) v = w_v[(long)c * D + h * dh + n - 2 * dh];
    else if (n == 3 * dh) v = w_g[(long)h * d + c];
    wp[e] = v;
  }
}

void launch_pack_proj(int dt, const void* w_q, const void* w_k, const void* w_v, const void* w_g, int d, int H,
                      int dh, void* wp, hipStream_t s) {
  const long total = (long)H * proj_cols(dh) * d;
  const int grid = (int)std::min<long>((total + 255) / 256, 4096);
  if (dt == BF16)
    hipLaunchKernelGGL(k_pack_proj<bf16>, dim3(grid), dim3(256), 0, s, (const bf16*)w_q, (const bf16*)w_k,
                       (const bf16*)w_v, (const bf16*)w_g, d, H, dh, (bf16*)wp);
  else
    hipLaunchKernelGGL(k_pack_proj<float>, dim3(grid), dim3(256), 0, s, (const float*)w_q, (const float*)w_k,
                       (const float*)w_v, (const float*)w_g, d, H, dh, (float*)wp);
}

// ============================================================== fused conv + projection
// One block = 128 packed tokens x one head; four waves of 32 rows, each wave
// holding all 3*dh/16 + 1 output tiles of its rows. k runs over d in chunks of
// 128 bytes per row staged in LDS; the A chunk is produced by the causal conv
// straight from x (never written to HBM in the forward).
template <typename T> struct GemmCfg {
  static constexpr int BK = 128 / (int)sizeof(T);   // k elements per LDS chunk
  static constexpr int LD = BK + 16 / (int)sizeof(T);  // LDS row pitch (16 B pad)
};

template <typename T, int DH, bool BWD>
__global__ __launch_bounds__(256) void k_proj(const T* __restrict__ x, const int32_t* __restrict__ cu, int nseq,
                                              int T_, int d, int H, const T* __restrict__ conv_w,
                                              const T* __restrict__ wp, const float* __restrict__ b_g,
                                              T* __restrict__ q_out, T* __restrict__ k_out, T* __restrict__ v_out,
                                              float* __restrict__ g_out, T* __restrict__ xt_out) {
  constexpr int BM = 128;
  constexpr int FB = DH / 16;          // 16-wide feature blocks per head
  constexpr int NT = 3 * FB + 1;       // + gate tile
  constexpr int NP = NT * 16;
  constexpr int BK = GemmCfg<T>::BK, LD = GemmCfg<T>::LD;
  constexpr int G8 = BK / 8;
  constexpr int AIT = BM * G8 / 256;
  __shared__ __align__(16) T As[BM * LD];
  __shared__ __align__(16) T Bs[NP * LD];

  const int mtiles = (T_ + BM - 1) / BM;
  const int lid = xcd_logical_block(blockIdx.x, mtiles * H);
  if (lid >= mtiles * H) return;
  const int mt = lid / H, h = lid - mt * H;
  const int m0 = mt * BM;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int D = H * DH;

  int arow[AIT], apos[AIT], ag8[AIT];
#pragma unroll
  for (int i = 0; i < AIT; ++i) {
    const int it = tid + 256 * i;
    arow[i] = it / G8;
    ag8[i] = it % G8;
    const int t = m0 + arow[i];
    apos[i] = t < T_ ? pos_in_seq(cu, nseq, t) : -1;
  }

  f32x4 acc[2][NT];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mi][nt] = zero4();

  const T* wph = wp + (size_t)h * NP * d;
  for (int k0 = 0; k0 < d; k0 += BK) {
#pragma unroll
    for (int i = 0; i < AIT; ++i) {
      const int c = k0 + ag8[i] * 8;
      const int t = m0 + arow[i];
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = 0.f;
      if (apos[i] >= 0 && c < d) {
        float wv[32];  // conv_w[c + j][k] at wv[4 * j + k]
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const Frag8<T> f = frag_load(conv_w + (size_t)c * 4 + 8 * m);
#pragma unroll
          for (int e = 0; e < 8; ++e) wv[8 * m + e] = frag_get(f, e);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int sh = 3 - k;  // tap k reads the token sh steps back
          if (sh > apos[i]) continue;
          const Frag8<T> xv = frag_load(x + (size_t)(t - sh) * d + c);
#pragma unroll
          for (int j = 0; j < 8; ++j) o[j] += wv[4 * j + k] * frag_get(xv, j);
        }
      }
      const Frag8<T> f = frag_from<T>(o);
      frag_store(As + arow[i] * LD + ag8[i] * 8, f);
      if (BWD && h == 0 && t < T_ && c < d) frag_store(xt_out + (size_t)t * d + c, f);
    }
    for (int it = tid; it < NP * G8; it += 256) {
      const int n = it / G8, g8 = it - n * G8;
      const int c = k0 + g8 * 8;
      const Frag8<T> f = c < d ? frag_load(wph + (size_t)n * d + c) : frag_zero<T>();
      frag_store(Bs + n * LD + g8 * 8, f);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      Frag8<T> a[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) a[mi] = frag_load(As + (32 * w + 16 * mi + col) * LD + ks + 8 * grp);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const Frag8<T> b = frag_load(Bs + (16 * nt + col) * LD + ks + 8 * grp);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) mma8(acc[mi][nt], a[mi], b);
      }
    }
    __syncthreads();
  }

  const float bg = b_g[h];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int rbase = m0 + 32 * w + 16 * mi + 4 * grp;
    float g[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) g[r] = col0_bcast(sigmoidf_(acc[mi][NT - 1][r] + bg), lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = rbase + r;
      if (t >= T_) continue;
      T* qrow = q_out + (size_t)t * D + h * DH + col;
      T* krow = k_out + (size_t)t * D + h * DH + col;
      T* vrow = v_out + (size_t)t * D + h * DH + col;
#pragma unroll
      for (int f = 0; f < FB; ++f) {
        qrow[16 * f] = from_f<T>(phi_elu1(acc[mi][f][r]));
        const float kf = phi_elu1(acc[mi][FB + f][r]);
        krow[16 * f] = from_f<T>(BWD ? kf : g[r] * kf);
        vrow[16 * f] = from_f<T>(acc[mi][2 * FB + f][r]);
      }
      if (BWD && col == 0) g_out[(size_t)t * H + h] = g[r];
    }
  }
}

template <typename T, int DH, bool BWD>
static void proj_t(const void* x, const int32_t* cu, int N, int T_, int d, int H, const void* conv_w, const void* wp,
                   const float* b_g, void* q, void* k, void* v, float* g, void* xt, hipStream_t s) {
  const int n = ((T_ + 127) / 128) * H;
  hipLaunchKernelGGL((k_proj<T, DH, BWD>), dim3(xcd_grid(n)), dim3(256), 0, s, (const T*)x, cu, N, T_, d, H,
                     (const T*)conv_w, (const T*)wp, b_g, (T*)q, (T*)k, (T*)v, g, (T*)xt);
}

void launch_proj(int dt, int dh, bool bwd, const void* x, const int32_t* cu, int N, int T, int d, int H,
                 const void* conv_w, const void* wp, const float* b_g, void* q_out, void* k_out, void* v_out,
                 float* g_out, void* xt_out, hipStream_t s) {
#define GBLA_PROJ(TT, DD, BB) proj_t<TT, DD, BB>(x, cu, N, T, d, H, conv_w, wp, b_g, q_out, k_out, v_out, g_out, xt_out, s)
  if (dt == BF16) {
    if (dh == 64) { if (bwd) GBLA_PROJ(bf16, 64, true); else GBLA_PROJ(bf16, 64, false); }
    else          { if (bwd) GBLA_PROJ(bf16, 32, true); else GBLA_PROJ(bf16, 32, false); }
  } else {
    if (dh == 64) { if (bwd) GBLA_PROJ(float, 64, true); else GBLA_PROJ(float, 64, false); }
    else          { if (bwd) GBLA_PROJ(float, 32, true); else GBLA_PROJ(float, 32, false); }
  }
#undef GBLA_PROJ
}

// ============================================================== split-L state reduction
// Block = one chunk (<= kChunk tokens of one sequence) x one head. Each wave
// takes 16 tokens at a time, loads g*phi(k) and v in C-tile order (lane holds
// feature lane%16 of tokens 4*(lane/16)+0..3) and contracts over the tokens with
// K=16 MFMAs, accumulating the whole dh x dh partial state. The four wave
// partials are summed in a fixed order through LDS.
template <typename T, int DH>
__global__ __launch_bounds__(256) void k_state_partial(const T* __restrict__ ka, const T* __restrict__ va,
                                                       const int* __restrict__ nchunks,
                                                       const Chunk* __restrict__ tab, int max_slots, int H,
                                                       float* __restrict__ partial) {
  constexpr int FB = DH / 16;
  constexpr int E = DH * DH + DH;
  __shared__ float red[E];
  const int lid = xcd_logical_block(blockIdx.x, max_slots * H);
  if (lid >= max_slots * H) return;
  const int slot = lid / H, h = lid - slot * H;
  if (slot >= *nchunks) return;
  const Chunk ch = tab[slot];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int D = H * DH;

  f32x4 sacc[FB][FB];
  float zacc[FB];
#pragma unroll
  for (int a = 0; a < FB; ++a) {
    zacc[a] = 0.f;
#pragma unroll
    for (int b = 0; b < FB; ++b) sacc[a][b] = zero4();
  }
  for (int t0 = ch.start + 16 * w; t0 < ch.end; t0 += 64) {
    float kv[FB][4], vv[FB][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + 4 * grp + j;
      const bool ok = t < ch.end;
      const size_t base = (size_t)(ok ? t : ch.start) * D + h * DH + col;
#pragma unroll
      for (int b = 0; b < FB; ++b) {
        kv[b][j] = ok ? to_f<T>(ka[base + 16 * b]) : 0.f;
        vv[b][j] = ok ? to_f<T>(va[base + 16 * b]) : 0.f;
      }
    }
#pragma unroll
    for (int a = 0; a < FB; ++a) {
      zacc[a] += (kv[a][0] + kv[a][1]) + (kv[a][2] + kv[a][3]);
#pragma unroll
      for (int b = 0; b < FB; ++b) mma4<T>(sacc[a][b], kv[a], vv[b]);
    }
  }
#pragma unroll
  for (int a = 0; a < FB; ++a) {
    zacc[a] += __shfl_xor(zacc[a], 16, 64);
    zacc[a] += __shfl_xor(zacc[a], 32, 64);
  }
  // fixed-order cross-wave sum: wave 0 stores, waves 1..3 add in turn
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int a = 0; a < FB; ++a) {
#pragma unroll
        for (int b = 0; b < FB; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int idx = (16 * a + 4 * grp + r) * DH + 16 * b + col;
            red[idx] = ww == 0 ? sacc[a][b][r] : red[idx] + sacc[a][b][r];
          }
        if (grp == 0) {
          const int idx = DH * DH + 16 * a + col;
          red[idx] = ww == 0 ? zacc[a] : red[idx] + zacc[a];
        }
      }
    }
    __syncthreads();
  }
  float* out = partial + ((size_t)slot * H + h) * E;
  for (int e = tid; e < E; e += 256) out[e] = red[e];
}

void launch_state_partial(int dt, int dh, const void* ka, const void* va, const int* nchunks, const Chunk* tab,
                          int max_slots, int H, float* partial, hipStream_t s) {
  const dim3 grid(xcd_grid(max_slots * H));
#define GBLA_SP(TT, DD) hipLaunchKernelGGL((k_state_partial<TT, DD>), grid, dim3(256), 0, s, (const TT*)ka, \
                                           (const TT*)va, nchunks, tab, max_slots, H, partial)
  if (dt == BF16) { if (dh == 64) GBLA_SP(bf16, 64); else GBLA_SP(bf16, 32); }
  else            { if (dh == 64) GBLA_SP(float, 64); else GBLA_SP(float, 32); }
#undef GBLA_SP
}

// ============================================================== combine
// out[b][h][e] = sum of partial[slot][h][e] over the chunks of sequence b, in
// chunk order (deterministic).
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ partial, const int* __restrict__ nchunks,
                                                 const int* __restrict__ chunk_off, int N, int H, int E,
                                                 float* __restrict__ out) {
  const int b = blockIdx.x / H, h = blockIdx.x - b * H;
  const int nc = *nchunks;
  const int c0 = min(chunk_off[b], nc), c1 = min(chunk_off[b + 1], nc);
  for (int e = threadIdx.x; e < E; e += 256) {
    float s = 0.f;
    for (int c = c0; c < c1; ++c) s += partial[((size_t)c * H + h) * E + e];
    out[((size_t)b * H + h) * E + e] = s;
  }
}

void launch_combine(const float* partial, const int* nchunks, const int* chunk_off, int N, int H, int elems,
                    float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_combine, dim3(N * H), dim3(256), 0, s, partial, nchunks, chunk_off, N, H, elems, out);
}

// ============================================================== readout
// Stages [S | z] of the chunk's sequence in LDS as the B operand (column n of
// S, column dh = z), split into a high and a low bfloat16 part for bf16 so the
// state keeps ~16 mantissa bits; A = phi(q) rows straight from HBM.
template <typename T> struct SplitState { static constexpr int parts = 2; };
template <> struct SplitState<float> { static constexpr int parts = 1; };

template <typename T, int DH, int NROWS>
__device__ __forceinline__ void stage_state_T(T* __restrict__ Bs, int ld, const float* __restrict__ S,
                                              const float* __restrict__ z, int tid) {
  // Bs[part][n][i] = S[i][n] (n < DH), z[i] (n == DH), 0 (DH < n < NROWS)
  for (int e = tid; e < NROWS * DH; e += 256) {
    const int n = e / DH, i = e - n * DH;
    const float v = n < DH ? S[i * DH + n] : (n == DH ? z[i] : 0.f);
    const T hi = from_f<T>(v);
    Bs[n * ld + i] = hi;
    if (SplitState<T>::parts == 2) Bs[NROWS * ld + n * ld + i] = from_f<T>(v - to_f<T>(hi));
  }
}

template <typename T, int DH>
__global__ __launch_bounds__(256) void k_readout(const T* __restrict__ qa, const float* __restrict__ saved,
                                                 const int* __restrict__ nchunks, const Chunk* __restrict__ tab,
                                                 int max_slots, int H, T* __restrict__ y) {
  constexpr int FB = DH / 16;
  constexpr int NR = DH + 16;
  constexpr int LD = DH + 16 / (int)sizeof(T);
  constexpr int P = SplitState<T>::parts;
  constexpr int E = DH * DH + DH;
  __shared__ __align__(16) T Bs[P * NR * LD];
  const int lid = xcd_logical_block(blockIdx.x, max_slots * H);
  if (lid >= max_slots * H) return;
  const int slot = lid / H, h = lid - slot * H;
  if (slot >= *nchunks) return;
  const Chunk ch = tab[slot];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int D = H * DH;
  const float* st = saved + ((size_t)ch.seq * H + h) * E;
  stage_state_T<T, DH, NR>(Bs, LD, st, st + DH * DH, tid);
  __syncthreads();

  for (int t0 = ch.start + 16 * w; t0 < ch.end; t0 += 64) {
    const int ta = t0 + col;  // A-operand row of this lane
    Frag8<T> a[DH / 32];
#pragma unroll
    for (int s = 0; s < DH / 32; ++s)
      a[s] = ta < ch.end ? frag_load(qa + (size_t)ta * D + h * DH + 32 * s + 8 * grp) : frag_zero<T>();
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
      const float den = col0_bcast(acc[FB][r], lane);
      const int t = t0 + 4 * grp + r;
      if (t < ch.end) {
        const float inv = 1.f / den;
        T* yrow = y + (size_t)t * D + h * DH + col;
#pragma unroll
        for (int nt = 0; nt < FB; ++nt) yrow[16 * nt] = from_f<T>(acc[nt][r] * inv);
      }
    }
  }
}

void launch_readout(int dt, int dh, const void* qa, const float* saved, const int* nchunks, const Chunk* tab,
                    int max_slots, int H, void* y, hipStream_t s) {
  const dim3 grid(xcd_grid(max_slots * H));
#define GBLA_RO(TT, DD) hipLaunchKernelGGL((k_readout<TT, DD>), grid, dim3(256), 0, s, (const TT*)qa, saved, \
                                           nchunks, tab, max_slots, H, (TT*)y)
  if (dt == BF16) { if (dh == 64) GBLA_RO(bf16, 64); else GBLA_RO(bf16, 32); }
  else            { if (dh == 64) GBLA_RO(float, 64); else GBLA_RO(float, 32); }
#undef GBLA_RO
}

}  // namespace gbla
