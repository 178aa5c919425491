// GBLA backward kernels for gfx950.
//
// Reverse mode of the forward (Eqs. (4)-(6) of "Gated Bidirectional Linear
// Attention for Generative Retrieval"), per sequence b and head h, with
// q~ = phi(q), k~ = g phi(k), den_i = q~_i . z, y_i = q~_i^T S / den_i:
//   dn_i = dy_i / den_i,  dden_i = -(dy_i . y_i) / den_i
//   dq~_i = S dn_i + dden_i z        dS = sum_i q~_i dn_i^T,  dz = sum_i dden_i q~_i
//   dk~_j = dS v_j + dz              dv_j = dS^T k~_j
//   dk = g dk~ (.) phi'(k),  dg_j = phi(k_j) . dk~_j,  ds = dg g (1 - g),  dq = dq~ (.) phi'(q)
// with phi'(u) = min(1, phi(u)) for phi = elu + 1. Then the projection chain rule
//   dX~ = [dQ|dK|dV|ds] [W_Q|W_K|W_V|w_g^T]^T,  dW = X~^T [dQ|dK|dV|ds],  db_g = sum_t ds
// and the conv chain rule.
//
// Kernels:
//   (k_proj in backward mode recomputes phi(q), phi(k), v, g and writes x~)
//   k_bwd_dstate  per (chunk, head): y, dn, dden, dq -> G; partial [dS | dz]
//   k_bwd_token   per (chunk, head): dk, dv, ds -> G; partial db_g
//   k_gemm_nt     dX~ = G Wt^T (MFMA)
//   k_gemm_tn     split-token partials of X~^T G (MFMA), then k_dw_reduce
//   k_conv_bwd    dx and per-block partial dconv_w, then k_dconv_reduce
#include "internal.h"

namespace gbla {

template <typename T> struct Parts { static constexpr int n = 2; };  // bf16: hi + lo split of fp32 matrices
template <> struct Parts<float> { static constexpr int n = 1; };

// Bs[p][row][col] (ld pitch) <- split(M[row][col]) for a dh x dh fp32 matrix,
// transposed when TR (Bs[p][col][row] = M[row][col]).
template <typename T, int DH, bool TR>
__device__ __forceinline__ void stage_mat(T* __restrict__ Bs, int ld, const float* __restrict__ M, int tid) {
  for (int e = tid; e < DH * DH; e += 256) {
    const int r = e / DH, c = e - r * DH;
    const float v = M[e];
    const int o = TR ? c * ld + r : r * ld + c;
    const T hi = from_f<T>(v);
    Bs[o] = hi;
    if (Parts<T>::n == 2) Bs[DH * ld + o] = from_f<T>(v - to_f<T>(hi));
  }
}

// fixed-order sum of per-wave dh x dh C-tile accumulators (+ a per-lane vector) into red[]
template <int DH>
__device__ __forceinline__ void wave_reduce_state(float* red, const f32x4 (&acc)[DH / 16][DH / 16],
                                                  const float (&vec)[DH / 16], int w, int grp, int col) {
  constexpr int FB = DH / 16;
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int a = 0; a < FB; ++a) {
#pragma unroll
        for (int b = 0; b < FB; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int idx = (16 * a + 4 * grp + r) * DH + 16 * b + col;
            red[idx] = ww == 0 ? acc[a][b][r] : red[idx] + acc[a][b][r];
          }
        if (grp == 0) {
          const int idx = DH * DH + 16 * a + col;
          red[idx] = ww == 0 ? vec[a] : red[idx] + vec[a];
        }
      }
    }
    __syncthreads();
  }
}

// ============================================================== dS, dz and dq
template <typename T, int DH>
__global__ __launch_bounds__(256) void k_bwd_dstate(const T* __restrict__ qa, const T* __restrict__ dy,
                                                    const float* __restrict__ saved, const int* __restrict__ nchunks,
                                                    const Chunk* __restrict__ tab, int max_slots, int H, int Kp,
                                                    float* __restrict__ partial, T* __restrict__ G) {
  constexpr int FB = DH / 16;
  constexpr int NR = DH + 16;
  constexpr int LD = DH + 16 / (int)sizeof(T);
  constexpr int P = Parts<T>::n;
  constexpr int E = DH * DH + DH;
  __shared__ __align__(16) T Bsz[P * NR * LD];  // [S | z] as B of q~ [S|z]:  Bsz[n][i]
  __shared__ __align__(16) T Brm[P * DH * LD];  // S as B of dn S^T:          Brm[a][n] = S[a][n]
  __shared__ __align__(16) T dns[4 * 16 * LD];  // per-wave dn rows
  __shared__ float zs[DH];
  __shared__ float red[E];

  const int lid = xcd_logical_block(blockIdx.x, max_slots * H);
  if (lid >= max_slots * H) return;
  const int slot = lid / H, h = lid - slot * H;
  if (slot >= *nchunks) return;
  const Chunk ch = tab[slot];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int D = H * DH;
  const float* st = saved + ((size_t)ch.seq * H + h) * E;
  for (int e = tid; e < NR * DH; e += 256) {
    const int n = e / DH, i = e - n * DH;
    const float v = n < DH ? st[i * DH + n] : (n == DH ? st[DH * DH + i] : 0.f);
    const T hi = from_f<T>(v);
    Bsz[n * LD + i] = hi;
    if (P == 2) Bsz[NR * LD + n * LD + i] = from_f<T>(v - to_f<T>(hi));
  }
  stage_mat<T, DH, false>(Brm, LD, st, tid);
  for (int e = tid; e < DH; e += 256) zs[e] = st[DH * DH + e];
  __syncthreads();

  f32x4 dS[FB][FB];
  float dz[FB];
#pragma unroll
  for (int a = 0; a < FB; ++a) {
    dz[a] = 0.f;
#pragma unroll
    for (int b = 0; b < FB; ++b) dS[a][b] = zero4();
  }
  T* dnw = dns + w * 16 * LD;

  for (int tb = ch.start; tb < ch.end; tb += 64) {  // uniform trip count (barriers inside)
    const int t0 = tb + 16 * w;
    const int ta = t0 + col;
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
          mma8(acc[nt], a[s], frag_load(Bsz + p * NR * LD + (16 * nt + col) * LD + 32 * s + 8 * grp));
    }
    float qv[FB][4], dn[FB][4], dden[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 4 * grp + r;
      const bool ok = t < ch.end;
      const float den = col0_bcast(acc[FB][r], lane);
      const float inv = ok ? 1.f / den : 0.f;
      const size_t base = (size_t)(ok ? t : ch.start) * D + h * DH + col;
      float p = 0.f, dyv[FB];
#pragma unroll
      for (int nt = 0; nt < FB; ++nt) {
        dyv[nt] = ok ? to_f<T>(dy[base + 16 * nt]) : 0.f;
        qv[nt][r] = ok ? to_f<T>(qa[base + 16 * nt]) : 0.f;
        p += dyv[nt] * (acc[nt][r] * inv);
      }
      p = row16_sum(p);
      dden[r] = -p * inv;
#pragma unroll
      for (int nt = 0; nt < FB; ++nt) {
        dn[nt][r] = dyv[nt] * inv;
        dnw[(4 * grp + r) * LD + 16 * nt + col] = from_f<T>(dn[nt][r]);
      }
    }
    __syncthreads();
    Frag8<T> dnf[DH / 32];
#pragma unroll
    for (int s = 0; s < DH / 32; ++s) dnf[s] = frag_load(dnw + col * LD + 32 * s + 8 * grp);
#pragma unroll
    for (int nt = 0; nt < FB; ++nt) {
      f32x4 dq = zero4();
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int s = 0; s < DH / 32; ++s)
          mma8(dq, dnf[s], frag_load(Brm + p * DH * LD + (16 * nt + col) * LD + 32 * s + 8 * grp));
      const float za = zs[16 * nt + col];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 4 * grp + r;
        if (t < ch.end) {
          const float v = (dq[r] + dden[r] * za) * fminf(1.f, qv[nt][r]);
          G[(size_t)t * Kp + h * DH + 16 * nt + col] = from_f<T>(v);
        }
      }
    }
#pragma unroll
    for (int ia = 0; ia < FB; ++ia) {
      dz[ia] += (dden[0] * qv[ia][0] + dden[1] * qv[ia][1]) + (dden[2] * qv[ia][2] + dden[3] * qv[ia][3]);
#pragma unroll
      for (int nb = 0; nb < FB; ++nb) mma4<T>(dS[ia][nb], qv[ia], dn[nb]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < FB; ++a) {
    dz[a] += __shfl_xor(dz[a], 16, 64);
    dz[a] += __shfl_xor(dz[a], 32, 64);
  }
  wave_reduce_state<DH>(red, dS, dz, w, grp, col);
  float* out = partial + ((size_t)slot * H + h) * E;
  for (int e = tid; e < E; e += 256) out[e] = red[e];
}

void launch_bwd_dstate(int dt, int dh, const void* qa, const void* dy, const float* saved, const int* nchunks,
                       const Chunk* tab, int max_slots, int H, int Kp, float* partial, void* G, hipStream_t s) {
  const dim3 grid(xcd_grid(max_slots * H));
#define GBLA_BD(TT, DD) hipLaunchKernelGGL((k_bwd_dstate<TT, DD>), grid, dim3(256), 0, s, (const TT*)qa, \
                                           (const TT*)dy, saved, nchunks, tab, max_slots, H, Kp, partial, (TT*)G)
  if (dt == BF16) { if (dh == 64) GBLA_BD(bf16, 64); else GBLA_BD(bf16, 32); }
  else            { if (dh == 64) GBLA_BD(float, 64); else GBLA_BD(float, 32); }
#undef GBLA_BD
}

// ============================================================== dk, dv, ds
template <typename T, int DH>
__global__ __launch_bounds__(256) void k_bwd_token(const T* __restrict__ ka, const T* __restrict__ va,
                                                   const float* __restrict__ ga, const float* __restrict__ dsz,
                                                   const int* __restrict__ nchunks, const Chunk* __restrict__ tab,
                                                   int max_slots, int H, int Kp, T* __restrict__ G,
                                                   float* __restrict__ dbg_part) {
  constexpr int FB = DH / 16;
  constexpr int LD = DH + 16 / (int)sizeof(T);
  constexpr int P = Parts<T>::n;
  constexpr int E = DH * DH + DH;
  __shared__ __align__(16) T Srm[P * DH * LD];  // dS as B of v dS^T: Srm[i][n] = dS[i][n]
  __shared__ __align__(16) T Str[P * DH * LD];  // dS as B of k~ dS:  Str[n][i] = dS[i][n]
  __shared__ float dzs[DH];
  __shared__ float wsum[4];

  const int lid = xcd_logical_block(blockIdx.x, max_slots * H);
  if (lid >= max_slots * H) return;
  const int slot = lid / H, h = lid - slot * H;
  if (slot >= *nchunks) return;
  const Chunk ch = tab[slot];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int D = H * DH;
  const float* st = dsz + ((size_t)ch.seq * H + h) * E;
  stage_mat<T, DH, false>(Srm, LD, st, tid);
  stage_mat<T, DH, true>(Str, LD, st, tid);
  for (int e = tid; e < DH; e += 256) dzs[e] = st[DH * DH + e];
  __syncthreads();

  float dbg = 0.f;
  const int gcol0 = 3 * D + H;  // first zero-pad column of G
  for (int t0 = ch.start + 16 * w; t0 < ch.end; t0 += 64) {
    const int ta = t0 + col;
    const bool okA = ta < ch.end;
    const float gA = okA ? ga[(size_t)ta * H + h] : 0.f;
    Frag8<T> vf[DH / 32], kf[DH / 32];
#pragma unroll
    for (int s = 0; s < DH / 32; ++s) {
      const size_t o = (size_t)(okA ? ta : ch.start) * D + h * DH + 32 * s + 8 * grp;
      vf[s] = okA ? frag_load(va + o) : frag_zero<T>();
      const Frag8<T> pk = okA ? frag_load(ka + o) : frag_zero<T>();
      float kt[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) kt[e] = gA * frag_get(pk, e);
      kf[s] = frag_from<T>(kt);
    }
    f32x4 dkt[FB], dvv[FB];
#pragma unroll
    for (int nt = 0; nt < FB; ++nt) {
      dkt[nt] = zero4();
      dvv[nt] = zero4();
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int s = 0; s < DH / 32; ++s) {
          mma8(dkt[nt], vf[s], frag_load(Srm + p * DH * LD + (16 * nt + col) * LD + 32 * s + 8 * grp));
          mma8(dvv[nt], kf[s], frag_load(Str + p * DH * LD + (16 * nt + col) * LD + 32 * s + 8 * grp));
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 4 * grp + r;
      const bool ok = t < ch.end;
      const size_t base = (size_t)(ok ? t : ch.start) * D + h * DH + col;
      const float g = ok ? ga[(size_t)t * H + h] : 0.f;
      float kv[FB], dk[FB], dg = 0.f;
#pragma unroll
      for (int nt = 0; nt < FB; ++nt) {
        kv[nt] = ok ? to_f<T>(ka[base + 16 * nt]) : 0.f;
        dk[nt] = dkt[nt][r] + dzs[16 * nt + col];
        dg += kv[nt] * dk[nt];
      }
      dg = row16_sum(dg);
      if (ok) {
        T* grow = G + (size_t)t * Kp;
#pragma unroll
        for (int nt = 0; nt < FB; ++nt) {
          grow[D + h * DH + 16 * nt + col] = from_f<T>(g * dk[nt] * fminf(1.f, kv[nt]));
          grow[2 * D + h * DH + 16 * nt + col] = from_f<T>(dvv[nt][r]);
        }
        const float ds = dg * g * (1.f - g);
        if (col == 0) {
          grow[3 * D + h] = from_f<T>(ds);
          dbg += ds;
        }
        if (h == 0)
          for (int c = gcol0 + col; c < Kp; c += 16) grow[c] = from_f<T>(0.f);
      }
    }
  }
  dbg += __shfl_xor(dbg, 16, 64);
  dbg += __shfl_xor(dbg, 32, 64);
  if (lane == 0) wsum[w] = dbg;
  __syncthreads();
  if (tid == 0) dbg_part[(size_t)slot * H + h] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
}

void launch_bwd_token(int dt, int dh, const void* ka, const void* va, const float* ga, const float* dsz,
                      const int* nchunks, const Chunk* tab, int max_slots, int H, int Kp, void* G, float* dbg_part,
                      hipStream_t s) {
  const dim3 grid(xcd_grid(max_slots * H));
#define GBLA_BT(TT, DD) hipLaunchKernelGGL((k_bwd_token<TT, DD>), grid, dim3(256), 0, s, (const TT*)ka, \
                                           (const TT*)va, ga, dsz, nchunks, tab, max_slots, H, Kp, (TT*)G, dbg_part)
  if (dt == BF16) { if (dh == 64) GBLA_BT(bf16, 64); else GBLA_BT(bf16, 32); }
  else            { if (dh == 64) GBLA_BT(float, 64); else GBLA_BT(float, 32); }
#undef GBLA_BT
}

// ============================================================== weight packing for dX~
// wt[c][n] = [W_Q[c,:] | W_K[c,:] | W_V[c,:] | w_g[:,c] | 0]
template <typename T>
__global__ void k_pack_wt(const T* __restrict__ w_q, const T* __restrict__ w_k, const T* __restrict__ w_v,
                          const T* __restrict__ w_g, int d, int H, int dh, int Kp, T* __restrict__ wt) {
  const int D = H * dh;
  const long total = (long)d * Kp;
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < total; e += (long)gridDim.x * blockDim.x) {
    const int c = (int)(e / Kp), n = (int)(e - (long)c * Kp);
    T v = from_f<T>(0.f);
    if (n < D) v = w_q[(long)c * D + n];
    else if (n < 2 * D) v = w_k[(long)c * D + n - D];
    else if (n < 3 * D) v = w_v[(long)c * D + n - 2 * D];
    else if (n < 3 * D + H) v = w_g[(long)(n - 3 * D) * d + c];
    wt[e] = v;
  }
}

void launch_pack_wt(int dt, const void* w_q, const void* w_k, const void* w_v, const void* w_g, int d, int H,
                    int dh, int Kp, void* wt, hipStream_t s) {
  const long total = (long)d * Kp;
  const int grid = (int)std::min<long>((total + 255) / 256, 4096);
  if (dt == BF16)
    hipLaunchKernelGGL(k_pack_wt<bf16>, dim3(grid), dim3(256), 0, s, (const bf16*)w_q, (const bf16*)w_k,
                       (const bf16*)w_v, (const bf16*)w_g, d, H, dh, Kp, (bf16*)wt);
  else
    hipLaunchKernelGGL(k_pack_wt<float>, dim3(grid), dim3(256), 0, s, (const float*)w_q, (const float*)w_k,
                       (const float*)w_v, (const float*)w_g, d, H, dh, Kp, (float*)wt);
}

// ============================================================== dX~ = G Wt^T
// C[M][N] = A[M][K] B[N][K]^T, both operands k-contiguous; 128x128 block tile,
// 2x2 waves of 64x64, fp32 output. Requires K % 8 == 0.
template <typename T>
__global__ __launch_bounds__(256) void k_gemm_nt(const T* __restrict__ A, const T* __restrict__ B, int M, int N,
                                                 int K, float* __restrict__ C) {
  constexpr int BM = 128, BN = 128;
  constexpr int BK = 128 / (int)sizeof(T), LD = BK + 16 / (int)sizeof(T), G8 = BK / 8;
  __shared__ __align__(16) T As[BM * LD];
  __shared__ __align__(16) T Bs[BN * LD];
  const int mtiles = (M + BM - 1) / BM, ntiles = (N + BN - 1) / BN;
  const int lid = xcd_logical_block(blockIdx.x, mtiles * ntiles);
  if (lid >= mtiles * ntiles) return;
  const int mt = lid / ntiles, nt = lid - mt * ntiles;
  const int m0 = mt * BM, n0 = nt * BN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int wm = w >> 1, wn = w & 1;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero4();

  for (int k0 = 0; k0 < K; k0 += BK) {
    for (int it = tid; it < BM * G8; it += 256) {
      const int r = it / G8, g8 = it - r * G8;
      const int c = k0 + g8 * 8;
      const bool okA = (m0 + r) < M && c < K;
      frag_store(As + r * LD + g8 * 8, okA ? frag_load(A + (size_t)(m0 + r) * K + c) : frag_zero<T>());
      const bool okB = (n0 + r) < N && c < K;
      frag_store(Bs + r * LD + g8 * 8, okB ? frag_load(B + (size_t)(n0 + r) * K + c) : frag_zero<T>());
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      Frag8<T> a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = frag_load(As + (64 * wm + 16 * i + col) * LD + ks + 8 * grp);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = frag_load(Bs + (64 * wn + 16 * j + col) * LD + ks + 8 * grp);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma8(acc[i][j], a[i], b[j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 64 * wm + 16 * i + 4 * grp + r;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + 64 * wn + 16 * j + col;
        if (n < N) C[(size_t)m * N + n] = acc[i][j][r];
      }
    }
}

void launch_gemm_dx(int dt, const void* G, const void* wt, int T, int d, int Kp, float* dxt, hipStream_t s) {
  const int n = ((T + 127) / 128) * ((d + 127) / 128);
  if (dt == BF16)
    hipLaunchKernelGGL(k_gemm_nt<bf16>, dim3(xcd_grid(n)), dim3(256), 0, s, (const bf16*)G, (const bf16*)wt, T, d,
                       Kp, dxt);
  else
    hipLaunchKernelGGL(k_gemm_nt<float>, dim3(xcd_grid(n)), dim3(256), 0, s, (const float*)G, (const float*)wt, T,
                       d, Kp, dxt);
}

// ============================================================== dW = X~^T G (split over tokens)
// part[ks][m][n] = sum over tokens t of split ks of A[t][m] B[t][n]. Both
// operands are token-major, so the LDS tiles are written transposed (pairs of
// tokens per 32-bit store) and read k-contiguous.
template <typename T> __device__ __forceinline__ void store_pair(T* p, float a, float b);
template <> __device__ __forceinline__ void store_pair<bf16>(bf16* p, float a, float b) {
  *reinterpret_cast<uint32_t*>(p) = (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}
template <> __device__ __forceinline__ void store_pair<float>(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
}

template <typename T>
__global__ __launch_bounds__(256) void k_gemm_tn(const T* __restrict__ A, const T* __restrict__ B, int Tn, int M,
                                                 int N, int tok_per_split, int nsplit, float* __restrict__ part) {
  constexpr int BM = 128, BN = 128, BKT = 32;
  constexpr int LD = BKT + 16 / (int)sizeof(T);
  __shared__ __align__(16) T As[BM * LD];
  __shared__ __align__(16) T Bs[BN * LD];
  const int mtiles = (M + BM - 1) / BM, ntiles = (N + BN - 1) / BN;
  const int total = mtiles * ntiles * nsplit;
  const int lid = xcd_logical_block(blockIdx.x, total);
  if (lid >= total) return;
  const int ks = lid / (mtiles * ntiles);
  const int rem = lid - ks * mtiles * ntiles;
  const int mt = rem / ntiles, nt = rem - mt * ntiles;
  const int m0 = mt * BM, n0 = nt * BN;
  const int tbeg = ks * tok_per_split, tend = min(Tn, tbeg + tok_per_split);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int wm = w >> 1, wn = w & 1;
  const int pr = tid >> 4, c8 = tid & 15;  // loader: token pair pr, 8-column group c8

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero4();

  for (int t0 = tbeg; t0 < tend; t0 += BKT) {
    const int ta = t0 + 2 * pr, tb = ta + 1;
    {
      const int m = m0 + 8 * c8;
      const bool okc = m < M;
      const Frag8<T> f0 = okc && ta < tend ? frag_load(A + (size_t)ta * M + m) : frag_zero<T>();
      const Frag8<T> f1 = okc && tb < tend ? frag_load(A + (size_t)tb * M + m) : frag_zero<T>();
#pragma unroll
      for (int j = 0; j < 8; ++j) store_pair<T>(As + (8 * c8 + j) * LD + 2 * pr, frag_get(f0, j), frag_get(f1, j));
    }
    {
      const int n = n0 + 8 * c8;
      const bool okc = n < N;
      const Frag8<T> f0 = okc && ta < tend ? frag_load(B + (size_t)ta * N + n) : frag_zero<T>();
      const Frag8<T> f1 = okc && tb < tend ? frag_load(B + (size_t)tb * N + n) : frag_zero<T>();
#pragma unroll
      for (int j = 0; j < 8; ++j) store_pair<T>(Bs + (8 * c8 + j) * LD + 2 * pr, frag_get(f0, j), frag_get(f1, j));
    }
    __syncthreads();
    Frag8<T> a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = frag_load(As + (64 * wm + 16 * i + col) * LD + 8 * grp);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = frag_load(Bs + (64 * wn + 16 * j + col) * LD + 8 * grp);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mma8(acc[i][j], a[i], b[j]);
    __syncthreads();
  }
  float* out = part + (size_t)ks * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 64 * wm + 16 * i + 4 * grp + r;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + 64 * wn + 16 * j + col;
        if (n < N) out[(size_t)m * N + n] = acc[i][j][r];
      }
    }
}

void launch_gemm_dw(int dt, const void* xt, const void* G, int T, int d, int Kp, int nsplit, float* part,
                    hipStream_t s) {
  const int tps = ((T + nsplit - 1) / nsplit + 31) / 32 * 32;
  const int n = ((d + 127) / 128) * ((Kp + 127) / 128) * nsplit;
  if (dt == BF16)
    hipLaunchKernelGGL(k_gemm_tn<bf16>, dim3(xcd_grid(n)), dim3(256), 0, s, (const bf16*)xt, (const bf16*)G, T, d,
                       Kp, tps, nsplit, part);
  else
    hipLaunchKernelGGL(k_gemm_tn<float>, dim3(xcd_grid(n)), dim3(256), 0, s, (const float*)xt, (const float*)G, T,
                       d, Kp, tps, nsplit, part);
}

__global__ void k_dw_reduce(const float* __restrict__ part, int nsplit, int d, int H, int dh, int Kp,
                            float* __restrict__ dw_q, float* __restrict__ dw_k, float* __restrict__ dw_v,
                            float* __restrict__ dw_g) {
  const int D = H * dh;
  const long total = (long)d * Kp;
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < total; e += (long)gridDim.x * blockDim.x) {
    const int c = (int)(e / Kp), n = (int)(e - (long)c * Kp);
    if (n >= 3 * D + H) continue;
    float s = 0.f;
    for (int k = 0; k < nsplit; ++k) s += part[(size_t)k * total + e];
    if (n < D) dw_q[(long)c * D + n] = s;
    else if (n < 2 * D) dw_k[(long)c * D + n - D] = s;
    else if (n < 3 * D) dw_v[(long)c * D + n - 2 * D] = s;
    else dw_g[(long)(n - 3 * D) * d + c] = s;
  }
}

void launch_dw_reduce(const float* part, int nsplit, int d, int H, int dh, int Kp, float* dw_q, float* dw_k,
                      float* dw_v, float* dw_g, hipStream_t s) {
  const long total = (long)d * Kp;
  const int grid = (int)std::min<long>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(k_dw_reduce, dim3(grid), dim3(256), 0, s, part, nsplit, d, H, dh, Kp, dw_q, dw_k, dw_v, dw_g);
}

__global__ void k_dbg_reduce(const float* __restrict__ part, const int* __restrict__ nchunks, int H,
                             float* __restrict__ db_g) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  const int nc = *nchunks;
  float s = 0.f;
  for (int c = 0; c < nc; ++c) s += part[(size_t)c * H + h];
  db_g[h] = s;
}

void launch_dbg_reduce(const float* dbg_part, const int* nchunks, int H, float* db_g, hipStream_t s) {
  hipLaunchKernelGGL(k_dbg_reduce, dim3((H + 255) / 256), dim3(256), 0, s, dbg_part, nchunks, H, db_g);
}

// ============================================================== conv backward
// Thread = 8 channels x 8 consecutive tokens; block = 64 channels x 256 tokens.
//   dx_u[c]       = sum_k w[c][k] dx~_{u+3-k}[c]      (u+3-k inside u's sequence)
//   dconv_w[c][k] = sum_t dx~_t[c] x_{t-3+k}[c]       (t-3+k inside t's sequence)
constexpr int kConvRows = 256;
int conv_bwd_row_blocks(int T) { return (T + kConvRows - 1) / kConvRows; }

template <typename T>
__global__ __launch_bounds__(256) void k_conv_bwd(const float* __restrict__ dxt, const T* __restrict__ x,
                                                  const int32_t* __restrict__ cu, int nseq, int T_, int d,
                                                  const T* __restrict__ conv_w, T* __restrict__ dx,
                                                  float* __restrict__ part) {
  __shared__ float red[32][8 * 8 * 4 + 1];
  const int rb = blockIdx.x, cb = blockIdx.y;
  const int tid = threadIdx.x, c8 = tid & 7, run = tid >> 3;
  const int c = cb * 64 + c8 * 8;
  float dw[8][4];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k) dw[j][k] = 0.f;
  if (c < d) {
    float wv[8][4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const Frag8<T> f = frag_load(conv_w + (size_t)c * 4 + 8 * m);
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[(8 * m + e) >> 2][(8 * m + e) & 3] = frag_get(f, e);
    }
    const int u0 = rb * kConvRows + run * 8;
    for (int u = u0; u < min(u0 + 8, T_); ++u) {
      const int end = seq_end_of(cu, nseq, u, T_);
      const int pos = pos_in_seq(cu, nseq, u);
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = 0.f;
      float g[8];
      const float4 g0 = *reinterpret_cast<const float4*>(dxt + (size_t)u * d + c);
      const float4 g1 = *reinterpret_cast<const float4*>(dxt + (size_t)u * d + c + 4);
      g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w; g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int sh = 3 - k;
        // dx: output token u + sh reads x_u through tap k
        if (u + sh < end) {
          const float4 a = *reinterpret_cast<const float4*>(dxt + (size_t)(u + sh) * d + c);
          const float4 b = *reinterpret_cast<const float4*>(dxt + (size_t)(u + sh) * d + c + 4);
          o[0] += wv[0][k] * a.x; o[1] += wv[1][k] * a.y; o[2] += wv[2][k] * a.z; o[3] += wv[3][k] * a.w;
          o[4] += wv[4][k] * b.x; o[5] += wv[5][k] * b.y; o[6] += wv[6][k] * b.z; o[7] += wv[7][k] * b.w;
        }
        // dconv_w: output token u read x_{u-sh} through tap k
        if (sh <= pos) {
          const Frag8<T> xv = frag_load(x + (size_t)(u - sh) * d + c);
#pragma unroll
          for (int j = 0; j < 8; ++j) dw[j][k] += g[j] * frag_get(xv, j);
        }
      }
      frag_store(dx + (size_t)u * d + c, frag_from<T>(o));
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k) red[run][c8 * 32 + j * 4 + k] = dw[j][k];
  __syncthreads();
  // 64 channels x 4 taps = 256 outputs, one per thread, summed over the 32 runs in order
  const int oc = tid >> 2, ok = tid & 3;
  const int cc = cb * 64 + oc;
  float s = 0.f;
  for (int r = 0; r < 32; ++r) s += red[r][(oc >> 3) * 32 + (oc & 7) * 4 + ok];
  if (cc < d) part[((size_t)rb * d + cc) * 4 + ok] = s;
}

void launch_conv_bwd(int dt, const float* dxt, const void* x, const int32_t* cu, int N, int T, int d,
                     const void* conv_w, void* dx, float* dconv_part, hipStream_t s) {
  const dim3 grid(conv_bwd_row_blocks(T), (d + 63) / 64);
  if (dt == BF16)
    hipLaunchKernelGGL(k_conv_bwd<bf16>, grid, dim3(256), 0, s, dxt, (const bf16*)x, cu, N, T, d,
                       (const bf16*)conv_w, (bf16*)dx, dconv_part);
  else
    hipLaunchKernelGGL(k_conv_bwd<float>, grid, dim3(256), 0, s, dxt, (const float*)x, cu, N, T, d,
                       (const float*)conv_w, (float*)dx, dconv_part);
}

__global__ void k_dconv_reduce(const float* __restrict__ part, int nparts, int d, float* __restrict__ out) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= d * 4) return;
  float s = 0.f;
  for (int p = 0; p < nparts; ++p) s += part[(size_t)p * d * 4 + e];
  out[e] = s;
}

void launch_dconv_reduce(const float* dconv_part, int nparts, int d, float* dconv_w, hipStream_t s) {
  hipLaunchKernelGGL(k_dconv_reduce, dim3((d * 4 + 255) / 256), dim3(256), 0, s, dconv_part, nparts, d, dconv_w);
}

}  // namespace gbla
