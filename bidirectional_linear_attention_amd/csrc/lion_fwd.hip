// LION-s selective-decay bidirectional linear attention, chunkwise, for gfx950.
//
// "Linear Attention for Efficient Bidirectional Sequence Modeling" (method
// details): M = M^F + M^B - I with M^F_ij = prod_{k=j+1..i} lambda_k and
// M^B_ij = prod_{k=i+1..j} lambda_k, lambda_i = sigmoid(w x_i + b) (Lion-s),
// feature map phi(x) = (SiLU(x) + 0.5) / ||SiLU(x) + 0.5||, and
// Y = Scale(phi(Q) phi(K)^T (.) M) V with Scale = row normalisation.
// With A_i = sum_{k<=i} log lambda_k every mask entry is exp(-|A_i - A_j|).
//
// Chunkwise evaluation with chunks of C tokens inside each sequence (chunk c
// covers [s_c, e_c), A~ is the prefix of log lambda inside the chunk and
// L_c = A~ at the chunk's last token). For a token i of chunk c:
//   num_i = sum_{j in c} exp(-|A~_i - A~_j|) (q~_i . k~_j) [v_j | 1]         (intra)
//         + exp(A~_i)       q~_i^T SF_c                                       (earlier chunks)
//         + exp(L_c - A~_i) q~_i^T SB_c                                       (later chunks)
//   SF_{c+1} = exp(L_c) SF_c + U_c,  U_c = sum_{j in c} exp(L_c - A~_j) k~_j [v_j | 1]^T
//   SB_{c-1} = exp(L_c) SB_c + W_c,  W_c = sum_{j in c} exp(A~_j)       k~_j [v_j | 1]^T
//   y_i = num_i[:dh] / num_i[dh]
// Every exponent is <= 0, so no factor overflows whatever the sequence length.
//
// Kernels:
//   k_lion_chunk_state  per (chunk, head): U_c and W_c (MFMA over the chunk's
//                       tokens), L_c. The backward runs the same kernel with
//                       (q~, g^) in place of (k~, [v | 1]).
//   k_lion_scan         per (sequence, head, state element): SF_c and SB_c, in place
//   k_lion_readout      per (chunk, head): y and the row sums r = num[dh]
#include "internal.h"
#include "lion_internal.h"

namespace gbla {

// ---------------------------------------------------------------- chunk states
// MODE 0 (forward):  rows R = phi(k) [dh], columns V = [v | 1 | 0..]       (NC = dh + 16)
// MODE 1 (backward): rows R = phi(q) [dh], columns V = g^ = [dy / r | -(dy . y) / r | 0..]
// out[slot][h][0][E] = U = sum_j exp(L - A~_j) R_j V_j^T,  out[..][1][E] = W = sum_j exp(A~_j) R_j V_j^T,
// laid out as [dh x dh] followed by the extra column (index dh) as a dh-vector.
template <typename T, int DH, int MODE>
__global__ __launch_bounds__(256) void k_lion_chunk_state(const T* __restrict__ rsrc, const T* __restrict__ vsrc,
                                                          const T* __restrict__ ysrc, const float* __restrict__ rsum,
                                                          const float* __restrict__ logl,
                                                          const int* __restrict__ nchunks,
                                                          const Chunk* __restrict__ tab, int max_slots, int H,
                                                          float* __restrict__ out, float* __restrict__ lam_out) {
  constexpr int C = kLionChunk;
  constexpr int FB = DH / 16, NB = FB + 1;
  constexpr int TILES = FB * NB, TPW = (TILES + 3) / 4;
  constexpr int PAD = 16 / (int)sizeof(T);
  constexpr int LDR = DH + PAD, LDC = 16 * NB + PAD;
  constexpr int E = DH * DH + DH;
  constexpr int V8 = DH / 8, NV = (C * V8 + 255) / 256;
  __shared__ __align__(16) T Rs[C * LDR];
  __shared__ __align__(16) T Vs[C * LDC];
  __shared__ float As[C], wU[C], wW[C];
  __shared__ float Ls;
  const int lid = xcd_logical_block(blockIdx.x, max_slots * H);
  if (lid >= max_slots * H) return;
  const int slot = lid / H, h = lid - slot * H;
  if (slot >= *nchunks) return;
  const Chunk ch = tab[slot];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, grp = lane >> 4;
  const int D = H * DH;

  chunk_decay_prefix<C>(logl, ch, H, h, As, &Ls, tid);
  for (int e = tid; e < C * 16; e += 256) {  // extra column block; in MODE 1 column dh is written below
    const int r = e >> 4, c = e & 15;
    if (MODE == 0 || c > 0) Vs[r * LDC + DH + c] = from_f<T>(MODE == 0 && c == 0 && ch.start + r < ch.end ? 1.f : 0.f);
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int it = tid + 256 * v;
    if (it >= C * V8) continue;
    const int r = it / V8, c = (it % V8) * 8, t = ch.start + r;
    const bool ok = t < ch.end;
    const size_t o = (size_t)(ok ? t : ch.start) * D + h * DH + c;
    float u[8], p[8];
    const Frag8<T> fr = ok ? frag_load(rsrc + o) : frag_zero<T>();
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = frag_get(fr, j);
    phi_lion8<V8>(u, p, ok);
    frag_store(Rs + r * LDR + c, frag_from<T>(p));
    if (MODE == 0) {
      frag_store(Vs + r * LDC + c, ok ? frag_load(vsrc + o) : frag_zero<T>());
    } else {  // g^ from dy (vsrc), y (ysrc) and the row sum r
      const Frag8<T> fd = ok ? frag_load(vsrc + o) : frag_zero<T>();
      const Frag8<T> fy = ok ? frag_load(ysrc + o) : frag_zero<T>();
      const float inv = ok ? 1.f / rsum[(size_t)t * H + h] : 0.f;
      float g[8], dd = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        g[j] = frag_get(fd, j) * inv;
        dd += frag_get(fd, j) * frag_get(fy, j);
      }
#pragma unroll
      for (int m = 1; m < V8; m <<= 1) dd += __shfl_xor(dd, m, 64);
      frag_store(Vs + r * LDC + c, frag_from<T>(g));
      if (c == 0) Vs[r * LDC + DH] = from_f<T>(-dd * inv);
    }
  }
  __syncthreads();
  if (tid < C) {
    const bool ok = ch.start + tid < ch.end;
    wU[tid] = ok ? __expf(Ls - As[tid]) : 0.f;
    wW[tid] = ok ? __expf(As[tid]) : 0.f;
  }
  __syncthreads();

  f32x4 accU[TPW], accW[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) accU[u] = accW[u] = zero4();
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tile = w + 4 * u;
    if (tile >= TILES) continue;
    const int ib = tile / NB, nb = tile - ib * NB;
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 32) {
      const Frag8<T> a = frag_kmajor<T>(Rs, LDR, k0 + 8 * grp, 16 * ib, lane);
      const Frag8<T> b = frag_kmajor<T>(Vs, LDC, k0 + 8 * grp, 16 * nb, lane);
      float au[8], aw[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {  // token k0 + 8 grp + m carries the two decay weights
        const float x = frag_get(a, m);
        au[m] = x * wU[k0 + 8 * grp + m];
        aw[m] = x * wW[k0 + 8 * grp + m];
      }
      mma8(accU[u], frag_from<T>(au), b);
      mma8(accW[u], frag_from<T>(aw), b);
    }
  }
  float* o = out + ((size_t)slot * H + h) * 2 * E;
  const int col = lane & 15;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tile = w + 4 * u;
    if (tile >= TILES) continue;
    const int ib = tile / NB, nb = tile - ib * NB;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ib + 4 * grp + r;
      if (nb < FB) {
        o[i * DH + 16 * nb + col] = accU[u][r];
        o[E + i * DH + 16 * nb + col] = accW[u][r];
      } else if (col == 0) {
        o[DH * DH + i] = accU[u][r];
        o[E + DH * DH + i] = accW[u][r];
      }
    }
  }
  if (MODE == 0 && lam_out && tid == 0) lam_out[(size_t)slot * H + h] = Ls;
}

void launch_lion_chunk_state(int dt, int dh, int mode, const void* rsrc, const void* vsrc, const void* ysrc,
                             const float* rsum, const float* logl, const int* nchunks, const Chunk* tab,
                             int max_slots, int H, float* out, float* lam_out, hipStream_t s) {
  const dim3 grid(xcd_grid(max_slots * H));
#define LION_CS(TT, DD, MM) hipLaunchKernelGGL((k_lion_chunk_state<TT, DD, MM>), grid, dim3(256), 0, s,          \
                                               (const TT*)rsrc, (const TT*)vsrc, (const TT*)ysrc, rsum, logl, \
                                               nchunks, tab, max_slots, H, out, lam_out)
  if (dt == BF16) {
    if (dh == 64) { if (mode == 0) LION_CS(bf16, 64, 0); else LION_CS(bf16, 64, 1); }
    else          { if (mode == 0) LION_CS(bf16, 32, 0); else LION_CS(bf16, 32, 1); }
  } else {
    if (dh == 64) { if (mode == 0) LION_CS(float, 64, 0); else LION_CS(float, 64, 1); }
    else          { if (mode == 0) LION_CS(float, 32, 0); else LION_CS(float, 32, 1); }
  }
#undef LION_CS
}

// ---------------------------------------------------------------- scan over chunks
// For every (sequence, head, element e): replace U_c by SF_c (the state that
// enters chunk c from the left) and W_c by SB_c (from the right), in chunk order.
__global__ __launch_bounds__(256) void k_lion_scan(float* __restrict__ st, const float* __restrict__ lam,
                                                   const int* __restrict__ nchunks, const int* __restrict__ chunk_off,
                                                   int N, int H, int E) {
  const int eblocks = (E + 255) / 256;
  const int bh = blockIdx.x / eblocks, b = bh / H, h = bh - b * H;
  const int e = (blockIdx.x - bh * eblocks) * 256 + threadIdx.x;
  if (b >= N || e >= E) return;
  const int nc = *nchunks;
  const int c0 = min(chunk_off[b], nc), c1 = min(chunk_off[b + 1], nc);
  float sf = 0.f;
  for (int c = c0; c < c1; ++c) {
    float* p = st + ((size_t)c * H + h) * 2 * E + e;
    const float u = *p;
    *p = sf;
    sf = __expf(lam[(size_t)c * H + h]) * sf + u;
  }
  float sb = 0.f;
  for (int c = c1 - 1; c >= c0; --c) {
    float* p = st + ((size_t)c * H + h) * 2 * E + E + e;
    const float w = *p;
    *p = sb;
    sb = __expf(lam[(size_t)c * H + h]) * sb + w;
  }
}

void launch_lion_scan(float* st, const float* lam, const int* nchunks, const int* chunk_off, int N, int H, int E,
                      hipStream_t s) {
  hipLaunchKernelGGL(k_lion_scan, dim3(((E + 255) / 256) * N * H), dim3(256), 0, s, st, lam, nchunks, chunk_off, N,
                     H, E);
}

// ---------------------------------------------------------------- readout
// Block = (chunk, head); wave w owns query rows 16 w .. 16 w + 15 of the chunk.
template <typename T, int DH>
__global__ __launch_bounds__(256) void k_lion_readout(const T* __restrict__ qr, const T* __restrict__ kr,
                                                      const T* __restrict__ vr, const float* __restrict__ logl,
                                                      const float* __restrict__ st, const int* __restrict__ nchunks,
                                                      const Chunk* __restrict__ tab, int max_slots, int H,
                                                      T* __restrict__ y, float* __restrict__ rsum) {
  constexpr int C = kLionChunk;
  constexpr int FB = DH / 16, NB = FB + 1, NR = DH + 16;
  constexpr int PAD = 16 / (int)sizeof(T);
  constexpr int LDR = DH + PAD, LDC = 16 * NB + PAD, LDP = C + PAD;
  constexpr int P2 = sizeof(T) == 2 ? 2 : 1;
  constexpr int E = DH * DH + DH;
  constexpr int V8 = DH / 8, NV = (C * V8 + 255) / 256;
  __shared__ __align__(16) T Qs[C * LDR];
  __shared__ __align__(16) T Ks[C * LDR];
  __shared__ __align__(16) T Vs[C * LDC];
  __shared__ __align__(16) T Ps[4 * 16 * LDP];
  __shared__ __align__(16) T SF[P2 * NR * LDR];
  __shared__ __align__(16) T SB[P2 * NR * LDR];
  __shared__ float As[C];
  __shared__ float Ls;
  const int lid = xcd_logical_block(blockIdx.x, max_slots * H);
  if (lid >= max_slots * H) return;
  const int slot = lid / H, h = lid - slot * H;
  if (slot >= *nchunks) return;
  const Chunk ch = tab[slot];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int D = H * DH;

  chunk_decay_prefix<C>(logl, ch, H, h, As, &Ls, tid);
  const float* sp = st + ((size_t)slot * H + h) * 2 * E;
  stage_state<T, DH, NR>(SF, nullptr, LDR, sp, sp + DH * DH, tid, 256);
  stage_state<T, DH, NR>(SB, nullptr, LDR, sp + E, sp + E + DH * DH, tid, 256);
  for (int e = tid; e < C * 16; e += 256) {
    const int r = e >> 4, c = e & 15;
    Vs[r * LDC + DH + c] = from_f<T>(c == 0 && ch.start + r < ch.end ? 1.f : 0.f);
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int it = tid + 256 * v;
    if (it >= C * V8) continue;
    const int r = it / V8, c = (it % V8) * 8, t = ch.start + r;
    const bool ok = t < ch.end;
    const size_t o = (size_t)(ok ? t : ch.start) * D + h * DH + c;
    float u[8], p[8];
    Frag8<T> f = ok ? frag_load(qr + o) : frag_zero<T>();
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = frag_get(f, j);
    phi_lion8<V8>(u, p, ok);
    frag_store(Qs + r * LDR + c, frag_from<T>(p));
    f = ok ? frag_load(kr + o) : frag_zero<T>();
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = frag_get(f, j);
    phi_lion8<V8>(u, p, ok);
    frag_store(Ks + r * LDR + c, frag_from<T>(p));
    frag_store(Vs + r * LDC + c, ok ? frag_load(vr + o) : frag_zero<T>());
  }
  __syncthreads();

  const int r0 = 16 * w;
  Frag8<T> aq[DH / 32];
#pragma unroll
  for (int s = 0; s < DH / 32; ++s) aq[s] = frag_load(Qs + (r0 + col) * LDR + 32 * s + 8 * grp);
  // intra-chunk similarities, masked by the decay: P = (q~ k~^T) (.) exp(-|A~_i - A~_j|)
  T* Pw = Ps + w * 16 * LDP;
#pragma unroll
  for (int nt = 0; nt < C / 16; ++nt) {
    f32x4 g = zero4();
#pragma unroll
    for (int s = 0; s < DH / 32; ++s) mma8(g, aq[s], frag_load(Ks + (16 * nt + col) * LDR + 32 * s + 8 * grp));
    const int j = 16 * nt + col;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = r0 + 4 * grp + r;
      Pw[(4 * grp + r) * LDP + j] = from_f<T>(g[r] * __expf(-fabsf(As[i] - As[j])));
    }
  }
  __syncthreads();
  f32x4 num[NB], fw[NB], bw[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    num[nb] = fw[nb] = bw[nb] = zero4();
#pragma unroll
    for (int s = 0; s < C / 32; ++s)
      mma8(num[nb], frag_load(Pw + col * LDP + 32 * s + 8 * grp), frag_kmajor<T>(Vs, LDC, 32 * s + 8 * grp, 16 * nb, lane));
#pragma unroll
    for (int p = 0; p < P2; ++p)
#pragma unroll
      for (int s = 0; s < DH / 32; ++s) {
        mma8(fw[nb], aq[s], frag_load(SF + p * NR * LDR + (16 * nb + col) * LDR + 32 * s + 8 * grp));
        mma8(bw[nb], aq[s], frag_load(SB + p * NR * LDR + (16 * nb + col) * LDR + 32 * s + 8 * grp));
      }
  }
  const float L = Ls;
  float ef[4], eb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float a = As[r0 + 4 * grp + r];
    ef[r] = __expf(a);
    eb[r] = __expf(L - a);
  }
  __syncthreads();  // every wave is done with Qs (A operands above); reuse its rows for y
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = r0 + 4 * grp + r;
    const float den = col0_bcast(num[FB][r] + ef[r] * fw[FB][r] + eb[r] * bw[FB][r], lane);
    const bool ok = ch.start + i < ch.end;
    const float inv = ok ? 1.f / den : 0.f;
#pragma unroll
    for (int nb = 0; nb < FB; ++nb)
      Qs[i * LDR + 16 * nb + col] = from_f<T>((num[nb][r] + ef[r] * fw[nb][r] + eb[r] * bw[nb][r]) * inv);
    if (ok && col == 0) rsum[(size_t)(ch.start + i) * H + h] = den;
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int it = tid + 256 * v;
    if (it >= C * V8) continue;
    const int r = it / V8, c = (it % V8) * 8, t = ch.start + r;
    if (t < ch.end) frag_store(y + (size_t)t * D + h * DH + c, frag_load(Qs + r * LDR + c));
  }
}

void launch_lion_readout(int dt, int dh, const void* q, const void* k, const void* v, const float* logl,
                         const float* st, const int* nchunks, const Chunk* tab, int max_slots, int H, void* y,
                         float* rsum, hipStream_t s) {
  const dim3 grid(xcd_grid(max_slots * H));
#define LION_RO(TT, DD) hipLaunchKernelGGL((k_lion_readout<TT, DD>), grid, dim3(256), 0, s, (const TT*)q, \
                                           (const TT*)k, (const TT*)v, logl, st, nchunks, tab, max_slots, H, \
                                           (TT*)y, rsum)
  if (dt == BF16) { if (dh == 64) LION_RO(bf16, 64); else LION_RO(bf16, 32); }
  else            { if (dh == 64) LION_RO(float, 64); else LION_RO(float, 32); }
#undef LION_RO
}

}  // namespace gbla
