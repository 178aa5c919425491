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
// each stored transposed: E = (dh + 1) rows n of dh values a, element [n][a] = (R^T V)[a][n];
// row dh is the extra column (index dh of V).
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
  Chunk ch;
  if (!block_chunk(nchunks, tab, slot, ch)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, grp = lane >> 4;
  const int D = H * DH;

  const float la = chunk_decay_load<C>(logl, ch, H, h, tid);
  for (int e = tid; e < C * 16; e += 256) {  // extra column block; in MODE 1 column dh is written below
    const int r = e >> 4, c = e & 15;
    if (MODE == 0 || c > 0) Vs[r * LDC + DH + c] = from_f<T>(MODE == 0 && c == 0 && ch.start + r < ch.end ? 1.f : 0.f);
  }
  // every load of the staging is issued before any of it is used
  Frag8<T> fr[NV], fv[NV], fy[NV];
  float rs[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int it = tid + 256 * v;
    const int r = it / V8, c = (it % V8) * 8, t = ch.start + r;
    const bool ok = it < C * V8 && t < ch.end;
    const size_t o = (size_t)(ok ? t : ch.start) * D + h * DH + c;
    fr[v] = ok ? frag_load(rsrc + o) : frag_zero<T>();
    fv[v] = ok ? frag_load(vsrc + o) : frag_zero<T>();
    if (MODE == 1) {
      fy[v] = ok ? frag_load(ysrc + o) : frag_zero<T>();
      rs[v] = ok ? rsum[(size_t)t * H + h] : 1.f;
    }
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int it = tid + 256 * v;
    if (it >= C * V8) continue;
    const int r = it / V8, c = (it % V8) * 8, t = ch.start + r;
    const bool ok = t < ch.end;
    float u[8], p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = frag_get(fr[v], j);
    phi_lion8<V8>(u, p, ok);
    frag_store(Rs + r * LDR + c, frag_from<T>(p));
    if (MODE == 0) {
      frag_store(Vs + r * LDC + c, fv[v]);
    } else {  // g^ from dy (vsrc), y (ysrc) and the row sum r
      const Frag8<T> fd = fv[v];
      const Frag8<T> fy1 = fy[v];
      const float inv = ok ? fast_rcp(rs[v]) : 0.f;
      float g[8], dd = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        g[j] = frag_get(fd, j) * inv;
        dd += frag_get(fd, j) * frag_get(fy1, j);
      }
      dd = lane_group_sum<V8>(dd);
      frag_store(Vs + r * LDC + c, frag_from<T>(g));
      if (c == 0) Vs[r * LDC + DH] = from_f<T>(-dd * inv);
    }
  }
  chunk_decay_scan<C>(la, As, &Ls, tid);
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
  // states are stored transposed, [n][a] (n = column feature, row n = dh is the
  // extra column), so each state is one contiguous run of E floats: the tiles
  // are gathered in LDS (a lane's 4 rows a of column n are one 16-byte store)
  // and the run leaves as whole 1 KB wave stores, U then W
  constexpr int LDO = DH + 4;
  __shared__ __align__(16) float Ost[(DH + 1) * LDO];
  float* o = out + ((size_t)slot * H + h) * 2 * E;
  const int col = lane & 15;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tile = w + 4 * u;
      if (tile >= TILES) continue;
      const int ib = tile / NB, nb = tile - ib * NB;
      const int n = nb < FB ? 16 * nb + col : DH;
      if (nb < FB || col == 0) *reinterpret_cast<f32x4*>(Ost + n * LDO + 16 * ib + 4 * grp) = half ? accW[u] : accU[u];
    }
    __syncthreads();
    for (int f = tid; f < E / 4; f += 256) {
      const int n = f / (DH / 4), a = 4 * (f % (DH / 4));
      *reinterpret_cast<float4*>(o + half * E + 4 * f) = *reinterpret_cast<const float4*>(Ost + n * LDO + a);
    }
    __syncthreads();
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
// The two walks touch disjoint halves of each chunk's state, so they run
// together: each round issues the loads of kScanBatch chunks of the forward
// walk and of the backward walk before either carry advances, and the walk
// pays one memory latency per round.
// With a row image (rows != null), the dh x dh part of each result (e < dh^2)
// is written rounded to TO into rows [slot][H][2][dh^2] instead, for a consumer
// that stages the state in TO anyway; the extra row stays in place in fp32.
constexpr int kScanBatch = 16;

template <typename TO>
__global__ __launch_bounds__(256) void k_lion_scan(float* __restrict__ st, const float* __restrict__ lam,
                                                   const int* __restrict__ nchunks, const int* __restrict__ chunk_off,
                                                   int N, int H, int E, TO* __restrict__ rows, int DD) {
  constexpr int B = kScanBatch;
  const int eblocks = (E + 255) / 256;
  const int bh = blockIdx.x / eblocks, b = bh / H, h = bh - b * H;
  const int e = (blockIdx.x - bh * eblocks) * 256 + threadIdx.x;
  if (b >= N || e >= E) return;
  const int nc = *nchunks;
  const int c0 = min(chunk_off[b], nc), c1 = min(chunk_off[b + 1], nc);
  const size_t cs = (size_t)H * 2 * E;  // stride between consecutive chunks
  float* base = st + (size_t)h * 2 * E + e;
  const bool img = rows != nullptr && e < DD;
  const size_t rcs = (size_t)H * 2 * DD;  // chunk stride of the row image
  TO* rbase = img ? rows + (size_t)h * 2 * DD + e : nullptr;
  float sf = 0.f, sb = 0.f;
  for (int k = 0; c0 + k < c1; k += B) {
    const int cf = c0 + k, cb = c1 - 1 - k;  // first chunk of the round: forward walk, backward walk
    float u[B], gu[B], w[B], gw[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int c = cf + j, d = cb - j;
      u[j] = c < c1 ? base[(size_t)c * cs] : 0.f;
      gu[j] = c < c1 ? lam[(size_t)c * H + h] : 0.f;
      w[j] = d >= c0 ? base[(size_t)d * cs + E] : 0.f;
      gw[j] = d >= c0 ? lam[(size_t)d * H + h] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int c = cf + j, d = cb - j;
      if (c < c1) {
        if (img) rbase[(size_t)c * rcs] = from_f<TO>(sf);
        else base[(size_t)c * cs] = sf;
        sf = __expf(gu[j]) * sf + u[j];
      }
      if (d >= c0) {
        if (img) rbase[(size_t)d * rcs + DD] = from_f<TO>(sb);
        else base[(size_t)d * cs + E] = sb;
        sb = __expf(gw[j]) * sb + w[j];
      }
    }
  }
}

void launch_lion_scan(float* st, const float* lam, const int* nchunks, const int* chunk_off, int N, int H, int E,
                      int dt, void* rows, int dh, hipStream_t s) {
  const dim3 grid(((E + 255) / 256) * N * H);
  if (dt == BF16 && rows)
    hipLaunchKernelGGL(k_lion_scan<bf16>, grid, dim3(256), 0, s, st, lam, nchunks, chunk_off, N, H, E, (bf16*)rows,
                       dh * dh);
  else
    hipLaunchKernelGGL(k_lion_scan<float>, grid, dim3(256), 0, s, st, lam, nchunks, chunk_off, N, H, E,
                       (float*)rows, dh * dh);
}

// ---------------------------------------------------------------- readout
// Block = (chunk, head), 4 waves.
//  Phase 1: wave w forms rows 16 w .. 16 w + 15 of P = (q~ k~^T) (.) exp(-|A~_i - A~_j|)
//           in LDS, with their row sums, and the dots q~_i . z of both carried
//           states; together they give the denominators r_i.
//  Phase 2: wave w produces output columns 16 ct .. 16 ct + 15 for its row tiles:
//           P V plus e^{A~_i} q~_i^T SF + e^{L - A~_i} q~_i^T SB, over r_i. Its slice of
//           SF and SB ([n][a] in HBM, n = 16 ct + lane % 16) is loaded straight into
//           MFMA B fragments (split into high and low bf16 parts for bf16).

// 8 floats -> high and low parts (bf16: ~16 mantissa bits together; float: exact, low = 0)
__device__ __forceinline__ void split8(const float (&v)[8], Frag8<bf16>& hi, Frag8<bf16>& lo) {
  float l[8];
  hi = frag_from<bf16>(v);
#pragma unroll
  for (int m = 0; m < 8; ++m) l[m] = v[m] - frag_get(hi, m);
  lo = frag_from<bf16>(l);
}
__device__ __forceinline__ void split8(const float (&v)[8], Frag8<float>& hi, Frag8<float>& lo) {
  hi = frag_from<float>(v);
  lo = frag_zero<float>();
}

template <typename T, int DH>
__global__ __launch_bounds__(256) void k_lion_readout(const T* __restrict__ qr, const T* __restrict__ kr,
                                                      const T* __restrict__ vr, const float* __restrict__ logl,
                                                      const float* __restrict__ st, const int* __restrict__ nchunks,
                                                      const Chunk* __restrict__ tab, int max_slots, int H,
                                                      T* __restrict__ y, float* __restrict__ rsum) {
  constexpr int C = kLionChunk;
  constexpr int FB = DH / 16;    // 16-wide column tiles of the output
  constexpr int WPC = 4 / FB;    // waves per column tile
  constexpr int RTW = 4 / WPC;   // row tiles per wave in phase 2
  constexpr int KS = DH / 32;    // 32-wide k steps over the features
  constexpr int PAD = 16 / (int)sizeof(T);
  constexpr int LDR = DH + PAD, LDP = C + PAD;
  constexpr int P2 = sizeof(T) == 2 ? 2 : 1;
  constexpr int E = DH * DH + DH;
  constexpr int V8 = DH / 8, NV = (C * V8 + 255) / 256;
  static_assert(FB * WPC == 4 && RTW * WPC == 4, "4 waves cover the 4 x FB output tiles");
  __shared__ __align__(16) T Qs[C * LDR];
  __shared__ __align__(16) T Ks[C * LDR];  // phi(k); y on output
  __shared__ __align__(16) T Vs[C * LDR];
  __shared__ __align__(16) T Ps[C * LDP];
  __shared__ __align__(16) float zS[2][DH];
  __shared__ float As[C], rowsum[C], zpart[C];
  __shared__ float Ls;
  const int lid = xcd_logical_block(blockIdx.x, max_slots * H);
  if (lid >= max_slots * H) return;
  const int slot = lid / H, h = lid - slot * H;
  Chunk ch;
  if (!block_chunk(nchunks, tab, slot, ch)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int D = H * DH;
  const int ct = w / WPC, rt0 = (w % WPC) * RTW;
  const float la = chunk_decay_load<C>(logl, ch, H, h, tid);

  // the token tiles' loads are all issued first, then the states' (nothing
  // waits on a load before every load of the staging is in flight)
  Frag8<T> fq[NV], fk[NV], fv[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int it = tid + 256 * v;
    const int r = it / V8, c = (it % V8) * 8, t = ch.start + r;
    const bool ok = it < C * V8 && t < ch.end;
    const size_t o = (size_t)(ok ? t : ch.start) * D + h * DH + c;
    fq[v] = ok ? frag_load(qr + o) : frag_zero<T>();
    fk[v] = ok ? frag_load(kr + o) : frag_zero<T>();
    fv[v] = ok ? frag_load(vr + o) : frag_zero<T>();
  }
  // this wave's slice of the carried states: column n = 16 ct + col, rows a = 32 s + 8 grp .. + 7
  const float* sp = st + ((size_t)slot * H + h) * 2 * E;
  float4 sv[2][KS][2];
#pragma unroll
  for (int dir = 0; dir < 2; ++dir)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float4* p = reinterpret_cast<const float4*>(sp + dir * E + (16 * ct + col) * DH + 32 * s + 8 * grp);
      sv[dir][s][0] = p[0];
      sv[dir][s][1] = p[1];
    }
  if (tid < DH / 2) {  // the extra rows (z) of both states
    const int dir = tid / (DH / 4), e4 = tid % (DH / 4);
    reinterpret_cast<float4*>(zS[dir])[e4] = reinterpret_cast<const float4*>(sp + dir * E + DH * DH)[e4];
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int it = tid + 256 * v;
    if (it >= C * V8) continue;
    const int r = it / V8, c = (it % V8) * 8, t = ch.start + r;
    const bool ok = t < ch.end;
    float u[8], p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = frag_get(fq[v], j);
    phi_lion8<V8>(u, p, ok);
    frag_store(Qs + r * LDR + c, frag_from<T>(p));
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = frag_get(fk[v], j);
    phi_lion8<V8>(u, p, ok);
    frag_store(Ks + r * LDR + c, frag_from<T>(p));
    frag_store(Vs + r * LDR + c, fv[v]);
  }
  chunk_decay_scan<C>(la, As, &Ls, tid);
  __syncthreads();
  const float L = Ls;

  // ---------------- phase 1: rows r0 .. r0 + 15 of P, row sums, q~ . z
  {
    const int r0 = 16 * w;
    Frag8<T> aq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) aq[s] = frag_load(Qs + (r0 + col) * LDR + 32 * s + 8 * grp);
    float zf = 0.f, zb = 0.f;  // partial dots of row r0 + col with the two z rows
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float q = frag_get(aq[s], m);
        zf += q * zS[0][32 * s + 8 * grp + m];
        zb += q * zS[1][32 * s + 8 * grp + m];
      }
    zf = add_xor32(add_xor16(zf));
    zb = add_xor32(add_xor16(zb));
    if (grp == 0) {
      const float a = As[r0 + col];
      zpart[r0 + col] = __expf(a) * zf + __expf(L - a) * zb;
    }
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < C / 16; ++nt) {
      f32x4 g = zero4();
#pragma unroll
      for (int s = 0; s < KS; ++s) mma8(g, aq[s], frag_load(Ks + (16 * nt + col) * LDR + 32 * s + 8 * grp));
      const int j = 16 * nt + col;
      const float aj = As[j];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = r0 + 4 * grp + r;
        const T pv = from_f<T>(g[r] * __expf(-fabsf(As[i] - aj)));
        Ps[i * LDP + j] = pv;
        rs[r] += to_f<T>(pv);  // the denominator sums the same rounded weights the numerator uses
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      rs[r] = row16_sum(rs[r]);
      if (col == 0) rowsum[r0 + 4 * grp + r] = rs[r];
    }
  }
  __syncthreads();
  if (tid < C && ch.start + tid < ch.end) rsum[(size_t)(ch.start + tid) * H + h] = rowsum[tid] + zpart[tid];

  // ---------------- phase 2: columns 16 ct .. 16 ct + 15, row tiles rt0 .. rt0 + RTW - 1
  Frag8<T> bF[P2][KS], bB[P2][KS], vb[C / 32];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    float f[8], b[8];
    f[0] = sv[0][s][0].x; f[1] = sv[0][s][0].y; f[2] = sv[0][s][0].z; f[3] = sv[0][s][0].w;
    f[4] = sv[0][s][1].x; f[5] = sv[0][s][1].y; f[6] = sv[0][s][1].z; f[7] = sv[0][s][1].w;
    b[0] = sv[1][s][0].x; b[1] = sv[1][s][0].y; b[2] = sv[1][s][0].z; b[3] = sv[1][s][0].w;
    b[4] = sv[1][s][1].x; b[5] = sv[1][s][1].y; b[6] = sv[1][s][1].z; b[7] = sv[1][s][1].w;
    Frag8<T> hi, lo;
    split8(f, hi, lo);
    bF[0][s] = hi;
    if (P2 == 2) bF[P2 - 1][s] = lo;
    split8(b, hi, lo);
    bB[0][s] = hi;
    if (P2 == 2) bB[P2 - 1][s] = lo;
  }
#pragma unroll
  for (int s = 0; s < C / 32; ++s) vb[s] = frag_kmajor<T>(Vs, LDR, 32 * s + 8 * grp, 16 * ct, lane);
  float yv[RTW][4];
#pragma unroll
  for (int q = 0; q < RTW; ++q) {
    const int rt = rt0 + q;
    f32x4 in = zero4(), fw = zero4(), bw = zero4();
#pragma unroll
    for (int s = 0; s < C / 32; ++s) mma8(in, frag_load(Ps + (16 * rt + col) * LDP + 32 * s + 8 * grp), vb[s]);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const Frag8<T> a = frag_load(Qs + (16 * rt + col) * LDR + 32 * s + 8 * grp);
#pragma unroll
      for (int p = 0; p < P2; ++p) {
        mma8(fw, a, bF[p][s]);
        mma8(bw, a, bB[p][s]);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * rt + 4 * grp + r;
      const float a = As[i];
      const float den = rowsum[i] + zpart[i];
      yv[q][r] = ch.start + i < ch.end ? (in[r] + __expf(a) * fw[r] + __expf(L - a) * bw[r]) * fast_rcp(den) : 0.f;
    }
  }
  // Ks is free since phase 1 (every wave passed the barrier after its last read)
#pragma unroll
  for (int q = 0; q < RTW; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) Ks[(16 * (rt0 + q) + 4 * grp + r) * LDR + 16 * ct + col] = from_f<T>(yv[q][r]);
  __syncthreads();
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int it = tid + 256 * v;
    if (it >= C * V8) continue;
    const int r = it / V8, c = (it % V8) * 8, t = ch.start + r;
    if (t < ch.end) frag_store(y + (size_t)t * D + h * DH + c, frag_load(Ks + r * LDR + c));
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
