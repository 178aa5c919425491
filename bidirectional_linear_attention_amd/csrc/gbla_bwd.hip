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
//   (without an activation cache, k_conv_fwd + k_proj recompute x~, g, phi(q), phi(k), v)
//   k_bwd_dstate  per (chunk, head): y, dn, dden, dq -> G; partial [dS | dz]
//   k_bwd_token   per (chunk, head): dk, dv, ds -> G; partial db_g
//   k_gemm_dx     dX~ = G Wt^T (pipelined MFMA), stored in the activation dtype
//   k_gemm_dw     split-token partials of X~^T G (pipelined MFMA), then k_dw_reduce
//   k_conv_bwd    dx and per-block partial dconv_w (summed by k_sum_parts)
#include "gemm.h"
#include <algorithm>

#include "internal.h"

namespace gbla {

template <typename T> struct Parts { static constexpr int n = 2; };  // bf16: hi + lo split of fp32 matrices
template <> struct Parts<float> { static constexpr int n = 1; };

// ============================================================== dS, dz and dq
// Block = one chunk x one head; tiles of 64 tokens of q~ and dy are staged in
// LDS with 16-byte loads, wave w works on tokens 16 w .. 16 w + 15 of a tile in
// the transposed orientation (C rows = features, C columns = tokens), so each
// lane holds 4 consecutive features of one token:
//   [num | den]^T = [S | z]^T q~^T        (MFMA, A = the staged transposed state)
//   dn = dy / den, dden = -(dy . y) / den (dy read as 8-byte quads)
//   dq~^T = S dn^T (+ z dden)             (K=16 MFMAs: dn stays in registers, A =
//                                          transposing reads of the staged state)
//   dq = dq~ (.) phi'(q) -> G             (8-byte stores)
//   [dS | dz] += q~^T [dn | dden]         (MFMA over the tile's tokens; each wave
//                                          owns a fixed set of output tiles)
// GATED (gated RMSNorm output, Eq. (7)): dy is the gradient of
// y = gamma (.) n (.) SiLU(r), n = O / rho, rho = sqrt(mean(O^2) + eps); with O
// = num / den recomputed above, the gradient of O replaces dy:
//   a = gamma (.) SiLU(r),  dO = (dy (.) a - n mean(n (.) dy (.) a)) / rho
//   dr = dy (.) gamma (.) n (.) SiLU'(r) -> G's R columns,  dgamma += dy (.) n (.) SiLU(r)
// (the means are row sums over the 4 lanes of a token, as for dy . y).
template <typename T, int DH, bool GATED>
__global__ __launch_bounds__(256) void k_bwd_dstate(const T* __restrict__ qa, const T* __restrict__ dy,
                                                    const float* __restrict__ saved, const int* __restrict__ nchunks,
                                                    const Chunk* __restrict__ tab, int max_slots, int H, int Kp,
                                                    float* __restrict__ partial, T* __restrict__ G,
                                                    const T* __restrict__ ra, const float* __restrict__ gamma,
                                                    float eps, float* __restrict__ dgam_part) {
  constexpr int FB = DH / 16, NB = FB + 1, NR = DH + 16;
  constexpr int PAD = 16 / (int)sizeof(T);
  constexpr int LD = DH + PAD, LDN = DH + 16 + PAD;
  constexpr int P = Parts<T>::n;
  constexpr int E = DH * DH + DH;
  constexpr int ST = 64, V8 = DH / 8, KS = DH / 32;
  constexpr int TILES = FB * NB, TPW = (TILES + 3) / 4;
  __shared__ __align__(16) T Sst[P * NR * LD];  // [S | z]^T: row n (row dh = z, rows > dh zero), column a
  __shared__ __align__(16) T qs[ST * LD];       // q~ tile (token-major)
  __shared__ __align__(16) T ys[ST * LD];       // dy tile
  __shared__ __align__(16) T dns[ST * LDN];     // [dn | dden | 0] (token-major)
  __shared__ __align__(16) T rs[GATED ? ST * LD : 8];  // R tile (gated output)
  __shared__ __align__(16) float gms[GATED ? DH : 4];   // gamma (gated output)
  __shared__ float zs[DH];

  const int lid = xcd_logical_block(blockIdx.x, max_slots * H);
  if (lid >= max_slots * H) return;
  const int slot = lid / H, h = lid - slot * H;
  if (slot >= *nchunks) return;
  const Chunk ch = tab[slot];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int D = H * DH;
  const float* st = saved + ((size_t)ch.seq * H + h) * E;
  stage_state<T, DH, NR>(Sst, nullptr, LD, st, st + DH * DH, tid);
  for (int e = tid; e < DH; e += 256) zs[e] = st[DH * DH + e];
  for (int e = tid; e < ST * 16; e += 256) dns[(e >> 4) * LDN + DH + (e & 15)] = from_f<T>(0.f);

  f32x4 accS[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) accS[u] = zero4();
  const int r0 = 16 * w;
  float dgam[FB][4];  // gated output: the lane's dgamma partial sums
#pragma unroll
  for (int nt = 0; nt < FB; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) dgam[nt][r] = 0.f;
  if constexpr (GATED)
    for (int e = tid; e < DH; e += 256) gms[e] = gamma ? gamma[e] : 1.f;

  constexpr int NV = (ST * V8 + 255) / 256;
  Frag8<T> pq[NV], py[NV], pr[NV];
  auto fetch = [&](int tb) {  // the next tile's loads are issued before the current tile is processed
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int it = tid + 256 * v, r = it / V8, c = (it % V8) * 8, t = tb + r;
      const bool ok = it < ST * V8 && t < ch.end;
      const size_t o = (size_t)(ok ? t : ch.start) * D + h * DH + c;
      pq[v] = ok ? frag_load(qa + o) : frag_zero<T>();
      py[v] = ok ? frag_load(dy + o) : frag_zero<T>();
      if constexpr (GATED) pr[v] = ok ? frag_load(ra + o) : frag_zero<T>();
    }
  };
  fetch(ch.start);
  for (int tb = ch.start; tb < ch.end; tb += ST) {  // uniform trip count (barriers inside)
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int it = tid + 256 * v, r = it / V8, c = (it % V8) * 8;
      if (it < ST * V8) {
        frag_store(qs + r * LD + c, pq[v]);
        frag_store(ys + r * LD + c, py[v]);
        if constexpr (GATED) frag_store(rs + r * LD + c, pr[v]);
      }
    }
    __syncthreads();
    if (tb + ST < ch.end) fetch(tb + ST);

    // [num | den]^T for tokens r0 .. r0 + 15: C[4 grp + r][col] = num[token r0 + col][16 nt + 4 grp + r]
    Frag8<T> bq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) bq[s] = frag_load(qs + (r0 + col) * LD + 32 * s + 8 * grp);
    f32x4 num[NB];
#pragma unroll
    for (int nt = 0; nt < NB; ++nt) {
      num[nt] = zero4();
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int s = 0; s < KS; ++s)
          mma8(num[nt], frag_load(Sst + p * NR * LD + (16 * nt + col) * LD + 32 * s + 8 * grp), bq[s]);
    }
    const int tok = r0 + col;
    const bool ok = tb + tok < ch.end;
    const float den = __shfl(num[FB][0], col, 64);  // row dh (z) sits in group 0, element 0
    const float inv = ok ? fast_rcp(den) : 0.f;
    if constexpr (GATED) {
      // the gradient of O replaces dy in the staged tile (each lane rewrites
      // its own token's features); O = num * inv and n = O * rinv are
      // recomputed from the live accumulators rather than kept
      float ss = 0.f;
#pragma unroll
      for (int nt = 0; nt < FB; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) ss += num[nt][r] * num[nt][r];
      ss *= inv * inv;
      ss = add_xor32(add_xor16(ss));
      const float rinv = ok ? fast_rsqrt(ss * (1.f / DH) + eps) : 0.f;
      const float nsc = inv * rinv;  // n = num * nsc
      float ndot = 0.f, dnv[FB][4];
#pragma unroll
      for (int nt = 0; nt < FB; ++nt) {
        const Quad<T> q = quad_load(ys + tok * LD + 16 * nt + 4 * grp);
        const Quad<T> rq = quad_load(rs + tok * LD + 16 * nt + 4 * grp);
        const float4 g4 = *reinterpret_cast<const float4*>(gms + 16 * nt + 4 * grp);
        const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
        float dr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float dout = quad_get(q, r), rv = quad_get(rq, r), sg = sigmoidf_(rv), sl = rv * sg;
          const float n = num[nt][r] * nsc, dg = dout * gv[r];
          dnv[nt][r] = dg * sl;  // gradient of n
          ndot += n * dnv[nt][r];
          dr[r] = dg * n * sg * (1.f + rv * (1.f - sg));
          dgam[nt][r] += dout * n * sl;
        }
        if (ok) quad_store(G + (size_t)(tb + tok) * Kp + 3 * D + h * DH + 16 * nt + 4 * grp, quad_from4<T>(dr));
      }
      ndot = add_xor32(add_xor16(ndot));
      const float c = ndot * (1.f / DH);
#pragma unroll
      for (int nt = 0; nt < FB; ++nt) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = rinv * (dnv[nt][r] - num[nt][r] * nsc * c);
        quad_store(ys + tok * LD + 16 * nt + 4 * grp, quad_from4<T>(v));
      }
    }
    float dyv[FB][4], pdot = 0.f;
#pragma unroll
    for (int nt = 0; nt < FB; ++nt) {
      const Quad<T> q = quad_load(ys + tok * LD + 16 * nt + 4 * grp);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dyv[nt][r] = quad_get(q, r);
        pdot += dyv[nt][r] * (num[nt][r] * inv);
      }
    }
    pdot = add_xor32(add_xor16(pdot));
    const float dden = -pdot * inv;
    Quad<T> dnq[FB];
#pragma unroll
    for (int nt = 0; nt < FB; ++nt) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = dyv[nt][r] * inv;
      dnq[nt] = quad_from4<T>(v);
      quad_store(dns + tok * LDN + 16 * nt + 4 * grp, dnq[nt]);
    }
    if (grp == 0) dns[tok * LDN + DH] = from_f<T>(dden);

    // dq~^T tile at: C[4 grp + r][col] = sum_n S[16 at + 4 grp + r][n] dn[tok][n]
#pragma unroll
    for (int at = 0; at < FB; ++at) {
      f32x4 dq = zero4();
#pragma unroll
      for (int nt = 0; nt < FB; ++nt)
#pragma unroll
        for (int p = 0; p < P; ++p)
          mma_q(dq, quad_kmajor<T>(Sst + p * NR * LD, LD, 16 * nt + 4 * grp, 16 * at, lane), dnq[nt]);
      const Quad<T> qv = quad_load(qs + tok * LD + 16 * at + 4 * grp);
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        o[r] = (dq[r] + dden * zs[16 * at + 4 * grp + r]) * fminf(1.f, quad_get(qv, r));
      if (ok) quad_store(G + (size_t)(tb + tok) * Kp + h * DH + 16 * at + 4 * grp, quad_from4<T>(o));
    }
    __syncthreads();  // [dn | dden] of all 64 tokens are in LDS

    // [dS | dz] tiles of this wave, contracted over the tile's tokens
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tile = w + 4 * u;
      if (tile >= TILES) continue;
      const int ia = tile / NB, nb = tile - ia * NB;
#pragma unroll
      for (int s = 0; s < ST / 32; ++s)
        mma8(accS[u], frag_kmajor<T>(qs, LD, 32 * s + 8 * grp, 16 * ia, lane),
             frag_kmajor<T>(dns, LDN, 32 * s + 8 * grp, 16 * nb, lane));
    }
    __syncthreads();  // the tiles are rewritten next
  }
  float* out = partial + ((size_t)slot * H + h) * E;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tile = w + 4 * u;
    if (tile >= TILES) continue;
    const int ia = tile / NB, nb = tile - ia * NB;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a = 16 * ia + 4 * grp + r;
      if (nb < FB) out[a * DH + 16 * nb + col] = accS[u][r];
      else if (col == 0) out[DH * DH + a] = accS[u][r];
    }
  }
  if constexpr (GATED) {
    if (dgam_part) {  // dgamma of the chunk: over the 16 tokens of a lane group, then over the 4 waves
      float* red = reinterpret_cast<float*>(qs);  // the tiles are free after the last barrier
#pragma unroll
      for (int nt = 0; nt < FB; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = dgam[nt][r];
          v = row16_sum(v);
          if (col == 0) red[w * DH + 16 * nt + 4 * grp + r] = v;
        }
      __syncthreads();
      if (tid < DH)
        dgam_part[((size_t)slot * H + h) * DH + tid] =
            (red[tid] + red[DH + tid]) + (red[2 * DH + tid] + red[3 * DH + tid]);
    }
  }
}

void launch_bwd_dstate(int dt, int dh, const void* qa, const void* dy, const float* saved, const int* nchunks,
                       const Chunk* tab, int max_slots, int H, int Kp, float* partial, void* G, hipStream_t s,
                       const void* ra, const float* gamma, float eps, float* dgam_part) {
  const dim3 grid(xcd_grid(max_slots * H));
#define GBLA_BD(TT, DD)                                                                                           \
  do {                                                                                                            \
    if (ra)                                                                                                       \
      hipLaunchKernelGGL((k_bwd_dstate<TT, DD, true>), grid, dim3(256), 0, s, (const TT*)qa, (const TT*)dy, saved, \
                         nchunks, tab, max_slots, H, Kp, partial, (TT*)G, (const TT*)ra, gamma, eps, dgam_part);  \
    else                                                                                                          \
      hipLaunchKernelGGL((k_bwd_dstate<TT, DD, false>), grid, dim3(256), 0, s, (const TT*)qa, (const TT*)dy,       \
                         saved, nchunks, tab, max_slots, H, Kp, partial, (TT*)G, (const TT*)ra, gamma, eps,       \
                         dgam_part);                                                                              \
  } while (0)
  if (dt == BF16) { if (dh == 64) GBLA_BD(bf16, 64); else GBLA_BD(bf16, 32); }
  else            { if (dh == 64) GBLA_BD(float, 64); else GBLA_BD(float, 32); }
#undef GBLA_BD
}

// ============================================================== dk, dv, ds
// Same tiling as k_bwd_dstate: phi(k), v and g of 64 tokens are staged in LDS;
//   dk~ = v dS^T + dz,  dv = k~ dS      (MFMA, A rows from LDS, k~ = g phi(k);
//                                        dS is staged once, row-major, and read
//                                        transposed for dv with the transposing
//                                        LDS read, so three blocks fit per CU)
//   dg = phi(k) . dk~,  dk = g dk~ (.) phi'(k),  ds = dg g (1 - g)
// dk and dv are staged over the wave's own phi(k) and v rows and written to G
// with 16-byte stores.
template <typename T, int DH, bool SOFTMAX>
__global__ __launch_bounds__(256) void k_bwd_token(const T* __restrict__ ka, const T* __restrict__ va,
                                                   const float* __restrict__ ga, const float* __restrict__ dsz,
                                                   const int* __restrict__ nchunks, const Chunk* __restrict__ tab,
                                                   int max_slots, int H, int Kp, int nseg, T* __restrict__ G,
                                                   float* __restrict__ dbg_part, const float* __restrict__ gmax) {
  constexpr int FB = DH / 16;
  constexpr int LD = DH + 16 / (int)sizeof(T);
  constexpr int P = Parts<T>::n;
  constexpr int E = DH * DH + DH;
  constexpr int ST = 64, V8 = DH / 8;
  __shared__ __align__(16) T Srm[P * DH * LD];  // dS[i][n]: B of v dS^T by rows, B of k~ dS by columns
  __shared__ __align__(16) T ks[ST * LD];       // phi(k) tile, then dk
  __shared__ __align__(16) T vs[ST * LD];       // v tile, then dv
  __shared__ float gs[ST];
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
  stage_state<T, DH, DH>(nullptr, Srm, LD, st, st + DH * DH, tid);
  for (int e = tid; e < DH; e += 256) dzs[e] = st[DH * DH + e];

  float dbg = 0.f;
  const int gs0 = nseg * D, gcol0 = gs0 + H;  // gate column of head 0; first padding column of G
  const int gcolr = (gcol0 + 7) / 8 * 8;       // padding columns the dX~ GEMM reads (zeroed)
  const int r0 = 16 * w;
  constexpr int NV = (ST * V8 + 255) / 256;
  Frag8<T> pk[NV], pv[NV];
  float pg = 0.f;
  auto fetch = [&](int tb) {  // the next tile's loads are issued before the current tile is processed
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int it = tid + 256 * v, r = it / V8, c = (it % V8) * 8, t = tb + r;
      const bool ok = it < ST * V8 && t < ch.end;
      const size_t o = (size_t)(ok ? t : ch.start) * D + h * DH + c;
      pk[v] = ok ? frag_load(ka + o) : frag_zero<T>();
      pv[v] = ok ? frag_load(va + o) : frag_zero<T>();
    }
    if (tid < ST) pg = tb + tid < ch.end ? ga[(size_t)(tb + tid) * H + h] : 0.f;  // gate or softmax logit
  };
  fetch(ch.start);
  const float gm = SOFTMAX ? gmax[(size_t)ch.seq * H + h] : 0.f;  // softmax gate: exp(s - largest logit)
  for (int tb = ch.start; tb < ch.end; tb += ST) {  // uniform trip count (barriers inside)
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int it = tid + 256 * v, r = it / V8, c = (it % V8) * 8;
      if (it < ST * V8) {
        frag_store(ks + r * LD + c, pk[v]);
        frag_store(vs + r * LD + c, pv[v]);
      }
    }
    if (tid < ST) gs[tid] = SOFTMAX ? (tb + tid < ch.end ? __expf(pg - gm) : 0.f) : pg;
    __syncthreads();
    if (tb + ST < ch.end) fetch(tb + ST);
    const float gA = gs[r0 + col];
    Frag8<T> vf[DH / 32], kf[DH / 32];
#pragma unroll
    for (int s = 0; s < DH / 32; ++s) {
      vf[s] = frag_load(vs + (r0 + col) * LD + 32 * s + 8 * grp);
      const Frag8<T> pk = frag_load(ks + (r0 + col) * LD + 32 * s + 8 * grp);
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
          mma8(dvv[nt], kf[s], frag_kmajor<T>(Srm + p * DH * LD, LD, 32 * s + 8 * grp, 16 * nt, lane));
        }
    }
    float dkv[FB][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = r0 + 4 * grp + r;
      const int t = tb + row;
      const bool ok = t < ch.end;
      const float g = gs[row];
      float kv[FB], dk[FB], dg = 0.f;
#pragma unroll
      for (int nt = 0; nt < FB; ++nt) {
        kv[nt] = to_f<T>(ks[row * LD + 16 * nt + col]);
        dk[nt] = dkt[nt][r] + dzs[16 * nt + col];
        dg += kv[nt] * dk[nt];
      }
      dg = row16_sum(dg);
#pragma unroll
      for (int nt = 0; nt < FB; ++nt) dkv[nt][r] = g * dk[nt] * fminf(1.f, kv[nt]);
      // sigmoid gate: dg g (1 - g); softmax gate (unnormalised g, the output is
      // invariant to the normaliser): dg g
      const float ds = SOFTMAX ? dg * g : dg * g * (1.f - g);
      if (ok && col == 0) {
        G[(size_t)t * Kp + gs0 + h] = from_f<T>(ds);
        dbg += ds;
      }
      if (ok && h == 0)
        for (int c = gcol0 + col; c < gcolr; c += 16) G[(size_t)t * Kp + c] = from_f<T>(0.f);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int nt = 0; nt < FB; ++nt) {
        ks[(r0 + 4 * grp + r) * LD + 16 * nt + col] = from_f<T>(dkv[nt][r]);
        vs[(r0 + 4 * grp + r) * LD + 16 * nt + col] = from_f<T>(dvv[nt][r]);
      }
    __syncthreads();
    for (int it = tid; it < ST * V8; it += 256) {
      const int r = it / V8, c = (it % V8) * 8;
      const int t = tb + r;
      if (t < ch.end) {
        frag_store(G + (size_t)t * Kp + D + h * DH + c, frag_load(ks + r * LD + c));
        frag_store(G + (size_t)t * Kp + 2 * D + h * DH + c, frag_load(vs + r * LD + c));
      }
    }
    __syncthreads();
  }
  dbg = add_xor32(add_xor16(dbg));
  if (lane == 0) wsum[w] = dbg;
  __syncthreads();
  if (tid == 0) dbg_part[(size_t)slot * H + h] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
}

void launch_bwd_token(int dt, int dh, const void* ka, const void* va, const float* ga, const float* dsz,
                      const int* nchunks, const Chunk* tab, int max_slots, int H, int Kp, int nseg, void* G,
                      float* dbg_part, const float* gmax, hipStream_t s) {
  const dim3 grid(xcd_grid(max_slots * H));
#define GBLA_BT(TT, DD)                                                                                      \
  do {                                                                                                       \
    if (gmax)                                                                                                \
      hipLaunchKernelGGL((k_bwd_token<TT, DD, true>), grid, dim3(256), 0, s, (const TT*)ka, (const TT*)va, ga, \
                         dsz, nchunks, tab, max_slots, H, Kp, nseg, (TT*)G, dbg_part, gmax);                 \
    else                                                                                                     \
      hipLaunchKernelGGL((k_bwd_token<TT, DD, false>), grid, dim3(256), 0, s, (const TT*)ka, (const TT*)va,   \
                         ga, dsz, nchunks, tab, max_slots, H, Kp, nseg, (TT*)G, dbg_part, gmax);             \
  } while (0)
  if (dt == BF16) { if (dh == 64) GBLA_BT(bf16, 64); else GBLA_BT(bf16, 32); }
  else            { if (dh == 64) GBLA_BT(float, 64); else GBLA_BT(float, 32); }
#undef GBLA_BT
}

// ============================================================== weight packing for dX~
// wt[p][n] = [W_Q[c,:] | W_K[c,:] | W_V[c,:] | (W_R[c,:]) | w_g[:,c] | 0] for
// channel c = tile_row_perm(p) (zero rows for c >= d; wt_rows(d) rows in all).
// Thread = 8 consecutive columns n (16-byte loads and stores in the weight
// column blocks, which start at multiples of 32; element-wise in the gate and
// padding columns). With a schedule (sc.cu non-null) the last block builds the
// chunk table instead.
template <typename T>
__global__ __launch_bounds__(256) void k_pack_wt(const T* __restrict__ w_q, const T* __restrict__ w_k,
                                                 const T* __restrict__ w_v, const T* __restrict__ w_r,
                                                 const T* __restrict__ w_g, int d, int H, int dh, int Kp,
                                                 T* __restrict__ wt, Sched sc) {
  const int nblk = gridDim.x - (sc.cu ? 1 : 0);  // packing blocks
  if (sc.cu && (int)blockIdx.x == nblk) {
    schedule_block<256>(sc);
    return;
  }
  const int D = H * dh, GD = (w_r ? 4 : 3) * D;  // first gate column
  const int per_row = Kp / 8, total = wt_rows(d) * per_row;  // < 2^31 (checked on the host)
  for (int e8 = blockIdx.x * blockDim.x + threadIdx.x; e8 < total; e8 += nblk * blockDim.x) {
    const int p = e8 / per_row, n = 8 * (e8 - p * per_row);
    const size_t e = (size_t)p * Kp + n;
    const int c = tile_row_perm(p);
    Frag8<T> v = frag_zero<T>();
    if (c < d) {
      if (n < GD) {
        const int seg = n / D;
        const T* src = seg == 0 ? w_q : (seg == 1 ? w_k : (seg == 2 ? w_v : w_r));
        v = frag_load(src + (long)c * D + n - seg * D);
      } else if (w_g) {  // no w_g: zero rows
        float f[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) f[u] = n + u < GD + H ? to_f<T>(w_g[(long)(n + u - GD) * d + c]) : 0.f;
        v = frag_from<T>(f);
      }
    }
    frag_store(wt + e, v);
  }
}

void launch_pack_wt(int dt, const void* w_q, const void* w_k, const void* w_v, const void* w_r, const void* w_g,
                    int d, int H, int dh, int Kp, void* wt, const Sched& sc, hipStream_t s) {
  const long total = (long)wt_rows(d) * Kp / 8;
  const int grid = (int)std::min<long>((total + 255) / 256, 4096) + (sc.cu ? 1 : 0);
  if (dt == BF16)
    hipLaunchKernelGGL(k_pack_wt<bf16>, dim3(grid), dim3(256), 0, s, (const bf16*)w_q, (const bf16*)w_k,
                       (const bf16*)w_v, (const bf16*)w_r, (const bf16*)w_g, d, H, dh, Kp, (bf16*)wt, sc);
  else
    hipLaunchKernelGGL(k_pack_wt<float>, dim3(grid), dim3(256), 0, s, (const float*)w_q, (const float*)w_k,
                       (const float*)w_v, (const float*)w_r, (const float*)w_g, d, H, dh, Kp, (float*)wt, sc);
}

// ============================================================== dX~ = G Wt^T
// Computed transposed, dX~^T = Wt G^T: A = the packed Wt (rows = channels in
// tile_row_perm order), B = G (rows = tokens). A lane's tiles 2i and 2i+1 then
// hold 8 consecutive channels of one token, stored as one vector straight from
// registers (no LDS staging, no barrier). bf16: 256 x 256 tiles of 16 waves of
// 64 x 64 (one block per CU; a 64 x 64 wave tile keeps the LDS operand reads per
// MFMA low, and 16 waves hide their latency).
template <typename T> struct DxCfg;
template <> struct DxCfg<bf16> { using S = DlShape<256, 256, 64, 4, 4, 2>; static constexpr bool DL = true; };
template <> struct DxCfg<float> { using S = GemmShape<float, 128, 64, 32, 2, 2>; static constexpr bool DL = false; };

// Kp is the row pitch of G and Wt; the k loop reads Kr <= Kp columns.
template <typename T>
__global__ __launch_bounds__((DxCfg<T>::S::NTHREADS)) void k_gemm_dx(const T* __restrict__ G,
                                                                     const T* __restrict__ wt, int T_, int d, int Kp,
                                                                     int Kr, T* __restrict__ dxt) {
  using S = typename DxCfg<T>::S;
  constexpr bool DL = DxCfg<T>::DL;
  static_assert(S::BM % 32 == 0 && S::WTM % 32 == 0, "whole 32-row channel groups per wave");
  __shared__ __align__(16) T smem[DL ? S::STAGE : 2 * S::STAGE];
  __shared__ __align__(16) T smem1[DL ? S::STAGE : 8];
  const int dp = wt_rows(d);
  const int mtiles = (T_ + S::BN - 1) / S::BN, ntiles = (dp + S::BM - 1) / S::BM;
  const int lid = xcd_logical_block(blockIdx.x, mtiles * ntiles);
  if (lid >= mtiles * ntiles) return;
  const int mt = lid / ntiles, nt = lid - mt * ntiles;
  const int m0 = mt * S::BN, n0 = nt * S::BM;  // first token, first channel row
  f32x4 acc[S::FM][S::FN];
  if constexpr (DL)
    gemm_nt_dl<S>(wt + (size_t)n0 * Kp, Kp, min(S::BM, dp - n0), G + (size_t)m0 * Kp, Kp, min(S::BN, T_ - m0), Kr,
                  smem, smem1, smem1, smem1, acc);
  else
    gemm_nt_mainloop<T, S>(wt + (size_t)n0 * Kp, Kp, min(S::BM, dp - n0), G + (size_t)m0 * Kp, Kp,
                           min(S::BN, T_ - m0), Kr, smem, acc);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 15, grp = lane >> 4;
  const int wm = w / S::WGN, wn = w % S::WGN;
#pragma unroll
  for (int i2 = 0; i2 < S::FM / 2; ++i2) {
    const int c = n0 + wm * S::WTM + 32 * i2 + 8 * grp;  // the lane's 8 channels c .. c + 7 (d % 8 == 0)
#pragma unroll
    for (int j = 0; j < S::FN; ++j) {
      const int t = m0 + wn * S::WTN + 16 * j + col;
      float v[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = acc[2 * i2][j][r];
        v[4 + r] = acc[2 * i2 + 1][j][r];
      }
      if (t < T_ && c < d) frag_store(dxt + (size_t)t * d + c, frag_from<T>(v));
    }
  }
}

void launch_gemm_dx(int dt, const void* G, const void* wt, int T, int d, int Kp, int Kr, void* dxt, hipStream_t s) {
  if (dt == BF16) {
    using S = DxCfg<bf16>::S;
    const int n = ((T + S::BN - 1) / S::BN) * ((wt_rows(d) + S::BM - 1) / S::BM);
    if (n) hipLaunchKernelGGL(k_gemm_dx<bf16>, dim3(xcd_grid(n)), dim3(S::NTHREADS), 0, s, (const bf16*)G,
                              (const bf16*)wt, T, d, Kp, Kr, (bf16*)dxt);
  } else {
    using S = DxCfg<float>::S;
    const int n = ((T + S::BN - 1) / S::BN) * ((wt_rows(d) + S::BM - 1) / S::BM);
    if (n) hipLaunchKernelGGL(k_gemm_dx<float>, dim3(xcd_grid(n)), dim3(S::NTHREADS), 0, s, (const float*)G,
                              (const float*)wt, T, d, Kp, Kr, (float*)dxt);
  }
}

// ============================================================== dW = X~^T G (split over tokens)
// part[ks][m][n] = sum over the tokens of split ks of X~[t][m] G[t][n]; both
// operands are token-major and are transposed while staged in LDS. bf16: 256 x
// 256 tiles of 16 waves of 64 x 64, one block per CU.
template <typename T> struct DwCfg;
template <> struct DwCfg<bf16> { using S = DlShapeTN<256, 256, 64, 4, 4, 2>; static constexpr bool DL = true; };
template <> struct DwCfg<float> { using S = GemmShapeTN<float, 64, 128, 32, 2, 2>; static constexpr bool DL = false; };

int dw_tiles(int dt, int d, int Kp) {
  if (dt == BF16) {
    using S = DwCfg<bf16>::S;
    return ((d + S::BM - 1) / S::BM) * ((Kp + S::BN - 1) / S::BN);
  }
  using S = DwCfg<float>::S;
  return ((d + S::BM - 1) / S::BM) * ((Kp + S::BN - 1) / S::BN);
}

// token splits of the dW GEMM: bf16 (one 16-wave block per CU) as many as
// fill one round of the 256 CUs, float as many as fill two rounds of two
// resident blocks; at least 1024 tokens per split, at most 64
int dw_splits(int dt, int d, int Kp, int T) {
  const int tiles = dw_tiles(dt, d, Kp);
  int ns = std::max(1, (dt == BF16 ? 256 : 1024) / tiles);
  ns = std::min(ns, std::max(1, (T + 1023) / 1024));
  return std::max(1, std::min(ns, 64));
}

template <typename T>
__global__ __launch_bounds__((DwCfg<T>::S::NTHREADS)) void k_gemm_dw(const T* __restrict__ xt, const T* __restrict__ G,
                                                                   int T_, int d, int Kp, int tok_per_split,
                                                                   int nsplit, float* __restrict__ part) {
  using S = typename DwCfg<T>::S;
  constexpr bool DL = DwCfg<T>::DL;
  __shared__ __align__(16) T smem[DL ? S::STAGE : 2 * S::STAGE];
  __shared__ __align__(16) T smem1[DL ? S::STAGE : 8];
  const int mtiles = (d + S::BM - 1) / S::BM, ntiles = (Kp + S::BN - 1) / S::BN;
  const int total = mtiles * ntiles * nsplit;
  const int lid = xcd_logical_block(blockIdx.x, total);
  if (lid >= total) return;
  const int ks = lid / (mtiles * ntiles);
  const int rem = lid - ks * mtiles * ntiles;
  const int mt = rem / ntiles, nt = rem - mt * ntiles;
  const int m0 = mt * S::BM, n0 = nt * S::BN;
  const int tbeg = ks * tok_per_split, tend = min(T_, tbeg + tok_per_split);
  f32x4 acc[S::FM][S::FN];
  if constexpr (DL)
    gemm_tn_dl<S>(xt + m0, d, min(S::BM, d - m0), G + n0, Kp, min(S::BN, Kp - n0), tbeg, tend, smem, smem1, smem1,
                  smem1, acc);
  else
    gemm_tn_mainloop<T, S>(xt + m0, d, min(S::BM, d - m0), G + n0, Kp, min(S::BN, Kp - n0), tbeg, tend, smem, acc);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 15, grp = lane >> 4;
  const int wm = w / S::WGN, wn = w % S::WGN;
  float* out = part + (size_t)ks * d * Kp;
#pragma unroll
  for (int i = 0; i < S::FM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * S::WTM + 16 * i + 4 * grp + r;
      if (m >= d) continue;
#pragma unroll
      for (int j = 0; j < S::FN; ++j) {
        const int n = n0 + wn * S::WTN + 16 * j + col;
        if (n < Kp) out[(size_t)m * Kp + n] = acc[i][j][r];
      }
    }
}

void launch_gemm_dw(int dt, const void* xt, const void* G, int T, int d, int Kp, int nsplit, float* part,
                    hipStream_t s) {
  const int tps = ((T + nsplit - 1) / nsplit + 31) / 32 * 32;
  const int n = dw_tiles(dt, d, Kp) * nsplit;
  if (dt == BF16)
    hipLaunchKernelGGL(k_gemm_dw<bf16>, dim3(xcd_grid(n)), dim3(DwCfg<bf16>::S::NTHREADS), 0, s, (const bf16*)xt,
                       (const bf16*)G, T, d, Kp, tps, nsplit, part);
  else
    hipLaunchKernelGGL(k_gemm_dw<float>, dim3(xcd_grid(n)), dim3(DwCfg<float>::S::NTHREADS), 0, s,
                       (const float*)xt, (const float*)G, T, d, Kp, tps, nsplit, part);
}

// dW[c][n] = sum over the splits of part[k][c][n], four consecutive n per
// thread (Kp % 4 == 0; the Q, K, V and R column blocks start at multiples of
// 32, so a quad never straddles two of them), in split order (deterministic).
__global__ __launch_bounds__(256) void k_dw_reduce(const float* __restrict__ part, int nsplit, int d, int H,
                                                   int dh, int Kp, float* __restrict__ dw_q,
                                                   float* __restrict__ dw_k, float* __restrict__ dw_v,
                                                   float* __restrict__ dw_r, float* __restrict__ dw_g) {
  const int D = H * dh, GD = (dw_r ? 4 : 3) * D;  // first gate column
  const long total = (long)d * Kp, quads = total / 4;
  for (long qi = blockIdx.x * (long)blockDim.x + threadIdx.x; qi < quads; qi += (long)gridDim.x * blockDim.x) {
    const long e = 4 * qi;
    const int c = (int)(e / Kp), n = (int)(e - (long)c * Kp);
    if (n >= GD + H) continue;
    float4 s = *reinterpret_cast<const float4*>(part + e);
    for (int k = 1; k < nsplit; ++k) {
      const float4 p = *reinterpret_cast<const float4*>(part + (size_t)k * total + e);
      s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
    }
    if (n < GD) {
      const int seg = n / D;
      float* dst = seg == 0 ? dw_q : (seg == 1 ? dw_k : (seg == 2 ? dw_v : dw_r));
      *reinterpret_cast<float4*>(dst + (long)c * D + n - seg * D) = s;
    } else if (dw_g) {
      const float v[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (n + u < GD + H) dw_g[(long)(n + u - GD) * d + c] = v[u];
    }
  }
}

void launch_dw_reduce(const float* part, int nsplit, int d, int H, int dh, int Kp, float* dw_q, float* dw_k,
                      float* dw_v, float* dw_r, float* dw_g, hipStream_t s) {
  const long quads = (long)d * Kp / 4;
  const int grid = (int)std::min<long>((quads + 255) / 256, 8192);
  hipLaunchKernelGGL(k_dw_reduce, dim3(grid), dim3(256), 0, s, part, nsplit, d, H, dh, Kp, dw_q, dw_k, dw_v, dw_r,
                     dw_g);
}

// ============================================================== the backward's final reductions
// One launch for the three sums that close the backward, each over its own
// range of blocks, each in a fixed order: the dW split-K partials (float4 per
// thread, as k_dw_reduce), the conv-backward row-block partials of dconv_w,
// and the per-chunk partials of db_g (and of dgamma with the gated output).
__global__ __launch_bounds__(256) void k_bwd_finalize(BwdFinalize f) {
  int b = blockIdx.x;
  if (b < f.dw_blocks) {
    const int D = f.H * f.dh, GD = (f.dw_r ? 4 : 3) * D;
    const long total = (long)f.d * f.Kp, quads = total / 4;
    for (long qi = b * 256L + threadIdx.x; qi < quads; qi += (long)f.dw_blocks * 256) {
      const long e = 4 * qi;
      const int c = (int)(e / f.Kp), n = (int)(e - (long)c * f.Kp);
      if (n >= GD + f.H) continue;
      float4 s = *reinterpret_cast<const float4*>(f.dw_part + e);
      for (int k = 1; k < f.nsplit; ++k) {
        const float4 p = *reinterpret_cast<const float4*>(f.dw_part + (size_t)k * total + e);
        s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
      }
      if (n < GD) {
        const int seg = n / D;
        float* dst = seg == 0 ? f.dw_q : (seg == 1 ? f.dw_k : (seg == 2 ? f.dw_v : f.dw_r));
        *reinterpret_cast<float4*>(dst + (long)c * D + n - seg * D) = s;
      } else if (f.dw_g) {
        const float v[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (n + u < GD + f.H) f.dw_g[(long)(n + u - GD) * f.d + c] = v[u];
      }
    }
    return;
  }
  b -= f.dw_blocks;
  const int dconv_blocks = f.d;  // 4 d elements, 4 per block
  if (b < dconv_blocks) {
    sum_parts_block<4>(f.dconv_part, 4 * f.d, f.conv_rb, f.dconv_w, b);
    return;
  }
  b -= dconv_blocks;
  const int nc = *f.nchunks;
  const int dbg_blocks = (f.H + 3) / 4;
  if (b < dbg_blocks) {
    sum_parts_block<4>(f.dbg_part, f.H, nc, f.db_g, b);
    return;
  }
  b -= dbg_blocks;
  if (f.dgamma) sum_parts_block<4>(f.dgam_part, f.dh, nc * f.H, f.dgamma, b);
}

void launch_bwd_finalize(const BwdFinalize& f, hipStream_t s) {
  const int grid = f.dw_blocks + f.d + (f.H + 3) / 4 + (f.dgamma ? (f.dh + 3) / 4 : 0);
  hipLaunchKernelGGL(k_bwd_finalize, dim3(grid), dim3(256), 0, s, f);
}

int bwd_finalize_dw_blocks(int d, int Kp) {
  const long quads = (long)d * Kp / 4;
  return (int)std::min<long>((quads + 255) / 256, 8192);
}

// ============================================================== conv backward
// Thread = 8 channels x kConvRun consecutive tokens; block = 64 channel groups
// (512 channels) x 4 runs. Both windows slide in registers: dx~ rows u..u+3
// (for dx) and x rows u-3..u (for dconv_w); sequence bounds come from a cursor.
//   dx_u[c]       = sum_k w[c][k] dx~_{u+3-k}[c]      (u+3-k inside u's sequence)
//   dconv_w[c][k] = sum_t dx~_t[c] x_{t-3+k}[c]       (t-3+k inside t's sequence)
constexpr int kConvRun = 32;
constexpr int kConvBatch = 4;  // tokens per unrolled, prefetched batch
constexpr int kConvRows = 4 * kConvRun;
int conv_bwd_row_blocks(int T) { return (T + kConvRows - 1) / kConvRows; }

template <typename T>
__device__ __forceinline__ void load8f(const T* p, float (&v)[8]) {
  const Frag8<T> f = frag_load(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = frag_get(f, j);
}

template <typename T>
__global__ __launch_bounds__(256) void k_conv_bwd(const T* __restrict__ dxt, const T* __restrict__ x,
                                                  const int32_t* __restrict__ cu, int nseq, int T_, int d,
                                                  const T* __restrict__ conv_w, T* __restrict__ dx,
                                                  float* __restrict__ part) {
  constexpr int B = kConvBatch, RP = 33;  // tokens per unrolled batch; padded pitch of red[]
  __shared__ float red[4][64 * RP];
  const int rb = blockIdx.x, cb = blockIdx.y;
  const int tid = threadIdx.x, cg = tid & 63, run = tid >> 6;
  const int c = cb * 512 + cg * 8;
  float dw[8][4];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k) dw[j][k] = 0.f;
  const int u0 = rb * kConvRows + run * kConvRun;
  const int u1 = min(u0 + kConvRun, T_);
  if (c < d && u0 < u1) {
    float wv[8][4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const Frag8<T> f = frag_load(conv_w + (size_t)c * 4 + 8 * m);
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[(8 * m + e) >> 2][(8 * m + e) & 3] = frag_get(f, e);
    }
    // sliding windows: gw[s] = dx~_{u+s} (s = 0..2), xw[s] = x_{u-1-s} (s = 0..2); zero outside [0, T)
    float gw[3][8], xw[3][8];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int tg = u0 + s, tx = u0 - 1 - s;
      if (tg < T_) load8f(dxt + (size_t)tg * d + c, gw[s]);
      else
#pragma unroll
        for (int j = 0; j < 8; ++j) gw[s][j] = 0.f;
      if (tx >= 0) load8f(x + (size_t)tx * d + c, xw[s]);
      else
#pragma unroll
        for (int j = 0; j < 8; ++j) xw[s][j] = 0.f;
    }
    // the rows of a batch (dx~_{u+3}, x_u for its B tokens u) are loaded together, one batch ahead
    Frag8<T> fa[2][B], fb[2][B];
    auto fetch = [&](int buf, int ub) {
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const int tg = ub + 3 + i, tx = ub + i;
        fa[buf][i] = tg < T_ ? frag_load(dxt + (size_t)tg * d + c) : frag_zero<T>();
        fb[buf][i] = tx < u1 ? frag_load(x + (size_t)tx * d + c) : frag_zero<T>();
      }
    };
    SeqCursor cur(cu, nseq, u0, T_);
    auto compute = [&](int buf, int ub) {
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const int u = ub + i;
        if (u >= u1) break;
        float g3[8], x0[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          g3[j] = frag_get(fa[buf][i], j);
          x0[j] = frag_get(fb[buf][i], j);
        }
        const int end = cur.end(u), pos = cur.pos(u);
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // output token u + 3 - k reads x_u through tap k; token u read x_{u-sh} through tap 3 - sh
          float a = u + 3 < end ? wv[j][0] * g3[j] : 0.f;
          if (u + 2 < end) a += wv[j][1] * gw[2][j];
          if (u + 1 < end) a += wv[j][2] * gw[1][j];
          a += wv[j][3] * gw[0][j];
          o[j] = a;
          dw[j][3] += gw[0][j] * x0[j];
          if (pos >= 1) dw[j][2] += gw[0][j] * xw[0][j];
          if (pos >= 2) dw[j][1] += gw[0][j] * xw[1][j];
          if (pos >= 3) dw[j][0] += gw[0][j] * xw[2][j];
        }
        frag_store(dx + (size_t)u * d + c, frag_from<T>(o));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          gw[0][j] = gw[1][j]; gw[1][j] = gw[2][j]; gw[2][j] = g3[j];
          xw[2][j] = xw[1][j]; xw[1][j] = xw[0][j]; xw[0][j] = x0[j];
        }
      }
    };
    fetch(0, u0);
    for (int ub = u0; ub < u1; ub += 2 * B) {
      if (ub + B < u1) fetch(1, ub + B);
      compute(0, ub);
      if (ub + 2 * B < u1) fetch(0, ub + 2 * B);
      if (ub + B < u1) compute(1, ub + B);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k) red[run][cg * RP + j * 4 + k] = dw[j][k];
  __syncthreads();
  // 512 channels x 4 taps, summed over the 4 runs in a fixed order
  for (int e = tid; e < 512 * 4; e += 256) {
    const int cc = cb * 512 + (e >> 2);
    const int li = (e >> 5) * RP + (e & 31);  // channel group e / 32, element (channel % 8) * 4 + tap
    if (cc < d) part[((size_t)rb * d + cc) * 4 + (e & 3)] = (red[0][li] + red[1][li]) + (red[2][li] + red[3][li]);
  }
}

void launch_conv_bwd(int dt, const void* dxt, const void* x, const int32_t* cu, int N, int T, int d,
                     const void* conv_w, void* dx, float* dconv_part, hipStream_t s) {
  const dim3 grid(conv_bwd_row_blocks(T), (d + 511) / 512);
  if (grid.x == 0) return;
  if (dt == BF16)
    hipLaunchKernelGGL(k_conv_bwd<bf16>, grid, dim3(256), 0, s, (const bf16*)dxt, (const bf16*)x, cu, N, T, d,
                       (const bf16*)conv_w, (bf16*)dx, dconv_part);
  else
    hipLaunchKernelGGL(k_conv_bwd<float>, grid, dim3(256), 0, s, (const float*)dxt, (const float*)x, cu, N, T, d,
                       (const float*)conv_w, (float*)dx, dconv_part);
}

}  // namespace gbla
