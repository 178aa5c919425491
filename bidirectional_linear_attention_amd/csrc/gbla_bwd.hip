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
//   k_combine     the sum of those partials; its extra blocks pack the dX~ weights
//                 (pack_wt_range; k_pack_wt is the same as a launch of its own, for LION)
//   k_bwd_token   per (chunk, head): dk, dv, ds -> G; partial db_g
//   k_gemm_dx     dX~ = G Wt^T (pipelined MFMA); for GBLA its epilogue applies the
//                 conv's chain rule to the tile (dx, dconv_w partials), so dX~
//                 never reaches HBM; for LION dX~ is dx
//   k_gemm_dw     split-token partials of X~^T G (pipelined MFMA)
//   k_bwd_finalize the split-K sum of dW, the dconv_w / db_g / dgamma partial
//                 sums and dx of the three tokens at each token-tile seam
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
  // pitches (elements): LD for the dy and R tiles (row reads only); LDT = DH + 16
  // (40 dwords at d_h = 64, bf16) for the tiles that the transposing reads use:
  // the state (read by 16-row groups) and q~, [dn | dden] (read by frag_kmajor_4g)
  constexpr int LD = DH + PAD, LDT = DH + 16, LDN = DH + 16;
  constexpr int P = Parts<T>::n;
  constexpr int E = DH * DH + DH;
  constexpr int ST = 64, V8 = DH / 8, KS = DH / 32;
  constexpr int TILES = FB * NB, TPW = (TILES + 3) / 4;
  // One pool: [S | z]^T (row n = state row, row dh = z, rows > dh zero; the high
  // part, then the low part) followed by the q~ tile. Rows dh + 1 .. of the low
  // part overlap the q~ tile: they only feed output rows that are never used
  // (num rows past dh), so they may hold anything.
  constexpr int SST = (P * NR - (P - 1) * (NR - DH - 1)) * LDT, QS = ST * LDT;
  __shared__ __align__(16) T pool[SST + QS];
  T* const Sst = pool;
  T* const qs = pool + SST;
  __shared__ __align__(16) T ys[ST * LD];       // dy tile
  __shared__ __align__(16) T dns[ST * LDN];     // [dn | dden | 0] (token-major)
  __shared__ __align__(16) T rs[GATED ? ST * LD : 8];  // R tile (gated output)
  __shared__ __align__(16) float gms[GATED ? DH : 4];   // gamma (gated output)
  __shared__ float zs[DH];

  const int lid = xcd_logical_block(blockIdx.x, max_slots * H);
  if (lid >= max_slots * H) return;
  const int slot = lid / H, h = lid - slot * H;
  Chunk ch;
  if (!block_chunk(nchunks, tab, slot, ch)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int D = H * DH;
  const float* st = saved + ((size_t)ch.seq * H + h) * E;
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
  fetch(ch.start);  // the first tile loads while the state is staged
  stage_state<T, DH, NR>(Sst, nullptr, LDT, st, st + DH * DH, tid);
  __syncthreads();  // the state's low-part rows past dh that overlap the q~ tile are written before it
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

  for (int tb = ch.start; tb < ch.end; tb += ST) {  // uniform trip count (barriers inside)
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int it = tid + 256 * v, r = it / V8, c = (it % V8) * 8;
      if (it < ST * V8) {
        frag_store(qs + r * LDT + c, pq[v]);
        frag_store(ys + r * LD + c, py[v]);
        if constexpr (GATED) frag_store(rs + r * LD + c, pr[v]);
      }
    }
    __syncthreads();
    if (tb + ST < ch.end) fetch(tb + ST);

    // [num | den]^T for tokens r0 .. r0 + 15: C[4 grp + r][col] = num[token r0 + col][16 nt + 4 grp + r]
    Frag8<T> bq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) bq[s] = frag_load(qs + (r0 + col) * LDT + 32 * s + 8 * grp);
    f32x4 num[NB];
#pragma unroll
    for (int nt = 0; nt < NB; ++nt) {
      num[nt] = zero4();
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int s = 0; s < KS; ++s)
          mma8(num[nt], frag_load(Sst + p * NR * LDT + (16 * nt + col) * LDT + 32 * s + 8 * grp), bq[s]);
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
          mma_q(dq, quad_kmajor<T>(Sst + p * NR * LDT, LDT, 16 * nt + 4 * grp, 16 * at, lane), dnq[nt]);
      const Quad<T> qv = quad_load(qs + tok * LDT + 16 * at + 4 * grp);
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
        mma8(accS[u], frag_kmajor_4g<T>(qs, LDT, 32 * s, 16 * ia, lane),
             frag_kmajor_4g<T>(dns, LDN, 32 * s, 16 * nb, lane));
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
constexpr int kBwdTokenSets = 2;
template <typename T, int DH, bool SOFTMAX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))  // two tile sets within 168 registers
void k_bwd_token(const T* __restrict__ ka, const T* __restrict__ va, const float* __restrict__ ga,
                 const float* __restrict__ dsz, const int* __restrict__ nchunks, const Chunk* __restrict__ tab,
                 int max_slots, int H, int Kp, int nseg, T* __restrict__ G, float* __restrict__ dbg_part,
                 const float* __restrict__ gmax) {
  constexpr int FB = DH / 16;
  constexpr int LD = DH + 16 / (int)sizeof(T);
  constexpr int LDS_ = DH + 16;  // 40 dwords at d_h = 64 (bf16): conflict-free transposing reads of dS
  constexpr int P = Parts<T>::n;
  constexpr int E = DH * DH + DH;
  constexpr int ST = 64, V8 = DH / 8;
  __shared__ __align__(16) T Srm[P * DH * LDS_];  // dS[i][n]: B of v dS^T by rows, B of k~ dS by columns
  __shared__ __align__(16) T ks[ST * LD];       // phi(k) tile, then dk
  __shared__ __align__(16) T vs[ST * LD];       // v tile, then dv
  __shared__ float gs[ST];
  __shared__ float dzs[DH];
  __shared__ float wsum[4];

  const int lid = xcd_logical_block(blockIdx.x, max_slots * H);
  if (lid >= max_slots * H) return;
  const int slot = lid / H, h = lid - slot * H;
  Chunk ch;
  if (!block_chunk(nchunks, tab, slot, ch)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int D = H * DH;
  const float* st = dsz + ((size_t)ch.seq * H + h) * E;

  float dbg = 0.f;
  const int gs0 = nseg * D, gcol0 = gs0 + H;  // gate column of head 0; first padding column of G
  const int gcolr = (gcol0 + 7) / 8 * 8;       // padding columns the dX~ GEMM reads (zeroed)
  const int r0 = 16 * w;
  // The tile walk is unrolled (a chunk has at most kChunk / ST tiles); SETS
  // tiles are in flight, each in a register set of its own, and rows past the
  // chunk read as zeros (stores there are dropped) through buffer range checks:
  // no branch surrounds a tile load, so each tile's wait leaves the later
  // tiles' loads in flight.
  constexpr int NV = ST * V8 / 256, TILES = kChunk / ST, SETS = kBwdTokenSets;
  static_assert(ST * V8 % 256 == 0 && kChunk % ST == 0, "whole vectors per thread, whole tiles per chunk");
  const int n = ch.end - ch.start;
  const size_t o0 = (size_t)ch.start * D + h * DH;
  const RowBuf<T> kb(ka + o0, n, D, DH), vb(va + o0, n, D, DH);
  const RowBuf<T> gb(G + (size_t)ch.start * Kp, n, Kp, Kp);
  const RowScalar gate(ga + (size_t)ch.start * H + h, n, H);
  Frag8<T> pk[SETS][NV], pv[SETS][NV];
  float pg[SETS];
  auto fetch = [&](int i) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int it = tid + 256 * v, r = ST * i + it / V8, c = (it % V8) * 8;
      pk[i % SETS][v] = kb.load(r, c);
      pv[i % SETS][v] = vb.load(r, c);
    }
    pg[i % SETS] = gate.load(ST * i + (tid & (ST - 1)));  // gate or softmax logit (used by tid < ST)
  };
#pragma unroll
  for (int i = 0; i < SETS; ++i) fetch(i);  // the first tiles load while dS is staged
  const float gm = SOFTMAX ? gmax[(size_t)ch.seq * H + h] : 0.f;  // softmax gate: exp(s - largest logit)
  stage_state<T, DH, DH>(nullptr, Srm, LDS_, st, st + DH * DH, tid);
  for (int e = tid; e < DH; e += 256) dzs[e] = st[DH * DH + e];
#pragma unroll
  for (int i = 0; i < TILES; ++i) {
    if (ST * i >= n) break;  // uniform (barriers inside)
    const int tb = ch.start + ST * i;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int it = tid + 256 * v, r = it / V8, c = (it % V8) * 8;
      frag_store(ks + r * LD + c, pk[i % SETS][v]);
      frag_store(vs + r * LD + c, pv[i % SETS][v]);
    }
    const float pgv = pg[i % SETS];
    if (tid < ST) gs[tid] = SOFTMAX ? (tb + tid < ch.end ? __expf(pgv - gm) : 0.f) : pgv;
    __syncthreads();
    if (i + SETS < TILES) fetch(i + SETS);
    const float gA = gs[r0 + col];
    // kf: k~ of the lane's token with the k (feature) assignment of frag_kmajor_4g,
    // features 32 s + 4 grp + e and 32 s + 16 + 4 grp + e (e < 4), the B side's
    // transposing reads of dS then being conflict-free
    Frag8<T> vf[DH / 32], kf[DH / 32];
#pragma unroll
    for (int s = 0; s < DH / 32; ++s) {
      vf[s] = frag_load(vs + (r0 + col) * LD + 32 * s + 8 * grp);
      const Quad<T> k0 = quad_load(ks + (r0 + col) * LD + 32 * s + 4 * grp);
      const Quad<T> k1 = quad_load(ks + (r0 + col) * LD + 32 * s + 16 + 4 * grp);
      float kt[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kt[e] = gA * quad_get(k0, e);
        kt[4 + e] = gA * quad_get(k1, e);
      }
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
          mma8(dkt[nt], vf[s], frag_load(Srm + p * DH * LDS_ + (16 * nt + col) * LDS_ + 32 * s + 8 * grp));
          mma8(dvv[nt], kf[s], frag_kmajor_4g<T>(Srm + p * DH * LDS_, LDS_, 32 * s, 16 * nt, lane));
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
#pragma unroll
    for (int v = 0; v < NV; ++v) {  // rows past the chunk are dropped
      const int it = tid + 256 * v, r = it / V8, c = (it % V8) * 8;
      gb.store(ST * i + r, D + h * DH + c, frag_load(ks + r * LD + c));
      gb.store(ST * i + r, 2 * D + h * DH + c, frag_load(vs + r * LD + c));
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
// as a launch of its own (LION-s); the GBLA backward runs pack_wt_range as
// extra blocks of the combine launch instead
template <typename T>
__global__ __launch_bounds__(256) void k_pack_wt(WtPack<T> pk, Sched sc) {
  if (sc.cu && (int)blockIdx.x == pk.blocks) {
    schedule_block<256>(sc);
    return;
  }
  pack_wt_range(pk, blockIdx.x);
}

void launch_pack_wt(int dt, const void* w_q, const void* w_k, const void* w_v, const void* w_r, const void* w_g,
                    int d, int H, int dh, int Kp, void* wt, const Sched& sc, hipStream_t s) {
  const WtPackArgs a{w_q, w_k, w_v, w_r, w_g, d, H, dh, Kp, wt};
  const int grid = wt_pack_blocks(d, Kp) + (sc.cu ? 1 : 0);
  if (dt == BF16) hipLaunchKernelGGL(k_pack_wt<bf16>, dim3(grid), dim3(256), 0, s, wt_pack_of<bf16>(a), sc);
  else hipLaunchKernelGGL(k_pack_wt<float>, dim3(grid), dim3(256), 0, s, wt_pack_of<float>(a), sc);
}

// ============================================================== dX~ = G Wt^T
// Computed transposed, dX~^T = Wt G^T: A = the packed Wt (rows = channels in
// tile_row_perm order), B = G (rows = tokens). A lane's tiles 2i and 2i+1 then
// hold 8 consecutive channels of one token, stored as one vector straight from
// registers (no LDS staging, no barrier). bf16: 256 x 256 tiles of 16 waves of
// 64 x 64 (one block per CU; a 64 x 64 wave tile keeps the LDS operand reads per
// MFMA low, and 16 waves hide their latency).
// A batch whose 256-token tiles would leave compute units idle (fewer tiles than
// 256; the B = 32, L = 1024, d = 256 workload has 128) takes 128-token tiles
// of 8 waves instead (SMALL), so that every compute unit gets a block.
template <typename T, bool SMALL = false> struct DxCfg;
template <> struct DxCfg<bf16, false> { using S = DlShape<256, 256, 64, 4, 4, 2>; static constexpr bool DL = true; };
template <> struct DxCfg<bf16, true> { using S = DlShape<256, 128, 64, 4, 2, 2>; static constexpr bool DL = true; };
template <bool SMALL> struct DxCfg<float, SMALL> {
  using S = GemmShape<float, 128, 64, 32, 2, 2>;
  static constexpr bool DL = false;
};
constexpr int kDxFillTiles = 256;  // compute units of the MI355X

// Kp is the row pitch of G and Wt; the k loop reads Kr <= Kp columns.
//
// CONV = false (LION): the tile of dX~ = dx is stored as it is.
// CONV = true (GBLA): the epilogue applies the vector-Jacobian product of the
// causal conv (Eq. (4)) to the block's tile of dX~ (BN tokens x BM channels),
// which never goes to HBM:
//   dx_u[c]       = sum_k w[c][k] dX~_{u+3-k}[c]    (u+3-k inside u's sequence)
//   dconv_w[c][k] = sum_t dX~_t[c] x_{t-3+k}[c]     (t-3+k inside t's sequence)
// The tile goes to LDS (rounded to the activation dtype, as dX~ would be
// stored), then each thread slides a 4-row window over RL consecutive tokens of
// one 8-channel group. dx of the tile's last three tokens needs the next tile's
// first three rows of dX~, so every tile also writes its first and last three
// rows to `edge` and dx of those three tokens is formed by k_bwd_finalize (the
// last tile of the batch has no successor: its rows past T are zero and it
// writes all of its dx). dconv_w gets one partial per token tile, summed in a
// fixed order by k_bwd_finalize.
constexpr float kZero4[4] = {0.f, 0.f, 0.f, 0.f};

struct DxConv {
  const void* x;           // [T][d] conv input (dtype)
  const int32_t* cu;       // [N+1] sequence offsets
  int nseq;
  const void* conv_w;      // [d][4] (dtype)
  float* dconv_part;       // [token tiles][d][4]
  void* edge;              // [token tiles][6][d] (dtype): dX~ rows 0..2, then BN-3..BN-1 of every tile
};

template <typename T, class S>
__device__ __forceinline__ void dx_conv_epilogue(const f32x4 (&acc)[S::FM][S::FN], T* lo, T* hi, int m0, int n0,
                                                 int mt, int T_, int d, T* __restrict__ dx, const DxConv& cv) {
  constexpr int BT = S::BN, BC = S::BM, CH = BC / 8, NT = S::NTHREADS;
  constexpr int NQ = BC / 4, RUNS = NT / NQ, RL = BT / RUNS;  // 4-channel quads; token runs of RL
  static_assert(NT % NQ == 0 && BT % RUNS == 0 && RL >= 4 && RL % 4 == 0, "thread runs tile the token axis");
  constexpr int HALF = (BT / 2) * BC * (int)sizeof(T) / 4;  // floats in one token half of the tile
  static_assert(RUNS * NQ * 16 <= 2 * HALF, "room for the dconv_w partials where the tile was");
  const T* __restrict__ x = static_cast<const T*>(cv.x);
  // row r of the dX~ tile (token m0 + r): chunk q (8 channels) at row(r) + 8 * (q ^ (r % CH))
  auto row = [&](int r) -> T* { return r < BT / 2 ? lo + r * BC : hi + (r - BT / 2) * BC; };
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int wm = w / S::WGN, wn = w % S::WGN;
#pragma unroll
  for (int i2 = 0; i2 < S::FM / 2; ++i2) {
    const int q = (wm * S::WTM + 32 * i2) / 8 + grp;
#pragma unroll
    for (int j = 0; j < S::FN; ++j) {
      const int r = wn * S::WTN + 16 * j + col;
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = acc[2 * i2][j][e];
        v[4 + e] = acc[2 * i2 + 1][j][e];
      }
      frag_store(row(r) + 8 * (q ^ (r % CH)), frag_from<T>(v));
    }
  }
  __syncthreads();

  // the tile's first and last three rows, for the dx of the previous tile's and
  // this tile's last three tokens
  for (int e = tid; e < 6 * CH; e += NT) {
    const int er = e / CH, eq = e % CH, r = er < 3 ? er : BT - 6 + er;
    if (n0 + 8 * eq < d)
      frag_store(static_cast<T*>(cv.edge) + ((size_t)mt * 6 + er) * d + n0 + 8 * eq,
                 frag_load(row(r) + 8 * (eq ^ (r % CH))));
  }
  const int qd = tid % NQ, run = tid / NQ;
  const int c = n0 + 4 * qd, u0 = run * RL, t0 = m0 + u0;
  const int qoff = 8 * ((qd >> 1)) + 4 * (qd & 1);  // before the row swizzle
  const bool last_tile = m0 + BT >= T_;
  float dw[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k) dw[j][k] = 0.f;
  if (c < d && t0 < T_) {
    // taps of the 4 channels: w[c + j][k] = element (4 j + k) % 8 of wf[(4 j + k) / 8]
    Frag8<T> wf[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) wf[m] = frag_load(static_cast<const T*>(cv.conv_w) + (size_t)c * 4 + 8 * m);
    auto wtap = [&](int j, int k) { return frag_get(wf[(4 * j + k) >> 3], (4 * j + k) & 7); };
    // x rows slide through xw[0..3] = x_{t-3} .. x_t, loaded 4 rows ahead of use
    auto xrow = [&](int t) { return t >= 0 && t < T_ ? quad_load(x + (size_t)t * d + c) : quad_from4<T>(kZero4); };
    Quad<T> xw[4] = {quad_from4<T>(kZero4), xrow(t0 - 3), xrow(t0 - 2), xrow(t0 - 1)};
    Quad<T> xb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xb[i] = xrow(t0 + i);
    // the window g0..g3 = dX~ rows u .. u + 3 of the tile (zero past its end)
    auto tile_row = [&](int r) {
      return r < BT ? quad_load(row(r) + (qoff ^ (8 * (r % CH)))) : quad_from4<T>(kZero4);
    };
    Quad<T> g0 = tile_row(u0), g1 = tile_row(u0 + 1), g2 = tile_row(u0 + 2);
    SeqCursor cur(cv.cu, cv.nseq, t0, T_);
#pragma unroll
    for (int i = 0; i < RL; ++i) {
      const int u = u0 + i, t = m0 + u;
      if (t >= T_) break;
      xw[0] = xw[1];
      xw[1] = xw[2];
      xw[2] = xw[3];
      xw[3] = xb[i % 4];
      if (i % 4 == 3 && i + 1 < RL) {
#pragma unroll
        for (int k = 0; k < 4; ++k) xb[k] = xrow(t + 1 + k);
      }
      const Quad<T> g3 = tile_row(u + 3);
      const int end = cur.end(t), pos = cur.pos(t);
      if (u + 3 < BT || last_tile) {
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float a = t + 3 < end ? wtap(j, 0) * quad_get(g3, j) : 0.f;
          if (t + 2 < end) a += wtap(j, 1) * quad_get(g2, j);
          if (t + 1 < end) a += wtap(j, 2) * quad_get(g1, j);
          a += wtap(j, 3) * quad_get(g0, j);
          o[j] = a;
        }
        quad_store(dx + (size_t)t * d + c, quad_from4<T>(o));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float gv = quad_get(g0, j);
        dw[j][3] += gv * quad_get(xw[3], j);
        if (pos >= 1) dw[j][2] += gv * quad_get(xw[2], j);
        if (pos >= 2) dw[j][1] += gv * quad_get(xw[1], j);
        if (pos >= 3) dw[j][0] += gv * quad_get(xw[0], j);
      }
      g0 = g1;
      g1 = g2;
      g2 = g3;
    }
  }
  __syncthreads();  // the tile is no longer read: its LDS takes the dconv_w partials [RUNS][NQ][16]
  auto red_at = [&](int rr, int qq, int e) -> float& {
    const int i = (rr * NQ + qq) * 16 + e;
    return i < HALF ? reinterpret_cast<float*>(lo)[i] : reinterpret_cast<float*>(hi)[i - HALF];
  };
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k) red_at(run, qd, j * 4 + k) = dw[j][k];
  __syncthreads();
  for (int e = tid; e < BC * 4; e += NT) {
    const int cl = e >> 2, k = e & 3;
    float sum = 0.f;
    for (int rr = 0; rr < RUNS; ++rr) sum += red_at(rr, cl >> 2, (cl & 3) * 4 + k);
    if (n0 + cl < d) cv.dconv_part[((size_t)mt * d + n0 + cl) * 4 + k] = sum;
  }
}

template <typename T, bool CONV, bool SMALL>
__global__ __launch_bounds__((DxCfg<T, SMALL>::S::NTHREADS)) void k_gemm_dx(const T* __restrict__ G,
                                                                            const T* __restrict__ wt, int T_, int d,
                                                                            int Kp, int Kr, T* __restrict__ out,
                                                                            DxConv cv) {
  using S = typename DxCfg<T, SMALL>::S;
  constexpr bool DL = DxCfg<T, SMALL>::DL;
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
  if constexpr (CONV) {
    // the tile's token halves in the two stage buffers (bf16), or both in the one buffer (float)
    static_assert(!DL || (S::BN / 2) * S::BM <= S::STAGE, "a token half of the tile fits one stage");
    static_assert(DL || S::BN * S::BM <= 2 * S::STAGE, "the tile fits the stage buffer");
    dx_conv_epilogue<T, S>(acc, smem, DL ? smem1 : smem + (S::BN / 2) * S::BM, m0, n0, mt, T_, d, out, cv);
    return;
  }
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
      if (t < T_ && c < d) frag_store(out + (size_t)t * d + c, frag_from<T>(v));
    }
  }
}

static bool dx_small(int dt, int T, int d) {
  using S = DxCfg<bf16, false>::S;
  return dt == BF16 && (long)((T + S::BN - 1) / S::BN) * ((wt_rows(d) + S::BM - 1) / S::BM) < kDxFillTiles;
}
int dx_token_tile_rows(int dt, int T, int d) {
  if (dt != BF16) return DxCfg<float>::S::BN;
  return dx_small(dt, T, d) ? DxCfg<bf16, true>::S::BN : DxCfg<bf16, false>::S::BN;
}
int dx_token_tiles(int dt, int T, int d) {
  const int bn = dx_token_tile_rows(dt, T, d);
  return (T + bn - 1) / bn;
}

template <typename TT, bool SMALL>
static void gemm_dx_t(const void* G, const void* wt, int T, int d, int Kp, int Kr, void* out, const DxConv* cv,
                      hipStream_t s) {
  using S = typename DxCfg<TT, SMALL>::S;
  const int n = ((T + S::BN - 1) / S::BN) * ((wt_rows(d) + S::BM - 1) / S::BM);
  if (n == 0) return;
  if (cv)
    hipLaunchKernelGGL((k_gemm_dx<TT, true, SMALL>), dim3(xcd_grid(n)), dim3(S::NTHREADS), 0, s, (const TT*)G,
                       (const TT*)wt, T, d, Kp, Kr, (TT*)out, *cv);
  else
    hipLaunchKernelGGL((k_gemm_dx<TT, false, SMALL>), dim3(xcd_grid(n)), dim3(S::NTHREADS), 0, s, (const TT*)G,
                       (const TT*)wt, T, d, Kp, Kr, (TT*)out, DxConv{});
}
template <typename TT>
static void gemm_dx_any(int dt, const void* G, const void* wt, int T, int d, int Kp, int Kr, void* out,
                        const DxConv* cv, hipStream_t s) {
  if (dx_small(dt, T, d)) gemm_dx_t<TT, true>(G, wt, T, d, Kp, Kr, out, cv, s);
  else gemm_dx_t<TT, false>(G, wt, T, d, Kp, Kr, out, cv, s);
}

void launch_gemm_dx(int dt, const void* G, const void* wt, int T, int d, int Kp, int Kr, void* dxt, hipStream_t s) {
  if (dt == BF16) gemm_dx_any<bf16>(dt, G, wt, T, d, Kp, Kr, dxt, nullptr, s);
  else gemm_dx_t<float, false>(G, wt, T, d, Kp, Kr, dxt, nullptr, s);
}

void launch_gemm_dx_conv(int dt, const void* G, const void* wt, int T, int d, int Kp, int Kr, const void* x,
                         const int32_t* cu, int N, const void* conv_w, void* dx, float* dconv_part, void* edge,
                         hipStream_t s) {
  const DxConv cv{x, cu, N, conv_w, dconv_part, edge};
  if (dt == BF16) gemm_dx_any<bf16>(dt, G, wt, T, d, Kp, Kr, dx, &cv, s);
  else gemm_dx_t<float, false>(G, wt, T, d, Kp, Kr, dx, &cv, s);
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
// resident blocks; at least 512 tokens per split, at most 64
int dw_splits(int dt, int d, int Kp, int T) {
  const int tiles = dw_tiles(dt, d, Kp);
  int ns = std::max(1, (dt == BF16 ? 256 : 1024) / tiles);
  ns = std::min(ns, std::max(1, (T + 511) / 512));
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
// dx of tokens u = m0 + BT - 3 + i (i < 3) of token tile mt: their conv window
// dX~ rows u .. u + 3 straddles tiles mt and mt + 1, whose edge rows hold them
// (tile mt's last three rows, then tile mt + 1's first three). Same arithmetic,
// in the same order, as the dX~ GEMM's epilogue.
template <typename T>
__device__ void conv_tail_block(const BwdFinalize& f, int mt) {
  const T* edge = static_cast<const T*>(f.edge);
  const T* conv_w = static_cast<const T*>(f.conv_w);
  const int BT = f.tile_rows, d = f.d, G8 = d / 8;
  for (int e = threadIdx.x; e < 3 * G8; e += 256) {
    const int i = e / G8, c = 8 * (e % G8);
    const int t = mt * BT + BT - 3 + i;  // < T: tile mt is not the last
    int lo = 0, hi = f.nseq;  // t's sequence: the last b with cu[b] <= t
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (f.cu[mid] <= t) lo = mid; else hi = mid;
    }
    const int end = f.cu[lo + 1];
    // window rows t + s, s = 0..3: edge row 3 + i + s of tile mt while inside it, else row i + s - 3 of tile mt + 1
    Frag8<T> g[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const int r = i + s2;
      const size_t er = r < 3 ? (size_t)mt * 6 + 3 + r : (size_t)(mt + 1) * 6 + (r - 3);
      g[s2] = frag_load(edge + er * d + c);
    }
    Frag8<T> wf[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) wf[m] = frag_load(conv_w + (size_t)c * 4 + 8 * m);
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      auto wtap = [&](int k) { return frag_get(wf[(4 * j + k) >> 3], (4 * j + k) & 7); };
      float a = t + 3 < end ? wtap(0) * frag_get(g[3], j) : 0.f;
      if (t + 2 < end) a += wtap(1) * frag_get(g[2], j);
      if (t + 1 < end) a += wtap(2) * frag_get(g[1], j);
      a += wtap(3) * frag_get(g[0], j);
      o[j] = a;
    }
    frag_store(static_cast<T*>(f.dx) + (size_t)t * d + c, frag_from<T>(o));
  }
}

__global__ __launch_bounds__(256) void k_bwd_finalize(BwdFinalize f) {
  int b = blockIdx.x;
  if (b < f.dw_blocks) {
    const int D = f.H * f.dh, GD = (f.dw_r ? 4 : 3) * D;
    const long total = (long)f.d * f.Kp, quads = total / 4;
    for (long qi = b * 256L + threadIdx.x; qi < quads; qi += (long)f.dw_blocks * 256) {
      const long e = 4 * qi;
      const int c = (int)(e / f.Kp), n = (int)(e - (long)c * f.Kp);
      if (n >= GD + f.H) continue;
      // split k in order; the loads go out U at a time (one memory latency per U splits)
      constexpr int U = 8;
      float4 s = *reinterpret_cast<const float4*>(f.dw_part + e);
      for (int kb = 1; kb < f.nsplit; kb += U) {
        float4 p[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
          p[u] = kb + u < f.nsplit ? *reinterpret_cast<const float4*>(f.dw_part + (size_t)(kb + u) * total + e)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (kb + u >= f.nsplit) break;
          s.x += p[u].x; s.y += p[u].y; s.z += p[u].z; s.w += p[u].w;
        }
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
  const int dgam_blocks = f.dgamma ? (f.dh + 3) / 4 : 0;
  if (b < dgam_blocks) {
    sum_parts_block<4>(f.dgam_part, f.dh, nc * f.H, f.dgamma, b);
    return;
  }
  b -= dgam_blocks;
  if (f.edge && b < f.conv_rb - 1) {  // dx of the last three tokens of token tile b (not the batch's last)
    if (f.dt == BF16) conv_tail_block<bf16>(f, b);
    else conv_tail_block<float>(f, b);
  }
}

void launch_bwd_finalize(const BwdFinalize& f, hipStream_t s) {
  const int grid = f.dw_blocks + f.d + (f.H + 3) / 4 + (f.dgamma ? (f.dh + 3) / 4 : 0) +
                   (f.edge ? std::max(0, f.conv_rb - 1) : 0);
  hipLaunchKernelGGL(k_bwd_finalize, dim3(grid), dim3(256), 0, s, f);
}

int bwd_finalize_dw_blocks(int d, int Kp) {
  const long quads = (long)d * Kp / 4;
  return (int)std::min<long>((quads + 255) / 256, 8192);
}

}  // namespace gbla
