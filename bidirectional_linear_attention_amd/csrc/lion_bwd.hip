// LION-s chunkwise backward for gfx950.
//
// With P_ij = M_ij (q~_i . k~_j), r_i = sum_j P_ij, y_i = sum_j P_ij v_j / r_i and
// the upstream gradient dy, let g^_i = [dy_i / r_i | -(dy_i . y_i) / r_i] (a
// dh+1 vector, dN_i = its first dh entries) and v^_j = [v_j | 1]. Then
//   dP_ij = g^_i . v^_j
//   dq~_i = sum_j M_ij dP_ij k~_j,   dk~_j = sum_i M_ij dP_ij q~_i,   dv_j = sum_i P_ij dN_i
// and for the decay (M_ij = exp(-|A_i - A_j|), A non-increasing), with E_ij = dP_ij P_ij,
//   dA_t = sum_{j<t} (E_tj + E_jt) - sum_{j>t} (E_tj + E_jt),
//   dlog lambda_k = sum_{t>=k} dA_t (within the sequence),  da = dlog lambda (1 - lambda).
// Each sum over j splits like the forward into the chunk itself and the chunks
// before / after it. The inter-chunk parts use the forward states SF, SB for
// dq~ and the states HF, HB of sum_i decay q~_i g^_i^T (same recurrences) for dk~
// and dv; the inter-chunk parts of dA are dot products of q~ and k~ with those
// inter-chunk gradients (e.g. sum_{j before c} E_tj = q~_t . dq~_t(from SF)).
//
// dlog lambda_t splits at the end e_c of t's chunk c: the suffix of dA inside
// the chunk, plus sum_{u > e_c} dA_u. In that second sum every pair of tokens
// both after e_c enters twice with opposite signs, so it equals the sum of F_uj
// = E_uj + E_ju over the pairs u > e_c >= j that straddle the chunk end:
//   Z'_c = sum_{j in c} Y_j + Z_c,   Y_j = sum_{u after c} F_uj,
//   Z_c  = sum_{u after c, j before c} F_uj = e^{L_c} (<SF_c, HB_c> + <HF_c, SB_c>)
// (Frobenius products of the states entering chunk c, L_c its total log decay).
// Taking it in that form instead of summing dA over all later chunks keeps the
// rounding error of dlog lambda independent of the sequence length: summed over
// later chunks, the rounding residues of pairs that cancel in exact arithmetic
// would accumulate with the number of chunks.
//
// k_lion_bwd_token   per (chunk, head): dq, dk, dv (through the feature-map
//                    vector-Jacobian product) into G, chunk-local suffix sums
//                    of dA and the chunk's straddling sum Z'_c
// k_lion_da          per chunk: da = (local suffix + Z'_c)(1 - lambda) into G,
//                    and a partial sum for db_lam
#include "internal.h"
#include "lion_internal.h"

namespace gbla {

// phi(u) = (SiLU(u) + 0.5) / n: given p = phi(u), n and d = dphi, returns du
__device__ __forceinline__ float phi_lion_vjp(float u, float p, float inv_n, float d, float dot) {
  const float sg = sigmoidf_(u);
  return (d - p * dot) * inv_n * (sg * (1.f + u * (1.f - sg)));
}

// a carried state, stored transposed ([n][a]: row n = column feature n, dh
// values of the row feature a; row dh = the extra column), staged as the LDS
// tile [n][a] for n < dh (pitch ld, a multiple of 4) plus the extra row as
// floats; S is 16-byte aligned. state_rows_load issues the loads into
// registers, state_rows_store writes them (4 elements per 8- or 16-byte LDS
// store), so the loads can be issued well before the tile is needed.
template <int DH> struct StateRegs {
  static constexpr int V4 = DH * DH / 4, PER = (V4 + 255) / 256;
  float4 r[PER];
  float x;
};
template <int DH>
__device__ __forceinline__ void state_rows_load(StateRegs<DH>& g, const float* __restrict__ S, int tid) {
#pragma unroll
  for (int k = 0; k < StateRegs<DH>::PER; ++k) {
    const int e4 = tid + 256 * k;
    g.r[k] = e4 < StateRegs<DH>::V4 ? reinterpret_cast<const float4*>(S)[e4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  g.x = tid < DH ? S[DH * DH + tid] : 0.f;
}
template <typename T, int DH>
__device__ __forceinline__ void state_rows_store(const StateRegs<DH>& g, T* R, int ld, float* extra, int tid) {
#pragma unroll
  for (int k = 0; k < StateRegs<DH>::PER; ++k) {
    const int e4 = tid + 256 * k;
    if (e4 >= StateRegs<DH>::V4) continue;
    const int n = (4 * e4) / DH, a = (4 * e4) % DH;
    const float v[4] = {g.r[k].x, g.r[k].y, g.r[k].z, g.r[k].w};
    quad_store(R + n * ld + a, quad_from4<T>(v));
  }
  if (tid < DH) extra[tid] = g.x;
}
// the same staging from a state whose dh x dh part is already rounded to T
// (the row image of the scan, rows [n][a] contiguous) and whose extra row is
// the fp32 X: the loads move 4 T per lane and the LDS stores need no conversion
template <typename T, int DH> struct ImageRegs {
  static constexpr int V4 = DH * DH / 4, PER = (V4 + 255) / 256;
  Quad<T> r[PER];
  float x;
};
template <typename T, int DH>
__device__ __forceinline__ void image_rows_load(ImageRegs<T, DH>& g, const T* __restrict__ S,
                                                const float* __restrict__ X, int tid) {
  static_assert(ImageRegs<T, DH>::V4 % 256 == 0, "every lane loads PER quads");
#pragma unroll
  for (int k = 0; k < ImageRegs<T, DH>::PER; ++k) g.r[k] = quad_load<T>(S + 4 * (tid + 256 * k));
  g.x = tid < DH ? X[tid] : 0.f;
}
template <typename T, int DH>
__device__ __forceinline__ void image_rows_store(const ImageRegs<T, DH>& g, T* R, int ld, float* extra, int tid) {
#pragma unroll
  for (int k = 0; k < ImageRegs<T, DH>::PER; ++k) {
    const int e4 = tid + 256 * k;
    const int n = (4 * e4) / DH, a = (4 * e4) % DH;
    quad_store(R + n * ld + a, g.r[k]);
  }
  if (tid < DH) extra[tid] = g.x;
}
// this thread's share of the Frobenius product of a fp32 state and a state
// image (the same elements of both: the quads e4 = tid + 256 k and extra entry tid)
template <typename T, int DH>
__device__ __forceinline__ float state_image_dot(const StateRegs<DH>& s, const ImageRegs<T, DH>& g, int tid) {
  static_assert(StateRegs<DH>::PER == ImageRegs<T, DH>::PER, "same element split");
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < StateRegs<DH>::PER; ++k) {
    const float4 a = s.r[k];
    acc += a.x * quad_get(g.r[k], 0) + a.y * quad_get(g.r[k], 1) + a.z * quad_get(g.r[k], 2) +
           a.w * quad_get(g.r[k], 3);
  }
  return acc + (tid < DH ? s.x * g.x : 0.f);
}
template <typename T, int DH>
__device__ __forceinline__ void stage_state_rows(T* R, int ld, float* extra, const float* __restrict__ S, int tid) {
  StateRegs<DH> g;
  state_rows_load<DH>(g, S, tid);
  state_rows_store<T, DH>(g, R, ld, extra, tid);
}

// Block = (chunk, head), 4 waves; wave w owns rows 16 w .. 16 w + 15 of the chunk
// (query rows in phase 1, key rows in phase 2). The extra column of [v | 1] and
// of g^ enters every contraction as a rank-1 term, so all MFMA widths are dh.
// Two blocks per CU (the occupancy hint keeps the registers of the phase-2
// state prefetch within 256 per lane).
template <typename T, int DH>
__global__ __launch_bounds__(256, 2) void k_lion_bwd_token(
    const T* __restrict__ qr, const T* __restrict__ kr, const T* __restrict__ vr, const float* __restrict__ logl,
    const T* __restrict__ yv, const T* __restrict__ dy, const float* __restrict__ rsum, const float* __restrict__ st,
    const float* __restrict__ hst, const T* __restrict__ hrows, const int* __restrict__ nchunks,
    const Chunk* __restrict__ tab, int max_slots, int H, int Kp, T* __restrict__ G, float* __restrict__ dA_loc,
    float* __restrict__ dA_tot) {
  constexpr int C = kLionChunk;
  constexpr int FB = DH / 16;
  constexpr int PAD = 16 / (int)sizeof(T);
  constexpr int LDR = DH + PAD, LDP = C + PAD;
  constexpr int E = DH * DH + DH;
  constexpr int V8 = DH / 8, NV = (C * V8 + 255) / 256;
  __shared__ __align__(16) T Qs[C * LDR];   // phi(q); dk on output
  __shared__ __align__(16) T Ks[C * LDR];   // phi(k); dq on output
  __shared__ __align__(16) T Vs[C * LDR];   // v; dv on output
  __shared__ __align__(16) T Gs[C * LDR];   // dy / r
  __shared__ __align__(16) T PD[2 * C * LDP];    // P, then dP (.) M; dq (float) at the output
  __shared__ __align__(16) T SFB[2 * DH * LDR];  // SF then SB ([n][a]), later HF then HB; dk (float)
  T* const Pt = PD;
  T* const Dt = PD + C * LDP;
  T* const SFs = SFB;
  T* const SBs = SFB + DH * LDR;
  // the gradients of phi(q) and phi(k), kept in float for the feature-map VJP
  // at the output (both regions are free by then)
  static_assert(2 * C * LDP * sizeof(T) >= (DH == 64 ? 1 : 2) * C * DH * sizeof(float) &&
                    (DH != 64 || 2 * DH * LDR * sizeof(T) >= C * DH * sizeof(float)),
                "room for the float gradients");
  float* const dqf = reinterpret_cast<float*>(PD);
  float* const dkf = DH == 64 ? reinterpret_cast<float*>(SFB) : reinterpret_cast<float*>(PD) + C * DH;
  __shared__ float xF[DH], xB[DH];          // extra columns of the staged states
  __shared__ float As[C], nq[C], nk[C], gden[C], vone[C], dAq[C], dAk[C], dotq[C], dotk[C], Yq[C], Yk[C];
  __shared__ float colpart[4][C];
  __shared__ float Ls, zpart[4];

  const int lid = xcd_logical_block(blockIdx.x, max_slots * H);
  if (lid >= max_slots * H) return;
  const int slot = lid / H, h = lid - slot * H;
  Chunk ch;
  if (!block_chunk(nchunks, tab, slot, ch)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int D = H * DH;
  const int r0 = 16 * w;

  // ---------------- phase 0: staging
  const float la = chunk_decay_load<C>(logl, ch, H, h, tid);
  const float* sp = st + ((size_t)slot * H + h) * 2 * E;
  const T* img = hrows + ((size_t)slot * H + h) * 2 * (DH * DH);
  const float* ext = hst + ((size_t)slot * H + h) * 2 * E + DH * DH;
  // every global load of the phase is issued before any of it is used: the
  // token tiles, then the four states, so the phase pays one memory latency
  Frag8<T> fq[NV], fk[NV], fv[NV], fd[NV], fy[NV];
  float rinv[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int it = tid + 256 * v;
    const int r = it / V8, c = (it % V8) * 8, t = ch.start + r;
    const bool ok = it < C * V8 && t < ch.end;
    const size_t o = (size_t)(ok ? t : ch.start) * D + h * DH + c;
    fq[v] = ok ? frag_load(qr + o) : frag_zero<T>();
    fk[v] = ok ? frag_load(kr + o) : frag_zero<T>();
    fv[v] = ok ? frag_load(vr + o) : frag_zero<T>();
    fd[v] = ok ? frag_load(dy + o) : frag_zero<T>();
    fy[v] = ok ? frag_load(yv + o) : frag_zero<T>();
    rinv[v] = ok ? rsum[(size_t)t * H + h] : 1.f;
  }
  StateRegs<DH> sf, sb;
  ImageRegs<T, DH> hb, hf;
  state_rows_load<DH>(sf, sp, tid);
  image_rows_load<T, DH>(hb, img + DH * DH, ext + E, tid);
  state_rows_load<DH>(sb, sp + E, tid);
  image_rows_load<T, DH>(hf, img, ext, tid);
  // this thread's terms of <SF, HB> + <HF, SB> (fp32 S; H as the scan rounded it)
  float zdot = state_image_dot<T, DH>(sf, hb, tid) + state_image_dot<T, DH>(sb, hf, tid);
  state_rows_store<T, DH>(sf, SFs, LDR, xF, tid);
  state_rows_store<T, DH>(sb, SBs, LDR, xB, tid);
  zdot = add_xor32(add_xor16(row16_sum(zdot)));
  if (lane == 0) zpart[w] = zdot;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int it = tid + 256 * v;
    if (it >= C * V8) continue;
    const int r = it / V8, c = (it % V8) * 8, t = ch.start + r;
    const bool ok = t < ch.end;
    float u[8], p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = frag_get(fq[v], j);
    float n = phi_lion8<V8>(u, p, ok);
    frag_store(Qs + r * LDR + c, frag_from<T>(p));
    if (c == 0) nq[r] = ok ? n : 1.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = frag_get(fk[v], j);
    n = phi_lion8<V8>(u, p, ok);
    frag_store(Ks + r * LDR + c, frag_from<T>(p));
    if (c == 0) nk[r] = ok ? n : 1.f;
    frag_store(Vs + r * LDR + c, fv[v]);
    const float inv = ok ? fast_rcp(rinv[v]) : 0.f;
    float g[8], dd = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      g[j] = frag_get(fd[v], j) * inv;
      dd += frag_get(fd[v], j) * frag_get(fy[v], j);
    }
    dd = lane_group_sum<V8>(dd);
    frag_store(Gs + r * LDR + c, frag_from<T>(g));
    if (c == 0) {
      gden[r] = -dd * inv;
      vone[r] = ok ? 1.f : 0.f;
    }
  }
  chunk_decay_scan<C>(la, As, &Ls, tid);
  __syncthreads();
  const float L = Ls;

  // ---------------- phase 1: query rows i = r0 + 4 grp + r
  float dqo[FB][4];
  ImageRegs<T, DH> hreg[2];
  {
    Frag8<T> aq[DH / 32], ag[DH / 32];
#pragma unroll
    for (int s = 0; s < DH / 32; ++s) {
      aq[s] = frag_load(Qs + (r0 + col) * LDR + 32 * s + 8 * grp);
      ag[s] = frag_load(Gs + (r0 + col) * LDR + 32 * s + 8 * grp);
    }
    float gd[4], ef[4], eb[4], sgn[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float a = As[r0 + 4 * grp + r];
      gd[r] = gden[r0 + 4 * grp + r];
      ef[r] = __expf(a);
      eb[r] = __expf(L - a);
    }
#pragma unroll
    for (int nt = 0; nt < C / 16; ++nt) {
      f32x4 g = zero4(), dp = zero4();
#pragma unroll
      for (int s = 0; s < DH / 32; ++s) {
        mma8(g, aq[s], frag_load(Ks + (16 * nt + col) * LDR + 32 * s + 8 * grp));
        mma8(dp, ag[s], frag_load(Vs + (16 * nt + col) * LDR + 32 * s + 8 * grp));
      }
      const int j = 16 * nt + col;
      const float aj = As[j], oj = vone[j];
      float cp = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = r0 + 4 * grp + r;
        const float m = __expf(-fabsf(As[i] - aj));
        const float dpf = dp[r] + gd[r] * oj;
        const float P = g[r] * m, e = dpf * P;
        Pt[i * LDP + j] = from_f<T>(P);
        Dt[i * LDP + j] = from_f<T>(dpf * m);
        sgn[r] += j < i ? e : (j > i ? -e : 0.f);  // towards dA_i
        cp += i < j ? e : (i > j ? -e : 0.f);      // towards dA_j
      }
      cp = add_xor32(add_xor16(cp));
      if (grp == 0) colpart[w][j] = cp;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sgn[r] = row16_sum(sgn[r]);
    __syncthreads();  // Pt, Dt complete
    // the states of phase 2 load while this phase finishes
    image_rows_load<T, DH>(hreg[0], img, ext, tid);
    image_rows_load<T, DH>(hreg[1], img + DH * DH, ext + E, tid);

    f32x4 dq[FB];
    float inter[4] = {0.f, 0.f, 0.f, 0.f}, dot[4] = {0.f, 0.f, 0.f, 0.f}, later[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < FB; ++nt) {
      f32x4 in = zero4(), fw = zero4(), bw = zero4();
#pragma unroll
      for (int s = 0; s < C / 32; ++s)
        mma8(in, frag_load(Dt + (r0 + col) * LDP + 32 * s + 8 * grp),
             frag_kmajor<T>(Ks, LDR, 32 * s + 8 * grp, 16 * nt, lane));
#pragma unroll
      for (int s = 0; s < DH / 32; ++s) {
        mma8(fw, ag[s], frag_kmajor<T>(SFs, LDR, 32 * s + 8 * grp, 16 * nt, lane));
        mma8(bw, ag[s], frag_kmajor<T>(SBs, LDR, 32 * s + 8 * grp, 16 * nt, lane));
      }
      const float zf = xF[16 * nt + col], zb = xB[16 * nt + col];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = r0 + 4 * grp + r;
        const float f = ef[r] * (fw[r] + gd[r] * zf), b = eb[r] * (bw[r] + gd[r] * zb);
        dq[nt][r] = in[r] + f + b;
        const float p = to_f<T>(Qs[i * LDR + 16 * nt + col]);
        inter[r] += p * (f - b);
        later[r] += p * b;
        dot[r] += p * dq[nt][r];
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      inter[r] = row16_sum(inter[r]);
      later[r] = row16_sum(later[r]);
      dot[r] = row16_sum(dot[r]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = r0 + 4 * grp + r;
      const bool ok = ch.start + i < ch.end;
#pragma unroll
      for (int nt = 0; nt < FB; ++nt) dqo[nt][r] = dq[nt][r];  // the gradient of phi(q); its VJP runs at the output
      if (col == 0) {
        dAq[i] = ok ? sgn[r] + inter[r] : 0.f;
        Yq[i] = ok ? later[r] : 0.f;
        dotq[i] = dot[r];
      }
    }
  }
  __syncthreads();  // every wave is done with SF / SB

  // ---------------- phase 2: key rows j = r0 + 4 grp + r
  image_rows_store<T, DH>(hreg[0], SFs, LDR, xF, tid);
  image_rows_store<T, DH>(hreg[1], SBs, LDR, xB, tid);
  if (tid < C) dAk[tid] = (colpart[0][tid] + colpart[1][tid]) + (colpart[2][tid] + colpart[3][tid]);
  __syncthreads();
  float dko[FB][4];
  f32x4 dv[FB];
  {
    Frag8<T> ak[DH / 32], av[DH / 32];
#pragma unroll
    for (int s = 0; s < DH / 32; ++s) {
      ak[s] = frag_load(Ks + (r0 + col) * LDR + 32 * s + 8 * grp);
      av[s] = frag_load(Vs + (r0 + col) * LDR + 32 * s + 8 * grp);
    }
    float ef[4], eb[4], oj[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float a = As[r0 + 4 * grp + r];
      ef[r] = __expf(a);
      eb[r] = __expf(L - a);
      oj[r] = vone[r0 + 4 * grp + r];
    }
    f32x4 dk[FB];
    float inter[4] = {0.f, 0.f, 0.f, 0.f}, dot[4] = {0.f, 0.f, 0.f, 0.f}, later[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < FB; ++nt) {
      f32x4 ik = zero4(), iv = zero4(), fk = zero4(), bk = zero4(), fv = zero4(), bv = zero4();
#pragma unroll
      for (int s = 0; s < C / 32; ++s) {
        mma8(ik, frag_kmajor<T>(Dt, LDP, 32 * s + 8 * grp, r0, lane),
             frag_kmajor<T>(Qs, LDR, 32 * s + 8 * grp, 16 * nt, lane));
        mma8(iv, frag_kmajor<T>(Pt, LDP, 32 * s + 8 * grp, r0, lane),
             frag_kmajor<T>(Gs, LDR, 32 * s + 8 * grp, 16 * nt, lane));
      }
#pragma unroll
      for (int s = 0; s < DH / 32; ++s) {
        mma8(fk, av[s], frag_kmajor<T>(SFs, LDR, 32 * s + 8 * grp, 16 * nt, lane));
        mma8(bk, av[s], frag_kmajor<T>(SBs, LDR, 32 * s + 8 * grp, 16 * nt, lane));
        mma8(fv, ak[s], frag_load(SFs + (16 * nt + col) * LDR + 32 * s + 8 * grp));
        mma8(bv, ak[s], frag_load(SBs + (16 * nt + col) * LDR + 32 * s + 8 * grp));
      }
      const float hf = xF[16 * nt + col], hb = xB[16 * nt + col];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = r0 + 4 * grp + r;
        const float f = ef[r] * (fk[r] + oj[r] * hf), b = eb[r] * (bk[r] + oj[r] * hb);
        dk[nt][r] = ik[r] + f + b;
        dv[nt][r] = iv[r] + ef[r] * fv[r] + eb[r] * bv[r];
        const float p = to_f<T>(Ks[j * LDR + 16 * nt + col]);
        inter[r] += p * (f - b);
        later[r] += p * b;
        dot[r] += p * dk[nt][r];
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      inter[r] = row16_sum(inter[r]);
      later[r] = row16_sum(later[r]);
      dot[r] = row16_sum(dot[r]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = r0 + 4 * grp + r;
      const bool ok = ch.start + j < ch.end;
#pragma unroll
      for (int nt = 0; nt < FB; ++nt) dko[nt][r] = dk[nt][r];  // the gradient of phi(k); its VJP runs at the output
      if (col == 0) {
        dAk[j] = ok ? dAk[j] + inter[r] : 0.f;
        Yk[j] = ok ? later[r] : 0.f;
        dotk[j] = dot[r];
      }
    }
  }
  __syncthreads();  // every wave is done reading the tiles; reuse them for the outputs
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = r0 + 4 * grp + r;
#pragma unroll
    for (int nt = 0; nt < FB; ++nt) {
      dqf[i * DH + 16 * nt + col] = dqo[nt][r];
      dkf[i * DH + 16 * nt + col] = dko[nt][r];
      Vs[i * LDR + 16 * nt + col] = from_f<T>(dv[nt][r]);
    }
  }
  __syncthreads();

  // ---------------- outputs
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int it = tid + 256 * v;
    if (it >= C * V8) continue;
    const int r = it / V8, c = (it % V8) * 8, t = ch.start + r;
    if (t < ch.end) {
      // feature-map VJP of 8 features of row r: raw q and k as 16-byte vectors
      const size_t o = (size_t)t * D + h * DH + c;
      const Frag8<T> uq = frag_load(qr + o), uk = frag_load(kr + o);
      const Frag8<T> pq = frag_load(Qs + r * LDR + c), pk = frag_load(Ks + r * LDR + c);
      const float inq = fast_rcp(nq[r]), ink = fast_rcp(nk[r]), dtq = dotq[r], dtk = dotk[r];
      float oq[8], ok8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        oq[j] = phi_lion_vjp(frag_get(uq, j), frag_get(pq, j), inq, dqf[r * DH + c + j], dtq);
        ok8[j] = phi_lion_vjp(frag_get(uk, j), frag_get(pk, j), ink, dkf[r * DH + c + j], dtk);
      }
      T* g = G + (size_t)t * Kp + h * DH + c;
      frag_store(g, frag_from<T>(oq));
      frag_store(g + D, frag_from<T>(ok8));
      frag_store(g + 2 * D, frag_load(Vs + r * LDR + c));
    }
  }
  if (tid < C) {  // chunk-local suffix sums of dA, and the chunk's straddling sum Z'_c
    const bool ok = ch.start + tid < ch.end;
    float a = ok ? dAq[tid] + dAk[tid] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_down(a, off, 64);
      if (tid + off < 64) a += o;
    }
    if (ok) dA_loc[(size_t)(ch.start + tid) * H + h] = a;
    float y = Yq[tid] + Yk[tid];  // 0 past the chunk's end
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) y += __shfl_xor(y, off, 64);
    if (tid == 0)
      dA_tot[(size_t)slot * H + h] = y + __expf(L) * ((zpart[0] + zpart[1]) + (zpart[2] + zpart[3]));
  }
}

void launch_lion_bwd_token(int dt, int dh, const void* q, const void* k, const void* v, const float* logl,
                           const void* y, const void* dy, const float* rsum, const float* st, const float* hst,
                           const void* hrows, const int* nchunks, const Chunk* tab, int max_slots, int H, int Kp,
                           void* G, float* dA_loc, float* dA_tot, hipStream_t s) {
  const dim3 grid(xcd_grid(max_slots * H));
#define LION_BT(TT, DD) hipLaunchKernelGGL((k_lion_bwd_token<TT, DD>), grid, dim3(256), 0, s, (const TT*)q,         \
                                           (const TT*)k, (const TT*)v, logl, (const TT*)y, (const TT*)dy, rsum, st, \
                                           hst, (const TT*)hrows, nchunks, tab, max_slots, H, Kp, (TT*)G,   \
                                           dA_loc, dA_tot)
  if (dt == BF16) { if (dh == 64) LION_BT(bf16, 64); else LION_BT(bf16, 32); }
  else            { if (dh == 64) LION_BT(float, 64); else LION_BT(float, 32); }
#undef LION_BT
}

// ---------------------------------------------------------------- decay gradient
// dlog lambda_t = dA_loc[t] (the suffix of dA inside t's chunk) + Z'_c (the
// chunk's straddling sum, dA_tot[slot]); da_t = dlog lambda_t (1 - lambda_t)
// goes to G column 3 D + h when the decay depends on x (else 0). One block per
// chunk also zeroes the padding columns of G the dX~ GEMM reads and writes the
// chunk's per-head sum of da (db partial).
template <typename T>
__global__ __launch_bounds__(256) void k_lion_da(const float* __restrict__ logl, const float* __restrict__ dA_loc,
                                                 const float* __restrict__ dA_tot, const int* __restrict__ nchunks,
                                                 const Chunk* __restrict__ tab, int H, int D, int Kp,
                                                 int write_da, T* __restrict__ G, float* __restrict__ db_part) {
  constexpr int C = kLionChunk;
  const int slot = blockIdx.x;
  Chunk ch;
  if (!block_chunk(nchunks, tab, slot, ch)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t = ch.start + lane;
  const bool ok = t < ch.end;
  for (int h = w; h < H; h += 4) {  // lane = token of the chunk
    float da = 0.f;
    if (ok) {
      const float ll = logl[(size_t)t * H + h];
      da = (dA_loc[(size_t)t * H + h] + dA_tot[(size_t)slot * H + h]) * -expm1f(ll);
      G[(size_t)t * Kp + 3 * D + h] = from_f<T>(write_da ? da : 0.f);
    }
    float sum = da;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (lane == 0) db_part[(size_t)slot * H + h] = sum;
  }
  const int g0 = 3 * D + H, P = (g0 + 7) / 8 * 8 - g0;  // the padding columns of G the dX~ GEMM reads
  for (int e = tid; e < C * P; e += 256) {
    const int r = e / P, c = g0 + e % P;
    if (ch.start + r < ch.end) G[(size_t)(ch.start + r) * Kp + c] = from_f<T>(0.f);
  }
}

void launch_lion_da(const float* logl, const float* dA_loc, const float* dA_tot, const int* nchunks, const Chunk* tab,
                    int max_slots, int H, int D, int Kp, int dt, bool write_da, void* G, float* db_part,
                    hipStream_t s) {
  if (dt == BF16)
    hipLaunchKernelGGL(k_lion_da<bf16>, dim3(max_slots), dim3(256), 0, s, logl, dA_loc, dA_tot, nchunks, tab, H, D,
                       Kp, (int)write_da, (bf16*)G, db_part);
  else
    hipLaunchKernelGGL(k_lion_da<float>, dim3(max_slots), dim3(256), 0, s, logl, dA_loc, dA_tot, nchunks, tab, H, D,
                       Kp, (int)write_da, (float*)G, db_part);
}

}  // namespace gbla
