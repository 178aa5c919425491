// Pipelined MFMA GEMM main loops for gfx950 (wave64, 16x16 MFMA tiles).
//
// A block computes a BM x BN tile of C = A B^T with WGM x WGN waves, each wave a
// (BM/WGM) x (BN/WGN) sub-tile held in registers as 16x16 C tiles. k advances
// in chunks of BK elements staged in two LDS buffers: while the MFMAs consume
// one buffer, the next chunk is already in flight from global memory into
// registers and is written to the other buffer afterwards, so there is one
// barrier per chunk.
//
// Two loaders:
//  * NT: A [M][lda] and B [N][ldb] are both k-contiguous (row-major along k);
//    rows are copied to LDS as 16-byte vectors.
//  * TN: A [K][lda] and B [K][ldb] are both k-major (token-major, k = token);
//    the LDS tiles keep that layout and the MFMA operands are read with the
//    transposing LDS read (frag_kmajor), so no transposed stores are needed.
#pragma once
#include "common.h"

namespace gbla {

// k chunks held in flight in registers by the main loops
constexpr int kPrefetchDepth = 3;

template <typename T, int BM_, int BN_, int BK_, int WGM_, int WGN_>
struct GemmShape {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
  static constexpr int NWAVES = WGM * WGN;
  static constexpr int NTHREADS = NWAVES * 64;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static constexpr int LD = BK + 16 / (int)sizeof(T);  // LDS row pitch (elements), 16-byte pad
  static constexpr int STAGE = (BM + BN) * LD;           // elements per LDS buffer
  static constexpr size_t LDS_BYTES = 2 * (size_t)STAGE * sizeof(T);
  static_assert(BK % 32 == 0, "k chunk must hold whole 32-wide MFMA steps");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be whole 16x16 tiles");
};

// acc += A_lds[wave rows] * B_lds[wave cols]^T over one BK chunk
template <typename T, class S>
__device__ __forceinline__ void mma_chunk(const T* __restrict__ As, const T* __restrict__ Bs, int wm, int wn,
                                          int col, int grp, f32x4 (&acc)[S::FM][S::FN]) {
#pragma unroll
  for (int ks = 0; ks < S::BK; ks += 32) {
    Frag8<T> a[S::FM];
#pragma unroll
    for (int i = 0; i < S::FM; ++i) a[i] = frag_load(As + (wm * S::WTM + 16 * i + col) * S::LD + ks + 8 * grp);
#pragma unroll
    for (int j = 0; j < S::FN; ++j) {
      const Frag8<T> b = frag_load(Bs + (wn * S::WTN + 16 * j + col) * S::LD + ks + 8 * grp);
#pragma unroll
      for (int i = 0; i < S::FM; ++i) mma8(acc[i][j], a[i], b);
    }
  }
}

// ---------------------------------------------------------------- NT main loop
// A: rows [0, ma) of a BM-row panel (pitch lda), B: rows [0, nb) of a BN-row
// panel (pitch ldb); k in [0, K), K % 8 == 0. Rows past ma / nb and k past K
// read as zero.
template <typename T, class S>
__device__ __forceinline__ void gemm_nt_mainloop(const T* __restrict__ A, int lda, int ma, const T* __restrict__ B,
                                                 int ldb, int nb, int K, T* __restrict__ smem,
                                                 f32x4 (&acc)[S::FM][S::FN]) {
  constexpr int G8 = S::BK / 8;
  constexpr int VA = (S::BM * G8 + S::NTHREADS - 1) / S::NTHREADS;
  constexpr int VB = (S::BN * G8 + S::NTHREADS - 1) / S::NTHREADS;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int wm = w / S::WGN, wn = w % S::WGN;
#pragma unroll
  for (int i = 0; i < S::FM; ++i)
#pragma unroll
    for (int j = 0; j < S::FN; ++j) acc[i][j] = zero4();

  // PF register sets: the loads of chunk c + PF - 1 are in flight while chunk c
  // is multiplied, so each load has PF - 1 chunks of MFMA work to arrive.
  constexpr int PF = kPrefetchDepth;
  Frag8<T> ra[PF][VA], rb[PF][VB];
  auto fetch = [&](int set, int k0) {
#pragma unroll
    for (int v = 0; v < VA; ++v) {
      const int it = tid + v * S::NTHREADS;
      const int r = it / G8, c = k0 + (it % G8) * 8;
      ra[set][v] = (it < S::BM * G8 && r < ma && c < K) ? frag_load(A + (size_t)r * lda + c) : frag_zero<T>();
    }
#pragma unroll
    for (int v = 0; v < VB; ++v) {
      const int it = tid + v * S::NTHREADS;
      const int r = it / G8, c = k0 + (it % G8) * 8;
      rb[set][v] = (it < S::BN * G8 && r < nb && c < K) ? frag_load(B + (size_t)r * ldb + c) : frag_zero<T>();
    }
  };
  auto stash = [&](int set, T* buf) {
#pragma unroll
    for (int v = 0; v < VA; ++v) {
      const int it = tid + v * S::NTHREADS;
      if (it < S::BM * G8) frag_store(buf + (it / G8) * S::LD + (it % G8) * 8, ra[set][v]);
    }
#pragma unroll
    for (int v = 0; v < VB; ++v) {
      const int it = tid + v * S::NTHREADS;
      if (it < S::BN * G8) frag_store(buf + S::BM * S::LD + (it / G8) * S::LD + (it % G8) * 8, rb[set][v]);
    }
  };

  const int nk = (K + S::BK - 1) / S::BK;
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (p < nk) fetch(p, p * S::BK);
  stash(0, smem);
  __syncthreads();
  for (int c0 = 0; c0 < nk; c0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {  // chunk c = c0 + p lives in register set p
      const int c = c0 + p;
      if (c < nk) {
        if (c > 0 && c + PF - 1 < nk) fetch((p + PF - 1) % PF, (c + PF - 1) * S::BK);
        const T* buf = smem + (c & 1) * S::STAGE;
        mma_chunk<T, S>(buf, buf + S::BM * S::LD, wm, wn, col, grp, acc);
        if (c + 1 < nk) stash((p + 1) % PF, smem + ((c + 1) & 1) * S::STAGE);
        __syncthreads();
      }
    }
  }
}

// ---------------------------------------------------------------- TN main loop
// LDS tiles stay k-major (row = k): global rows are copied as 16-byte vectors
// and the MFMA operands are read k-contiguous per column with frag_kmajor.
template <typename T, int BM_, int BN_, int BK_, int WGM_, int WGN_>
struct GemmShapeTN {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
  static constexpr int NWAVES = WGM * WGN;
  static constexpr int NTHREADS = NWAVES * 64;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static constexpr int LDA = BM + 16 / (int)sizeof(T), LDB = BN + 16 / (int)sizeof(T);
  static constexpr int STAGE = BK * (LDA + LDB);
  static_assert(BK % 32 == 0, "k chunk must hold whole 32-wide MFMA steps");
};

// A: k rows [k_begin, k_end) of a k-major matrix, columns [0, ma) of a BM-wide
// panel (pitch lda); B likewise with nb valid columns (pitch ldb). ma, nb and
// the pitches are multiples of 8; columns past ma / nb and k past k_end read 0.
template <typename T, class S>
__device__ __forceinline__ void gemm_tn_mainloop(const T* __restrict__ A, int lda, int ma, const T* __restrict__ B,
                                                 int ldb, int nb, int k_begin, int k_end, T* __restrict__ smem,
                                                 f32x4 (&acc)[S::FM][S::FN]) {
  constexpr int CA = S::BM / 8, CB = S::BN / 8;  // 8-column vectors per k row
  constexpr int VA = (CA * S::BK + S::NTHREADS - 1) / S::NTHREADS;
  constexpr int VB = (CB * S::BK + S::NTHREADS - 1) / S::NTHREADS;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, grp = lane >> 4;
  const int wm = w / S::WGN, wn = w % S::WGN;
#pragma unroll
  for (int i = 0; i < S::FM; ++i)
#pragma unroll
    for (int j = 0; j < S::FN; ++j) acc[i][j] = zero4();

  constexpr int PF = kPrefetchDepth;
  Frag8<T> ra[PF][VA], rb[PF][VB];
  auto fetch = [&](int set, int k0) {
#pragma unroll
    for (int v = 0; v < VA; ++v) {
      const int it = tid + v * S::NTHREADS;
      const int kr = it / CA, c = (it % CA) * 8, k = k0 + kr;
      ra[set][v] = (it < CA * S::BK && c < ma && k < k_end) ? frag_load(A + (size_t)k * lda + c) : frag_zero<T>();
    }
#pragma unroll
    for (int v = 0; v < VB; ++v) {
      const int it = tid + v * S::NTHREADS;
      const int kr = it / CB, c = (it % CB) * 8, k = k0 + kr;
      rb[set][v] = (it < CB * S::BK && c < nb && k < k_end) ? frag_load(B + (size_t)k * ldb + c) : frag_zero<T>();
    }
  };
  auto stash = [&](int set, T* buf) {
#pragma unroll
    for (int v = 0; v < VA; ++v) {
      const int it = tid + v * S::NTHREADS;
      if (it < CA * S::BK) frag_store(buf + (it / CA) * S::LDA + (it % CA) * 8, ra[set][v]);
    }
#pragma unroll
    for (int v = 0; v < VB; ++v) {
      const int it = tid + v * S::NTHREADS;
      if (it < CB * S::BK) frag_store(buf + S::BK * S::LDA + (it / CB) * S::LDB + (it % CB) * 8, rb[set][v]);
    }
  };
  auto compute = [&](const T* buf) {
    const T* As = buf;
    const T* Bs = buf + S::BK * S::LDA;
#pragma unroll
    for (int ks = 0; ks < S::BK; ks += 32) {
      Frag8<T> a[S::FM];
#pragma unroll
      for (int i = 0; i < S::FM; ++i) a[i] = frag_kmajor<T>(As, S::LDA, ks + 8 * grp, wm * S::WTM + 16 * i, lane);
#pragma unroll
      for (int j = 0; j < S::FN; ++j) {
        const Frag8<T> b = frag_kmajor<T>(Bs, S::LDB, ks + 8 * grp, wn * S::WTN + 16 * j, lane);
#pragma unroll
        for (int i = 0; i < S::FM; ++i) mma8(acc[i][j], a[i], b);
      }
    }
  };

  if (k_begin >= k_end) return;
  const int nk = (k_end - k_begin + S::BK - 1) / S::BK;
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (p < nk) fetch(p, k_begin + p * S::BK);
  stash(0, smem);
  __syncthreads();
  for (int c0 = 0; c0 < nk; c0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {  // chunk c = c0 + p lives in register set p
      const int c = c0 + p;
      if (c < nk) {
        if (c > 0 && c + PF - 1 < nk) fetch((p + PF - 1) % PF, k_begin + (c + PF - 1) * S::BK);
        compute(smem + (c & 1) * S::STAGE);
        if (c + 1 < nk) stash((p + 1) % PF, smem + ((c + 1) & 1) * S::STAGE);
        __syncthreads();
      }
    }
  }
}

}  // namespace gbla
