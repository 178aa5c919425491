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

// ---------------------------------------------------------------- NT main loop, direct-to-LDS (bf16)
// Same contract as gemm_nt_mainloop for bf16, built for gfx950:
//  * global -> LDS with buffer_load ... lds (16 bytes per lane, no register
//    round trip); rows past ma / nb and k past K read as zero through the
//    buffer range check (out-of-range lanes get an offset beyond the range);
//  * LDS rows are unpadded (BK bf16) and the 16-byte chunks of row r are
//    XOR-swizzled so that 16 lanes reading one chunk of 16 consecutive rows hit
//    16 distinct 4-bank groups;
//  * NS stages, one barrier per k chunk: wait for this wave's loads of chunk c,
//    barrier (every wave's loads of chunk c are in LDS and every wave is done
//    with chunk c - 1), issue the loads of chunk c + NS - 1 into the stage of
//    chunk c - 1, multiply chunk c. (A second barrier per chunk, to issue
//    before waiting, measured slower.)
template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int NS_>
struct DlShape {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_, NS = NS_;
  static constexpr int NWAVES = WGM * WGN, NTHREADS = NWAVES * 64;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN, FM = WTM / 16, FN = WTN / 16;
  static constexpr int CPR = BK / 8;        // 16-byte chunks per LDS row
  static constexpr int RPL = 64 / CPR;      // rows written by one 1 KB wave load
  static constexpr int LA = BM / RPL, LB = BN / RPL;
  // wave loads per wave per chunk; when they do not divide evenly, the last
  // waves issue one fewer (only with two stages, whose waits are vmcnt(0))
  static constexpr int LPW = (LA + LB + NWAVES - 1) / NWAVES;
  static constexpr bool EVEN = (LA + LB) % NWAVES == 0;
  static constexpr int STAGE = (BM + BN) * BK;    // bf16 elements per stage
  static_assert(BK == 32 || BK == 64, "16 or 8 rows per wave load");
  static_assert(BM % RPL == 0 && BN % RPL == 0, "whole wave loads");
  static_assert(EVEN || NS_ == 2, "uneven wave loads need the two-stage pipeline");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0 && NS >= 2 && NS <= 4, "tile shape");
  static_assert(LPW * (NS - 1) < 64, "vmcnt range");
};

// physical 16-byte chunk of logical chunk c in LDS row r (CPR chunks per row)
template <int CPR>
__device__ __forceinline__ int dl_swizzle(int r, int c) { return c ^ ((r / (16 / CPR)) % CPR); }

// s_waitcnt immediate that waits until at most n vector-memory operations are outstanding
__host__ __device__ constexpr int dl_vmcnt(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

typedef __attribute__((address_space(3))) void dl_lds_void;

// st[s] are NS distinct LDS arrays of S::STAGE elements (distinct objects let the
// compiler tell the stages apart when it orders LDS reads after LDS-DMA loads)
template <class S>
__device__ __forceinline__ void gemm_nt_dl(const bf16* __restrict__ A, int lda, int ma, const bf16* __restrict__ B,
                                           int ldb, int nb, int K, bf16* st0, bf16* st1, bf16* st2, bf16* st3,
                                           f32x4 (&acc)[S::FM][S::FN]) {
  constexpr int CPR = S::CPR, RPL = S::RPL, NS = S::NS;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w / S::WGN, wn = w % S::WGN;
#pragma unroll
  for (int i = 0; i < S::FM; ++i)
#pragma unroll
    for (int j = 0; j < S::FN; ++j) acc[i][j] = zero4();

  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, ma > 0 ? (ma - 1) * lda * 2 + K * 2 : 0, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void*)B, 0, nb > 0 ? (nb - 1) * ldb * 2 + K * 2 : 0, kBufferRsrcWord3);
  const int rr = lane / CPR, pp = lane % CPR;  // this lane's row in a wave load and physical chunk
  auto stage = [&](int s) -> bf16* { return s == 0 ? st0 : (s == 1 ? st1 : (s == 2 ? st2 : st3)); };
  auto issue = [&](int s, int k0) {
    bf16* base = stage(s);
#pragma unroll
    for (int j = 0; j < S::LPW; ++j) {
      const int li = w + S::NWAVES * j;  // wave-uniform
      if (!S::EVEN && li >= S::LA + S::LB) break;
      const bool isA = li < S::LA;
      const int r = (isA ? li : li - S::LA) * RPL + rr;
      const int c = dl_swizzle<CPR>(r, pp);
      const int k = k0 + 8 * c;
      const int ld = isA ? lda : ldb, rows = isA ? ma : nb;
      const unsigned off = (r < rows && k < K) ? (unsigned)(r * ld + k) * 2u : 0x80000000u;
      bf16* dst = base + (isA ? li * RPL * S::BK : S::BM * S::BK + (li - S::LA) * RPL * S::BK);
      if (isA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (dl_lds_void*)dst, 16, off, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (dl_lds_void*)dst, 16, off, 0, 0, 0);
    }
  };
  auto compute = [&](const bf16* buf) {
    const bf16* As = buf;
    const bf16* Bs = buf + S::BM * S::BK;
#pragma unroll
    for (int ks = 0; ks < S::BK / 32; ++ks) {
      Frag8<bf16> a[S::FM];
#pragma unroll
      for (int i = 0; i < S::FM; ++i) {
        const int r = wm * S::WTM + 16 * i + col;
        a[i] = frag_load(As + r * S::BK + 8 * dl_swizzle<CPR>(r, 4 * ks + grp));
      }
#pragma unroll
      for (int j = 0; j < S::FN; ++j) {
        const int r = wn * S::WTN + 16 * j + col;
        const Frag8<bf16> b = frag_load(Bs + r * S::BK + 8 * dl_swizzle<CPR>(r, 4 * ks + grp));
#pragma unroll
        for (int i = 0; i < S::FM; ++i) mma8(acc[i][j], a[i], b);
      }
    }
  };

  const int nk = (K + S::BK - 1) / S::BK;
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)  // chunks 0 .. NS - 2 in flight before the loop
    if (p < nk) issue(p, p * S::BK);
  for (int c = 0; c < nk; ++c) {
    if (c + NS - 2 < nk)
      __builtin_amdgcn_s_waitcnt(dl_vmcnt(S::LPW * (NS - 2)));  // this wave's loads of chunk c are done
    else
      __builtin_amdgcn_s_waitcnt(dl_vmcnt(0));
    __syncthreads();  // every wave's loads of chunk c are in LDS and every wave is done with chunk c - 1
    if (c + NS - 1 < nk) issue((c + NS - 1) % NS, (c + NS - 1) * S::BK);
    compute(stage(c % NS));
  }
  __syncthreads();  // the stages may be reused by the caller
}

// ---------------------------------------------------------------- persistent NT loop, direct-to-LDS (bf16)
// Operands of one work item (one C tile) of a persistent NT GEMM: A rows
// [0, ma) and B rows [0, nb), k in [0, K); the pitches are fixed per launch.
struct DlItem {
  const bf16* A;
  const bf16* B;
  int ma, nb;
};

// One block per CU walks its work items in order (item(i, it) fills `it` and
// returns false past the block's last item). The two-stage k-chunk pipeline of
// gemm_nt_dl runs on across items: the first chunk of the next item is loaded
// while the last chunk of the current one is multiplied and while the
// epilogue's stores leave, so a tile pays no pipeline fill. Chunks go in pairs,
// the first of a pair to st0, the second to st1: with compile-time stages the
// wait-count pass sees that the loads in flight into one stage do not alias the
// reads of the other. K % (2 BK) == 0 and K <= lda, ldb: a lane's offset within
// a chunk is the same for every item and chunk (the chunk's k goes in the
// scalar offset), and rows past ma / nb fall outside the buffer range and read
// as zero. The epilogue, epi(i, acc), must issue exactly NST vector-memory
// instructions per wave (buffer stores, whose range check drops what falls
// outside): the wait for the next item's first chunk lets those NST complete later.
template <class S, int NST, class ItemFn, class Epi>
__device__ __forceinline__ void gemm_nt_dl_persistent(int K, int lda, int ldb, ItemFn item, Epi epi, bf16* st0,
                                                      bf16* st1) {
  static_assert(S::NS == 2, "two stages");
  static_assert(NST < 64, "vmcnt range");
  static_assert(S::LA % S::NWAVES == 0 && S::LB % S::NWAVES == 0, "whole wave loads of A and of B per wave");
  constexpr int CPR = S::CPR, RPL = S::RPL, JA = S::LA / S::NWAVES, JB = S::LB / S::NWAVES;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w / S::WGN, wn = w % S::WGN;
  unsigned offa[JA], offb[JB];  // this lane's byte offset in wave load j of a chunk at k = 0
#pragma unroll
  for (int j = 0; j < JA; ++j) {
    const int r = (w + S::NWAVES * j) * RPL + lane / CPR;
    offa[j] = (unsigned)(r * lda + 8 * dl_swizzle<CPR>(r, lane % CPR)) * 2u;
  }
#pragma unroll
  for (int j = 0; j < JB; ++j) {
    const int r = (w + S::NWAVES * j) * RPL + lane / CPR;
    offb[j] = (unsigned)(r * ldb + 8 * dl_swizzle<CPR>(r, lane % CPR)) * 2u;
  }
  auto issue = [&](const DlItem& it, bf16* base, int k0) {
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void*)it.A, 0, it.ma * lda * 2, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)it.B, 0, it.nb * ldb * 2, kBufferRsrcWord3);
#pragma unroll
    for (int j = 0; j < JA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (dl_lds_void*)(base + (w + S::NWAVES * j) * RPL * S::BK), 16,
                                               offa[j], 2 * k0, 0, 0);
#pragma unroll
    for (int j = 0; j < JB; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (dl_lds_void*)(base + S::BM * S::BK + (w + S::NWAVES * j) * RPL * S::BK), 16, offb[j], 2 * k0, 0, 0);
  };
  f32x4 acc[S::FM][S::FN];
  auto compute = [&](const bf16* buf) {
    const bf16* As = buf;
    const bf16* Bs = buf + S::BM * S::BK;
#pragma unroll
    for (int ks = 0; ks < S::BK / 32; ++ks) {
      Frag8<bf16> a[S::FM];
#pragma unroll
      for (int i = 0; i < S::FM; ++i) {
        const int r = wm * S::WTM + 16 * i + col;
        a[i] = frag_load(As + r * S::BK + 8 * dl_swizzle<CPR>(r, 4 * ks + grp));
      }
#pragma unroll
      for (int j = 0; j < S::FN; ++j) {
        const int r = wn * S::WTN + 16 * j + col;
        const Frag8<bf16> b = frag_load(Bs + r * S::BK + 8 * dl_swizzle<CPR>(r, 4 * ks + grp));
#pragma unroll
        for (int i = 0; i < S::FM; ++i) mma8(acc[i][j], a[i], b);
      }
    }
  };

  const int nk = K / S::BK;
  DlItem cur, nxt;
  if (nk == 0 || !item(0, cur)) return;
  issue(cur, st0, 0);
  __builtin_amdgcn_s_waitcnt(dl_vmcnt(0));
  __syncthreads();
  for (int i = 0;; ++i) {
    const bool more = item(i + 1, nxt);
#pragma unroll
    for (int a = 0; a < S::FM; ++a)
#pragma unroll
      for (int b = 0; b < S::FN; ++b) acc[a][b] = zero4();
    for (int c = 0; c < nk; c += 2) {
      if (c > 0) {
        __builtin_amdgcn_s_waitcnt(dl_vmcnt(0));  // this wave's loads of chunk c are done
        __syncthreads();  // every wave's loads of chunk c are in LDS; every wave is done with chunk c - 1
      }
      issue(cur, st1, (c + 1) * S::BK);
      __builtin_amdgcn_sched_barrier(0);  // the loads leave before the multiplies, not after them
      compute(st0);
      __builtin_amdgcn_sched_barrier(0);  // and the multiplies stay ahead of the wait
      __builtin_amdgcn_s_waitcnt(dl_vmcnt(0));
      __syncthreads();
      if (c + 2 < nk)
        issue(cur, st0, (c + 2) * S::BK);
      else if (more)
        issue(nxt, st0, 0);
      __builtin_amdgcn_sched_barrier(0);
      compute(st1);
      __builtin_amdgcn_sched_barrier(0);
    }
    epi(i, acc);
    if (!more) break;
    cur = nxt;
    // the next item's first chunk is in: behind its loads only this item's NST stores may be in flight
    __builtin_amdgcn_s_waitcnt(dl_vmcnt(NST));
    __syncthreads();
  }
}

// ---------------------------------------------------------------- TN main loop, direct-to-LDS (bf16)
// Same contract as gemm_tn_mainloop for bf16: A [K][lda] and B [K][ldb] are
// k-major (token-major). LDS tiles keep that layout (row = k, BM or BN columns,
// unpadded) and the MFMA operands are read with the transposing LDS read. A
// transposing read fetches, per 16-lane group, 4 rows x 32 bytes; the 16-byte
// chunk q of row r is stored at chunk q ^ 2 g(r), g(r) = (r & 3) | ((r >> 1) & 4),
// so the 8 rows r and r + 8 read by two groups land in 16 distinct bank groups.
template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int NS_>
struct DlShapeTN {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_, NS = NS_;
  static constexpr int NWAVES = WGM * WGN, NTHREADS = NWAVES * 64;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN, FM = WTM / 16, FN = WTN / 16;
  static constexpr int CA = BM / 8, CB = BN / 8;          // 16-byte chunks per k row
  static constexpr int LA = BK * CA / 64, LB = BK * CB / 64;  // 1 KB wave loads per stage
  static constexpr int LPW = (LA + LB) / NWAVES;
  static constexpr int STAGE = BK * (BM + BN);
  static_assert(CA % 16 == 0 && CB % 16 == 0, "the swizzle permutes chunks within groups of 16");
  static_assert((BK * CA) % 64 == 0 && (BK * CB) % 64 == 0 && (LA + LB) % NWAVES == 0, "whole wave loads");
  static_assert(BK % 32 == 0 && WTM % 16 == 0 && WTN % 16 == 0 && NS >= 2 && NS <= 4, "tile shape");
  static_assert(LPW * (NS - 1) < 64, "vmcnt range");
};

__device__ __forceinline__ int dl_tn_swizzle(int r, int q) { return q ^ (2 * ((r & 3) | ((r >> 1) & 4))); }

// k-major operand (8 consecutive k of column cb + lane % 16) from a swizzled tile of W columns
template <int W>
__device__ __forceinline__ Frag8<bf16> frag_kmajor_swz(const bf16* tile, int kb, int cb, int lane) {
  const int j = lane & 15;
  uint2 part[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = kb + 4 * h + (j >> 2), c = cb + 4 * (j & 3);
    const bf16* p = tile + r * W + 8 * dl_tn_swizzle(r, c >> 3) + (c & 7);
    part[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_tr*)p));
  }
  Frag8<bf16> f;
  f.v = make_uint4(part[0].x, part[0].y, part[1].x, part[1].y);
  return f;
}

template <class S>
__device__ __forceinline__ void gemm_tn_dl(const bf16* __restrict__ A, int lda, int ma, const bf16* __restrict__ B,
                                           int ldb, int nb, int k_begin, int k_end, bf16* st0, bf16* st1, bf16* st2,
                                           bf16* st3, f32x4 (&acc)[S::FM][S::FN]) {
  constexpr int NS = S::NS;
  const int lane = threadIdx.x & 63, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w / S::WGN, wn = w % S::WGN;
#pragma unroll
  for (int i = 0; i < S::FM; ++i)
#pragma unroll
    for (int j = 0; j < S::FN; ++j) acc[i][j] = zero4();
  if (k_begin >= k_end) return;

  // the ranges cover rows k_begin .. k_end - 1 of each operand, columns 0 .. ma (nb) - 1
  const bf16* A0 = A + (size_t)k_begin * lda;
  const bf16* B0 = B + (size_t)k_begin * ldb;
  const int kn = k_end - k_begin;
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)A0, 0, ((kn - 1) * lda + ma) * 2, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void*)B0, 0, ((kn - 1) * ldb + nb) * 2, kBufferRsrcWord3);
  auto stage = [&](int s) -> bf16* { return s == 0 ? st0 : (s == 1 ? st1 : (s == 2 ? st2 : st3)); };
  auto issue = [&](int s, int k0) {  // k0 relative to k_begin
    bf16* base = stage(s);
#pragma unroll
    for (int j = 0; j < S::LPW; ++j) {
      const int li = w + S::NWAVES * j;  // wave-uniform
      const bool isA = li < S::LA;
      const int C = isA ? S::CA : S::CB;   // chunks per row
      const int e = (isA ? li : li - S::LA) * 64 + lane;  // chunk slot in the operand's stage tile
      const int r = e / C, p = e % C;      // k row and physical chunk
      const int q = dl_tn_swizzle(r, p);   // logical chunk held there
      const int k = k0 + r, col = 8 * q;
      const int ld = isA ? lda : ldb, cols = isA ? ma : nb;
      const unsigned off = (k < kn && col < cols) ? (unsigned)(k * ld + col) * 2u : 0x80000000u;
      bf16* dst = base + (isA ? li * 512 : S::BK * S::BM + (li - S::LA) * 512);
      if (isA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (dl_lds_void*)dst, 16, off, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (dl_lds_void*)dst, 16, off, 0, 0, 0);
    }
  };
  auto compute = [&](const bf16* buf) {
    const bf16* As = buf;
    const bf16* Bs = buf + S::BK * S::BM;
#pragma unroll
    for (int ks = 0; ks < S::BK; ks += 32) {
      Frag8<bf16> a[S::FM];
#pragma unroll
      for (int i = 0; i < S::FM; ++i) a[i] = frag_kmajor_swz<S::BM>(As, ks + 8 * grp, wm * S::WTM + 16 * i, lane);
#pragma unroll
      for (int j = 0; j < S::FN; ++j) {
        const Frag8<bf16> b = frag_kmajor_swz<S::BN>(Bs, ks + 8 * grp, wn * S::WTN + 16 * j, lane);
#pragma unroll
        for (int i = 0; i < S::FM; ++i) mma8(acc[i][j], a[i], b);
      }
    }
  };

  const int nk = (kn + S::BK - 1) / S::BK;
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < nk) issue(p, p * S::BK);
  for (int c = 0; c < nk; ++c) {
    if (c + NS - 2 < nk)
      __builtin_amdgcn_s_waitcnt(dl_vmcnt(S::LPW * (NS - 2)));
    else
      __builtin_amdgcn_s_waitcnt(dl_vmcnt(0));
    __syncthreads();
    if (c + NS - 1 < nk) issue((c + NS - 1) % NS, (c + NS - 1) * S::BK);
    compute(stage(c % NS));
  }
  __syncthreads();
}

}  // namespace gbla
