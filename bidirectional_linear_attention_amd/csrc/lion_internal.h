// LION-s chunkwise kernels: launchers and device helpers shared by the forward and backward (internal).
#pragma once
#include "internal.h"

namespace gbla {

// tokens per chunk of the chunkwise LION-s evaluation (one per lane of a wave)
constexpr int kLionChunk = 64;

// ---------------------------------------------------------------- tile staging helpers
// Rows of 8-element vectors: thread it handles row it / V8, columns 8 (it % V8)
// .. + 7, and the V8 threads of one row are consecutive lanes.

// phi(u) = (SiLU(u) + 0.5) / ||SiLU(u) + 0.5||_2 of one row, given this thread's 8
// raw values; returns the row norm. `valid` rows produce zeros.
template <int V8>
__device__ __forceinline__ float phi_lion8(const float (&u)[8], float (&out)[8], bool valid) {
  float f[8], ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    f[j] = u[j] * sigmoidf_(u[j]) + 0.5f;
    ss += f[j] * f[j];
  }
  ss = lane_group_sum<V8>(ss);
  const float rn = fast_rsqrt(ss);  // ss > 0: SiLU(u) + 0.5 >= 0.22 for every u
  const float n = ss * rn;
  const float inv = valid ? rn : 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = f[j] * inv;
  return n;
}

// Log-decay of the chunk's tokens -> inclusive prefix A~ (LDS) and the chunk
// total L (LDS); tokens past the chunk end count as log lambda = 0. Split in
// two so that the load is issued at block start and its latency hides behind
// the tile loads: chunk_decay_load on every thread (wave 0 loads, the others
// get 0), chunk_decay_scan on every thread before the barrier that publishes
// the staged tiles (wave 0 scans and writes).
template <int C>
__device__ __forceinline__ float chunk_decay_load(const float* __restrict__ logl, const Chunk& ch, int H, int h,
                                                  int tid) {
  static_assert(C == 64, "one token per lane of wave 0");
  const int t = ch.start + tid;
  return tid < 64 && t < ch.end ? logl[(size_t)t * H + h] : 0.f;
}

template <int C>
__device__ __forceinline__ void chunk_decay_scan(float a, float* As, float* Ls, int tid) {
  if (tid < 64) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(a, off, 64);
      if (tid >= off) a += o;
    }
    As[tid] = a;
    if (tid == 63) *Ls = a;
  }
}

void launch_lion_chunk_state(int dt, int dh, int mode, const void* rsrc, const void* vsrc, const void* ysrc,
                             const float* rsum, const float* logl, const int* nchunks, const Chunk* tab,
                             int max_slots, int H, float* out, float* lam_out, hipStream_t s);
// rows: null (every element in place, fp32) or the row image of the scan (the
// dh x dh part rounded to the data type dt, [slot][H][2][dh^2])
void launch_lion_scan(float* st, const float* lam, const int* nchunks, const int* chunk_off, int N, int H, int E,
                      int dt, void* rows, int dh, hipStream_t s);
void launch_lion_readout(int dt, int dh, const void* q, const void* k, const void* v, const float* logl,
                         const float* st, const int* nchunks, const Chunk* tab, int max_slots, int H, void* y,
                         float* rsum, hipStream_t s);
void launch_lion_bwd_token(int dt, int dh, const void* q, const void* k, const void* v, const float* logl,
                           const void* y, const void* dy, const float* rsum, const float* st, const float* hst,
                           const void* hrows, const int* nchunks, const Chunk* tab, int max_slots, int H, int Kp,
                           void* G, float* dA_loc, float* dA_tot, hipStream_t s);
// da into G (and its zero padding) and per-chunk partial sums of da [slot][H]
// (sum them over the first *nchunks slots); dA_tot holds each chunk's straddling sum
void launch_lion_da(const float* logl, const float* dA_loc, const float* dA_tot, const int* nchunks, const Chunk* tab,
                    int max_slots, int H, int D, int Kp, int dt, bool write_da, void* G, float* db_part,
                    hipStream_t s);

}  // namespace gbla
