// Device-side building blocks shared by the GBLA and LION-s kernels (gfx950).
//
// Conventions used by every kernel in this library:
//  * activations and weights are stored either as float or as bfloat16 (the
//    raw 16-bit pattern in a uint16_t); accumulation is always float;
//  * MFMA lane layouts (wave64, 16x16 output tiles):
//      - an A operand supplies row  i = lane % 16, a B operand column j = lane % 16;
//      - each lane supplies the same set of k indices for A and B, so any
//        consistent assignment of k to (lane / 16, element) gives the same sum;
//      - the output tile C holds C[4 * (lane / 16) + r][lane % 16] in element r.
//    A C tile can therefore be fed back as a K=16 operand (k = 4 * (lane / 16) + r)
//    without moving data between lanes ("C-reuse"), which is how token-axis
//    contractions are done on values already held in registers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gbla {

typedef uint16_t bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_v;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_v;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(bf16 v) { return __uint_as_float(((uint32_t)v) << 16); }

typedef float f32x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// float -> bfloat16, round to nearest even (the gfx950 conversion instruction)
__device__ __forceinline__ bf16 f2bf(float f) { return __builtin_bit_cast(bf16, (__bf16)f); }
// two floats -> a packed bfloat16 pair, a in the low half (one instruction)
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  const f32x2_v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

// hardware reciprocal and reciprocal square root (about 1 ulp): used where a
// result is normalised or squashed, never where a value is accumulated
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16>(bf16 v) { return bf2f(v); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return f2bf(v); }

// round a float to the storage precision of T, returned as float
template <typename T> __device__ __forceinline__ float round_to(float v) { return to_f<T>(from_f<T>(v)); }

// ---------------------------------------------------------------- 8-element fragments
// Eight consecutive elements of one row along k: the per-lane MFMA operand for
// a 32-wide k step (one 16x16x32 bf16 MFMA, or eight 16x16x4 f32 MFMAs).
template <typename T> struct Frag8;
template <> struct Frag8<bf16> { uint4 v; };
template <> struct Frag8<float> { float4 lo, hi; };

template <typename T> __device__ __forceinline__ Frag8<T> frag_zero();
template <> __device__ __forceinline__ Frag8<bf16> frag_zero<bf16>() { Frag8<bf16> f; f.v = make_uint4(0, 0, 0, 0); return f; }
template <> __device__ __forceinline__ Frag8<float> frag_zero<float>() {
  Frag8<float> f; f.lo = make_float4(0.f, 0.f, 0.f, 0.f); f.hi = f.lo; return f;
}

template <typename T> __device__ __forceinline__ Frag8<T> frag_load(const T* p);
template <> __device__ __forceinline__ Frag8<bf16> frag_load<bf16>(const bf16* p) {
  Frag8<bf16> f; f.v = *reinterpret_cast<const uint4*>(p); return f;
}
template <> __device__ __forceinline__ Frag8<float> frag_load<float>(const float* p) {
  Frag8<float> f; f.lo = reinterpret_cast<const float4*>(p)[0]; f.hi = reinterpret_cast<const float4*>(p)[1]; return f;
}
template <typename T> __device__ __forceinline__ void frag_store(T* p, const Frag8<T>& f);
template <> __device__ __forceinline__ void frag_store<bf16>(bf16* p, const Frag8<bf16>& f) {
  *reinterpret_cast<uint4*>(p) = f.v;
}
template <> __device__ __forceinline__ void frag_store<float>(float* p, const Frag8<float>& f) {
  reinterpret_cast<float4*>(p)[0] = f.lo; reinterpret_cast<float4*>(p)[1] = f.hi;
}

// Rows [0, n) of a row-major array (pitch ld elements), `width` elements of each
// from `base` on, seen through a buffer resource: a fragment load from a row at
// or past n returns zeros and a store there is dropped. Tile loops use it so that
// no branch surrounds their memory operations: around a branch the compiler's
// wait-count pass loses track of the loads in flight and waits for all of them
// at the next use, which leaves one tile in flight instead of two. Offsets are
// 32-bit (n * ld * sizeof(T) < 2^31); width % 8 == 0.
constexpr int kBufferRsrcWord3 = 0x00020000;
template <typename T> struct RowBuf {
  __amdgpu_buffer_rsrc_t r;
  int ld;
  __device__ __forceinline__ RowBuf(const T* base, int n, int ld_, int width) : ld(ld_) {
    r = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), 0,
                                          n > 0 ? ((n - 1) * ld_ + width) * (int)sizeof(T) : 0, kBufferRsrcWord3);
  }
  __device__ __forceinline__ Frag8<T> load(int row, int col) const;
  __device__ __forceinline__ void store(int row, int col, const Frag8<T>& f) const;
};
template <> __device__ __forceinline__ Frag8<bf16> RowBuf<bf16>::load(int row, int col) const {
  Frag8<bf16> f;
  f.v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (row * ld + col) * 2, 0, 0));
  return f;
}
template <> __device__ __forceinline__ Frag8<float> RowBuf<float>::load(int row, int col) const {
  const int o = (row * ld + col) * 4;
  Frag8<float> f;
  f.lo = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
  f.hi = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, o + 16, 0, 0));
  return f;
}
template <> __device__ __forceinline__ void RowBuf<bf16>::store(int row, int col, const Frag8<bf16>& f) const {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f.v), r, (row * ld + col) * 2, 0, 0);
}
template <> __device__ __forceinline__ void RowBuf<float>::store(int row, int col, const Frag8<float>& f) const {
  const int o = (row * ld + col) * 4;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f.lo), r, o, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f.hi), r, o + 16, 0, 0);
}

// element access of a fragment as float
__device__ __forceinline__ float frag_get(const Frag8<float>& f, int j) {
  const float* p = reinterpret_cast<const float*>(&f);
  return p[j];
}
__device__ __forceinline__ float frag_get(const Frag8<bf16>& f, int j) {
  const bf16* p = reinterpret_cast<const bf16*>(&f.v);
  return bf2f(p[j]);
}

// build a fragment from 8 floats (rounded to T)
template <typename T> __device__ __forceinline__ Frag8<T> frag_from(const float* v);
template <> __device__ __forceinline__ Frag8<float> frag_from<float>(const float* v) {
  Frag8<float> f; f.lo = make_float4(v[0], v[1], v[2], v[3]); f.hi = make_float4(v[4], v[5], v[6], v[7]); return f;
}
template <> __device__ __forceinline__ Frag8<bf16> frag_from<bf16>(const float* v) {
  Frag8<bf16> f;
  f.v = make_uint4(f2bf2(v[0], v[1]), f2bf2(v[2], v[3]), f2bf2(v[4], v[5]), f2bf2(v[6], v[7]));
  return f;
}

// acc += A(16x32) * B(32x16); a, b: this lane's 8 k-elements
__device__ __forceinline__ void mma8(f32x4& acc, const Frag8<bf16>& a, const Frag8<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a.v), __builtin_bit_cast(bf16x8_v, b.v),
                                                acc, 0, 0, 0);
}
__device__ __forceinline__ void mma8(f32x4& acc, const Frag8<float>& a, const Frag8<float>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
}

// acc += A(16x16) * B(16x16) with this lane's 4 k-elements given as floats
// (rounded to T first). Used with C-reuse operands: k = 4 * (lane / 16) + j.
template <typename T> __device__ __forceinline__ void mma4(f32x4& acc, const float* a, const float* b);
template <> __device__ __forceinline__ void mma4<bf16>(f32x4& acc, const float* a, const float* b) {
  const uint2 ap = make_uint2(f2bf2(a[0], a[1]), f2bf2(a[2], a[3]));
  const uint2 bp = make_uint2(f2bf2(b[0], b[1]), f2bf2(b[2], b[3]));
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_v, ap), __builtin_bit_cast(s16x4_v, bp),
                                                  acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mma4<float>(f32x4& acc, const float* a, const float* b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

// ---------------------------------------------------------------- k-major LDS operands
// tile is a k-major LDS tile (row = k, column = m or n; pitch ld elements).
// Lane (g = lane / 16, i = lane % 16) receives tile[kb + m][cb + i] for
// m = 0..3, where kb may differ between the four 16-lane groups.
//
// For 16-bit data this is one ds_read_b64_tr_b16: within each group of 16
// lanes, lane j addresses the 4 elements tile[kb + j/4][cb + 4(j%4) .. +3] and
// the hardware hands lane i the element (m, i%4) of the row loaded by lane
// 4m + i/4, i.e. tile[kb + m][cb + i]. ld and cb must be multiples of 4.
typedef short s16x4_tr __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_tr lds_s16x4_tr;

__device__ __forceinline__ uint2 tr_read4(const bf16* tile, int ld, int kb, int cb, int lane) {
  const int j = lane & 15;
  const bf16* p = tile + (kb + (j >> 2)) * ld + cb + 4 * (j & 3);
  const s16x4_tr r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_tr*)p);
  return __builtin_bit_cast(uint2, r);
}

// eight k values kb..kb+7 of column cb + lane % 16 as an MFMA fragment
template <typename T> __device__ __forceinline__ Frag8<T> frag_kmajor(const T* tile, int ld, int kb, int cb, int lane);
template <> __device__ __forceinline__ Frag8<bf16> frag_kmajor<bf16>(const bf16* tile, int ld, int kb, int cb,
                                                                    int lane) {
  const uint2 lo = tr_read4(tile, ld, kb, cb, lane), hi = tr_read4(tile, ld, kb + 4, cb, lane);
  Frag8<bf16> f;
  f.v = make_uint4(lo.x, lo.y, hi.x, hi.y);
  return f;
}
template <> __device__ __forceinline__ Frag8<float> frag_kmajor<float>(const float* tile, int ld, int kb, int cb,
                                                                      int lane) {
  const float* p = tile + kb * ld + cb + (lane & 15);
  Frag8<float> f;
  f.lo = make_float4(p[0], p[ld], p[2 * ld], p[3 * ld]);
  f.hi = make_float4(p[4 * ld], p[5 * ld], p[6 * ld], p[7 * ld]);
  return f;
}

// The same eight k values per lane as frag_kmajor for a 32-wide k step starting
// at row k0, assigned so that 16-lane group g reads rows k0 + 4 g .. k0 + 4 g + 3
// and k0 + 16 + 4 g .. k0 + 16 + 4 g + 3: each transposing read of the four
// groups then covers 16 consecutive rows, which row pitches of 40 or 72 dwords
// keep free of LDS bank conflicts (with rows k0 + 8 g .. as in frag_kmajor two
// groups always share banks). Both operands of an MFMA must use the same form.
template <typename T> __device__ __forceinline__ Frag8<T> frag_kmajor_4g(const T* tile, int ld, int k0, int cb, int lane);
template <> __device__ __forceinline__ Frag8<bf16> frag_kmajor_4g<bf16>(const bf16* tile, int ld, int k0, int cb,
                                                                        int lane) {
  const int g = lane >> 4;
  const uint2 lo = tr_read4(tile, ld, k0 + 4 * g, cb, lane), hi = tr_read4(tile, ld, k0 + 16 + 4 * g, cb, lane);
  Frag8<bf16> f;
  f.v = make_uint4(lo.x, lo.y, hi.x, hi.y);
  return f;
}
template <> __device__ __forceinline__ Frag8<float> frag_kmajor_4g<float>(const float* tile, int ld, int k0, int cb,
                                                                          int lane) {
  const float* p = tile + (k0 + 4 * (lane >> 4)) * ld + cb + (lane & 15);
  Frag8<float> f;
  f.lo = make_float4(p[0], p[ld], p[2 * ld], p[3 * ld]);
  f.hi = make_float4(p[16 * ld], p[17 * ld], p[18 * ld], p[19 * ld]);
  return f;
}

// ---------------------------------------------------------------- 4-element quads (K = 16 MFMA operands)
// Four consecutive k elements of one lane for a 16x16x16 MFMA (bf16: one 8-byte
// register pair; float: four 16x16x4 MFMAs). With the C-reuse assignment
// k = 4 * (lane / 16) + m, the 4 values a lane holds in a 16x16 C tile form
// a quad, so a C tile feeds the next contraction without leaving registers.
template <typename T> struct Quad;
template <> struct Quad<bf16> { uint2 v; };
template <> struct Quad<float> { float4 v; };

template <typename T> __device__ __forceinline__ Quad<T> quad_from4(const float* f);
template <> __device__ __forceinline__ Quad<bf16> quad_from4<bf16>(const float* f) {
  Quad<bf16> q; q.v = make_uint2(f2bf2(f[0], f[1]), f2bf2(f[2], f[3])); return q;
}
template <> __device__ __forceinline__ Quad<float> quad_from4<float>(const float* f) {
  Quad<float> q; q.v = make_float4(f[0], f[1], f[2], f[3]); return q;
}
__device__ __forceinline__ float quad_get(const Quad<float>& q, int m) { return reinterpret_cast<const float*>(&q.v)[m]; }
__device__ __forceinline__ float quad_get(const Quad<bf16>& q, int m) {
  return bf2f(reinterpret_cast<const bf16*>(&q.v)[m]);
}
// 4 consecutive elements at p (8-byte aligned for bf16, 16-byte for float)
template <typename T> __device__ __forceinline__ Quad<T> quad_load(const T* p);
template <> __device__ __forceinline__ Quad<bf16> quad_load<bf16>(const bf16* p) {
  Quad<bf16> q; q.v = *reinterpret_cast<const uint2*>(p); return q;
}
template <> __device__ __forceinline__ Quad<float> quad_load<float>(const float* p) {
  Quad<float> q; q.v = *reinterpret_cast<const float4*>(p); return q;
}
template <typename T> __device__ __forceinline__ void quad_store(T* p, const Quad<T>& q);
template <> __device__ __forceinline__ void quad_store<bf16>(bf16* p, const Quad<bf16>& q) {
  *reinterpret_cast<uint2*>(p) = q.v;
}
template <> __device__ __forceinline__ void quad_store<float>(float* p, const Quad<float>& q) {
  *reinterpret_cast<float4*>(p) = q.v;
}
// One float per row (pitch ld floats) of rows [0, n) from base, through a
// buffer resource: rows at or past n read as 0.
struct RowScalar {
  __amdgpu_buffer_rsrc_t r;
  int ld;
  __device__ __forceinline__ RowScalar(const float* base, int n, int ld_) : ld(ld_) {
    r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, n > 0 ? ((n - 1) * ld_ + 1) * 4 : 0,
                                          kBufferRsrcWord3);
  }
  __device__ __forceinline__ float load(int row) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, row * ld * 4, 0, 0));
  }
};
// acc += A(16x16) B(16x16) with this lane's quads of A (row lane % 16) and B (column lane % 16)
__device__ __forceinline__ void mma_q(f32x4& acc, const Quad<bf16>& a, const Quad<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_v, a.v), __builtin_bit_cast(s16x4_v, b.v),
                                                  acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_q(f32x4& acc, const Quad<float>& a, const Quad<float>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.x, b.v.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.y, b.v.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.z, b.v.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.w, b.v.w, acc, 0, 0, 0);
}

// k-major quad: lane (g = lane / 16, i = lane % 16) receives tile[kb + m][cb + i], m = 0..3
// (kb may differ between the groups; bf16: one transposing LDS read)
template <typename T> __device__ __forceinline__ Quad<T> quad_kmajor(const T* tile, int ld, int kb, int cb, int lane);
template <> __device__ __forceinline__ Quad<bf16> quad_kmajor<bf16>(const bf16* tile, int ld, int kb, int cb, int lane) {
  Quad<bf16> q; q.v = tr_read4(tile, ld, kb, cb, lane); return q;
}
template <> __device__ __forceinline__ Quad<float> quad_kmajor<float>(const float* tile, int ld, int kb, int cb,
                                                                      int lane) {
  const float* p = tile + kb * ld + cb + (lane & 15);
  Quad<float> q; q.v = make_float4(p[0], p[ld], p[2 * ld], p[3 * ld]); return q;
}

// ---------------------------------------------------------------- small helpers
__device__ __forceinline__ float sigmoidf_(float s) { return fast_rcp(1.f + __expf(-s)); }
// phi(u) = elu(u) + 1
// Row order of a weight operand that is used as the A (row) side of a GEMM
// whose output C[row][token] leaves straight from registers: in each group of
// 32 rows, row p of the operand holds output feature tile_row_perm(p). A lane
// (grp = lane / 16) holds C rows 4 grp .. 4 grp + 3 of the group's two 16-row
// tiles, i.e. rows p = 16 u + 4 grp + r (u = 0, 1; r = 0..3), which are then
// features 8 grp + 4 u + r: eight consecutive features, one vector store.
__host__ __device__ __forceinline__ int tile_row_perm(int p) {
  return (p & ~31) + 8 * ((p & 15) >> 2) + 4 * ((p >> 4) & 1) + (p & 3);
}

__device__ __forceinline__ float phi_elu1(float u) { return u > 0.f ? u + 1.f : __expf(u); }

// Workgroup i runs on XCD i % 8. Give every XCD a contiguous range of logical
// block ids so blocks that share inputs (the heads of one token tile) share an
// L2. The grid must hold 8 * ceil(n / 8) blocks; ids >= n are idle.
__device__ __forceinline__ int xcd_logical_block(int bid, int n) {
  const int per = (n + 7) >> 3;
  return (bid & 7) * per + (bid >> 3);
}
__host__ __device__ inline int xcd_grid(int n) { return ((n + 7) >> 3) << 3; }

// sum over the 16 lanes that share lane / 16
// ---------------------------------------------------------------- cross-lane sums
// Register to register: DPP moves within rows of 16 lanes, lane-half swaps
// across rows. Each step adds the same two partial sums as the xor butterfly
// (v += v[lane ^ m] for m = 1, 2, 4, ...), so the results equal it bit for bit
// and are the same in every lane of a group. The whole wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// quad permutations (lane ^ 1, lane ^ 2), mirrors of an 8-lane half and of a row,
// rotate a row by 8, broadcast lane 0 of the row
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppRowMirror = 0x140, kDppRowRor8 = 0x128,
              kDppRowBcast0 = 0x150;

// v summed over each aligned group of N lanes (N = 1, 2, 4, 8 or 16). Once the
// 4-lane sums are uniform in a quad, the half mirror pairs each quad with the
// other quad of its 8 lanes (as lane ^ 4 would), and once the 8-lane sums are
// uniform, the row mirror pairs the two halves of the row (as lane ^ 8 would).
template <int N>
__device__ __forceinline__ float lane_group_sum(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "groups of 1 to 16 lanes");
  if constexpr (N >= 2) v += dpp_f<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp_f<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_f<kDppRowMirror>(v);
  return v;
}
__device__ __forceinline__ float row16_sum(float v) { return lane_group_sum<16>(v); }
// v + v[lane ^ 16] and v + v[lane ^ 32]
__device__ __forceinline__ float add_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// value held by lane 16 * (lane / 16) (column 0 of this lane's C-tile rows)
__device__ __forceinline__ float col0_bcast(float v) { return dpp_f<kDppRowBcast0>(v); }

// Walks consecutive tokens t0, t0+1, ... tracking their sequence: pos(t) is
// t's position in its sequence and end(t) the sequence's end (exclusive,
// clamped to [t + 1, T]), with one binary search at t0 and an advance over the
// offsets only where a sequence boundary is crossed.
// Must be queried with non-decreasing t.
struct SeqCursor {
  const int32_t* cu;
  int nseq, T, b, start, stop;
  __device__ SeqCursor(const int32_t* cu_, int nseq_, int t0, int T_) : cu(cu_), nseq(nseq_), T(T_) {
    int lo = 0, hi = nseq;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu[mid] <= t0) lo = mid; else hi = mid;
    }
    b = lo;
    start = cu[b];
    stop = cu[b + 1];
  }
  __device__ __forceinline__ void seek(int t) {
    while (t >= stop && b + 1 < nseq) {
      ++b;
      start = stop;
      stop = cu[b + 1];
    }
  }
  __device__ __forceinline__ int pos(int t) {
    seek(t);
    const int p = t - start;
    return p < 0 ? 0 : (p > t ? t : p);
  }
  __device__ __forceinline__ int end(int t) {
    seek(t);
    return stop <= t ? t + 1 : (stop > T ? T : stop);
  }
};

// Stage a dh x dh float matrix M (row-major) and a vector z as MFMA B operands
// in LDS, split into a high and a low part for bfloat16 (P = 2) so the staged
// matrix keeps about 16 mantissa bits:
//   MT[p][n][i] = M[i][n] for n < DH; row DH holds z, rows DH+1 .. NR-1 are 0
//   MR[p][i][n] = M[i][n]
// Either destination may be null; part 1 of MT starts NR rows after part 0,
// part 1 of MR starts DH rows after part 0 (pitch ld elements; ld * sizeof(T)
// a multiple of 16). M and z must be 16-byte aligned.
// MT: a lane owns column n of M and a run of consecutive i, so its loads are
// coalesced across the lanes (consecutive n) and its LDS stores are whole
// 8- or 16-byte vectors along row n of MT (element-wise transposed stores
// would put the lanes of a wave on a handful of banks). MR: float4 loads of a
// row, stored as one vector each.
// stores n consecutive values (n * sizeof(T) a multiple of 8) as whole vectors
template <typename T, int N>
__device__ __forceinline__ void lds_store_run(T* dst, const T (&v)[N]) {
  constexpr int VE = 16 / (int)sizeof(T);
  if constexpr (N % VE == 0) {
#pragma unroll
    for (int k = 0; k < N; k += VE) {
      T tmp[VE];
#pragma unroll
      for (int j = 0; j < VE; ++j) tmp[j] = v[k + j];
      *reinterpret_cast<uint4*>(dst + k) = __builtin_bit_cast(uint4, tmp);
    }
  } else {
    static_assert(N * sizeof(T) == 8, "runs of 8 bytes or whole 16-byte vectors");
    *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, v);
  }
}

template <typename T, int DH, int NR, int NT = 256>
__device__ __forceinline__ void stage_state(T* MT, T* MR, int ld, const float* __restrict__ M,
                                            const float* __restrict__ z, int tid) {
  constexpr bool SPLIT = sizeof(T) == 2;
  static_assert(NT % DH == 0 && (DH * DH) % NT == 0, "whole columns per thread group");
  if (MT) {
    constexpr int IP = DH * DH / NT;  // consecutive i per thread
    const int n = tid % DH, i0 = (tid / DH) * IP;
    float v[IP];
#pragma unroll
    for (int k = 0; k < IP; ++k) v[k] = M[(size_t)(i0 + k) * DH + n];
    T hi[IP], lo[IP];
#pragma unroll
    for (int k = 0; k < IP; ++k) {
      hi[k] = from_f<T>(v[k]);
      lo[k] = from_f<T>(v[k] - to_f<T>(hi[k]));
    }
    lds_store_run(MT + n * ld + i0, hi);
    if (SPLIT) lds_store_run(MT + NR * ld + n * ld + i0, lo);
    for (int e = tid; e < (NR - DH) * DH; e += NT) {  // rows DH..: z in row DH, zeros below
      const int r = DH + e / DH, i = e % DH;
      const float u = r == DH ? z[i] : 0.f;
      const T h = from_f<T>(u);
      MT[r * ld + i] = h;
      if (SPLIT) MT[NR * ld + r * ld + i] = from_f<T>(u - to_f<T>(h));
    }
  }
  if (MR) {
    constexpr int V4 = DH * DH / 4, PER = (V4 + NT - 1) / NT;
    float4 rv[PER];  // every load is issued before the first conversion
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e4 = tid + k * NT;
      rv[k] = e4 < V4 ? reinterpret_cast<const float4*>(M)[e4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e4 = tid + k * NT;
      if (e4 >= V4) continue;
      const int i = (4 * e4) / DH, n = (4 * e4) % DH;
      const float4 r = rv[k];
      const float v[4] = {r.x, r.y, r.z, r.w};
      T hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hi[j] = from_f<T>(v[j]);
        lo[j] = from_f<T>(v[j] - to_f<T>(hi[j]));
      }
      lds_store_run(MR + i * ld + n, hi);
      if (SPLIT) lds_store_run(MR + DH * ld + i * ld + n, lo);
    }
  }
}

// out[e] = sum over p < P of in[p * E + e] for the EB elements of virtual block
// blk (256 threads: 256 / EB phases per element, eight independent partial sums
// per thread so the loads stay in flight). Fixed summation order.
template <int EB>
__device__ __forceinline__ void sum_parts_block(const float* __restrict__ in, int E, int P, float* __restrict__ out,
                                                int blk) {
  constexpr int PH = 256 / EB;
  __shared__ float red[PH][EB];
  const int el = threadIdx.x % EB, ph = threadIdx.x / EB;
  const int e = blk * EB + el;
  float a[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) a[u] = 0.f;
  if (e < E) {
    int p = ph;
    for (; p + 7 * PH < P; p += 8 * PH)
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] += in[(size_t)(p + u * PH) * E + e];
    for (int u = 0; p < P; p += PH, ++u) a[u] += in[(size_t)p * E + e];
  }
  red[ph][el] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  __syncthreads();
  if (ph == 0 && e < E) {
    float t = 0.f;
    for (int q = 0; q < PH; ++q) t += red[q][el];
    out[e] = t;
  }
}

// chunk table entry: one run of <= chunk tokens inside one sequence
struct Chunk { int seq, start, end, pad; };

}  // namespace gbla
