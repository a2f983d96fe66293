// msa_device.h -- device-side building blocks of the gfx950 MSA kernels.
//
// Internal to the GPU library.  MFMA wrappers for the two element types, the
// 8-element operand fragment every kernel uses, wave-level shuffles, and the
// total order of the block selection.
//
// MFMA operand convention used throughout: for both the 16x16 and the 32x32
// shapes a lane contributes 8 consecutive elements of the contraction axis
// (one 16-byte bf16 load, or one 32-byte fp32 load).  For bf16 this is exactly
// one v_mfma_f32_{16x16x32,32x32x16}_bf16.  For fp32 it is 8 fp32 MFMAs
// (v_mfma_f32_{16x16x4,32x32x2}_f32), the i-th consuming element i of every
// lane; summed over i they contract the same 8 * (lanes per row) elements.
// Since A and B always use the same lane -> k mapping, any permutation of the
// contraction axis inside one MFMA is harmless.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 128;    // key block size (tokens)
constexpr int kHeadDim = 128;  // main-branch head dim
constexpr int kList = 15;      // per-lane candidate list: topk - 1 for topk <= 16

template <typename T> struct Vec8;
template <> struct Vec8<bf16> { typedef bf16x8 type; };
template <> struct Vec8<float> { typedef f32x8 type; };

template <typename T>
using frag8 = typename Vec8<T>::type;

template <typename T>
__device__ __forceinline__ frag8<T> load8(const T* p) {
  return *reinterpret_cast<const frag8<T>*>(p);
}

template <typename T>
__device__ __forceinline__ frag8<T> zero8() {
  frag8<T> z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = T(0.0f);
  return z;
}

// acc[16x16] += A[16 x K] * B[K x 16]; lane l holds A row l%16, B column l%16,
// k-slots 8*(l/16) .. 8*(l/16)+7.  Output: lane l, reg r -> row 4*(l/16)+r,
// column l%16.
__device__ __forceinline__ f32x4 mma16(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
  return c;
}

// acc[32x32] += A[32 x K] * B[K x 32]; lane l holds A row l%32, B column l%32,
// k-slots 8*(l/32) .. +7.  Output: lane l, reg r -> row 8*(r/4)+4*(l/32)+(r%4),
// column l%32.
__device__ __forceinline__ f32x16 mma32(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32(const f32x8& a, const f32x8& b, f32x16 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, kWave); }
__device__ __forceinline__ int shfl_xor_i(int v, int mask) { return __shfl_xor(v, mask, kWave); }

// Selection order: (score, id) precedes (score', id') when the score is higher,
// or equal with a lower block id.  Invalid entries carry id < 0 and are last.
__device__ __forceinline__ bool precedes(float s, int i, float s2, int i2) {
  if (i2 < 0) return i >= 0;
  if (i < 0) return false;
  return (s > s2) || (s == s2 && i < i2);
}

// Wave-wide best (score, id) under `precedes`; every lane gets the result.
__device__ __forceinline__ void wave_best(float& s, int& i) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    float so = shfl_xor_f(s, m);
    int io = shfl_xor_i(i, m);
    if (precedes(so, io, s, i)) { s = so; i = io; }
  }
}

// Insert (v, c) into a descending list of kList entries when it beats the last
// one.  Blocks arrive in ascending id order, so a strict comparison keeps the
// earlier (lower) id ahead on equal scores: the lowest-id tie-break.
__device__ __forceinline__ void list_insert(float (&ls)[kList], int (&li)[kList], float v, int c) {
  if (!(v > ls[kList - 1])) return;
  bool gt[kList];
#pragma unroll
  for (int j = 0; j < kList; ++j) gt[j] = v > ls[j];
#pragma unroll
  for (int j = kList - 1; j > 0; --j) {
    float ns = gt[j - 1] ? ls[j - 1] : (gt[j] ? v : ls[j]);
    int ni = gt[j - 1] ? li[j - 1] : (gt[j] ? c : li[j]);
    ls[j] = ns;
    li[j] = ni;
  }
  if (gt[0]) { ls[0] = v; li[0] = c; }
}

// Insert (v, c) into a list kept sorted by `precedes` when it precedes the
// last entry (for candidates arriving in any order).
__device__ __forceinline__ void list_insert_ordered(float (&ls)[kList], int (&li)[kList], float v, int c) {
  if (!precedes(v, c, ls[kList - 1], li[kList - 1])) return;
  bool pr[kList];
#pragma unroll
  for (int j = 0; j < kList; ++j) pr[j] = precedes(v, c, ls[j], li[j]);
#pragma unroll
  for (int j = kList - 1; j > 0; --j) {
    float ns = pr[j - 1] ? ls[j - 1] : (pr[j] ? v : ls[j]);
    int ni = pr[j - 1] ? li[j - 1] : (pr[j] ? c : li[j]);
    ls[j] = ns;
    li[j] = ni;
  }
  if (pr[0]) { ls[0] = v; li[0] = c; }
}

// 64-bit selection key: the score's bits mapped to an order-preserving
// unsigned integer in the high word, the inverted block id in the low word, so
// a larger key precedes in the selection order (higher score, then lower id).
// Every finite score maps to a non-zero high word; 0 is "no entry".
__device__ __forceinline__ uint64_t sel_key(float s, int id) {
  const uint32_t b = __float_as_uint(s);
  const uint32_t hi = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)hi << 32) | (uint32_t)(0xffffffffu - (uint32_t)id);
}
__device__ __forceinline__ int sel_key_id(uint64_t k) { return (int)(0xffffffffu - (uint32_t)k); }

// Insert a key into a descending list of 16 keys when it beats the last one.
__device__ __forceinline__ void key_insert(uint64_t (&kl)[16], uint64_t v) {
  if (!(v > kl[15])) return;
  bool gt[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) gt[j] = v > kl[j];
#pragma unroll
  for (int j = 15; j > 0; --j) kl[j] = gt[j - 1] ? kl[j - 1] : (gt[j] ? v : kl[j]);
  if (gt[0]) kl[0] = v;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, kWave);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// Merge the descending 16-key lists of lanes l and l ^ m: every lane ends
// with the top 16 of the union, descending.  Elementwise max against the
// partner's reversed list keeps the top half (a bitonic sequence), which a
// 4-stage bitonic half-cleaner network sorts.
__device__ __forceinline__ void key_merge_xor(uint64_t (&kl)[16], int m) {
  uint64_t other[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) other[j] = shfl_xor_u64(kl[j], m);
#pragma unroll
  for (int j = 0; j < 16; ++j) kl[j] = kl[j] > other[15 - j] ? kl[j] : other[15 - j];
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if ((j & d) == 0) {
        const uint64_t x = kl[j], y = kl[j + d];
        kl[j] = x > y ? x : y;
        kl[j + d] = x > y ? y : x;
      }
}

// Remove the head of a list (shift left), padding with an invalid entry.
__device__ __forceinline__ void list_pop(float (&ls)[kList], int (&li)[kList]) {
#pragma unroll
  for (int j = 0; j < kList - 1; ++j) { ls[j] = ls[j + 1]; li[j] = li[j + 1]; }
  ls[kList - 1] = -__builtin_inff();
  li[kList - 1] = -1;
}

// Wave-level merge of per-lane descending lists: the first `take` entries of
// their union under `precedes` go to lanes 0..take-1 (`mine`), one per lane;
// returns how many valid entries were found.  Lane ids must be distinct
// across lanes (they are: lists cover disjoint block ranges).
__device__ __forceinline__ int wave_merge(float (&ls)[kList], int (&li)[kList], int take, int& mine) {
  const int lane = lane_id();
  mine = -1;
  int found = 0;
  for (int r = 0; r < take; ++r) {
    float s = ls[0];
    int i = li[0];
    wave_best(s, i);
    if (i < 0) break;
    if (li[0] == i) list_pop(ls, li);
    if (lane == r) mine = i;
    ++found;
  }
  return found;
}

// Write the final selection: `found` earlier ids held one per lane in lanes
// 0..found-1 plus the local block, ascending, padded with -1 to topk.
__device__ __forceinline__ void write_selection(int mine, int found, int local, int topk,
                                                int32_t* out) {
  const int lane = lane_id();
  int v = lane < found ? mine : (lane == found ? local : 0x7fffffff);
  const int cnt = found + 1;
  int rank = 0;
  for (int j = 0; j < cnt; ++j) {
    int o = __shfl(v, j, kWave);
    rank += (o < v) ? 1 : 0;
  }
  if (lane < cnt) out[rank] = v;
  if (lane >= cnt && lane < topk) out[lane] = -1;
}

template <typename T>
__device__ __forceinline__ T from_f32(float x) { return T(x); }

}  // namespace msa
