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
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 128;    // key block size (tokens)
constexpr int kHeadDim = 128;  // main-branch head dim

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// 8-bit floating point E4M3 (OCP: bias 7, 3 mantissa bits, no infinities),
// carried as raw bytes; only the MFMAs interpret them.
struct fp8e4m3 {
  uint8_t bits;
};

template <typename T> struct Vec8;
template <> struct Vec8<bf16> { typedef bf16x8 type; };
template <> struct Vec8<float> { typedef f32x8 type; };

template <typename T>
using frag8 = typename Vec8<T>::type;

template <typename T>
__device__ __forceinline__ frag8<T> load8(const T* p) {
  return *reinterpret_cast<const frag8<T>*>(p);
}

// Eight E4M3 values (8 bytes) widened to the bf16 MFMA operand.  Exact: every
// E4M3 value (subnormals, signed zero and NaN included) is a bf16 value.  The
// gfx950 conversion takes two bytes of a dword per instruction (scale 1).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 widen8_e4m3(u32x2 w) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight K/V elements of storage type TKV as the compute-type operand T: a
// plain load when the two agree, E4M3 widened to bf16 otherwise.
template <typename T, typename TKV>
__device__ __forceinline__ frag8<T> load8_kv(const TKV* p) {
  if constexpr (sizeof(TKV) == 1) {
    static_assert(sizeof(T) == 2, "E4M3 K/V is widened to bf16");
    return widen8_e4m3(*reinterpret_cast<const u32x2*>(p));
  } else {
    return load8(p);
  }
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

// fp8: 32x32x64 (lane l: A row l%32, k-slots 32*(l/32) .. +31, i.e. 32 bytes)
// and 16x16x32 (lane l: A row l%16, k-slots 8*(l/16) .. +7, 8 bytes); both
// E4M3 operands (format codes 0), fp32 accumulate, C layouts as for bf16.
__device__ __forceinline__ f32x16 mma32_fp8(const i32x8& a, const i32x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16_fp8(long a, long b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

// Direct memory-to-LDS load of 16 bytes per lane (gfx950), through a buffer
// resource over [base, base + bytes): lane i reads the 16 bytes at byte offset
// voff and they land at lds_base + 16 i; lds_base must be the same for the
// whole wave.  A lane whose 16 bytes are not inside the range reads zeros (the
// buffer unit's range check), so a wrong offset cannot reach other memory.  The
// load counts in vmcnt only: wait for it (s_waitcnt vmcnt) before a barrier
// that makes the data visible to other waves.  The global-address form of this
// load is taken by the compiler as an event of the LDS counter too, after which
// every wait for an LDS read becomes a wait for all of them; the buffer form is
// not.  The builtins exist only in the device pass; the host pass of a kernel
// body never runs this.
__device__ __forceinline__ void lds_load16(const void* base, int bytes, int voff, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  // word 3: 32-bit data format (required for untyped loads on this family)
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, 0, 0, 0);
#endif
}

// Transposed LDS read of 16-bit data (gfx950): every lane gives the address
// of four consecutive 16-bit values (8-byte aligned); lane 16 g + i receives,
// as element e, value i % 4 of the four at the address of lane 16 g + 4 e +
// i / 4.  With lane 16 g + 4 e + q pointing at row r0 + e, columns c0 + 4 q
// .. + 3 of a row-major tile, lane 16 g + i gets column c0 + i of rows r0 ..
// r0 + 3: a column fragment of an MFMA operand read from a row-major tile.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)p);
#else
  return bf16x4{};
#endif
}

// An 8-byte LDS store issued from an asm statement.  The compiler's
// wait-count pass orders its own LDS stores after any direct-to-LDS load
// still in flight that it cannot tell apart from the stored buffer, with a
// full vector-memory wait; this store never waits.  The caller must order it
// against other accesses of the same buffer by barriers (the LDS-counter wait
// of lds_barrier completes it; LDS operations complete in order, so the
// compiler's own LDS-counter waits are never made too short by it).
__device__ __forceinline__ void lds_store8(bf16* p, bf16x4 v) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16*)p;
  asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(v));
#endif
}

// Wait until every vector memory operation of this wave has completed
// (loads, stores, direct-to-LDS loads): s_waitcnt vmcnt(0), with the gfx9
// immediate (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8 left at
// their maxima).  Unlike the same instruction in an asm statement, the
// builtin is seen by the compiler's wait-count pass, which then knows that
// registers loaded earlier are complete and adds no waits of its own for
// them later (an asm wait left it waiting again, for everything in flight,
// inside loops).  It does not order memory accesses: follow it with a
// barrier or fence where the staged data is read.
__device__ __forceinline__ void vmem_wait_all() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0x0F70);
#endif
}
// The same, but leaving the N most recently issued operations in flight
// (s_waitcnt vmcnt(N), N < 16).
template <int N>
__device__ __forceinline__ void vmem_wait_all_but() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate of 4 bits");
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
#endif
}

// Workgroup barrier that orders LDS accesses only: the wave's own LDS
// writes are complete before it (lgkmcnt) and later LDS reads see the other
// waves' writes, while global loads and direct-to-LDS loads stay in flight
// across it.  A compiler fence would also wait for those: __syncthreads
// waits for every outstanding global access, and even a fence restricted to
// LDS waits for direct-to-LDS loads, which write LDS.  Data staged by such
// loads needs its own s_waitcnt vmcnt before the barrier that publishes it.
// The memory clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, kWave); }
// The value of lane l ^ 32 (the other half of the wave), by gfx950's
// permlane32 swap: a vector-ALU exchange, so unlike a shuffle through LDS it
// adds nothing to the LDS counter that later LDS waits would also drain
// (probed against the LDS shuffle on all 64 lanes).
__device__ __forceinline__ uint32_t xchg_halves_u32(uint32_t x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return lane_id() < 32 ? r[1] : r[0];
#else
  return x;
#endif
}
__device__ __forceinline__ float xchg_halves_f(float x) { return __uint_as_float(xchg_halves_u32(__float_as_uint(x))); }
__device__ __forceinline__ int shfl_xor_i(int v, int mask) { return __shfl_xor(v, mask, kWave); }

// 64-bit selection key: the score's bits mapped to an order-preserving
// unsigned integer in the high word, the inverted block id in the low word, so
// a larger key precedes in the selection order (higher score, then lower id).
// Every finite score maps to a non-zero high word; 0 is "no entry".
__device__ __forceinline__ uint64_t sel_key(float s, int id) {
  const uint32_t b = __float_as_uint(s);
  const uint32_t hi = b ^ (uint32_t)(((int32_t)b >> 31) | INT32_MIN);  // ~b if negative, else b | 2^31
  return ((uint64_t)hi << 32) | (uint32_t)(0xffffffffu - (uint32_t)id);
}
__device__ __forceinline__ int sel_key_id(uint64_t k) { return (int)(0xffffffffu - (uint32_t)k); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, kWave);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, kWave);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src, kWave);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src, kWave);
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

// Write the final selection: `found` earlier ids held one per lane in lanes
// 0..found-1 plus the local block, ascending, padded with -1 to topk.
__device__ __forceinline__ void write_selection(int mine, int found, int local, int topk,
                                                int32_t* out) {
  const int lane = lane_id();
  int v = lane < found ? mine : (lane == found ? local : 0x7fffffff);
  const int cnt = found + 1;  // <= 16
  // rank among the first cnt lanes, each value read as a scalar (no LDS
  // round trip per lane, unlike a shuffle); lanes from cnt on hold INT_MAX,
  // which is below no value
  int rank = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) rank += __builtin_amdgcn_readlane(v, j) < v ? 1 : 0;
  if (lane < cnt) out[rank] = v;
  if (lane >= cnt && lane < topk) out[lane] = -1;
}

template <typename T>
__device__ __forceinline__ T from_f32(float x) { return T(x); }

}  // namespace msa
