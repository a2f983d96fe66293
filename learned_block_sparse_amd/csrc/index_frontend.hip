// index_frontend.hip -- the index branch's front end: hidden states through a
// linear projection, an RMS norm and RoPE to the index-query heads (one per
// GQA group) and the shared index-key head, in one kernel.
//
// Method: "MiniMax Sparse Attention: let each query pick its own blocks",
// Figure 1 (projection, norm, RoPE, in that order, ahead of the score
// matrix); the atlas record of MiniMax M3, provenance notes on section 5.1
// (model width 3072; the main heads rotate 64 of their 128 dims).  The norm's
// kind and the rotary base are not given: the norm is an RMS norm over each
// head vector with a gain per dimension, the rotation turns the pair
// (i, i + rope_dim/2) by p * theta^(-2i/rope_dim) at the token's absolute
// position p, and theta and eps come from the caller.
//
// Schedule.  One workgroup computes one head (DI output dims) for 256 tokens
// (the heads of a token tile run back to back on one XCD, see the kernel):
// C^T[dim][token] = W_h[dim][:] . x[token][:], on 32x32x16 MFMAs with the
// head's dims as MFMA rows and tokens as columns.  Each of the 4 waves owns 64
// tokens (two column tiles) and all DI dims, so a token's whole head vector
// ends in one wave: the norm is a register sum plus one lane swap, and the
// rotation partner of dim i (i + rope_dim/2, a multiple of 32 away) sits in
// the same lane and register of another row tile.  The contraction runs in
// chunks of 32: the head's 32 weight columns are staged in LDS (shared by the
// 4 waves, double-buffered), while each lane reads its token's 16 consecutive
// values of the chunk straight from global memory (64 contiguous bytes per
// token and chunk over the two lane halves).  Both operands use the same
// lane -> k mapping inside a chunk (lane half h, MFMA s: k = 16h + 8s + 0..7),
// which any MFMA contraction allows.  32-wide chunks keep the accumulators,
// the prefetched fragments and the staged weights within 256 registers.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kFeThreads = 256;
constexpr int kFeCt = 2;                             // 32-token column tiles per wave
constexpr int kFeTokWave = 32 * kFeCt;               // tokens per wave
constexpr int kFeTok = kFeTokWave * (kFeThreads / kWave);
constexpr int kFeKc = 32;                            // contraction chunk
constexpr int kFeS = kFeKc / 16;                     // 8-element fragments per lane and chunk

struct FeArgs {
  const void* x;
  const void* w_q;
  const void* w_k;
  const float* gain_q;
  const float* gain_k;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int batch, G, d_model, rope_dim;
  int64_t total;
  double log2_theta;
  float eps;
  void* q_out;
  void* k_out;
};

template <typename T> struct FeLds;
template <> struct FeLds<bf16> { static constexpr int stride = kFeKc + 8; };   // 80-byte rows
template <> struct FeLds<float> { static constexpr int stride = kFeKc + 4; };  // 144-byte rows

__device__ __forceinline__ int fe_find(const int32_t* cu, int n, int64_t x) {
  int lo = 0, hi = n;  // cu[lo] <= x < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

template <typename TO>
__device__ __forceinline__ void fe_store4(TO* dst, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void fe_store4<bf16>(bf16* dst, float a, float b, float c, float d) {
  *reinterpret_cast<bf16x4*>(dst) = bf16x4{bf16(a), bf16(b), bf16(c), bf16(d)};
}
template <>
__device__ __forceinline__ void fe_store4<float>(float* dst, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{a, b, c, d};
}

// sin and cos of |x| <= pi/4 by their Taylor polynomials (through x^9 and
// x^10; truncation below 2e-9, so fp32 rounding dominates).
__device__ __forceinline__ void fe_sincos_small(float x, float& sn, float& cs) {
  const float x2 = x * x;
  sn = x * (1.f + x2 * (-1.f / 6.f + x2 * (1.f / 120.f + x2 * (-1.f / 5040.f + x2 * (1.f / 362880.f)))));
  cs = 1.f + x2 * (-0.5f + x2 * (1.f / 24.f + x2 * (-1.f / 720.f + x2 * (1.f / 40320.f - x2 * (1.f / 3628800.f)))));
}

// Rotation of column tile CT: the pair (i, i + 32*HT) for every dim i of the
// first HT row tiles, by the angle p * inv_freq[i].  The angle is split in
// fp64 into k quarter turns plus a rest |r| <= pi/4 (p reaches 2^20 and more,
// so fp32 could not hold the angle to 1e-7), then sin and cos of the rest
// are evaluated in fp32 and moved to quadrant k.
template <int RT, int HT, int CT>
__device__ __forceinline__ void fe_rope(f32x16 (&acc)[RT][kFeCt], int h, int64_t p, const double* inv_freq) {
#pragma unroll
  for (int rt = 0; rt < HT; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * rt + 8 * (r >> 2) + 4 * h + (r & 3);
      const double ang = (double)p * inv_freq[i];
      const double k = rint(ang * 0.63661977236758134308);  // 2 / pi
      const float rest = (float)(ang - k * 1.57079632679489661923);
      float s0, c0;
      fe_sincos_small(rest, s0, c0);
      const int quad = (int)((int64_t)k & 3);
      const float sn = quad == 0 ? s0 : quad == 1 ? c0 : quad == 2 ? -s0 : -c0;
      const float cs = quad == 0 ? c0 : quad == 1 ? -s0 : quad == 2 ? -c0 : s0;
      const float va = acc[rt][CT][r], vb = acc[rt + HT][CT][r];
      acc[rt][CT][r] = va * cs - vb * sn;
      acc[rt + HT][CT][r] = vb * cs + va * sn;
    }
}

// Epilogue of column tile CT (token t of this lane): RMS norm over the head's
// DI dims (16 per register tile in this lane, the rest in lane ^ 32), gain,
// rotation, store.
template <typename TO, int DI, int CT>
__device__ __forceinline__ void fe_finish(f32x16 (&acc)[DI / 32][kFeCt], const FeArgs& a, int head, int64_t t, int h,
                                          const double* inv_freq) {
  constexpr int RT = DI / 32;
  float ss = 0.f;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) ss += acc[rt][CT][r] * acc[rt][CT][r];
  ss += shfl_xor_f(ss, 32);
  if (t >= a.total || t >= a.cu_q[a.batch]) return;  // past the packed tokens: nothing to write
  const float inv = 1.0f / sqrtf(ss / (float)DI + a.eps);
  const float* gain = head < a.G ? a.gain_q : a.gain_k;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dim = 32 * rt + 8 * (r >> 2) + 4 * h + (r & 3);
      acc[rt][CT][r] = gain[dim] * (acc[rt][CT][r] * inv);
    }
  const int b = fe_find(a.cu_q, a.batch, t);
  const int64_t M = a.cu_q[b + 1] - a.cu_q[b];
  const int64_t N = a.cu_k[b + 1] - a.cu_k[b];
  const int64_t p = N - M + (t - a.cu_q[b]);
  if (a.rope_dim == 64) fe_rope<RT, 1, CT>(acc, h, p, inv_freq);
  else if (a.rope_dim == 128) fe_rope<RT, (RT >= 4 ? 2 : 1), CT>(acc, h, p, inv_freq);
  TO* dst;
  if (head < a.G) {
    dst = static_cast<TO*>(a.q_out) + (t * a.G + head) * DI;
  } else {
    if (p < 0 || p >= N) return;  // a token before the sequence start has no key row
    dst = static_cast<TO*>(a.k_out) + ((int64_t)a.cu_k[b] + p) * DI;
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      fe_store4<TO>(dst + 32 * rt + 8 * q4 + 4 * h, acc[rt][CT][4 * q4], acc[rt][CT][4 * q4 + 1],
                    acc[rt][CT][4 * q4 + 2], acc[rt][CT][4 * q4 + 3]);
}

template <typename T, typename TO, int DI>
__global__ __launch_bounds__(kFeThreads, sizeof(T) == 2 ? 2 : 1) void index_frontend(FeArgs a) {
  constexpr int RT = DI / 32;             // row tiles (32 dims each)
  constexpr int LS = FeLds<T>::stride;
  constexpr int V16 = 16 / sizeof(T);     // elements per 16-byte piece
  constexpr int PIECES = DI * kFeKc / V16 / kFeThreads;  // 16-byte pieces per thread per chunk
  __shared__ __attribute__((aligned(16))) T w_lds[2][DI * LS];

  // Workgroup i runs on XCD i % 8 (round-robin dispatch).  The G+1 heads of
  // token tile `tile` get ids 8 * ((tile / 8) * (G+1) + head) + tile % 8: they
  // are dispatched back to back on one XCD and read the tile's hidden states
  // through that XCD's L2 instead of each from HBM.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int head = slot % (a.G + 1);      // 0..G-1 query heads, G the key head
  const int64_t tile = (int64_t)(slot / (a.G + 1)) * 8 + xcd;
  if (tile * kFeTok >= a.total) return;   // padding of the last group of 8 tiles
  const T* w = head < a.G ? static_cast<const T*>(a.w_q) + (int64_t)head * DI * a.d_model
                          : static_cast<const T*>(a.w_k);
  const T* x = static_cast<const T*>(a.x);
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int col = lane & 31, h = lane >> 5;
  const int64_t t0 = tile * kFeTok + wave * kFeTokWave;
  // rows past the end read the last token (their results are not stored)
  const T* xp[kFeCt];
#pragma unroll
  for (int ct = 0; ct < kFeCt; ++ct) {
    const int64_t t = t0 + 32 * ct + col;
    xp[ct] = x + (t < a.total ? t : a.total - 1) * a.d_model + (kFeKc / 2) * h;
  }

  frag8<T> xr[kFeCt][kFeS], xn[kFeCt][kFeS];
  u32x4 wr[PIECES];
  auto load_w = [&](int kc) {
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int piece = threadIdx.x + u * kFeThreads;
      const int row = piece / (kFeKc / V16), c16 = piece % (kFeKc / V16);
      wr[u] = *reinterpret_cast<const u32x4*>(w + (int64_t)row * a.d_model + kc + c16 * V16);
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int piece = threadIdx.x + u * kFeThreads;
      const int row = piece / (kFeKc / V16), c16 = piece % (kFeKc / V16);
      *reinterpret_cast<u32x4*>(&w_lds[buf][row * LS + c16 * V16]) = wr[u];
    }
  };
  auto load_x = [&](frag8<T> (&dst)[kFeCt][kFeS], int kc) {
#pragma unroll
    for (int ct = 0; ct < kFeCt; ++ct)
#pragma unroll
      for (int s = 0; s < kFeS; ++s) dst[ct][s] = load8(xp[ct] + kc + 8 * s);
  };

  f32x16 acc[RT][kFeCt];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < kFeCt; ++ct) acc[rt][ct] = f32x16{};

  const int nc = a.d_model / kFeKc;
  load_w(0);
  load_x(xr, 0);
  store_w(0);
  __syncthreads();
  for (int c = 0; c < nc; ++c) {
    const bool more = c + 1 < nc;
    if (more) {
      load_w((c + 1) * kFeKc);
      load_x(xn, (c + 1) * kFeKc);
    }
    const T* wl = w_lds[c & 1];
#pragma unroll
    for (int s = 0; s < kFeS; ++s)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const frag8<T> av = load8(wl + (32 * rt + col) * LS + (kFeKc / 2) * h + 8 * s);
#pragma unroll
        for (int ct = 0; ct < kFeCt; ++ct) acc[rt][ct] = mma32(av, xr[ct][s], acc[rt][ct]);
      }
    if (more) {
      store_w((c + 1) & 1);
#pragma unroll
      for (int ct = 0; ct < kFeCt; ++ct)
#pragma unroll
        for (int s = 0; s < kFeS; ++s) xr[ct][s] = xn[ct][s];
    }
    __syncthreads();
  }

  // inverse frequencies theta^(-2i/rope_dim), once per workgroup (LDS is free
  // after the last barrier of the loop)
  __shared__ double inv_freq[64];
  if ((int)threadIdx.x < a.rope_dim / 2)
    inv_freq[threadIdx.x] = exp2(-2.0 * (double)threadIdx.x / (double)a.rope_dim * a.log2_theta);
  __syncthreads();
  const int64_t tw = t0 + col;
  fe_finish<TO, DI, 0>(acc, a, head, tw, h, inv_freq);
  if constexpr (kFeCt > 1) fe_finish<TO, DI, (kFeCt > 1 ? 1 : 0)>(acc, a, head, tw + 32, h, inv_freq);
}

template <typename T, typename TO>
static void launch_fe_t(const FeArgs& a, int DI, dim3 grid, hipStream_t st) {
  if (DI == 64) hipLaunchKernelGGL((index_frontend<T, TO, 64>), grid, dim3(kFeThreads), 0, st, a);
  else hipLaunchKernelGGL((index_frontend<T, TO, 128>), grid, dim3(kFeThreads), 0, st, a);
}

hipError_t launch_index_frontend(const FrontendLaunch& f, hipStream_t st) {
  if (f.total == 0) return hipSuccess;
  FeArgs a;
  a.x = f.x;
  a.w_q = f.w_q;
  a.w_k = f.w_k;
  a.gain_q = f.gain_q;
  a.gain_k = f.gain_k;
  a.cu_q = f.cu_q;
  a.cu_k = f.cu_k;
  a.batch = f.batch;
  a.G = f.G;
  a.d_model = f.d_model;
  a.rope_dim = f.rope_dim;
  a.total = f.total;
  a.log2_theta = log2((double)f.theta);
  a.eps = f.eps;
  a.q_out = f.q_out;
  a.k_out = f.k_out;
  const int64_t tiles8 = (f.total + 8 * kFeTok - 1) / (8 * kFeTok);  // groups of 8 token tiles
  const dim3 grid((unsigned)(tiles8 * 8 * (f.G + 1)));
  if (f.in_f32) {
    if (f.out_f32) launch_fe_t<float, float>(a, f.DI, grid, st);
    else launch_fe_t<float, bf16>(a, f.DI, grid, st);
  } else {
    if (f.out_f32) launch_fe_t<bf16, float>(a, f.DI, grid, st);
    else launch_fe_t<bf16, bf16>(a, f.DI, grid, st);
  }
  return hipGetLastError();
}

}  // namespace msa
