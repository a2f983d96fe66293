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
constexpr int kFeCt = 2;                             // 32-token column tiles per wave (forward)
constexpr int kFeTokWave = 32 * kFeCt;               // tokens per wave
constexpr int kFeTok = kFeTokWave * (kFeThreads / kWave);
constexpr int kFeBwdTok = 32 * (kFeThreads / kWave);  // backward recompute: one column tile per wave
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

// LDS layout of a staged weight chunk (rows = the head's dims, kFeKc values
// each), as the element offset of 16-byte piece c16 of a row.  bf16: 64-byte
// rows, unpadded, with the piece index XOR-ed by (row / 4) % 4, so both the
// staging writes (4 rows x 4 pieces per 16 lanes) and the MFMA fragment reads
// (16 rows at one piece) cover all 16 bank groups.  fp32: 144-byte padded
// rows.
template <typename T> struct FeLds;
template <> struct FeLds<bf16> {
  static constexpr int stride = kFeKc;
  static __device__ __forceinline__ int off(int row, int c16) { return row * kFeKc + ((c16 ^ ((row >> 2) & 3)) << 3); }
};
template <> struct FeLds<float> {
  static constexpr int stride = kFeKc + 4;
  static __device__ __forceinline__ int off(int row, int c16) { return row * (kFeKc + 4) + (c16 << 2); }
};

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
__device__ __forceinline__ void fe_angle(int64_t p, double inv_freq, float& sn, float& cs) {
  const double ang = (double)p * inv_freq;
  const double k = rint(ang * 0.63661977236758134308);  // 2 / pi
  const float rest = (float)(ang - k * 1.57079632679489661923);
  float s0, c0;
  fe_sincos_small(rest, s0, c0);
  // quadrant q = k mod 4: sin = (s0, c0, -s0, -c0)[q], cos = (c0, -s0, -c0, s0)[q],
  // selected without branches (odd q swaps, the sign bit is flipped)
  const uint32_t q = (uint32_t)(int)(k - 4.0 * floor(k * 0.25));
  const float bs = (q & 1u) ? c0 : s0;
  const float bc = (q & 1u) ? s0 : c0;
  sn = __uint_as_float(__float_as_uint(bs) ^ ((q & 2u) << 30));
  cs = __uint_as_float(__float_as_uint(bc) ^ (((q + 1u) & 2u) << 30));
}

template <int RT, int HT, int CT, int CTW>
__device__ __forceinline__ void fe_rope(f32x16 (&acc)[RT][CTW], int h, int64_t p, const double* inv_freq) {
#pragma unroll
  for (int rt = 0; rt < HT; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * rt + 8 * (r >> 2) + 4 * h + (r & 3);
      float sn, cs;
      fe_angle(p, inv_freq[i], sn, cs);
      const float va = acc[rt][CT][r], vb = acc[rt + HT][CT][r];
      acc[rt][CT][r] = va * cs - vb * sn;
      acc[rt + HT][CT][r] = vb * cs + va * sn;
    }
}

// Epilogue of column tile CT (token t of this lane): RMS norm over the head's
// DI dims (16 per register tile in this lane, the rest in lane ^ 32), gain,
// rotation, store.
template <typename TO, int DI, int CT, int CTW>
__device__ __forceinline__ void fe_finish(f32x16 (&acc)[DI / 32][CTW], const FeArgs& a, int head, int64_t t, int h,
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
  if (a.rope_dim == 64) fe_rope<RT, 1, CT, CTW>(acc, h, p, inv_freq);
  else if (a.rope_dim == 128) fe_rope<RT, (RT >= 4 ? 2 : 1), CT, CTW>(acc, h, p, inv_freq);
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

// Token tile and head of this workgroup.  Workgroup i runs on XCD i % 8
// (round-robin dispatch); the G+1 heads of token tile `tile` get ids
// 8 * ((tile / 8) * (G+1) + head) + tile % 8, so they are dispatched back to
// back on one XCD and read the tile's hidden states through that XCD's L2
// instead of each from HBM.
struct FeTile {
  int head;       // 0..G-1 query heads, G the key head
  int64_t tile;
};
__device__ __forceinline__ FeTile fe_tile(int G) {  // tile size: the kernel's own
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  return FeTile{slot % (G + 1), (int64_t)(slot / (G + 1)) * 8 + xcd};
}

// acc[rt][ct] = C^T tile: rows = the head's dims 32*rt + .., columns = the
// wave's tokens t0 + 32*ct + ...  (see the schedule at the top of the file).
// PD: chunks of x requested ahead of the one being multiplied.
template <typename T, int DI, int CTW, int PD = 1>
__device__ __forceinline__ void fe_gemm(const FeArgs& a, const T* w, int64_t t0, f32x16 (&acc)[DI / 32][CTW],
                                        T (&w_lds)[2][DI * FeLds<T>::stride]) {
  constexpr int RT = DI / 32;             // row tiles (32 dims each)
  constexpr int V16 = 16 / sizeof(T);     // elements per 16-byte piece
  constexpr int PIECES = DI * kFeKc / V16 / kFeThreads;  // 16-byte pieces per thread per chunk
  const T* x = static_cast<const T*>(a.x);
  const int lane = lane_id();
  const int col = lane & 31, h = lane >> 5;
  // rows past the end read the last token (their results are not stored)
  const T* xp[CTW];
#pragma unroll
  for (int ct = 0; ct < CTW; ++ct) {
    const int64_t t = t0 + 32 * ct + col;
    xp[ct] = x + (t < a.total ? t : a.total - 1) * a.d_model + (kFeKc / 2) * h;
  }

  frag8<T> xr[CTW][kFeS], xn[PD][CTW][kFeS];
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
      *reinterpret_cast<u32x4*>(&w_lds[buf][FeLds<T>::off(row, c16)]) = wr[u];
    }
  };
  auto load_x = [&](frag8<T> (&dst)[CTW][kFeS], int kc) {
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
      for (int s = 0; s < kFeS; ++s) dst[ct][s] = load8(xp[ct] + kc + 8 * s);
  };

#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) acc[rt][ct] = f32x16{};

  const int nc = a.d_model / kFeKc;
  load_w(0);
  load_x(xr, 0);
#pragma unroll
  for (int p = 0; p + 1 < PD; ++p)
    if (p + 1 < nc) load_x(xn[p], (p + 1) * kFeKc);
  store_w(0);
  __syncthreads();
  for (int c = 0; c < nc; ++c) {
    const bool more = c + 1 < nc;
    if (more) load_w((c + 1) * kFeKc);
    if (c + PD < nc) load_x(xn[PD - 1], (c + PD) * kFeKc);
    const T* wl = w_lds[c & 1];
#pragma unroll
    for (int s = 0; s < kFeS; ++s)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        // 8 elements = 16 bytes (bf16: one piece) or 32 bytes (fp32: two pieces)
        const frag8<T> av = load8(wl + FeLds<T>::off(32 * rt + col, ((kFeKc / 2) * h + 8 * s) / V16));
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) acc[rt][ct] = mma32(av, xr[ct][s], acc[rt][ct]);
      }
    if (more) {
      store_w((c + 1) & 1);
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
        for (int s = 0; s < kFeS; ++s) {
          xr[ct][s] = xn[0][ct][s];
#pragma unroll
          for (int p = 0; p + 1 < PD; ++p) xn[p][ct][s] = xn[p + 1][ct][s];
        }
    }
    __syncthreads();
  }
}

// Inverse frequencies theta^(-2i/rope_dim), once per workgroup.
__device__ __forceinline__ void fe_inv_freq(double* inv_freq, int rope_dim, double log2_theta) {
  if ((int)threadIdx.x < rope_dim / 2)
    inv_freq[threadIdx.x] = exp2(-2.0 * (double)threadIdx.x / (double)rope_dim * log2_theta);
  __syncthreads();
}

template <typename T, typename TO, int DI>
__global__ __launch_bounds__(kFeThreads, sizeof(T) == 2 ? 2 : 1) void index_frontend(FeArgs a) {
  __shared__ __attribute__((aligned(16))) T w_lds[2][DI * FeLds<T>::stride];
  __shared__ double inv_freq[64];
  const FeTile ft = fe_tile(a.G);
  if (ft.tile * kFeTok >= a.total) return;   // padding of the last group of 8 tiles
  const T* w = ft.head < a.G ? static_cast<const T*>(a.w_q) + (int64_t)ft.head * DI * a.d_model
                             : static_cast<const T*>(a.w_k);
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int64_t t0 = ft.tile * kFeTok + wave * kFeTokWave;
  f32x16 acc[DI / 32][kFeCt];
  fe_gemm<T, DI, kFeCt, 2>(a, w, t0, acc, w_lds);  // x two chunks ahead (three: no faster, four: spills)
  fe_inv_freq(inv_freq, a.rope_dim, a.log2_theta);
  const int64_t tw = t0 + (lane & 31);
  fe_finish<TO, DI, 0, kFeCt>(acc, a, ft.head, tw, lane >> 5, inv_freq);
  fe_finish<TO, DI, 1, kFeCt>(acc, a, ft.head, tw + 32, lane >> 5, inv_freq);
}

// ------------------------------------------------------------------ backward
//
// Parameter gradients for upstream gradients dq (of q_idx) and dk (of k_idx),
// the hidden states held constant (the alignment loss reaches only the index
// projections: a stop-gradient on the indexer's input, atlas record of
// MiniMax M3, summary paragraph).  Per head vector, n = y / r, z = gain * n,
// out = R z:  dz = R^T dout;  dgain += dz * n;  dn = dz * gain;
// dy = (dn - n (dn . n) / DI) / r;  dW_h += dy x^T.
//   fe_bwd_local   recomputes y with the forward's GEMM and turns dout into
//                  dy in its epilogue: dy goes out token-major in bf16 (the
//                  forward's store pattern), and each workgroup's gain
//                  partial (its tokens summed in a fixed order) into its own
//                  slot;
//   fe_bwd_dw      dW = dy^T x over the tokens, split over token ranges into
//                  fp32 partial slices (dy and x staged transposed in LDS);
//   fe_bwd_reduce, fe_bwd_gain
//                  sum the slices and the gain partials in a fixed order,
//                  so the results are bitwise reproducible.
struct FeBwdArgs {
  FeArgs f;                  // forward inputs and sizes
  const float* dq;           // [T, G, DI]
  const float* dk;           // key-gradient rows, read at cu_k[b] + p
  bf16* dy;                  // [tp, (G+1)*DI], token-major
  int64_t tp;                // tokens rounded up to whole 128-token tiles
  float* gain_part;          // [tiles*(G+1), DI]
  float* dw_part;            // [splits, (G+1)*DI, d_model]
  int splits;
  int chunks_per_split;      // 64-token chunks per split
  int64_t tiles;
  int di;                    // DI
  int mrows;                 // (G+1)*DI rows of dW
  float* dw_q;               // [G*DI, d_model]
  float* dw_k;               // [DI, d_model]
  float* dgain_q;            // [DI]
  float* dgain_k;            // [DI]
};

// Each pair turned back by -angle (the transpose of the rotation).
template <int RT, int HT>
__device__ __forceinline__ void fe_rope_back(f32x16 (&v)[RT], int h, int64_t p, const double* inv_freq) {
#pragma unroll
  for (int rt = 0; rt < HT; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * rt + 8 * (r >> 2) + 4 * h + (r & 3);
      float sn, cs;
      fe_angle(p, inv_freq[i], sn, cs);
      const float va = v[rt][r], vb = v[rt + HT][r];
      v[rt][r] = va * cs + vb * sn;
      v[rt + HT][r] = vb * cs - va * sn;
    }
}

// Epilogue of the wave's column tile.  The gain contributions dz * n are
// summed over the wave's 32 token lanes right away into red[dim] (the wave's
// own LDS row), which keeps registers for the accumulators and dz.
template <int DI>
__device__ __forceinline__ void fe_bwd_finish(f32x16 (&acc)[DI / 32][1], const FeBwdArgs& b, int head, int64_t t,
                                              int h, const double* inv_freq, const float* gain, float* red) {
  constexpr int CT = 0;
  constexpr int RT = DI / 32;
  const FeArgs& a = b.f;
  float ss = 0.f;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) ss += acc[rt][CT][r] * acc[rt][CT][r];
  ss += shfl_xor_f(ss, 32);
  const bool valid = t < a.total && t < a.cu_q[a.batch];
  const float inv = 1.0f / sqrtf(ss / (float)DI + a.eps);
  f32x16 dz[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) dz[rt] = f32x16{};
  if (valid) {
    const int sq = fe_find(a.cu_q, a.batch, t);
    const int64_t M = a.cu_q[sq + 1] - a.cu_q[sq];
    const int64_t N = a.cu_k[sq + 1] - a.cu_k[sq];
    const int64_t p = N - M + (t - a.cu_q[sq]);
    const float* src = nullptr;
    if (head < a.G) src = b.dq + (t * a.G + head) * DI;
    else if (p >= 0 && p < N) src = b.dk + ((int64_t)a.cu_k[sq] + p) * DI;
    if (src) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(src + 32 * rt + 8 * q4 + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) dz[rt][4 * q4 + e] = v[e];
        }
      if (a.rope_dim == 64) fe_rope_back<RT, 1>(dz, h, p, inv_freq);
      else if (a.rope_dim == 128) fe_rope_back<RT, (RT >= 4 ? 2 : 1)>(dz, h, p, inv_freq);
    }
  }
  // invalid lanes hold dz = 0 from here on, so they add nothing
  const int col = lane_id() & 31;
  float dot = 0.f;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dim = 32 * rt + 8 * (r >> 2) + 4 * h + (r & 3);
      const float nv = acc[rt][CT][r] * inv;
      float c = dz[rt][r] * nv;
#pragma unroll
      for (int m = 16; m >= 1; m >>= 1) c += shfl_xor_f(c, m);
      if (col == 0) red[dim] = c;
      const float dn = dz[rt][r] * gain[dim];
      dz[rt][r] = dn;
      dot += dn * nv;
      __builtin_amdgcn_sched_barrier(0);  // one element at a time: bounds the live registers
    }
  dot += shfl_xor_f(dot, 32);
  const float dm = dot / (float)DI;
  bf16* dst = b.dy + t * b.mrows + head * DI;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float dy[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * q4 + e;
        dy[e] = valid ? (dz[rt][r] - acc[rt][CT][r] * inv * dm) * inv : 0.f;
      }
      fe_store4<bf16>(dst + 32 * rt + 8 * q4 + 4 * h, dy[0], dy[1], dy[2], dy[3]);
    }
}

template <int DI>
__global__ __launch_bounds__(kFeThreads, 2) void fe_bwd_local(FeBwdArgs b) {
  constexpr int RT = DI / 32;
  const FeArgs& a = b.f;
  __shared__ __attribute__((aligned(16))) bf16 w_lds[2][DI * FeLds<bf16>::stride];
  __shared__ double inv_freq[64];
  __shared__ float red[kFeThreads / kWave][DI];
  __shared__ float gain[DI];
  const FeTile ft = fe_tile(a.G);
  if (ft.tile * kFeBwdTok >= a.total) return;   // padding of the last group of 8 tiles
  if ((int)threadIdx.x < DI) gain[threadIdx.x] = (ft.head < a.G ? a.gain_q : a.gain_k)[threadIdx.x];
  const bf16* w = ft.head < a.G ? static_cast<const bf16*>(a.w_q) + (int64_t)ft.head * DI * a.d_model
                                : static_cast<const bf16*>(a.w_k);
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int col = lane & 31, h = lane >> 5;
  const int64_t t0 = ft.tile * kFeBwdTok + wave * 32;
  f32x16 acc[RT][1];
  fe_gemm<bf16, DI, 1>(a, w, t0, acc, w_lds);
  fe_inv_freq(inv_freq, a.rope_dim, a.log2_theta);
  fe_bwd_finish<DI>(acc, b, ft.head, t0 + col, h, inv_freq, gain, red[wave]);
  __syncthreads();
  // gain partial of this workgroup: its waves in order
  if ((int)threadIdx.x < DI) {
    float v = 0.f;
#pragma unroll
    for (int wv = 0; wv < kFeThreads / kWave; ++wv) v += red[wv][threadIdx.x];
    b.gain_part[(ft.tile * (a.G + 1) + ft.head) * DI + threadIdx.x] = v;
  }
}

// dW[o][c] = sum_t dy[t][o] x[t][c] for one 128 x 128 output tile and one
// token range.  Both operands need 8 consecutive tokens per lane and both are
// token-major in memory, so both are staged transposed in LDS: each thread
// loads 4 tokens x 8 columns (four 16-byte loads) and writes 8 runs of 4
// tokens.  Waves 2 x 2, each 64 rows x 64 columns.  Inside a 64-token chunk,
// lane half h and MFMA s use tokens 32h + 8s + 0..7 on both operands.
constexpr int kDwTok = 64;
constexpr int kDwS = kDwTok + 4;  // transposed tile rows: 136 B (two 8-byte reads per operand, conflict-free)

__global__ __launch_bounds__(kFeThreads, 2) void fe_bwd_dw(FeBwdArgs b) {
  const FeArgs& a = b.f;
  __shared__ __attribute__((aligned(16))) bf16 a_lds[2][128 * kDwS];
  __shared__ __attribute__((aligned(16))) bf16 b_lds[2][128 * kDwS];
  const int n_ot = (b.mrows + 127) / 128, n_ct = (a.d_model + 127) / 128;
  const int ot = blockIdx.x % n_ot;
  const int ct = (blockIdx.x / n_ot) % n_ct;
  const int split = blockIdx.x / (n_ot * n_ct);
  const int o0 = 128 * ot, c0 = 128 * ct;
  const int64_t ch_lo = (int64_t)split * b.chunks_per_split;
  const int64_t ch_hi = min(ch_lo + b.chunks_per_split, b.tp / kDwTok);
  const bf16* x = static_cast<const bf16*>(a.x);
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int col = lane & 31, h = lane >> 5;
  const int wo = wave & 1, wc = wave >> 1;

  // staging unit of this thread: tokens 4*tq .. 4*tq+3 of the chunk, rows /
  // columns 8*oc .. 8*oc+7 of the tile (past the end: any valid ones, not stored)
  bf16x8 ar[4], br[4];
  const int tq = tid & 15, oc = tid >> 4;
  const int arow = min(o0 + 8 * oc, b.mrows - 8);
  const int bcol = min(c0 + 8 * oc, a.d_model - 8);
  auto load = [&](int64_t ch) {
    const int64_t k0 = ch * kDwTok;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = k0 + 4 * tq + j;
      ar[j] = load8(b.dy + t * b.mrows + arow);
      br[j] = load8(x + (t < a.total ? t : a.total - 1) * a.d_model + bcol);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      *reinterpret_cast<bf16x4*>(&a_lds[buf][(8 * oc + e) * kDwS + 4 * tq]) =
          bf16x4{ar[0][e], ar[1][e], ar[2][e], ar[3][e]};
      *reinterpret_cast<bf16x4*>(&b_lds[buf][(8 * oc + e) * kDwS + 4 * tq]) =
          bf16x4{br[0][e], br[1][e], br[2][e], br[3][e]};
    }
  };
  auto frag = [&](const bf16* p) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 4);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x16{};
  if (ch_lo < ch_hi) {
    load(ch_lo);
    store(0);
    __syncthreads();
    for (int64_t ch = ch_lo; ch < ch_hi; ++ch) {
      const int cur = (int)((ch - ch_lo) & 1);
      const bool more = ch + 1 < ch_hi;
      if (more) load(ch + 1);
#pragma unroll
      for (int st = 0; st < kDwTok / 16; ++st) {
        const int toff = 32 * h + 8 * st;
        bf16x8 av[2], bv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          av[i] = frag(&a_lds[cur][(64 * wo + 32 * i + col) * kDwS + toff]);
          bv[i] = frag(&b_lds[cur][(64 * wc + 32 * i + col) * kDwS + toff]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mma32(av[i], bv[j], acc[i][j]);
      }
      if (more) store(cur ^ 1);
      __syncthreads();
    }
  }
  // partial slice: lane holds rows 8(r/4) + 4h + r%4 of each 32-row tile, column col
  float* part = b.dw_part + (int64_t)split * b.mrows * a.d_model;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = c0 + 64 * wc + 32 * j + col;
      if (c >= a.d_model) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = o0 + 64 * wo + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        if (o < b.mrows) part[(int64_t)o * a.d_model + c] = acc[i][j][r];
      }
    }
}

// dW = the sum of the slices in split order (grid-stride in 4-float units).
__global__ __launch_bounds__(256) void fe_bwd_reduce(FeBwdArgs b) {
  const FeArgs& a = b.f;
  const int64_t n4 = (int64_t)b.mrows * a.d_model / 4;
  const int64_t qrows4 = (int64_t)a.G * b.di * a.d_model / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    f32x4 v = *reinterpret_cast<const f32x4*>(b.dw_part + 4 * i);
    for (int sp = 1; sp < b.splits; ++sp)
      v += *reinterpret_cast<const f32x4*>(b.dw_part + (int64_t)sp * b.mrows * a.d_model + 4 * i);
    if (i < qrows4) *reinterpret_cast<f32x4*>(b.dw_q + 4 * i) = v;
    else *reinterpret_cast<f32x4*>(b.dw_k + 4 * (i - qrows4)) = v;
  }
}

// The gains: workgroup i sums dim i over the workgroup partials, query heads
// into dgain_q and the key head into dgain_k.  Thread j takes the slots
// j, j + 256, ... in order, then a fixed pairwise tree in LDS.
__global__ __launch_bounds__(256) void fe_bwd_gain(FeBwdArgs b) {
  const int G1 = b.f.G + 1, i = blockIdx.x, j = threadIdx.x;
  __shared__ float sq[256], sk[256];
  float gq = 0.f, gk = 0.f;
  for (int64_t slot = j; slot < b.tiles * G1; slot += 256) {
    const float v = b.gain_part[slot * b.di + i];
    if (slot % G1 < G1 - 1) gq += v; else gk += v;
  }
  sq[j] = gq;
  sk[j] = gk;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (j < w) {
      sq[j] += sq[j + w];
      sk[j] += sk[j + w];
    }
    __syncthreads();
  }
  if (j == 0) {
    b.dgain_q[i] = sq[0];
    b.dgain_k[i] = sk[0];
  }
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

__global__ __launch_bounds__(256) void fe_fill_zero(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

static int64_t fe_cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static size_t fe_align(size_t x) { return (x + 255) / 256 * 256; }

FrontendBwdPlan plan_index_frontend_bwd(int64_t total, int d_model, int G, int DI) {
  FrontendBwdPlan pl;
  pl.tiles = fe_cdiv(total, kFeBwdTok);
  pl.tp = pl.tiles * kFeBwdTok;
  pl.mrows = (G + 1) * DI;
  const int64_t cells = fe_cdiv(pl.mrows, 128) * fe_cdiv(d_model, 128);
  const int64_t chunks = pl.tp / kDwTok;
  int64_t splits = chunks > 0 ? fe_cdiv(1024, cells) : 1;
  if (splits > chunks && chunks > 0) splits = chunks;
  pl.chunks_per_split = (int)(chunks > 0 ? fe_cdiv(chunks, splits) : 1);
  pl.splits = (int)(chunks > 0 ? fe_cdiv(chunks, pl.chunks_per_split) : 1);
  pl.dy_off = 0;
  pl.gain_off = fe_align((size_t)pl.mrows * pl.tp * sizeof(bf16));
  pl.dw_off = pl.gain_off + fe_align((size_t)pl.tiles * (G + 1) * DI * sizeof(float));
  pl.workspace_bytes = total > 0 ? pl.dw_off + fe_align((size_t)pl.splits * pl.mrows * d_model * sizeof(float)) : 0;
  return pl;
}

hipError_t launch_index_frontend_bwd(const FrontendBwdPlan& pl, const FrontendLaunch& f, const float* dq,
                                     const float* dk, float* dw_q, float* dw_k, float* dgain_q, float* dgain_k,
                                     void* ws, hipStream_t st) {
  if (f.total == 0) {
    const int64_t nq = (int64_t)f.G * f.DI * f.d_model, nk = (int64_t)f.DI * f.d_model;
    hipLaunchKernelGGL(fe_fill_zero, dim3(1024), dim3(256), 0, st, dw_q, nq);
    hipLaunchKernelGGL(fe_fill_zero, dim3(1024), dim3(256), 0, st, dw_k, nk);
    hipLaunchKernelGGL(fe_fill_zero, dim3(1), dim3(256), 0, st, dgain_q, (int64_t)f.DI);
    hipLaunchKernelGGL(fe_fill_zero, dim3(1), dim3(256), 0, st, dgain_k, (int64_t)f.DI);
    return hipGetLastError();
  }
  char* w = static_cast<char*>(ws);
  FeBwdArgs b;
  FeArgs& a = b.f;
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
  a.q_out = nullptr;
  a.k_out = nullptr;
  b.dq = dq;
  b.dk = dk;
  b.dy = reinterpret_cast<bf16*>(w + pl.dy_off);
  b.tp = pl.tp;
  b.gain_part = reinterpret_cast<float*>(w + pl.gain_off);
  b.dw_part = reinterpret_cast<float*>(w + pl.dw_off);
  b.splits = pl.splits;
  b.chunks_per_split = pl.chunks_per_split;
  b.tiles = pl.tiles;
  b.di = f.DI;
  b.mrows = pl.mrows;
  b.dw_q = dw_q;
  b.dw_k = dw_k;
  b.dgain_q = dgain_q;
  b.dgain_k = dgain_k;
  const dim3 grid_local((unsigned)(fe_cdiv(pl.tiles, 8) * 8 * (f.G + 1)));
  if (f.DI == 64) hipLaunchKernelGGL(fe_bwd_local<64>, grid_local, dim3(kFeThreads), 0, st, b);
  else hipLaunchKernelGGL(fe_bwd_local<128>, grid_local, dim3(kFeThreads), 0, st, b);
  const int64_t cells = fe_cdiv(pl.mrows, 128) * fe_cdiv(f.d_model, 128);
  hipLaunchKernelGGL(fe_bwd_dw, dim3((unsigned)(cells * pl.splits)), dim3(kFeThreads), 0, st, b);
  const int64_t n4 = (int64_t)pl.mrows * f.d_model / 4;
  const int64_t rg = fe_cdiv(n4, 256) < 2048 ? fe_cdiv(n4, 256) : 2048;
  hipLaunchKernelGGL(fe_bwd_reduce, dim3((unsigned)rg), dim3(256), 0, st, b);
  hipLaunchKernelGGL(fe_bwd_gain, dim3((unsigned)f.DI), dim3(256), 0, st, b);
  return hipGetLastError();
}

}  // namespace msa
