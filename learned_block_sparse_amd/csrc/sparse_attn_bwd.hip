// sparse_attn_bwd.hip -- gradients of the MSA main branch on gfx950.
//
// Method: "MiniMax Sparse Attention: let each query pick its own blocks",
// section "The mechanism, precisely": the main branch is ordinary softmax
// attention over the keys of the selected blocks, so its gradients are those
// of softmax attention restricted to that key set.  The atlas record of
// MiniMax M3 (summary, "What the report claims is novel") describes training
// with this main branch; the LSE the forward pass returns is what lets the
// backward pass recompute the probabilities without a second softmax pass.
//
// For a row, head h and attended key j, with P_j = exp(z_j - lse):
//   dP_j = dO . v_j,  delta = dO . O  (= sum_j P_j dP_j),  dS_j = P_j (dP_j - delta)
//   dq = scale sum_j dS_j k_j,  dk_j += scale dS_j q,  dv_j += P_j dO
// (dk, dv summed over every row and head of the group that attends j).
//
// Kernels (bf16 inputs, fp32 accumulation and fp32 gradients):
//   bwd_zero   dk = dv = 0 for the key rows of the call
//   bwd_delta  delta[row, head] = dO . O
//   bwd_sort   sorts each bucket's edge list (the lists the KV-outer forward
//              builds, placed by atomics in no fixed order), so the order in
//              which bwd_dkdv sums the edges, and so every rounding, is fixed
//   bwd_dkdv   KV-outer, one workgroup per (sequence, group, block) bucket of
//              the selection edge lists.  Each of the 4 waves owns 32 keys of
//              the block and keeps their K and V rows in registers as MFMA
//              operands; the edges run in pairs (2
//              queries x 16 heads = 32 MFMA rows), whose Q and dO are staged in
//              LDS twice, row-major for S = Q K^T and dP = dO V^T and
//              transposed for dV += P^T dO and dK += dS^T Q, so the P and dS
//              registers of the first two products are directly the A
//              operands of the last two.  dK and dV accumulate over the
//              bucket in registers and are added to the output once per
//              window of query rows.
//   bwd_dq     query-outer, one wave per (row, group) as in the forward
//              kernel: S^T = K Q^T and dP^T = V dO^T with the heads as the 16
//              MFMA columns, then dQ^T += K^T dS^T through a wave-private
//              transposed K tile.
// No atomics touch the arithmetic: every result is bitwise reproducible.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kBwdThreads = 256;
constexpr int kBwdRow = 136;      // LDS row of Q / dO for one MFMA row: 128 bf16 + 8 pad
constexpr int kBwdT = 36;         // LDS row of Q^T / dO^T for one dim: 32 columns + 4 pad
constexpr int kSortMax = 8192;    // edges of one bucket in one window (<= rows per window)
constexpr int kQtStride = 36;     // bwd_dq: wave-private K^T tile row (32 keys + 4 pad)
constexpr float kLog2e = 1.4426950408889634f;

struct BwdKernelArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const bf16* dout;
  const float* lse;
  const int32_t* block_idx;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int batch, G, Hq, topk, nb_max;
  int64_t rows_bound, row_lo;
  float scale, scale_log2;
  const int32_t* offsets;
  int32_t* edges;
  float* delta;
  float* dq;
  float* dk;
  float* dv;
};

__device__ __forceinline__ int bwd_find(const int32_t* cu, int n, int64_t x) {
  int lo = 0, hi = n;  // cu[lo] <= x < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// dk = dv = 0 over the call's key rows (cu_k[batch] of them), grid-stride.
__global__ __launch_bounds__(256) void bwd_zero(BwdKernelArgs a) {
  const int64_t n = (int64_t)a.cu_k[a.batch] * a.G * kHeadDim / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    reinterpret_cast<f32x4*>(a.dk)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    reinterpret_cast<f32x4*>(a.dv)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// delta[row, head] = sum_d dO * O: 32 threads per (row, head), 4 dims each.
__global__ __launch_bounds__(256) void bwd_delta(BwdKernelArgs a) {
  const int64_t rh = (int64_t)blockIdx.x * 8 + threadIdx.x / 32;
  if (rh >= a.rows_bound * a.Hq || rh / a.Hq >= a.cu_q[a.batch]) return;
  const int d0 = (threadIdx.x & 31) * 4;
  const bf16x4 o = *reinterpret_cast<const bf16x4*>(a.o + rh * kHeadDim + d0);
  const bf16x4 g = *reinterpret_cast<const bf16x4*>(a.dout + rh * kHeadDim + d0);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += (float)o[i] * (float)g[i];
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) s += __shfl_xor(s, m, 32);
  if ((threadIdx.x & 31) == 0) a.delta[rh] = s;
}

// One pair of edges, staged by the whole workgroup: each thread holds two
// 16-byte pieces of Q and two of dO (piece pc = tid + 256 u: MFMA row pc / 16,
// dims 8 (pc % 16) .. +7).
struct PairStage {
  bf16x8 q[2];
  bf16x8 g[2];
  float lse, delta;  // threads 0..31: MFMA row tid
  int pos;           // threads 0..1: position of query tid of the pair
};

__device__ __forceinline__ void bwd_load_pair(const BwdKernelArgs& a, PairStage& S, int e, int e_hi, int g, int R,
                                              int N, int M, int64_t q0) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int pc = tid + kBwdThreads * u;
    const int col = pc >> 4, d8 = (pc & 15) * 8;
    const int jq = col >> 4, h = col & 15;
    const bool ok = e + jq < e_hi && h < R;
    const int64_t t = ok ? a.row_lo + (a.edges[e + jq] >> 4) : 0;
    const int64_t off = (t * a.Hq + g * R + (ok ? h : 0)) * kHeadDim + d8;
    S.q[u] = ok ? load8(a.q + off) : zero8<bf16>();
    S.g[u] = ok ? load8(a.dout + off) : zero8<bf16>();
  }
  if (tid < 32) {
    const int jq = tid >> 4, h = tid & 15;
    const bool ok = e + jq < e_hi && h < R;
    const int64_t t = ok ? a.row_lo + (a.edges[e + jq] >> 4) : 0;
    // an empty MFMA row gets lse = +inf, so its probabilities are exactly 0
    S.lse = ok ? a.lse[t * a.Hq + g * R + h] * kLog2e : __builtin_inff();
    S.delta = ok ? a.delta[t * a.Hq + g * R + h] : 0.f;
  } else if (tid < 34) {
    const int jq = tid - 32;
    const bool ok = e + jq < e_hi;
    const int64_t t = ok ? a.row_lo + (a.edges[e + jq] >> 4) : 0;
    S.pos = ok ? (int)((int64_t)N - M + (t - q0)) : -1;
  }
}

struct BwdLds {
  bf16 q_rm[2][32 * kBwdRow];
  bf16 g_rm[2][32 * kBwdRow];
  bf16 q_t[2][kHeadDim * kBwdT];
  bf16 g_t[2][kHeadDim * kBwdT];
  float lse[2][32];
  float delta[2][32];
  int pos[2][2];
};

__device__ __forceinline__ void bwd_store_pair(BwdLds& L, int buf, const PairStage& S) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int pc = tid + kBwdThreads * u;
    const int col = pc >> 4, d8 = (pc & 15) * 8;
    *reinterpret_cast<bf16x8*>(&L.q_rm[buf][col * kBwdRow + d8]) = S.q[u];
    *reinterpret_cast<bf16x8*>(&L.g_rm[buf][col * kBwdRow + d8]) = S.g[u];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      L.q_t[buf][(d8 + e) * kBwdT + col] = S.q[u][e];
      L.g_t[buf][(d8 + e) * kBwdT + col] = S.g[u][e];
    }
  }
  if (tid < 32) {
    L.lse[buf][tid] = S.lse;
    L.delta[buf][tid] = S.delta;
  } else if (tid < 34) {
    L.pos[buf][tid - 32] = S.pos;
  }
}

// Sort each bucket's edge codes ascending (bitonic, in LDS), in place.  The
// lists are placed by atomics in no fixed order; sorting them fixes the order
// in which bwd_dkdv sums the edges, so dK and dV are reproducible bit for bit.
__global__ __launch_bounds__(kBwdThreads) void bwd_sort(BwdKernelArgs a) {
  __shared__ int32_t srt[kSortMax];
  const int nbk = a.batch * a.G * a.nb_max;
  const int bucket = blockIdx.x;
  if (bucket >= nbk) return;
  const int e_lo = a.offsets[bucket];
  const int n = a.offsets[bucket + 1] - e_lo;
  if (n <= 1) return;
  const int tid = threadIdx.x;
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  for (int i = tid; i < n2; i += kBwdThreads) srt[i] = i < n ? a.edges[e_lo + i] : 0x7fffffff;
  __syncthreads();
  for (int kk = 2; kk <= n2; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n2; i += kBwdThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const int32_t x = srt[i], y = srt[ixj];
          if ((x > y) == ((i & kk) == 0)) {
            srt[i] = y;
            srt[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < n; i += kBwdThreads) a.edges[e_lo + i] = srt[i];
}

__global__ __launch_bounds__(kBwdThreads) void bwd_dkdv(BwdKernelArgs a) {
  __shared__ __attribute__((aligned(16))) BwdLds L;
  const int nbk = a.batch * a.G * a.nb_max;
  const int bucket = blockIdx.x;
  if (bucket >= nbk) return;
  const int e_lo = a.offsets[bucket], e_hi = a.offsets[bucket + 1];
  const int n = e_hi - e_lo;
  if (n <= 0) return;
  const int c = bucket % a.nb_max;
  const int g = (bucket / a.nb_max) % a.G;
  const int b = bucket / (a.nb_max * a.G);
  const int64_t kb0 = a.cu_k[b];
  const int N = a.cu_k[b + 1] - a.cu_k[b];
  const int64_t q0 = a.cu_q[b];
  const int M = a.cu_q[b + 1] - a.cu_q[b];
  const int R = a.Hq / a.G;
  const int64_t rs = (int64_t)a.G * kHeadDim;
  const int tid = threadIdx.x;

  const int wave = tid >> 6;
  const int lane = lane_id();
  const int col = lane & 31;  // MFMA row of A / column of B and C
  const int a32 = lane >> 5;
  // this wave's 32 keys: K and V rows as the B operands of S = Q K^T and
  // dP = dO V^T (column = key, 8 dims per k-step half); rows past the
  // sequence end clamp to its last row and are masked (key > every p)
  const int key_blk = 32 * wave + col;
  const int key_seq = c * kBlock + key_blk;
  const int64_t krow = kb0 + (key_seq < N ? key_seq : N - 1);
  bf16x8 kf[kHeadDim / 16], vf[kHeadDim / 16];
#pragma unroll
  for (int ks = 0; ks < kHeadDim / 16; ++ks) {
    kf[ks] = load8(a.k + krow * rs + g * kHeadDim + 16 * ks + 8 * a32);
    vf[ks] = load8(a.v + krow * rs + g * kHeadDim + 16 * ks + 8 * a32);
  }
  f32x16 dk_acc[kHeadDim / 32], dv_acc[kHeadDim / 32];
#pragma unroll
  for (int dt = 0; dt < kHeadDim / 32; ++dt) {
    dk_acc[dt] = f32x16{};
    dv_acc[dt] = f32x16{};
  }

  const int npairs = (n + 1) / 2;
  PairStage S;
  bwd_load_pair(a, S, e_lo, e_hi, g, R, N, M, q0);
  bwd_store_pair(L, 0, S);
  __syncthreads();
  for (int pi = 0; pi < npairs; ++pi) {
    const int buf = pi & 1;
    const bool more = pi + 1 < npairs;
    if (more) bwd_load_pair(a, S, e_lo + 2 * (pi + 1), e_hi, g, R, N, M, q0);

    // S[row][key] and dP[row][key], rows = (query of the pair, head)
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 16; ++ks) {
      const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&L.q_rm[buf][col * kBwdRow + 16 * ks + 8 * a32]);
      const bf16x8 ga = *reinterpret_cast<const bf16x8*>(&L.g_rm[buf][col * kBwdRow + 16 * ks + 8 * a32]);
      s = mma32(qa, kf[ks], s);
      dp = mma32(ga, vf[ks], dp);
    }
    // C layout: this lane's key, rows 8 (r / 4) + 4 a32 + r % 4
    bf16x8 pa[2], dsa[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * a32 + (r & 3);
      const bool live = key_seq <= L.pos[buf][row >> 4];
      const float p = live ? __builtin_amdgcn_exp2f(s[r] * a.scale_log2 - L.lse[buf][row]) : 0.f;
      const float ds = p * (dp[r] - L.delta[buf][row]);
      pa[r >> 3][r & 7] = bf16(p);
      dsa[r >> 3][r & 7] = bf16(ds);
    }
    // dV[key][d] += sum_row P[row][key] dO[row][d]; dK likewise with dS and Q.
    // k-step s2 covers rows 16 s2 .. +15; slot i of lane half a32 is row
    // 16 s2 + 4 a32 + i (i < 4) or 16 s2 + 8 + 4 a32 + i - 4, matching the
    // registers 8 s2 .. 8 s2 + 7 above.
#pragma unroll
    for (int dt = 0; dt < kHeadDim / 32; ++dt) {
      const int d = 32 * dt + col;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int c0 = 16 * s2 + 4 * a32;
        const bf16x4 glo = *reinterpret_cast<const bf16x4*>(&L.g_t[buf][d * kBwdT + c0]);
        const bf16x4 ghi = *reinterpret_cast<const bf16x4*>(&L.g_t[buf][d * kBwdT + c0 + 8]);
        const bf16x4 qlo = *reinterpret_cast<const bf16x4*>(&L.q_t[buf][d * kBwdT + c0]);
        const bf16x4 qhi = *reinterpret_cast<const bf16x4*>(&L.q_t[buf][d * kBwdT + c0 + 8]);
        const bf16x8 gb = {glo[0], glo[1], glo[2], glo[3], ghi[0], ghi[1], ghi[2], ghi[3]};
        const bf16x8 qb = {qlo[0], qlo[1], qlo[2], qlo[3], qhi[0], qhi[1], qhi[2], qhi[3]};
        dv_acc[dt] = mma32(pa[s2], gb, dv_acc[dt]);
        dk_acc[dt] = mma32(dsa[s2], qb, dk_acc[dt]);
      }
    }
    if (more) bwd_store_pair(L, buf ^ 1, S);
    __syncthreads();
  }

  // ---- add this window's contribution: lane column d = 32 dt + col, rows =
  // keys 8 (r / 4) + 4 a32 + r % 4 of the wave's 32
#pragma unroll
  for (int dt = 0; dt < kHeadDim / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = c * kBlock + 32 * wave + 8 * (r >> 2) + 4 * a32 + (r & 3);
      if (kk >= N) continue;
      const int64_t off = (kb0 + kk) * rs + g * kHeadDim + 32 * dt + col;
      a.dk[off] += dk_acc[dt][r] * a.scale;
      a.dv[off] += dv_acc[dt][r];
    }
}

// K rows key0 + 32 ks .. +31 as the units of the transposed staging: unit
// u = (key quad u % 8, dim octet u / 8); lane handles u = lane and lane + 64.
__device__ __forceinline__ void bwd_load_k_chunk(const bf16* kseq, int64_t rs, int64_t key0, int64_t p, int ks,
                                                 int lane, bf16x8 (&r)[2][4]) {
#pragma unroll
  for (int uu = 0; uu < 2; ++uu) {
    const int u = lane + 64 * uu;
    const int kq = u & 7, o8 = u >> 3;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      int64_t key = key0 + 32 * ks + 4 * kq + jj;
      if (key > p) key = p;
      r[uu][jj] = load8(kseq + key * rs + 8 * o8);
    }
  }
}

__global__ __launch_bounds__(kBwdThreads) void bwd_dq(BwdKernelArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 kt_all[kBwdThreads / kWave][kHeadDim * kQtStride];
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  bf16* ktile = kt_all[wave];
  const int G = a.G;
  const int64_t item = (int64_t)blockIdx.x * (kBwdThreads / kWave) + wave;
  if (item >= a.rows_bound * G) return;
  const int64_t t = item % a.rows_bound;
  const int g = (int)(item / a.rows_bound);
  if (t >= a.cu_q[a.batch]) return;
  const int b = bwd_find(a.cu_q, a.batch, t);
  const int64_t q0 = a.cu_q[b];
  const int M = a.cu_q[b + 1] - a.cu_q[b];
  const int64_t kb0 = a.cu_k[b];
  const int N = a.cu_k[b + 1] - a.cu_k[b];
  const int64_t p = (int64_t)N - M + (t - q0);

  const int R = a.Hq / G;
  const int h = lane & 15;
  const int a4 = lane >> 4;
  const int hq = g * R + h;
  const bool head_ok = h < R;
  const int64_t qoff = (t * a.Hq + (head_ok ? hq : g * R)) * kHeadDim;
  // B operands Q^T and dO^T: column h, dims 32 ds + 8 a4 .. +7
  bf16x8 qf[kHeadDim / 32], gf[kHeadDim / 32];
#pragma unroll
  for (int ds = 0; ds < kHeadDim / 32; ++ds) {
    qf[ds] = head_ok ? load8(a.q + qoff + 32 * ds + 8 * a4) : zero8<bf16>();
    gf[ds] = head_ok ? load8(a.dout + qoff + 32 * ds + 8 * a4) : zero8<bf16>();
  }
  // per column (head): lse in log2 units (+inf for a missing head: P = 0) and delta
  const float lse2 = head_ok ? a.lse[t * a.Hq + hq] * kLog2e : __builtin_inff();
  const float dlt = head_ok ? a.delta[t * a.Hq + hq] : 0.f;

  f32x4 acc[kHeadDim / 16];
#pragma unroll
  for (int dt = 0; dt < kHeadDim / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (p >= 0) {
    const int64_t local = p / kBlock;
    const int32_t* sel = a.block_idx + (t * G + g) * a.topk;
    const int64_t rs = (int64_t)G * kHeadDim;
    const bf16* kseq = a.k + kb0 * rs + g * kHeadDim;
    const bf16* vseq = a.v + kb0 * rs + g * kHeadDim;
    for (int i = 0; i < a.topk; ++i) {
      const int c = sel[i];
      bool seen = false;  // Sel is a set
      for (int j = 0; j < i; ++j) seen = seen || sel[j] == c;
      if (c < 0 || c > local || seen) continue;
      const int64_t key0 = (int64_t)c * kBlock;

      // S^T and dP^T for the block's 8 tiles of 16 keys (A row = lane % 16)
      f32x4 st[kBlock / 16], dpt[kBlock / 16];
#pragma unroll
      for (int kt = 0; kt < kBlock / 16; ++kt) {
        int64_t key = key0 + 16 * kt + h;
        if (key > p) key = p;
        const bf16* kp = kseq + key * rs + 8 * a4;
        const bf16* vp = vseq + key * rs + 8 * a4;
        bf16x8 kfr[kHeadDim / 32], vfr[kHeadDim / 32];
#pragma unroll
        for (int ds = 0; ds < kHeadDim / 32; ++ds) {
          kfr[ds] = load8(kp + 32 * ds);
          vfr[ds] = load8(vp + 32 * ds);
        }
        f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < kHeadDim / 32; ++ds) {
          x = mma16(kfr[ds], qf[ds], x);
          y = mma16(vfr[ds], gf[ds], y);
        }
        st[kt] = x;
        dpt[kt] = y;
      }
      // dS^T = P^T (dP^T - delta); this lane: head h, keys 16 kt + 4 a4 + r
      const int64_t rel = p - key0 - 4 * a4;
      const int lim = rel > kBlock ? kBlock : (int)rel;
#pragma unroll
      for (int kt = 0; kt < kBlock / 16; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pr = (16 * kt + r > lim) ? 0.f : __builtin_amdgcn_exp2f(st[kt][r] * a.scale_log2 - lse2);
          st[kt][r] = pr * (dpt[kt][r] - dlt);
        }

      // dQ^T[d][h] += K^T[d][key] dS^T[key][h], 32 keys at a time
#pragma unroll
      for (int ks = 0; ks < kBlock / 32; ++ks) {
        bf16x8 kr[2][4];
        bwd_load_k_chunk(kseq, rs, key0, p, ks, lane, kr);
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
          const int u = lane + 64 * uu;
          const int kq = u & 7, o8 = u >> 3;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            bf16x4 w = {kr[uu][0][e], kr[uu][1][e], kr[uu][2][e], kr[uu][3][e]};
            *reinterpret_cast<bf16x4*>(ktile + (8 * o8 + e) * kQtStride + 4 * kq) = w;
          }
        }
        __builtin_amdgcn_wave_barrier();
        // B operand dS^T: slots r < 4 -> key 32 ks + 4 a4 + r, r >= 4 -> 32 ks + 16 + 4 a4 + r - 4
        bf16x8 pb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pb[r] = bf16(st[2 * ks][r]);
          pb[4 + r] = bf16(st[2 * ks + 1][r]);
        }
#pragma unroll
        for (int dt = 0; dt < kHeadDim / 16; ++dt) {
          const bf16* src = ktile + (16 * dt + h) * kQtStride + 4 * a4;
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(src);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(src + 16);
          const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc[dt] = mma16(va, pb, acc[dt]);
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  if (!head_ok) return;
  float* dq = a.dq + (t * a.Hq + hq) * kHeadDim;
#pragma unroll
  for (int dt = 0; dt < kHeadDim / 16; ++dt)
    *reinterpret_cast<f32x4*>(dq + 16 * dt + 4 * a4) = acc[dt] * a.scale;
}

BwdPlan plan_bwd(int batch, int max_q_len, int max_kv_len, int Hq, int G, int topk) {
  BwdPlan pl;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  pl.nb_max = (max_kv_len + kBlock - 1) / kBlock;
  pl.nbuckets = batch * G * pl.nb_max;
  pl.rows_bound = (int64_t)batch * max_q_len;
  const int64_t win = kvo_window_rows() < kSortMax ? kvo_window_rows() : kSortMax;
  pl.window = pl.rows_bound < win ? pl.rows_bound : win;
  const size_t nbk = (size_t)pl.nbuckets;
  size_t off = 0;
  pl.counts_off = off;  off += al(nbk * 4);
  pl.offsets_off = off; off += al((nbk + 1) * 4);
  pl.chunks_off = off;  off += al((nbk + 1) * 4);
  pl.cursor_off = off;  off += al(nbk * 4);
  pl.edges_off = off;   off += al((size_t)pl.window * G * topk * 4);
  pl.delta_off = off;   off += al((size_t)pl.rows_bound * Hq * 4);
  pl.workspace_bytes = off;
  return pl;
}

hipError_t launch_sparse_attn_bwd(const BwdPlan& pl, const BwdArgs& x, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  BwdKernelArgs a;
  a.q = static_cast<const bf16*>(x.fwd.q);
  a.k = static_cast<const bf16*>(x.fwd.k);
  a.v = static_cast<const bf16*>(x.fwd.v);
  a.o = static_cast<const bf16*>(x.o);
  a.dout = static_cast<const bf16*>(x.dout);
  a.lse = x.lse;
  a.block_idx = x.fwd.block_idx;
  a.cu_q = x.fwd.cu_q;
  a.cu_k = x.fwd.cu_k;
  a.batch = x.fwd.batch;
  a.G = x.fwd.Hkv;
  a.Hq = x.fwd.Hq;
  a.topk = x.fwd.topk;
  a.nb_max = pl.nb_max;
  a.rows_bound = pl.rows_bound;
  a.row_lo = 0;
  a.scale = x.fwd.scale;
  a.scale_log2 = x.fwd.scale * kLog2e;
  int32_t* counts = reinterpret_cast<int32_t*>(w + pl.counts_off);
  int32_t* offsets = reinterpret_cast<int32_t*>(w + pl.offsets_off);
  int32_t* chunks = reinterpret_cast<int32_t*>(w + pl.chunks_off);
  int32_t* cursor = reinterpret_cast<int32_t*>(w + pl.cursor_off);
  a.offsets = offsets;
  a.edges = reinterpret_cast<int32_t*>(w + pl.edges_off);
  a.delta = reinterpret_cast<float*>(w + pl.delta_off);
  a.dq = x.dq;
  a.dk = x.dk;
  a.dv = x.dv;

  hipLaunchKernelGGL(bwd_zero, dim3(2048), dim3(256), 0, st, a);
  hipLaunchKernelGGL(bwd_delta, dim3((unsigned)((pl.rows_bound * a.Hq + 7) / 8)), dim3(256), 0, st, a);
  for (int64_t r0 = 0; r0 < pl.rows_bound; r0 += pl.window) {
    const int64_t r1 = r0 + pl.window < pl.rows_bound ? r0 + pl.window : pl.rows_bound;
    hipError_t e = build_edge_lists(x.fwd, pl.nb_max, r0, r1, counts, offsets, chunks, cursor, a.edges, st);
    if (e != hipSuccess) return e;
    a.row_lo = r0;
    hipLaunchKernelGGL(bwd_sort, dim3((unsigned)pl.nbuckets), dim3(kBwdThreads), 0, st, a);
    hipLaunchKernelGGL(bwd_dkdv, dim3((unsigned)pl.nbuckets), dim3(kBwdThreads), 0, st, a);
  }
  a.row_lo = 0;
  const int64_t items = pl.rows_bound * a.G;
  hipLaunchKernelGGL(bwd_dq, dim3((unsigned)((items + 3) / 4)), dim3(kBwdThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace msa
