// sparse_attn.hip -- MSA main branch on gfx950: exact attention over the
// selected key blocks, plus the log-sum-exp combine of split selections.
//
// Method: "MiniMax Sparse Attention: let each query pick its own blocks",
// section "The mechanism, precisely" (main branch: exact attention over only
// the selected blocks; every head of a group reuses the group's block set)
// and the atlas record of MiniMax M3, summary and kernel list (standard
// scaled dot-product softmax; a two-phase combine over per-partial LSE
// buffers with no atomics; LSE produced by the forward pass).
//
// One wave owns one work item (query row, group, split) and all r <= 16 heads
// of that group: the heads are the 16 columns of a 16x16 MFMA tile, so every
// K/V element the wave gathers serves all heads of the group.  Scores are
// computed transposed, S^T = K Q^T (keys x heads): a lane's 4 output registers
// are 4 keys of one head, which makes the softmax row statistics a register
// reduction plus two lane swaps, and the P^T fragment of the following
// O^T += V^T P^T MFMA is exactly the registers the lane already holds.  V^T is
// staged through a wave-private LDS tile, written transposed (keys
// contiguous) so each MFMA operand is two 8-byte LDS reads.  Online softmax
// (FlashAttention-style running max / sum) works in log2 units with exp2.
// Waves never synchronise with each other.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kAttnThreads = 256;  // 4 independent waves

template <typename T>
struct VtTile {
  static constexpr int kStride = 32 + 4;  // 32 keys per d-row plus padding (elements)
  static constexpr int kElems = kHeadDim * kStride;
};

struct AttnKernelArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_idx;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int64_t* k_offsets;
  const int32_t* k_lens;
  int batch;
  int64_t rows_bound;
  int Hq, Hkv, topk, nsplit, bps;
  float scale_log2;  // softmax scale * log2(e)
  void* out;
  float* lse;
  float* block_lse;  // [rows, Hq, topk] or null
  float* part_o;
  float* part_lse;
};

__device__ __forceinline__ int find_row_seq(const int32_t* cu, int batch, int64_t row) {
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, float a, float b, float c, float d) {
  bf16x4 v = {bf16(a), bf16(b), bf16(c), bf16(d)};
  *reinterpret_cast<bf16x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
}

// Eight K/V elements in registers as loaded: the compute-type fragment, or
// for E4M3 storage the 8 raw bytes, widened to bf16 where they are used (so a
// block's K and V fit in registers together).
template <typename T, typename TKV> struct KvReg { using type = frag8<T>; };
template <> struct KvReg<bf16, fp8e4m3> { using type = u32x2; };
template <typename T, typename TKV>
using kvreg = typename KvReg<T, TKV>::type;

template <typename T, typename TKV>
__device__ __forceinline__ kvreg<T, TKV> load_kvreg(const TKV* p) {
  if constexpr (sizeof(TKV) == 1) return *reinterpret_cast<const u32x2*>(p);
  else return load8(p);
}
template <typename T, typename R>
__device__ __forceinline__ frag8<T> kv_op(const R& r) {
  if constexpr (sizeof(R) == 8) return widen8_e4m3(r);
  else return r;
}

// V rows key0 + 32ks .. +31 of one block into registers, as the units of the
// transposed staging: unit u = (key quad u%8, d octet u/8); lane handles
// u = lane and lane + 64.  Rows past p clamp to p (their P is 0).
template <typename T, typename TKV>
__device__ __forceinline__ void load_v_chunk(const TKV* vseq, int64_t row_stride, int64_t key0, int64_t p, int ks,
                                             int lane, kvreg<T, TKV> (&r)[2][4]) {
#pragma unroll
  for (int uu = 0; uu < 2; ++uu) {
    const int u = lane + 64 * uu;
    const int kq = u & 7, o8 = u >> 3;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      int64_t key = key0 + 32 * ks + 4 * kq + jj;
      if (key > p) key = p;
      r[uu][jj] = load_kvreg<T>(vseq + key * row_stride + 8 * o8);
    }
  }
}

// T: element type of q, out and the MFMA operands; TKV: storage type of K
// and V (T, or E4M3 widened to bf16 as it is loaded).
template <typename T, typename TKV>
__global__ __launch_bounds__(kAttnThreads, sizeof(T) == 2 ? 2 : 1) void sparse_attn_fwd(AttnKernelArgs args) {
  using V = VtTile<T>;
  __shared__ __attribute__((aligned(16))) T vt_all[kAttnThreads / kWave][V::kElems];
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  T* vt = vt_all[wave];

  const int G = args.Hkv;
  const int64_t item = (int64_t)blockIdx.x * (kAttnThreads / kWave) + wave;
  if (item >= args.rows_bound * G * args.nsplit) return;
  const int s = (int)(item % args.nsplit);
  const int64_t rest = item / args.nsplit;
  const int64_t t = rest % args.rows_bound;
  const int g = (int)(rest / args.rows_bound);

  int64_t q0, kb0;
  int M, N;
  if (args.cu_q) {
    if (t >= args.cu_q[args.batch]) return;
    const int b = find_row_seq(args.cu_q, args.batch, t);
    q0 = args.cu_q[b];
    M = args.cu_q[b + 1] - args.cu_q[b];
    kb0 = args.cu_k[b];
    N = args.cu_k[b + 1] - args.cu_k[b];
  } else {
    if (t >= args.batch) return;
    q0 = t;
    M = 1;
    kb0 = args.k_offsets[t];
    N = args.k_lens[t];
  }
  const int64_t p = (int64_t)N - M + (t - q0);

  const T* __restrict__ qg = static_cast<const T*>(args.q);
  const TKV* __restrict__ kg = static_cast<const TKV*>(args.k);
  const TKV* __restrict__ vg = static_cast<const TKV*>(args.v);
  const int R = args.Hq / G;
  const int h = lane & 15;     // head column of the MFMA tile
  const int a = lane >> 4;     // lane group: contraction slots 8a..8a+7
  const int hq = g * R + h;
  const bool head_ok = h < R;

  // B operand of S^T = K Q^T: Q^T[d][h], slots d = 32*ds + 8a .. +7.
  frag8<T> qf[kHeadDim / 32];
#pragma unroll
  for (int ds = 0; ds < kHeadDim / 32; ++ds)
    qf[ds] = head_ok ? load8(qg + (t * args.Hq + (head_ok ? hq : g * R)) * kHeadDim + 32 * ds + 8 * a)
                     : zero8<T>();

  f32x4 o[kHeadDim / 16];
#pragma unroll
  for (int dt = 0; dt < kHeadDim / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  const int i_lo = s * args.bps;
  const int i_hi = min(i_lo + args.bps, args.topk);
  // per-slot block LSEs: -inf unless the slot's block is attended (set below)
  float* blse = (args.block_lse && head_ok && a == 0) ? args.block_lse + (t * args.Hq + hq) * args.topk : nullptr;
  if (blse)
    for (int i = i_lo; i < i_hi; ++i) blse[i] = -__builtin_inff();
  if (p >= 0) {
    const int64_t local = p / kBlock;
    const int32_t* sel = args.block_idx + (t * G + g) * args.topk;
    const int64_t row_stride = (int64_t)G * kHeadDim;   // elements between tokens
    const TKV* kseq = kg + kb0 * row_stride + g * kHeadDim;
    const TKV* vseq = vg + kb0 * row_stride + g * kHeadDim;

    for (int i = i_lo; i < i_hi; ++i) {
      const int c = sel[i];
      bool seen = false;  // Sel is a set: a repeated id counts once
      for (int j = 0; j < i; ++j) seen = seen || sel[j] == c;
      if (c < 0 || c > local || seen) continue;
      const int64_t key0 = (int64_t)c * kBlock;
      const bool causal = (c == local);

      // ---- S^T[key][head] for the 128 keys of the block (8 tiles of 16 keys);
      // the first V chunk is requested right behind the K rows, and each
      // later chunk while the previous one is staged and multiplied, so a
      // block costs about two memory round trips instead of five.
      kvreg<T, TKV> kfr[kBlock / 16][kHeadDim / 32];
#pragma unroll
      for (int kt = 0; kt < kBlock / 16; ++kt) {
        int64_t key = key0 + 16 * kt + h;   // A operand row = lane % 16
        if (key > p) key = p;               // stay inside the sequence; masked below
        const TKV* kp = kseq + key * row_stride + 8 * a;
#pragma unroll
        for (int ds = 0; ds < kHeadDim / 32; ++ds) kfr[kt][ds] = load_kvreg<T>(kp + 32 * ds);
      }
      // E4M3 K/V: the raw bytes of the block's K rows and of all four V
      // chunks (128 keys) are requested together, one memory round trip per
      // block, and still fit two waves per SIMD (widened to bf16 only as
      // they are used).  Otherwise two chunk buffers: the first chunk is
      // requested with K and each later one a chunk ahead (for bf16 K/V the
      // four-chunk form measured no faster and spills).
      constexpr int kVBufs = sizeof(TKV) == 1 ? kBlock / 32 : 2;
      kvreg<T, TKV> vbuf[kVBufs][2][4];
      if constexpr (kVBufs == 2) {
        load_v_chunk<T>(vseq, row_stride, key0, p, 0, lane, vbuf[0]);
      } else {
#pragma unroll
        for (int ks = 0; ks < kBlock / 32; ++ks) load_v_chunk<T>(vseq, row_stride, key0, p, ks, lane, vbuf[ks]);
      }
      f32x4 st[kBlock / 16];
#pragma unroll
      for (int kt = 0; kt < kBlock / 16; ++kt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < kHeadDim / 32; ++ds) acc = mma16(kv_op<T>(kfr[kt][ds]), qf[ds], acc);
        st[kt] = acc;
      }

      // ---- online softmax (log2 units)
      // causal limit inside the block: key offsets above `lim` are masked
      const int64_t rel = p - key0 - 4 * a;
      const int lim = (!causal || rel > kBlock) ? kBlock : (int)rel;
      float mb = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < kBlock / 16; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = st[kt][r] * args.scale_log2;
          if (16 * kt + r > lim) x = -__builtin_inff();
          st[kt][r] = x;
          mb = fmaxf(mb, x);
        }
      mb = fmaxf(mb, shfl_xor_f(mb, 16));
      mb = fmaxf(mb, shfl_xor_f(mb, 32));
      const float m_new = fmaxf(m_run, mb);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < kHeadDim / 16; ++dt) o[dt] *= alpha;
      float l_blk = 0.f;
#pragma unroll
      for (int kt = 0; kt < kBlock / 16; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(st[kt][r] - m_new);
          st[kt][r] = e;
          l_blk += e;
        }
      l_run += l_blk;
      if (args.block_lse) {
        // this block alone: ln sum_j exp(z_j) = m_new ln 2 + ln sum_e, the sum over the 4 lane groups
        float lb = l_blk + shfl_xor_f(l_blk, 16);
        lb += shfl_xor_f(lb, 32);
        if (blse) blse[i] = m_new * 0.69314718055994530942f + logf(lb);
      }

      // ---- O^T[d][head] += V^T[d][key] P^T[key][head], 32 keys at a time
#pragma unroll
      for (int ks = 0; ks < kBlock / 32; ++ks) {
        if (kVBufs == 2 && ks + 1 < kBlock / 32)
          load_v_chunk<T>(vseq, row_stride, key0, p, ks + 1, lane, vbuf[(ks + 1) % kVBufs]);
        // Stage V rows key0+32ks .. +31 transposed: vt[d][key], keys contiguous.
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
          const int u = lane + 64 * uu;
          const int kq = u & 7, o8 = u >> 3;
          frag8<T> r4[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) r4[jj] = kv_op<T>(vbuf[ks % kVBufs][uu][jj]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            T* dst = vt + (8 * o8 + e) * V::kStride + 4 * kq;
            if constexpr (sizeof(T) == 2) {
              bf16x4 w = {r4[0][e], r4[1][e], r4[2][e], r4[3][e]};
              *reinterpret_cast<bf16x4*>(dst) = w;
            } else {
              f32x4 w = {r4[0][e], r4[1][e], r4[2][e], r4[3][e]};
              *reinterpret_cast<f32x4*>(dst) = w;
            }
          }
        }
        __builtin_amdgcn_wave_barrier();

        // B operand P^T: slots i<4 -> key 32ks+4a+i (tile 2ks), i>=4 -> 32ks+16+4a+i-4.
        frag8<T> pb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pb[r] = T(st[2 * ks][r]);
          pb[4 + r] = T(st[2 * ks + 1][r]);
        }
#pragma unroll
        for (int dt = 0; dt < kHeadDim / 16; ++dt) {
          const T* src = vt + (16 * dt + h) * V::kStride + 4 * a;
          frag8<T> va;
          if constexpr (sizeof(T) == 2) {
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(src);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(src + 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) { va[r] = lo[r]; va[4 + r] = hi[r]; }
          } else {
            const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) { va[r] = lo[r]; va[4 + r] = hi[r]; }
          }
          o[dt] = mma16(va, pb, o[dt]);
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
  }

  // ---- finalize: l is lane-partial over the 4 lane groups of a head
  float l_tot = l_run + shfl_xor_f(l_run, 16);
  l_tot += shfl_xor_f(l_tot, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  const float lse_val = l_tot > 0.f ? m_run * 0.69314718055994530942f + logf(l_tot) : -__builtin_inff();
  if (!head_ok) return;
  const int64_t rh = t * args.Hq + hq;
  if (args.nsplit == 1) {
    T* out = static_cast<T*>(args.out) + rh * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < kHeadDim / 16; ++dt)
      store4<T>(out + 16 * dt + 4 * a, o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
    if (args.lse && a == 0) args.lse[rh] = lse_val;
  } else {
    float* po = args.part_o + (rh * args.nsplit + s) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < kHeadDim / 16; ++dt)
      store4<float>(po + 16 * dt + 4 * a, o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
    if (a == 0) args.part_lse[rh * args.nsplit + s] = lse_val;
  }
}

// Two-phase combine: lse = ln sum_s exp(lse_s), o = sum_s exp(lse_s - lse) o_s,
// summed in split order (deterministic, no atomics); empty chunks (lse_s =
// -inf) are skipped.  32 threads per (row, head), 4 dims each.  Every
// chunk's LSE and partial output are requested at once, before the row
// count is known (rows past it are in the workspace but never stored), so
// the kernel waits for one memory round trip.
template <typename T>
__global__ __launch_bounds__(256) void attn_combine(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_lse,
                                                    const int32_t* __restrict__ cu_q, int batch,
                                                    int64_t rows_bound, int Hq, int nsplit, T* __restrict__ out,
                                                    float* __restrict__ lse) {
  const int64_t rh = (int64_t)blockIdx.x * 8 + threadIdx.x / 32;
  const int d0 = (threadIdx.x % 32) * 4;
  if (rh >= rows_bound * Hq) return;
  const float* pl = part_lse + rh * nsplit;
  const float* po = part_o + rh * nsplit * kHeadDim + d0;
  float ls[16];
  f32x4 ov[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int sc = min(s, nsplit - 1);  // in bounds; chunks past nsplit are masked below
    ls[s] = pl[sc];
    ov[s] = *reinterpret_cast<const f32x4*>(po + sc * kHeadDim);
  }
  const int64_t nrows = cu_q ? cu_q[batch] : batch;
  if (rh / Hq >= nrows) return;
  float mx = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    if (s >= nsplit) ls[s] = -__builtin_inff();
    mx = fmaxf(mx, ls[s]);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = -__builtin_inff();
  if (mx != -__builtin_inff()) {
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s) sum += expf(ls[s] - mx);
    L = mx + logf(sum);
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if (ls[s] != -__builtin_inff()) acc += expf(ls[s] - L) * ov[s];
  }
  store4<T>(out + rh * kHeadDim + d0, acc[0], acc[1], acc[2], acc[3]);
  if (lse && d0 == 0) lse[rh] = L;
}

template <typename T, typename TKV>
static hipError_t launch_attn_t(const AttnPlan& pl, const AttnArgs& a, void* ws, hipStream_t st) {
  AttnKernelArgs k;
  k.q = a.q; k.k = a.k; k.v = a.v; k.block_idx = a.block_idx;
  k.cu_q = a.cu_q; k.cu_k = a.cu_k; k.k_offsets = a.k_offsets; k.k_lens = a.k_lens;
  k.batch = a.batch; k.rows_bound = pl.rows_bound;
  k.Hq = a.Hq; k.Hkv = a.Hkv; k.topk = a.topk; k.nsplit = pl.nsplit; k.bps = pl.bps;
  k.scale_log2 = a.scale * 1.4426950408889634f;
  k.out = a.out; k.lse = a.lse; k.block_lse = a.block_lse;
  char* w = static_cast<char*>(ws);
  k.part_o = pl.nsplit > 1 ? reinterpret_cast<float*>(w) : nullptr;
  k.part_lse = pl.nsplit > 1 ? reinterpret_cast<float*>(w + pl.part_o_bytes) : nullptr;
  const int64_t items = pl.rows_bound * a.Hkv * pl.nsplit;
  hipLaunchKernelGGL((sparse_attn_fwd<T, TKV>), dim3((unsigned)((items + 3) / 4)), dim3(kAttnThreads), 0, st, k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.nsplit == 1) return e;
  const int64_t rh = pl.rows_bound * a.Hq;
  hipLaunchKernelGGL(attn_combine<T>, dim3((unsigned)((rh + 7) / 8)), dim3(256), 0, st, k.part_o, k.part_lse,
                     a.cu_q, a.batch, pl.rows_bound, a.Hq, pl.nsplit, static_cast<T*>(a.out), a.lse);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const AttnPlan& pl, int dtype, int kv_dtype, const AttnArgs& a, void* ws,
                              hipStream_t st) {
  const bool kv8 = kv_dtype == 2;  // bf16 q/out with E4M3 K/V
  if (pl.kvouter) {
    if (dtype != 0) return launch_attn_kvouter(pl, kv8, a, ws, st);
    // fp32 inputs: the query-outer schedule with one chunk (needs no workspace)
    AttnPlan q1 = pl;
    q1.kvouter = false;
    q1.nsplit = 1;
    q1.bps = a.topk;
    return launch_attn_t<float, float>(q1, a, ws, st);
  }
  if (dtype == 0) return launch_attn_t<float, float>(pl, a, ws, st);
  return kv8 ? launch_attn_t<bf16, fp8e4m3>(pl, a, ws, st) : launch_attn_t<bf16, bf16>(pl, a, ws, st);
}

}  // namespace msa
