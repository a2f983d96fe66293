// sparse_attn_kvouter.hip -- KV-outer schedule of the MSA main branch (prefill).
//
// Method: "MiniMax Sparse Attention: let each query pick its own blocks",
// section "The mechanism, precisely" (exact attention over the selected
// blocks; all heads of a group share the group's blocks).  Schedule: the
// atlas record of MiniMax M3, kernel list (KV-outer sparse attention with
// query gathering, pre-scheduled chunking of hot blocks, a two-phase combine
// over per-partial LSE buffers with no atomics, LSE fused into the forward).
//
// Why KV-outer on gfx950: each (query, group, block) edge needs a 64 KB K/V
// block.  Gathering it per query costs 64 KB of cache traffic per 1 MFLOP of
// MFMA work; staging each block in LDS once and running every query that
// selected it costs ~12 KB per edge instead (the query's 4 KB Q and a 4 KB
// bf16 partial written and read back).
//
// Steps for one window of query rows (the host loops over windows so the
// partial buffer stays bounded):
//   kvo_zero / kvo_bucket<false> (count) / kvo_scan / kvo_bucket<true> (place)
//       invert the selection into per-(sequence, group, block) edge lists and
//       cut each list into chunks of kKvoChunk edges (the pre-scheduled
//       chunking: hot blocks get several workgroups).  Atomics only count and
//       place edges; every result lands in a slot fixed by (row, group,
//       position in the selection), so outputs do not depend on the order.
//   kvo_attn
//       one workgroup per chunk: the K and V blocks (32 KB each) are staged in
//       LDS once; each wave runs two queries at a time through 32x32x16 MFMAs
//       (2 queries x 16 heads = 32 columns): S^T = K Q^T (keys x columns), a
//       softmax over the block per column, O^T = V^T P^T with V staged
//       transposed (keys contiguous) once per workgroup, so each operand is
//       two 8-byte LDS reads.  Each edge writes its normalised partial output
//       (bf16) and its LSE (fp32).
//   kvo_combine
//       per (row, group): lse = ln sum_i exp(lse_i), o = sum_i exp(lse_i - lse) o_i
//       over the selection slots in order.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kKvoThreads = 256;
constexpr int kKvoChunk = kEdgeChunk;  // edges per attention workgroup
constexpr int kKStride = 136;   // LDS row of K: 128 bf16 + 8 pad (272 B: 16-byte reads of 16 rows hit distinct banks)
constexpr int kVtStride = 132;  // LDS row of V^T (one dim, 128 keys): 264 B, so 32 rows read at one key offset hit distinct banks
constexpr int kRmax = 16;       // heads per group held by one partial slot

struct KvoArgs {
  const bf16* q;
  const void* k;  // bf16, or E4M3 (widened to bf16 as it is staged)
  const void* v;
  const int32_t* block_idx;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int batch, G, Hq, topk, nb_max;
  int64_t row_lo, row_hi;
  float scale_log2;
  int32_t* counts;
  int32_t* offsets;
  int32_t* chunk_start;
  int32_t* chunk_bucket;  // bucket of each chunk (filled by kvo_scan when set)
  int32_t* cursor;
  int32_t* edges;
  bf16* part_o;
  float* part_lse;
  bf16* out;
  float* lse;
  float* block_lse;
};

__device__ __forceinline__ int kvo_find(const int32_t* cu, int n, int64_t x) {
  int lo = 0, hi = n;  // cu[lo] <= x < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

struct RowInfo {
  int b;
  int64_t p;
};

__device__ __forceinline__ RowInfo kvo_row(const KvoArgs& a, int64_t t) {
  RowInfo r;
  r.b = kvo_find(a.cu_q, a.batch, t);
  const int M = a.cu_q[r.b + 1] - a.cu_q[r.b];
  const int N = a.cu_k[r.b + 1] - a.cu_k[r.b];
  r.p = (int64_t)N - M + (t - a.cu_q[r.b]);
  return r;
}

__global__ __launch_bounds__(256) void kvo_zero(int32_t* counts, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) counts[i] = 0;
}

// Validity of the (up to 16) entries of one selection row, as a bit mask: an
// entry is attended when it names a block at or before the local block and
// does not repeat an earlier entry of the row (Sel is a set).
__device__ __forceinline__ unsigned kvo_row_mask(const int32_t* sel, int topk, int64_t local, int nb_max,
                                                 int (&c)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) c[i] = i < topk ? sel[i] : -1;
  unsigned mask = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    bool ok = c[i] >= 0 && c[i] <= local && c[i] < nb_max;
#pragma unroll
    for (int j = 0; j < i; ++j) ok = ok && (c[j] != c[i]);
    mask |= ok ? (1u << i) : 0u;
  }
  return mask;
}

// Count the edges per (sequence, group, block) bucket, or place them.  One
// thread per (row, group).  When the buckets fit in LDS, a workgroup first
// aggregates its 256 rows' edges there (the 64 rows of a query block share
// their local block, so this removes most same-address global atomics), then
// issues one global atomic per non-empty bucket; in the placing pass that
// atomic reserves the workgroup's range of the bucket's list.
constexpr int kLdsBuckets = 32768;  // 128 KB: one workgroup per CU, and a window's 8192 rows need <= 32 G of them

template <bool kScatter>
__global__ __launch_bounds__(256) void kvo_bucket(KvoArgs a, int nbk) {
  __shared__ int s_cnt[kLdsBuckets];  // counts; in the placing pass then each bucket's base in the list
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t t = a.row_lo + item / a.G;
  const int g = (int)(item % a.G);
  bool live = item < (a.row_hi - a.row_lo) * a.G && t < a.cu_q[a.batch];
  unsigned mask = 0;
  int c[16];
  int base = 0;
  if (live) {
    const RowInfo ri = kvo_row(a, t);
    if (ri.p >= 0) {
      mask = kvo_row_mask(a.block_idx + (t * a.G + g) * a.topk, a.topk, ri.p / kBlock, a.nb_max, c);
      base = (ri.b * a.G + g) * a.nb_max;
    }
  }
  const int32_t code0 = (int32_t)((t - a.row_lo) << 4);
  if (nbk > kLdsBuckets) {  // too many buckets for LDS: global atomics per edge
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (!(mask & (1u << i))) continue;
      if (kScatter) a.edges[atomicAdd(&a.cursor[base + c[i]], 1)] = code0 | i;
      else atomicAdd(&a.counts[base + c[i]], 1);
    }
    return;
  }
  for (int j = threadIdx.x; j < nbk; j += 256) s_cnt[j] = 0;
  __syncthreads();
  int rk[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) rk[i] = (mask & (1u << i)) ? atomicAdd(&s_cnt[base + c[i]], 1) : 0;
  __syncthreads();
  for (int j = threadIdx.x; j < nbk; j += 256) {
    const int n = s_cnt[j];
    if (n == 0) continue;
    if (kScatter) s_cnt[j] = atomicAdd(&a.cursor[j], n);
    else atomicAdd(&a.counts[j], n);
  }
  if (!kScatter) return;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (mask & (1u << i)) a.edges[s_cnt[base + c[i]] + rk[i]] = code0 | i;
}

// Exclusive scans of the edge counts and of the chunk counts, one workgroup.
__global__ __launch_bounds__(1024) void kvo_scan(KvoArgs a, int nbk) {
  __shared__ int s_e[1024];
  __shared__ int s_c[1024];
  const int tid = threadIdx.x;
  const int seg = (nbk + 1023) / 1024;
  const int lo = min(tid * seg, nbk), hi = min(lo + seg, nbk);
  int se = 0, sc = 0;
  for (int j = lo; j < hi; ++j) {
    const int n = a.counts[j];
    se += n;
    sc += (n + kKvoChunk - 1) / kKvoChunk;
  }
  s_e[tid] = se;
  s_c[tid] = sc;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int ve = tid >= off ? s_e[tid - off] : 0;
    const int vc = tid >= off ? s_c[tid - off] : 0;
    __syncthreads();
    s_e[tid] += ve;
    s_c[tid] += vc;
    __syncthreads();
  }
  int oe = s_e[tid] - se, oc = s_c[tid] - sc;  // exclusive prefix of this thread's range
  for (int j = lo; j < hi; ++j) {
    const int n = a.counts[j];
    a.offsets[j] = oe;
    a.cursor[j] = oe;
    a.chunk_start[j] = oc;
    const int nc = (n + kKvoChunk - 1) / kKvoChunk;
    if (a.chunk_bucket)
      for (int q = 0; q < nc; ++q) a.chunk_bucket[oc + q] = j;
    oe += n;
    oc += nc;
  }
  if (tid == 1023) {
    a.offsets[nbk] = s_e[1023];
    a.chunk_start[nbk] = s_c[1023];
  }
}

// A selection slot's partial output: 16 heads x 128 dims in bf16, stored
// run-major: the 16-byte run of dims 8 r .. 8 r + 7 of head h at element
// kvo_run_off(r, h).  A run's 16 heads are adjacent (256 bytes), so the
// attention kernel's stores (16 heads of one run per half-wave) and the
// combine's loads (16 heads of one run per quarter-wave) each cover whole
// cache lines; head-major rows made every access touch all 32 lines of a slot.
__device__ __forceinline__ int kvo_run_off(int r, int h) { return (r * kRmax + h) * 8; }

struct PairQ {
  bf16x8 q[kHeadDim / 16];  // B operand Q^T: column (jq, h), slots d = 16*ks + 8*a32 .. +7
  int code;                 // (row in window) << 4 | selection slot
  bool has;                 // this lane's column holds an edge
};

__device__ __forceinline__ void kvo_load_pair(const KvoArgs& a, PairQ& P, int e, int e_hi, int jq, int h, int a32,
                                              int g, int R) {
  P.has = false;
  P.code = 0;
  if (e >= e_hi) return;
  P.has = e + jq < e_hi;
  P.code = a.edges[P.has ? e + jq : e];
  const bool ok = P.has && h < R;
  const bf16* qp = a.q + ((a.row_lo + (P.code >> 4)) * a.Hq + g * R + (ok ? h : 0)) * kHeadDim + 8 * a32;
#pragma unroll
  for (int ks = 0; ks < kHeadDim / 16; ++ks) P.q[ks] = ok ? load8(qp + 16 * ks) : zero8<bf16>();
}

// One pair of edges (two queries x 16 heads) against the staged block; while
// the PV MFMAs run, P is refilled with the pair at e_pf.
__device__ __forceinline__ void kvo_pair(const KvoArgs& a, PairQ& P, int e_pf, int e_hi, const bf16* k_lds,
                                         const bf16* vt_lds, int c, int g, int R, int N, int M, int64_t q0,
                                         int col, int a32, int jq, int h) {
  const int64_t p = (int64_t)N - M + (a.row_lo + (P.code >> 4) - q0);
    // S^T[key][col] for the 128 keys: 4 tiles of 32 keys
    f32x16 st[kBlock / 32];
#pragma unroll
    for (int kt = 0; kt < kBlock / 32; ++kt) {
      st[kt] = f32x16{};
      const bf16* arow = k_lds + (32 * kt + col) * kKStride + 8 * a32;
#pragma unroll
      for (int ks = 0; ks < kHeadDim / 16; ++ks)
        st[kt] = mma32(*reinterpret_cast<const bf16x8*>(arow + 16 * ks), P.q[ks], st[kt]);
      __builtin_amdgcn_sched_barrier(0);  // keep each tile's LDS reads next to its MFMAs
    }

    // softmax over the block, per column (the other half of the keys sits in lane ^ 32)
    // causal limit inside the block: key offsets above `lim` are masked
    // (lim >= 127 - 4*a32 means nothing in this lane is masked)
    const int64_t rel = p - (int64_t)c * kBlock - 4 * a32;
    const int lim = rel > kBlock ? kBlock : (int)rel;
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < kBlock / 32; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = st[kt][r] * a.scale_log2;
        if (32 * kt + 8 * (r >> 2) + (r & 3) > lim) x = -__builtin_inff();
        st[kt][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, xchg_halves_f(mx));
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < kBlock / 32; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float ex = __builtin_amdgcn_exp2f(st[kt][r] - mx);
        st[kt][r] = ex;
        sum += ex;
      }
    sum += xchg_halves_f(sum);

    // P^T as bf16 B operands: k-step kk covers keys 32*kt + 16*m + 8*(i/4) + 4*a32 + i%4
    // (kt = kk/2, m = kk%2), which are exactly this lane's S^T registers 8m .. 8m+7.
    bf16x8 pb[kBlock / 16];
#pragma unroll
    for (int kk = 0; kk < kBlock / 16; ++kk)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[kk][i] = bf16(st[kk >> 1][8 * (kk & 1) + i]);
    __builtin_amdgcn_sched_barrier(0);

    // qf is free once S^T is done: fetch the pair two steps ahead into it
    const int64_t trel = P.code >> 4;
    const int slot_i = P.code & 15;
    const bool colok = P.has && h < R;
    kvo_load_pair(a, P, e_pf, e_hi, jq, h, a32, g, R);
    __builtin_amdgcn_sched_barrier(0);

    const float inv = 1.0f / sum;
    const int64_t slot = (trel * a.G + g) * a.topk + slot_i;
    bf16* po = a.part_o + slot * kRmax * kHeadDim;  // the slot's partial, run-major (kvo_run_off)
    // O^T[d][col] = V^T[d][key] P^T[key][col], 32 dims at a time
#pragma unroll
    for (int dt = 0; dt < kHeadDim / 32; ++dt) {
      f32x16 o = {};
#pragma unroll
      for (int kk = 0; kk < kBlock / 16; ++kk) {
        const int kb1 = 32 * (kk >> 1) + 16 * (kk & 1) + 4 * a32;
        // A operand V^T: row d = 32*dt + lane%32, keys kb1 .. kb1+3 and kb1+8 .. kb1+11
        const bf16* src = vt_lds + (32 * dt + col) * kVtStride + kb1;
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(src);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(src + 8);
        bf16x8 va;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          va[i] = lo[i];
          va[4 + i] = hi[i];
        }
        o = mma32(va, pb[kk], o);
        if (kk & 1) __builtin_amdgcn_sched_barrier(0);
      }
      // Lanes col and col+32 hold alternate 4-dim runs of the same 32 dims;
      // swap halves so each lane stores two 16-byte runs of 8 dims.  The 16
      // heads of one run are adjacent in the partial, so each store writes
      // whole 256-byte pieces.
      u32x2 pk[4];
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        bf16x4 wv = {bf16(o[4 * qd] * inv), bf16(o[4 * qd + 1] * inv), bf16(o[4 * qd + 2] * inv),
                     bf16(o[4 * qd + 3] * inv)};
        pk[qd] = __builtin_bit_cast(u32x2, wv);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const u32x2 mine = a32 ? pk[2 * m + 1] : pk[2 * m];   // run this lane stores
        const u32x2 give = a32 ? pk[2 * m] : pk[2 * m + 1];   // run the partner stores
        u32x2 got;
        got[0] = xchg_halves_u32(give[0]);
        got[1] = xchg_halves_u32(give[1]);
        if (colok) {
          const u32x4 run = a32 ? u32x4{got[0], got[1], mine[0], mine[1]} : u32x4{mine[0], mine[1], got[0], got[1]};
          *reinterpret_cast<u32x4*>(po + kvo_run_off(4 * dt + 2 * m + a32, h)) = run;
        }
      }
    }
    if (colok && a32 == 0) a.part_lse[slot * kRmax + h] = mx * 0.69314718055994530942f + logf(sum);
}

template <typename TKV>
__global__ __launch_bounds__(kKvoThreads, 2) void kvo_attn(KvoArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 k_lds[kBlock * kKStride];
  __shared__ __attribute__((aligned(16))) bf16 vt_lds[kHeadDim * kVtStride];
  const int nbk = a.batch * a.G * a.nb_max;
  const int w = blockIdx.x;
  if (w >= a.chunk_start[nbk]) return;
  const int bucket = a.chunk_bucket[w];  // one read (a search of chunk_start was a chain of ~log2(nbk) reads)
  const int chunk = w - a.chunk_start[bucket];
  const int c = bucket % a.nb_max;
  const int g = (bucket / a.nb_max) % a.G;
  const int b = bucket / (a.nb_max * a.G);
  const int e_lo = a.offsets[bucket] + chunk * kKvoChunk;
  const int e_hi = min(e_lo + kKvoChunk, a.offsets[bucket + 1]);
  const int64_t kb0 = a.cu_k[b];
  const int N = a.cu_k[b + 1] - a.cu_k[b];
  const int64_t q0 = a.cu_q[b];
  const int M = a.cu_q[b + 1] - a.cu_q[b];
  const int64_t rs = (int64_t)a.G * kHeadDim;
  const TKV* kg = static_cast<const TKV*>(a.k);
  const TKV* vg = static_cast<const TKV*>(a.v);

  // ---- stage K row-major and V transposed (rows past the sequence end clamp
  // to its last row; their scores are masked)
  {
    bf16x8 kr[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int piece = threadIdx.x + u * kKvoThreads;
      const int row = piece >> 4, col = (piece & 15) * 8;
      const int64_t key = min(c * kBlock + row, N - 1);
      kr[u] = load8_kv<bf16>(kg + (kb0 + key) * rs + g * kHeadDim + col);
    }
    // V unit = (key quad kq, dim octet o8): 4 rows x 8 dims, written as 8 runs of 4 keys
    bf16x8 vr[2][4];
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const int u = threadIdx.x + uu * kKvoThreads;
      const int kq = u & 31, o8 = u >> 5;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int64_t key = min(c * kBlock + 4 * kq + jj, N - 1);
        vr[uu][jj] = load8_kv<bf16>(vg + (kb0 + key) * rs + g * kHeadDim + 8 * o8);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int piece = threadIdx.x + u * kKvoThreads;
      const int row = piece >> 4, col = (piece & 15) * 8;
      *reinterpret_cast<bf16x8*>(k_lds + row * kKStride + col) = kr[u];
    }
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const int u = threadIdx.x + uu * kKvoThreads;
      const int kq = u & 31, o8 = u >> 5;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 w4 = {vr[uu][0][e], vr[uu][1][e], vr[uu][2][e], vr[uu][3][e]};
        *reinterpret_cast<bf16x4*>(vt_lds + (8 * o8 + e) * kVtStride + 4 * kq) = w4;
      }
    }
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int col = lane & 31;   // MFMA column (query jq, head h); also the A-operand row
  const int a32 = lane >> 5;   // contraction slots 8*a32 .. 8*a32+7
  const int jq = col >> 4, h = col & 15;
  const int R = a.Hq / a.G;

  // Pairs of edges per wave, software-pipelined two pairs deep: the Q
  // fragments of pair i+2 load while pair i runs its PV MFMAs.
  constexpr int kPairStride = 2 * (kKvoThreads / kWave);
  const int e0 = e_lo + 2 * wave;
  PairQ A, B;
  kvo_load_pair(a, A, e0, e_hi, jq, h, a32, g, R);
  kvo_load_pair(a, B, e0 + kPairStride, e_hi, jq, h, a32, g, R);
  for (int e = e0; e < e_hi; e += 2 * kPairStride) {
    kvo_pair(a, A, e + 2 * kPairStride, e_hi, k_lds, vt_lds, c, g, R, N, M, q0, col, a32, jq, h);
    if (e + kPairStride >= e_hi) break;
    kvo_pair(a, B, e + 3 * kPairStride, e_hi, k_lds, vt_lds, c, g, R, N, M, q0, col, a32, jq, h);
  }
}

// Fixed-order LSE combine of the selection slots: one wave per (row, group);
// lane = (head lane % 16, 32 dims at 32 * (lane / 16)).  The row's selection and slot
// LSEs are read once; the partial loads of all slots are independent.
__global__ __launch_bounds__(256) void kvo_combine(KvoArgs a) {
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (a.row_hi - a.row_lo) * a.G) return;
  const int64_t trel = item / a.G;
  const int g = (int)(item % a.G);
  const int64_t t = a.row_lo + trel;
  if (t >= a.cu_q[a.batch]) return;
  const int lane = lane_id();
  const int h = lane & 15, q = lane >> 4, d0 = 32 * q;
  const int R = a.Hq / a.G;
  if (h >= R) return;
  const RowInfo ri = kvo_row(a, t);
  int c[16];
  const unsigned mask = ri.p >= 0 ? kvo_row_mask(a.block_idx + (t * a.G + g) * a.topk, a.topk, ri.p / kBlock,
                                                 a.nb_max, c)
                                  : 0u;
  const int64_t slot0 = (trel * a.G + g) * a.topk;
  bf16* out = a.out + (t * a.Hq + g * R + h) * kHeadDim + d0;
  float ls[16];
  float mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ls[i] = (mask & (1u << i)) ? a.part_lse[(slot0 + i) * kRmax + h] : -__builtin_inff();
    mx = fmaxf(mx, ls[i]);
  }
  if (a.block_lse && q == 0) {
    float* bl = a.block_lse + (t * a.Hq + g * R + h) * a.topk;
    for (int i = 0; i < a.topk; ++i) bl[i] = ls[i];
  }
  if (mask == 0u) {
#pragma unroll
    for (int j = 0; j < 32; j += 4) *reinterpret_cast<bf16x4*>(out + j) = bf16x4{bf16(0.f), bf16(0.f), bf16(0.f), bf16(0.f)};
    if (a.lse && q == 0) a.lse[t * a.Hq + g * R + h] = -__builtin_inff();
    return;
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += (mask & (1u << i)) ? expf(ls[i] - mx) : 0.f;
  const float L = mx + logf(sum);
  // Branch-free over the 16 slots so all partial loads can be in flight at
  // once: an unused slot reads the first used one with weight 0.
  const int first = __builtin_ctz(mask);
  float acc[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) acc[j] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool use = (mask >> i) & 1u;
    const float wgt = use ? expf(ls[i] - L) : 0.f;
    const bf16* src = a.part_o + (slot0 + (use ? i : first)) * kRmax * kHeadDim;
    bf16x8 v8[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v8[j] = load8(src + kvo_run_off(4 * q + j, h));
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[8 * j + u] += wgt * (float)v8[j][u];
  }
#pragma unroll
  for (int j = 0; j < 32; j += 4)
    *reinterpret_cast<bf16x4*>(out + j) = bf16x4{bf16(acc[j]), bf16(acc[j + 1]), bf16(acc[j + 2]), bf16(acc[j + 3])};
  if (a.lse && q == 0) a.lse[t * a.Hq + g * R + h] = L;
}

// Each bucket's edge codes sorted ascending (row in the window, then slot):
// the placing pass above leaves them in the order the atomics handed out, and
// a consumer that sums over a bucket's edges (the backward's dK / dV, the KL
// loss's index-key gradient) needs one fixed order to be bitwise
// reproducible.  A row selects a block at most once, so a bucket's rows are
// distinct: each edge sets its row's bit in an LDS bitmap of the window's
// rows (and records its slot by row), and a prefix count of the bitmap gives
// every row its rank.  One workgroup per bucket.
constexpr int kSortCap = 8192;  // rows of a window

__global__ __launch_bounds__(256) void kvo_sort(const int32_t* __restrict__ offsets, int32_t* __restrict__ edges,
                                                int nbk) {
  __shared__ uint32_t bits[kSortCap / 32];
  __shared__ uint8_t slot_of[kSortCap];
  __shared__ int wsum[4];
  const int bucket = blockIdx.x;
  if (bucket >= nbk) return;
  const int lo = offsets[bucket];
  const int n = offsets[bucket + 1] - lo;
  if (n <= 1) return;
  const int tid = threadIdx.x;
  bits[tid] = 0u;  // kSortCap / 32 == 256 words, one per thread
  __syncthreads();
  for (int i = tid; i < n; i += 256) {
    const int code = edges[lo + i];
    const int row = code >> 4;
    slot_of[row] = (uint8_t)(code & 15);
    atomicOr(&bits[row >> 5], 1u << (row & 31));
  }
  __syncthreads();
  // exclusive prefix of the words' popcounts: within the wave, then across
  const uint32_t w = bits[tid];
  const int cnt = __builtin_popcount(w);
  const int lane = tid & 63;
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[tid >> 6] = incl;
  __syncthreads();
  int base = incl - cnt;
  for (int k = 0; k < (tid >> 6); ++k) base += wsum[k];
  uint32_t m = w;
  while (m != 0u) {
    const int bit = __builtin_ctz(m);
    m &= m - 1u;
    const int row = 32 * tid + bit;
    edges[lo + base] = (row << 4) | slot_of[row];
    ++base;
  }
}

// Edge lists of query rows [a.row_lo, a.row_hi): counts, offsets, chunk
// starts and the edges themselves, per (sequence, group, block) bucket.
static void launch_edge_lists(const KvoArgs& a, int nbk, hipStream_t st) {
  const unsigned eg = (unsigned)(((a.row_hi - a.row_lo) * a.G + 255) / 256);
  hipLaunchKernelGGL(kvo_zero, dim3((unsigned)((nbk + 255) / 256)), dim3(256), 0, st, a.counts, nbk);
  hipLaunchKernelGGL(kvo_bucket<false>, dim3(eg), dim3(256), 0, st, a, nbk);
  hipLaunchKernelGGL(kvo_scan, dim3(1), dim3(1024), 0, st, a, nbk);
  hipLaunchKernelGGL(kvo_bucket<true>, dim3(eg), dim3(256), 0, st, a, nbk);
}

hipError_t build_edge_lists(const AttnArgs& x, int nb_max, int64_t row_lo, int64_t row_hi, int32_t* counts,
                            int32_t* offsets, int32_t* chunk_start, int32_t* chunk_bucket, int32_t* cursor,
                            int32_t* edges, bool sorted, hipStream_t st) {
  if (row_hi - row_lo > kSortCap) return hipErrorInvalidValue;
  KvoArgs a{};
  a.block_idx = x.block_idx;
  a.cu_q = x.cu_q;
  a.cu_k = x.cu_k;
  a.batch = x.batch;
  a.G = x.Hkv;
  a.Hq = x.Hq;
  a.topk = x.topk;
  a.nb_max = nb_max;
  a.row_lo = row_lo;
  a.row_hi = row_hi;
  a.counts = counts;
  a.offsets = offsets;
  a.chunk_start = chunk_start;
  a.chunk_bucket = chunk_bucket;
  a.cursor = cursor;
  a.edges = edges;
  const int nbk = x.batch * x.Hkv * nb_max;
  launch_edge_lists(a, nbk, st);
  if (sorted) hipLaunchKernelGGL(kvo_sort, dim3((unsigned)nbk), dim3(256), 0, st, offsets, edges, nbk);
  return hipGetLastError();
}

hipError_t launch_attn_kvouter(const AttnPlan& pl, bool kv_e4m3, const AttnArgs& x, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  KvoArgs a;
  a.q = static_cast<const bf16*>(x.q);
  a.k = x.k;
  a.v = x.v;
  a.block_idx = x.block_idx;
  a.cu_q = x.cu_q;
  a.cu_k = x.cu_k;
  a.batch = x.batch;
  a.G = x.Hkv;
  a.Hq = x.Hq;
  a.topk = x.topk;
  a.nb_max = pl.nb_max;
  a.scale_log2 = x.scale * 1.4426950408889634f;
  a.counts = reinterpret_cast<int32_t*>(w + pl.kvo_counts_off);
  a.offsets = reinterpret_cast<int32_t*>(w + pl.kvo_offsets_off);
  a.chunk_start = reinterpret_cast<int32_t*>(w + pl.kvo_chunks_off);
  a.chunk_bucket = reinterpret_cast<int32_t*>(w + pl.kvo_cbucket_off);
  a.cursor = reinterpret_cast<int32_t*>(w + pl.kvo_cursor_off);
  a.edges = reinterpret_cast<int32_t*>(w + pl.kvo_edges_off);
  a.part_o = reinterpret_cast<bf16*>(w + pl.kvo_part_o_off);
  a.part_lse = reinterpret_cast<float*>(w + pl.kvo_part_lse_off);
  a.out = static_cast<bf16*>(x.out);
  a.lse = x.lse;
  a.block_lse = x.block_lse;
  const int nbk = pl.kvo_nbuckets;
  for (int64_t r0 = 0; r0 < pl.rows_bound; r0 += pl.kvo_window) {
    a.row_lo = r0;
    a.row_hi = r0 + pl.kvo_window < pl.rows_bound ? r0 + pl.kvo_window : pl.rows_bound;
    const int64_t entries = (a.row_hi - a.row_lo) * a.G * a.topk;
    launch_edge_lists(a, nbk, st);
    const int64_t ub = entries / kKvoChunk + (entries < nbk ? entries : nbk) + 1;
    if (kv_e4m3) hipLaunchKernelGGL(kvo_attn<fp8e4m3>, dim3((unsigned)ub), dim3(kKvoThreads), 0, st, a);
    else hipLaunchKernelGGL(kvo_attn<bf16>, dim3((unsigned)ub), dim3(kKvoThreads), 0, st, a);
    const int64_t items = (a.row_hi - a.row_lo) * a.G;
    hipLaunchKernelGGL(kvo_combine, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t kvo_part_slot_bytes() { return (size_t)kRmax * kHeadDim * sizeof(bf16); }
int kvo_window_rows() { return 8192; }

}  // namespace msa
