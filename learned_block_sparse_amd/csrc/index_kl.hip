// index_kl.hip -- KL alignment loss of the MSA index branch on gfx950.
//
// Method: "MiniMax Sparse Attention: let each query pick its own blocks",
// section "Two design choices" (the index is trained by an auxiliary KL loss
// that aligns the index branch's block scores with the main attention's
// distribution over blocks, behind a stop-gradient, so only the index
// projections learn) and the atlas record of MiniMax M3, summary (the target
// is the group-averaged main-branch distribution).
//
// For query row t and group g, over the attended slots i of its selection
// (Sel taken as a set), with c_i the slot's block:
//   A_i = mean over the group's heads h of exp(block_lse[t, h, i] - lse[t, h])
//         the share of the head's attention in block c_i (from the forward
//         call's per-slot block LSEs: nothing of the main branch is recomputed)
//   S_i = max over the attended keys j of block c_i of q_idx[t, g] . k_idx[j]
//         (fp32; j*_i = the lowest key reaching the max)
//   loss[t, g] = KL(A || softmax(S)) = sum_i A_i (ln A_i - ln softmax(S)_i)
// and the gradients of sum_{t, g} loss[t, g]: dS_i = softmax(S)_i sum_k A_k - A_i,
// dq_idx[t, g] = sum_i dS_i k_idx[j*_i], dk_idx[j*_i] += dS_i q_idx[t, g].
//
// Kernels, per window of at most 8192 query rows (the selection edge lists of
// the KV-outer schedule, built by the same kernels):
//   kl_scores  one workgroup per chunk of <= 64 edges of a (sequence, group,
//              block) bucket: the block's 128 index keys staged in LDS once,
//              S^T = K q_idx^T on 32x32 MFMAs (32 edges per wave as the
//              columns), then each column's causal max and argmax, written to
//              the edge's selection slot
//   kl_loss    one wave per (row, group): A, softmax(S), loss, dS per slot and
//              dq_idx (lanes over the index dims)
//   kl_dk      one workgroup per (sequence, block): for each group in order,
//              the bucket's edges sorted in LDS by (argmax key, code), so each
//              key's contributions are one segment summed in code order by
//              that key's threads; added to dk_idx once per window
// No atomics touch the arithmetic: results are bitwise reproducible.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kKlWindow = 8192;  // query rows per edge-list window
constexpr int kKlSortMax = kKlWindow;
// kl_dk's sort keys: argmax key (7 bits) above the edge code (row in the window << 4 | slot)
constexpr int kKlCodeBits = 17;
static_assert((kKlWindow << 4) <= (1 << kKlCodeBits) && kBlock <= (1 << (31 - kKlCodeBits)),
              "kl_dk sort key fields");
constexpr float kKlNegInf = -__builtin_inff();
constexpr int kRmaxKl = 16;  // query heads per group at most

struct KlArgs {
  const void* q_idx;
  const void* k_idx;
  const int32_t* block_idx;
  const float* lse;
  const float* block_lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int batch, G, Hq, DI, topk, nb_max;
  int64_t rows_bound, row_lo, row_hi;
  const int32_t* offsets;
  const int32_t* chunk_start;
  const int32_t* edges;
  float* s_slot;    // [window rows, G, topk] index score of each attended slot
  int32_t* j_slot;  // [window rows, G, topk] argmax key within the block (0..127)
  float* ds_slot;   // [window rows, G, topk] dS of each attended slot
  float* loss;
  float* dq_idx;
  float* dk_idx;
};

__device__ __forceinline__ int kl_find(const int32_t* cu, int n, int64_t x) {
  int lo = 0, hi = n;  // cu[lo] <= x < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Attended slots of one selection row (Sel as a set): id >= 0, at or before
// the local block, not a repeat of an earlier slot.
__device__ __forceinline__ unsigned kl_row_mask(const int32_t* sel, int topk, int64_t local) {
  unsigned mask = 0;
  for (int i = 0; i < topk; ++i) {
    const int c = sel[i];
    bool ok = c >= 0 && c <= local;
    for (int j = 0; j < i; ++j) ok = ok && sel[j] != c;
    mask |= ok ? (1u << i) : 0u;
  }
  return mask;
}

__global__ __launch_bounds__(256) void kl_zero(KlArgs a) {
  const int64_t n = (int64_t)a.cu_k[a.batch] * a.DI;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) a.dk_idx[i] = 0.f;
}

// ------------------------------------------------------------- kl_scores
template <typename T, int DI>
__global__ __launch_bounds__(128) void kl_scores(KlArgs a) {
  constexpr int kRow = DI + 16 / (int)sizeof(T);  // one key row + 16 bytes of padding
  __shared__ __attribute__((aligned(16))) T k_lds[kBlock * kRow];
  const int nbk = a.batch * a.G * a.nb_max;
  const int w = blockIdx.x;
  if (w >= a.chunk_start[nbk]) return;
  const int bucket = kl_find(a.chunk_start, nbk, w);
  const int chunk = w - a.chunk_start[bucket];
  const int c = bucket % a.nb_max;
  const int g = (bucket / a.nb_max) % a.G;
  const int b = bucket / (a.nb_max * a.G);
  const int e_lo = a.offsets[bucket] + chunk * kEdgeChunk;
  const int e_hi = min(e_lo + kEdgeChunk, a.offsets[bucket + 1]);
  const int64_t kb0 = a.cu_k[b];
  const int N = a.cu_k[b + 1] - a.cu_k[b];
  const int64_t q0 = a.cu_q[b];
  const int M = a.cu_q[b + 1] - a.cu_q[b];
  const T* kg = static_cast<const T*>(a.k_idx);
  const T* qg = static_cast<const T*>(a.q_idx);

  // stage the block's index keys (rows past the sequence end clamp to its
  // last row; they lie past every query's position and are masked)
  constexpr int kPieces = kBlock * DI / 8;  // 8 elements each
  for (int pc = threadIdx.x; pc < kPieces; pc += 128) {
    const int row = pc / (DI / 8), col = (pc % (DI / 8)) * 8;
    const int64_t key = min(c * kBlock + row, N - 1);
    *reinterpret_cast<frag8<T>*>(k_lds + row * kRow + col) = load8(kg + (kb0 + key) * DI + col);
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int col = lane & 31;
  const int a32 = lane >> 5;
  const int e = e_lo + 32 * wave + col;  // this lane's column (edge)
  const bool has = e < e_hi;
  const int code = has ? a.edges[e] : 0;
  const int64_t t = a.row_lo + (code >> 4);
  const int64_t p = has ? (int64_t)N - M + (t - q0) : -1;
  // B operand q_idx^T: column = edge, dims 16 ks + 8 a32 .. +7
  frag8<T> qf[DI / 16];
#pragma unroll
  for (int ks = 0; ks < DI / 16; ++ks)
    qf[ks] = has ? load8(qg + (t * a.G + g) * DI + 16 * ks + 8 * a32) : zero8<T>();

  float best = kKlNegInf;
  int bj = 0;
#pragma unroll
  for (int kt = 0; kt < kBlock / 32; ++kt) {
    f32x16 st = {};
    const T* arow = k_lds + (32 * kt + col) * kRow + 8 * a32;
#pragma unroll
    for (int ks = 0; ks < DI / 16; ++ks) st = mma32(load8(arow + 16 * ks), qf[ks], st);
    // C layout: column = edge, rows = keys 32 kt + 8 (r / 4) + 4 a32 + r % 4 (ascending in r)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * kt + 8 * (r >> 2) + 4 * a32 + (r & 3);
      const bool live = (int64_t)c * kBlock + key <= p;
      if (live && st[r] > best) {  // strict: the lowest key keeps a tie
        best = st[r];
        bj = key;
      }
    }
  }
  // merge with the lane holding the column's other keys (lane ^ 32)
  const float ob = __shfl_xor(best, 32, kWave);
  const int oj = __shfl_xor(bj, 32, kWave);
  if (ob > best || (ob == best && oj < bj)) {
    best = ob;
    bj = oj;
  }
  if (has && a32 == 0) {
    const int64_t slot = ((int64_t)(code >> 4) * a.G + g) * a.topk + (code & 15);
    a.s_slot[slot] = best;
    a.j_slot[slot] = bj;
  }
}

// ---------------------------------------------------------------- kl_loss
// One wave per (row, group); lane l holds index dims l and l + 64.
template <typename T>
__global__ __launch_bounds__(256) void kl_loss(KlArgs a) {
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (a.row_hi - a.row_lo) * a.G) return;
  const int64_t trel = item / a.G;
  const int g = (int)(item % a.G);
  const int64_t t = a.row_lo + trel;
  if (t >= a.cu_q[a.batch]) return;
  const int lane = lane_id();
  const int bq = kl_find(a.cu_q, a.batch, t);
  const int64_t kb0 = a.cu_k[bq];
  const int64_t p = (int64_t)(a.cu_k[bq + 1] - a.cu_k[bq]) - (a.cu_q[bq + 1] - a.cu_q[bq]) + (t - a.cu_q[bq]);
  const int32_t* sel = a.block_idx + (t * a.G + g) * a.topk;
  const unsigned mask = p >= 0 ? kl_row_mask(sel, a.topk, p / kBlock) : 0u;
  const int R = a.Hq / a.G;
  const int64_t slot0 = (trel * a.G + g) * a.topk;

  // A_i: lane i (< topk) owns slot i; the r heads' shares are averaged
  float Ai = 0.f, Si = kKlNegInf;
  const bool mine = lane < a.topk && ((mask >> lane) & 1u);
  if (mine) {
    // all heads' loads in flight together, then summed in head order (R <= 16)
    float e[kRmaxKl];
#pragma unroll
    for (int hh = 0; hh < kRmaxKl; ++hh) {
      const int64_t rh = t * a.Hq + g * R + (hh < R ? hh : 0);
      e[hh] = __expf(a.block_lse[rh * a.topk + lane] - a.lse[rh]);
    }
#pragma unroll
    for (int hh = 0; hh < kRmaxKl; ++hh)
      if (hh < R) Ai += e[hh];
    Ai /= (float)R;
    Si = a.s_slot[slot0 + lane];
  }
  // softmax of S over the attended slots, sum of A, loss (wave reductions)
  float m = Si;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  float ez = mine ? __expf(Si - m) : 0.f;
  float z = ez, asum = Ai;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    z += __shfl_xor(z, o, kWave);
    asum += __shfl_xor(asum, o, kWave);
  }
  const float logI = mine ? Si - m - __logf(z) : 0.f;
  float li = (mine && Ai > 0.f) ? Ai * (__logf(Ai) - logI) : 0.f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) li += __shfl_xor(li, o, kWave);
  const float dsi = mine ? (ez / z) * asum - Ai : 0.f;
  if (mine) a.ds_slot[slot0 + lane] = dsi;
  if (lane == 0) a.loss[t * a.G + g] = mask ? li : 0.f;

  // dq_idx = sum_i dS_i k_idx[j*_i], slots in order.  The key rows of all
  // slots are loaded first (an unattended slot reads the first attended
  // slot's row and is not summed), so their loads are in flight together.
  const T* kg = static_cast<const T*>(a.k_idx);
  float acc0 = 0.f, acc1 = 0.f;
  if (mask != 0u) {
    const int first = __builtin_ctz(mask);
    float kv0[16], kv1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int ii = (i < a.topk && ((mask >> i) & 1u)) ? i : first;
      const int64_t key = kb0 + (int64_t)sel[ii] * kBlock + a.j_slot[slot0 + ii];
      kv0[i] = (float)kg[key * a.DI + lane];
      kv1[i] = lane + 64 < a.DI ? (float)kg[key * a.DI + lane + 64] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < a.topk && ((mask >> i) & 1u)) {
        const float ds = __shfl(dsi, i, kWave);
        acc0 += ds * kv0[i];
        if (lane + 64 < a.DI) acc1 += ds * kv1[i];
      }
    }
  }
  float* dq = a.dq_idx + (t * a.G + g) * a.DI;
  dq[lane] = acc0;
  if (lane + 64 < a.DI) dq[lane + 64] = acc1;
}

// ------------------------------------------------------------------ kl_dk
// One workgroup per (sequence, block), 256 threads: thread (key j = tid / 2,
// half = tid % 2) owns dims 64 half .. 64 half + 63 of dk_idx[j].  For each
// group in order, the bucket's edges are keyed (argmax j* << 17 | code) and
// sorted in LDS, so each key's edges form one segment in code order; the
// thread sums its key's segment in that order.  Segments come from a count
// of edges per key and its prefix sum.
template <typename T, int DI>
__global__ __launch_bounds__(256) void kl_dk(KlArgs a) {
  __shared__ int32_t keys[kKlSortMax];
  __shared__ int32_t seg[kBlock + 1];
  constexpr int kHalf = DI / 2;
  const int sb = blockIdx.x;  // sequence * nb_max + block
  if (sb >= a.batch * a.nb_max) return;
  const int c = sb % a.nb_max;
  const int b = sb / a.nb_max;
  const int tid = threadIdx.x;
  const int j = tid >> 1, half = tid & 1;
  const T* qg = static_cast<const T*>(a.q_idx);
  bool any = false;
  for (int g = 0; g < a.G; ++g) {
    const int bucket = (b * a.G + g) * a.nb_max + c;
    any = any || a.offsets[bucket + 1] > a.offsets[bucket];
  }
  if (!any) return;
  float acc[kHalf];
#pragma unroll
  for (int d = 0; d < kHalf; ++d) acc[d] = 0.f;
  for (int g = 0; g < a.G; ++g) {
    const int bucket = (b * a.G + g) * a.nb_max + c;
    const int e_lo = a.offsets[bucket];
    const int n = a.offsets[bucket + 1] - e_lo;
    if (n == 0) continue;
    int n2 = 1;
    while (n2 < n) n2 <<= 1;
    __syncthreads();  // keys / seg of the previous group are no longer read
    for (int i = tid; i < n2; i += 256) {
      int32_t k = 0x7fffffff;
      if (i < n) {
        const int code = a.edges[e_lo + i];
        const int64_t slot = ((int64_t)(code >> 4) * a.G + g) * a.topk + (code & 15);
        k = (a.j_slot[slot] << kKlCodeBits) | code;
      }
      keys[i] = k;
    }
    if (tid <= kBlock) seg[tid] = 0;
    __syncthreads();
    for (int kk = 2; kk <= n2; kk <<= 1) {
      for (int jj = kk >> 1; jj > 0; jj >>= 1) {
        for (int i = tid; i < n2; i += 256) {
          const int ixj = i ^ jj;
          if (ixj > i) {
            const int32_t x = keys[i], y = keys[ixj];
            if ((x > y) == ((i & kk) == 0)) {
              keys[i] = y;
              keys[ixj] = x;
            }
          }
        }
        __syncthreads();
      }
    }
    // segment starts: the first sorted position of each key (keys ascend)
    for (int i = tid; i < n; i += 256) {
      const int kj = keys[i] >> kKlCodeBits;
      if (i == 0 || (keys[i - 1] >> kKlCodeBits) != kj) seg[kj] = i + 1;  // +1: 0 marks "no edge"
    }
    __syncthreads();
    const int s0 = seg[j] - 1;
    if (s0 >= 0) {
      int s1 = s0 + 1;  // end of this key's segment
      while (s1 < n && (keys[s1] >> kKlCodeBits) == j) ++s1;
      // kBatch edges' rows are loaded together, then summed in segment order
      // (a batch past the end re-reads the segment's last edge, not summed;
      // 2 measured faster than 4, which costs the kernel a wave per SIMD)
      constexpr int kBatch = 2;
      for (int i0 = s0; i0 < s1; i0 += kBatch) {
        float ds[kBatch];
        frag8<T> v[kBatch][kHalf / 8];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int code = keys[min(i0 + u, s1 - 1)] & ((1 << kKlCodeBits) - 1);
          const int64_t slot = ((int64_t)(code >> 4) * a.G + g) * a.topk + (code & 15);
          ds[u] = a.ds_slot[slot];
          const T* qrow = qg + ((a.row_lo + (code >> 4)) * a.G + g) * DI + kHalf * half;
#pragma unroll
          for (int d8 = 0; d8 < kHalf; d8 += 8) v[u][d8 / 8] = load8(qrow + d8);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (i0 + u < s1) {
#pragma unroll
            for (int d8 = 0; d8 < kHalf; d8 += 8)
#pragma unroll
              for (int w = 0; w < 8; ++w) acc[d8 + w] += ds[u] * (float)v[u][d8 / 8][w];
          }
        }
      }
    }
  }
  const int64_t kb0 = a.cu_k[b];
  const int N = a.cu_k[b + 1] - a.cu_k[b];
  if (c * kBlock + j < N) {
    float* dst = a.dk_idx + (kb0 + c * kBlock + j) * DI + kHalf * half;
#pragma unroll
    for (int d = 0; d < kHalf; ++d) dst[d] += acc[d];
  }
}

KlPlan plan_kl(int batch, int max_q_len, int max_kv_len, int G, int topk) {
  KlPlan pl;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  pl.nb_max = (max_kv_len + kBlock - 1) / kBlock;
  pl.nbuckets = batch * G * pl.nb_max;
  pl.rows_bound = (int64_t)batch * max_q_len;
  pl.window = pl.rows_bound < kKlWindow ? pl.rows_bound : kKlWindow;
  const size_t nbk = (size_t)pl.nbuckets;
  const size_t slots = (size_t)pl.window * G * topk;
  size_t off = 0;
  pl.counts_off = off;  off += al(nbk * 4);
  pl.offsets_off = off; off += al((nbk + 1) * 4);
  pl.chunks_off = off;  off += al((nbk + 1) * 4);
  pl.cursor_off = off;  off += al(nbk * 4);
  pl.edges_off = off;   off += al(slots * 4);
  pl.s_off = off;       off += al(slots * 4);
  pl.j_off = off;       off += al(slots * 4);
  pl.ds_off = off;      off += al(slots * 4);
  pl.workspace_bytes = off;
  return pl;
}

template <typename T, int DI>
static hipError_t launch_kl_t(const KlPlan& pl, const KlLaunch& x, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  KlArgs a;
  a.q_idx = x.q_idx;
  a.k_idx = x.k_idx;
  a.block_idx = x.attn.block_idx;
  a.lse = x.lse;
  a.block_lse = x.block_lse;
  a.cu_q = x.attn.cu_q;
  a.cu_k = x.attn.cu_k;
  a.batch = x.attn.batch;
  a.G = x.attn.Hkv;
  a.Hq = x.attn.Hq;
  a.DI = DI;
  a.topk = x.attn.topk;
  a.nb_max = pl.nb_max;
  a.rows_bound = pl.rows_bound;
  int32_t* counts = reinterpret_cast<int32_t*>(w + pl.counts_off);
  int32_t* offsets = reinterpret_cast<int32_t*>(w + pl.offsets_off);
  int32_t* chunks = reinterpret_cast<int32_t*>(w + pl.chunks_off);
  int32_t* cursor = reinterpret_cast<int32_t*>(w + pl.cursor_off);
  int32_t* edges = reinterpret_cast<int32_t*>(w + pl.edges_off);
  a.offsets = offsets;
  a.chunk_start = chunks;
  a.edges = edges;
  a.s_slot = reinterpret_cast<float*>(w + pl.s_off);
  a.j_slot = reinterpret_cast<int32_t*>(w + pl.j_off);
  a.ds_slot = reinterpret_cast<float*>(w + pl.ds_off);
  a.loss = x.loss;
  a.dq_idx = x.dq_idx;
  a.dk_idx = x.dk_idx;
  hipLaunchKernelGGL(kl_zero, dim3(1024), dim3(256), 0, st, a);
  for (int64_t r0 = 0; r0 < pl.rows_bound; r0 += pl.window) {
    const int64_t r1 = r0 + pl.window < pl.rows_bound ? r0 + pl.window : pl.rows_bound;
    hipError_t e = build_edge_lists(x.attn, pl.nb_max, r0, r1, counts, offsets, chunks, cursor, edges, st);
    if (e != hipSuccess) return e;
    a.row_lo = r0;
    a.row_hi = r1;
    const int64_t entries = (r1 - r0) * a.G * a.topk;
    const int64_t ub = entries / kEdgeChunk + (entries < pl.nbuckets ? entries : pl.nbuckets) + 1;
    hipLaunchKernelGGL((kl_scores<T, DI>), dim3((unsigned)ub), dim3(128), 0, st, a);
    hipLaunchKernelGGL(kl_loss<T>, dim3((unsigned)(((r1 - r0) * a.G + 3) / 4)), dim3(256), 0, st, a);
    hipLaunchKernelGGL((kl_dk<T, DI>), dim3((unsigned)(a.batch * pl.nb_max)), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_index_kl(const KlPlan& pl, int dtype, int DI, const KlLaunch& x, void* ws, hipStream_t st) {
  if (dtype == 0) return DI == 64 ? launch_kl_t<float, 64>(pl, x, ws, st) : launch_kl_t<float, 128>(pl, x, ws, st);
  return DI == 64 ? launch_kl_t<bf16, 64>(pl, x, ws, st) : launch_kl_t<bf16, 128>(pl, x, ws, st);
}

}  // namespace msa
