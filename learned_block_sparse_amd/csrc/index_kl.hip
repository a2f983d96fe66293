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
//   kl_loss    16 lanes per (row, group), four per wave: A, softmax(S),
//              loss, dS per slot and dq_idx (lanes over the index dims)
//   kl_dk      workgroups per (sequence, block) and range of its keys, each
//              wave owning a few keys: it reads the block's edges (group by
//              group, each bucket sorted) 64 at a time, picks those whose
//              argmax is one of its keys by a ballot, and adds dS q_idx to its
//              LDS accumulator rows in edge order; added to dk_idx once per
//              window
// No atomics touch the arithmetic: results are bitwise reproducible.
#include <type_traits>

#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kKlWindow = 8192;  // query rows per edge-list window
// kl_dk's sort keys: argmax key (7 bits) above the edge code (row in the window << 4 | slot)
constexpr int kKlCodeBits = 17;
static_assert((kKlWindow << 4) <= (1 << kKlCodeBits) && kBlock <= (1 << (31 - kKlCodeBits)),
              "kl_dk sort key fields");
constexpr int kKlGShift = kKlCodeBits + 7;  // edge keys: group above the argmax key (7 bits) and the code
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
  const int32_t* chunk_bucket;  // bucket of each edge chunk
  const int32_t* edges;
  float* s_slot;      // [window rows, G, topk] index score of each attended slot
  int32_t* j_slot;    // [window rows, G, topk] argmax key within the block (0..127)
  int32_t* pos_slot;  // [window rows, G, topk] position of the slot's edge in the edge lists
  int32_t* key_edge;  // [edges] per edge-list position: group << 24 | argmax << 17 | code
  float* ds_edge;     // [edges] per edge-list position: dS of the edge's slot
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


// ------------------------------------------------------------- kl_scores
template <typename T, int DI>
__global__ __launch_bounds__(128) void kl_scores(KlArgs a) {
  constexpr int kRow = DI + 16 / (int)sizeof(T);  // one key row + 16 bytes of padding
  __shared__ __attribute__((aligned(16))) T k_lds[kBlock * kRow];
  const int nbk = a.batch * a.G * a.nb_max;
  const int w = blockIdx.x;
  if (w >= a.chunk_start[nbk]) return;
  const int bucket = a.chunk_bucket[w];
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
    a.pos_slot[slot] = e;
    a.key_edge[e] = (g << kKlGShift) | (bj << kKlCodeBits) | code;
  }
}

// ---------------------------------------------------------------- kl_loss
// Four (row, group) items per wave, 16 lanes each: lane l of an item owns
// selection slot l (its attended flag, A, S, dS) and index dims
// DI / 16 * l .. + DI / 16 - 1 of dq_idx, so each slot's argmax key row is
// read as one 16-byte (bf16, DI 128) piece per lane, all 16 slots' pieces in
// flight together, then summed in slot order.
template <typename T>
__global__ __launch_bounds__(256) void kl_loss(KlArgs a) {
  constexpr int kItemLanes = 16;
  const int lane = lane_id();
  const int l = lane & (kItemLanes - 1);
  const int base = lane & ~(kItemLanes - 1);
  const int64_t item = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  const int64_t nitems = (a.row_hi - a.row_lo) * a.G;
  const int64_t trel = item < nitems ? item / a.G : 0;
  const int g = item < nitems ? (int)(item % a.G) : 0;
  const int64_t t = a.row_lo + trel;
  const bool live = item < nitems && t < a.cu_q[a.batch];
  const int bq = kl_find(a.cu_q, a.batch, live ? t : 0);
  const int64_t kb0 = a.cu_k[bq];
  const int64_t p = (int64_t)(a.cu_k[bq + 1] - a.cu_k[bq]) - (a.cu_q[bq + 1] - a.cu_q[bq]) + (t - a.cu_q[bq]);
  const int R = a.Hq / a.G;
  const int64_t slot0 = (trel * a.G + g) * a.topk;
  // slot l attended: an id at or before the local block, not repeating an
  // earlier slot of the row (Sel is a set)
  const int cid = (live && l < a.topk) ? a.block_idx[(t * a.G + g) * a.topk + l] : -1;
  bool mine = live && p >= 0 && cid >= 0 && cid <= p / kBlock;
#pragma unroll
  for (int k = 0; k < kItemLanes; ++k) {
    const int other = __shfl(cid, base + k, kWave);
    mine = mine && !(k < l && other == cid);
  }
  // A_l: the heads' shares of block c_l, averaged; all heads' loads in flight
  // together, summed in head order (R <= 16)
  float Ai = 0.f, Si = kKlNegInf;
  int jl = 0, pos = 0;
  if (mine) {
    float e[kRmaxKl];
#pragma unroll
    for (int hh = 0; hh < kRmaxKl; ++hh) {
      const int64_t rh = t * a.Hq + g * R + (hh < R ? hh : 0);
      e[hh] = a.block_lse[rh * a.topk + l] - a.lse[rh];
    }
#pragma unroll
    for (int hh = 0; hh < kRmaxKl; ++hh)
      if (hh < R) Ai += __expf(e[hh]);
    Ai /= (float)R;
    Si = a.s_slot[slot0 + l];
    jl = a.j_slot[slot0 + l];
    pos = a.pos_slot[slot0 + l];
  }
  // softmax of S over the attended slots, sum of A, loss (16-lane reductions)
  float m = Si;
#pragma unroll
  for (int o = kItemLanes / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  const float ez = mine ? __expf(Si - m) : 0.f;
  float z = ez, asum = Ai;
#pragma unroll
  for (int o = kItemLanes / 2; o >= 1; o >>= 1) {
    z += __shfl_xor(z, o, kWave);
    asum += __shfl_xor(asum, o, kWave);
  }
  const float logI = mine ? Si - m - __logf(z) : 0.f;
  float li = (mine && Ai > 0.f) ? Ai * (__logf(Ai) - logI) : 0.f;
#pragma unroll
  for (int o = kItemLanes / 2; o >= 1; o >>= 1) li += __shfl_xor(li, o, kWave);
  const float dsi = mine ? (ez / z) * asum - Ai : 0.f;
  if (mine) a.ds_edge[pos] = dsi;
  const unsigned any = __ballot(mine) >> base & 0xffffu;
  if (live && l == 0) a.loss[t * a.G + g] = any ? li : 0.f;

  // dq_idx = sum_i dS_i k_idx[j*_i]: this lane's dims of every slot's key row
  // (an unattended slot reads this item's first attended row, not summed)
  constexpr int kDims = 8;  // elements per lane and load (DI 128; DI 64 uses the first half of the lanes)
  const T* kg = static_cast<const T*>(a.k_idx);
  const bool dim_ok = kDims * l < a.DI;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  if (any) {
    const int first = __builtin_ctz(any);
    frag8<T> kv[kItemLanes];
#pragma unroll
    for (int i = 0; i < kItemLanes; ++i) {
      const int src = ((any >> i) & 1u) ? i : first;
      const int ci = __shfl(cid, base + src, kWave);
      const int ji = __shfl(jl, base + src, kWave);
      const int64_t key = kb0 + (int64_t)ci * kBlock + ji;
      kv[i] = dim_ok ? load8(kg + key * a.DI + kDims * l) : zero8<T>();
    }
#pragma unroll
    for (int i = 0; i < kItemLanes; ++i) {
      const float ds = __shfl(dsi, base + i, kWave);
      if ((any >> i) & 1u) {
        acc0 += ds * f32x4{(float)kv[i][0], (float)kv[i][1], (float)kv[i][2], (float)kv[i][3]};
        acc1 += ds * f32x4{(float)kv[i][4], (float)kv[i][5], (float)kv[i][6], (float)kv[i][7]};
      }
    }
  }
  if (live && dim_ok) {
    float* dq = a.dq_idx + (t * a.G + g) * a.DI + kDims * l;
    *reinterpret_cast<f32x4*>(dq) = acc0;
    *reinterpret_cast<f32x4*>(dq + 4) = acc1;
  }
}

// ------------------------------------------------------------------ kl_dk
// `split` workgroups per (sequence, block), each 128 / split of the block's
// keys; each of the 4 waves owns a quarter of those keys and works alone (no
// barriers).  The edges of the block's buckets, group by group and each
// bucket in its sorted (row, slot) order, form one sequence.  A wave
//   1. reads it 4 x 64 positions at a time (lane i: a position's key and dS,
//      all loads in flight together) and lists, in position order, the edges
//      whose argmax is one of its keys (ballot + compaction into LDS), until
//      its list could overflow;
//   2. applies the listed edges in order, kKlApply at a time: their q_idx
//      rows are loaded together (lane l: dims DI / 64 * l ..), then
//      dk[j*] += dS * q_idx[row, g] is added to the wave's accumulator rows in
//      LDS.
// Each key is summed by one wave over its edges in (group, row, slot) order.
constexpr int kKlKeysWave = 16;  // most keys per wave (split >= 2)
constexpr int kKlList = 256;     // listed edges per wave before they are applied
constexpr int kKlApply = 32;     // q_idx rows in flight per wave

template <typename T, int DI>
struct KlLane {  // this lane's DI / 64 dims of an index row, as loaded
  static constexpr int kN = DI / 64;
  using Raw = typename std::conditional<sizeof(T) * kN == 4, uint32_t,
                                        typename std::conditional<sizeof(T) * kN == 8, u32x2, T>::type>::type;
  Raw raw;
  __device__ __forceinline__ void load(const T* row, int lane) {
    raw = *reinterpret_cast<const Raw*>(row + kN * lane);
  }
  __device__ __forceinline__ float get(int i) const {
    const T* p = reinterpret_cast<const T*>(&raw);
    return (float)p[i];
  }
};

template <typename T, int DI>
__global__ __launch_bounds__(256) void kl_dk(KlArgs a, int split) {
  constexpr int kN = DI / 64;
  __shared__ float s_acc[4][kKlKeysWave * DI];
  __shared__ int32_t s_lk[4][kKlList];
  __shared__ float s_ld[4][kKlList];
  const int r = blockIdx.x % split;
  const int sb = blockIdx.x / split;  // sequence * nb_max + block
  if (sb >= a.batch * a.nb_max) return;
  const int c = sb % a.nb_max;
  const int b = sb / a.nb_max;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int keys_wave = kBlock / split / 4;
  const int k0 = r * (kBlock / split) + wave * keys_wave;  // this wave's first key
  float* acc = s_acc[wave];
  int32_t* lk = s_lk[wave];
  float* ld = s_ld[wave];
  const T* qg = static_cast<const T*>(a.q_idx);
  // the block's edge sequence: group g's bucket holds positions [pre[g], pre[g + 1]),
  // which are edge-list positions ebase[g] .. (uniform values)
  int pre[kRmaxKl + 1], ebase[kRmaxKl];
  pre[0] = 0;
#pragma unroll
  for (int g = 0; g < kRmaxKl; ++g) {
    const int bucket = (b * a.G + (g < a.G ? g : 0)) * a.nb_max + c;
    ebase[g] = a.offsets[bucket];
    pre[g + 1] = pre[g] + (g < a.G ? a.offsets[bucket + 1] - ebase[g] : 0);
  }
  const int total = pre[kRmaxKl];
  const int64_t kb0 = a.cu_k[b];
  const int N = a.cu_k[b + 1] - a.cu_k[b];
  if (total == 0) {
    // no edge in this window: the first window writes the keys' rows as zero
    if (a.row_lo == 0)
      for (int kk = 0; kk < keys_wave && c * kBlock + k0 + kk < N; ++kk)
        for (int d = lane; d < DI; d += kWave) a.dk_idx[(kb0 + c * kBlock + k0 + kk) * DI + d] = 0.f;
    return;
  }
  for (int i = lane; i < keys_wave * DI; i += kWave) acc[i] = 0.f;

  // key and dS of sequence position f
  auto load_meta = [&](int f, int32_t& key, float& ds) {
    key = -1;
    ds = 0.f;
    if (f >= total) return;
    int e = f;
#pragma unroll
    for (int g = 0; g < kRmaxKl; ++g)
      if (f >= pre[g] && f < pre[g + 1]) e = ebase[g] + f - pre[g];
    key = a.key_edge[e];
    ds = a.ds_edge[e];
  };
  int f0 = 0;
  while (f0 < total) {
    // 1. list this wave's edges in position order
    int cnt = 0;
    while (f0 < total && cnt + 4 * kWave <= kKlList) {
      int32_t k4[4];
      float d4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) load_meta(f0 + u * kWave + lane, k4[u], d4[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kj = (k4[u] >> kKlCodeBits) & 127;
        const bool hit = k4[u] >= 0 && kj >= k0 && kj < k0 + keys_wave;
        const uint64_t m = __ballot(hit);
        if (hit) {
          const int slot =
              cnt + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
          lk[slot] = k4[u];
          ld[slot] = d4[u];
        }
        cnt += __builtin_popcountll(m);
      }
      f0 += 4 * kWave;
    }
    // 2. apply them in order
    for (int i0 = 0; i0 < cnt; i0 += kKlApply) {
      KlLane<T, DI> q[kKlApply];
#pragma unroll
      for (int u = 0; u < kKlApply; ++u) {
        const int32_t ku = lk[min(i0 + u, cnt - 1)];
        const int g = ku >> kKlGShift;
        const int row = (ku & ((1 << kKlCodeBits) - 1)) >> 4;
        q[u].load(qg + ((a.row_lo + row) * a.G + g) * DI, lane);
      }
      __builtin_amdgcn_sched_barrier(0);  // the loads stay in flight together
#pragma unroll
      for (int u = 0; u < kKlApply; ++u) {
        if (i0 + u >= cnt) break;
        const int32_t ku = lk[i0 + u];
        const float du = ld[i0 + u];
        float* arow = acc + (((ku >> kKlCodeBits) & 127) - k0) * DI + kN * lane;
#pragma unroll
        for (int i = 0; i < kN; ++i) arow[i] += du * q[u].get(i);
      }
    }
  }
  for (int kk = 0; kk < keys_wave; ++kk) {
    if (c * kBlock + k0 + kk >= N) break;
    float* dst = a.dk_idx + (kb0 + c * kBlock + k0 + kk) * DI + kN * lane;
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const float v = acc[kk * DI + kN * lane + i];
      dst[i] = a.row_lo == 0 ? v : dst[i] + v;  // the first window writes outright
    }
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
  pl.cbucket_off = off; off += al((slots / kEdgeChunk + (slots < nbk ? slots : nbk) + 1) * 4);
  pl.s_off = off;       off += al(slots * 4);
  pl.j_off = off;       off += al(slots * 4);
  pl.pos_off = off;     off += al(slots * 4);
  pl.key_off = off;     off += al(slots * 4);
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
  int32_t* cbucket = reinterpret_cast<int32_t*>(w + pl.cbucket_off);
  a.offsets = offsets;
  a.chunk_start = chunks;
  a.chunk_bucket = cbucket;
  a.edges = edges;
  a.s_slot = reinterpret_cast<float*>(w + pl.s_off);
  a.j_slot = reinterpret_cast<int32_t*>(w + pl.j_off);
  a.pos_slot = reinterpret_cast<int32_t*>(w + pl.pos_off);
  a.key_edge = reinterpret_cast<int32_t*>(w + pl.key_off);
  a.ds_edge = reinterpret_cast<float*>(w + pl.ds_off);
  a.loss = x.loss;
  a.dq_idx = x.dq_idx;
  a.dk_idx = x.dk_idx;
  for (int64_t r0 = 0; r0 < pl.rows_bound; r0 += pl.window) {
    const int64_t r1 = r0 + pl.window < pl.rows_bound ? r0 + pl.window : pl.rows_bound;
    hipError_t e = build_edge_lists(x.attn, pl.nb_max, r0, r1, counts, offsets, chunks, cbucket, cursor, edges, true, st);
    if (e != hipSuccess) return e;
    a.row_lo = r0;
    a.row_hi = r1;
    const int64_t entries = (r1 - r0) * a.G * a.topk;
    const int64_t ub = entries / kEdgeChunk + (entries < pl.nbuckets ? entries : pl.nbuckets) + 1;
    hipLaunchKernelGGL((kl_scores<T, DI>), dim3((unsigned)ub), dim3(128), 0, st, a);
    hipLaunchKernelGGL(kl_loss<T>, dim3((unsigned)(((r1 - r0) * a.G + 15) / 16)), dim3(256), 0, st, a);
    // keys per workgroup: 64, or fewer when there are few blocks (the first
    // window of a long prefill), so that the blocks' long edge sequences are
    // spread over more workgroups
    const int64_t nblk = (int64_t)a.batch * pl.nb_max;
    const int split = nblk >= 256 ? 2 : nblk >= 128 ? 4 : 8;
    hipLaunchKernelGGL((kl_dk<T, DI>), dim3((unsigned)(nblk * split)), dim3(256), 0, st, a, split);
  }
  return hipGetLastError();
}

hipError_t launch_index_kl(const KlPlan& pl, int dtype, int DI, const KlLaunch& x, void* ws, hipStream_t st) {
  if (dtype == 0) return DI == 64 ? launch_kl_t<float, 64>(pl, x, ws, st) : launch_kl_t<float, 128>(pl, x, ws, st);
  return DI == 64 ? launch_kl_t<bf16, 64>(pl, x, ws, st) : launch_kl_t<bf16, 128>(pl, x, ws, st);
}

}  // namespace msa
