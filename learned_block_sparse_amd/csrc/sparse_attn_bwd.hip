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
//   bwd_zero   dk = dv = 0 for the key rows no selection of the first query
//              window reaches (the rows of every other block are written
//              outright by that window's bwd_dkdv / bwd_dkdv_reduce, and later
//              windows add to them)
//   bwd_delta  delta[row, head] = dO . O
//   bwd_dkv_scan  chunk starts of bwd_dkdv: each bucket of the selection
//              edge lists (the lists the KV-outer forward builds, here sorted
//              per bucket, so the order in which edges are summed is fixed) is
//              cut into chunks of at most kDkvChunk edges; buckets of more
//              than one chunk (planted blocks, the early blocks of the first
//              query window, which nearly every row picks) also get one
//              partial slot per chunk
//   bwd_dkdv   KV-outer, one workgroup per chunk, 8 waves: two per key tile
//              of 32 keys sharing a SIMD, one keeping the tile's K rows as MFMA
//              operands (S = Q K^T, P, dV += P^T dO), the other its V rows
//              (dP = dO V^T, dS = P (dP - delta) with P passed through LDS,
//              dK += dS^T Q).  The edges run in quads (4 queries x 16 heads =
//              64 MFMA rows) whose Q and dO rows are staged once in LDS by
//              direct-to-LDS loads, a quad ahead; the second products read
//              them transposed.  dS also goes to LDS key-major; during the
//              next quad each B wave computes 32 dims of dQ^T = K^T dS^T over
//              the block's 128 keys into an LDS stage, from which each A wave
//              writes one edge's rows (4 KB, whole cache lines) to the bf16
//              partial of its selection slot.  dK and dV accumulate over the
//              chunk in registers; a bucket's only chunk adds them to the
//              output, the chunks of a longer bucket write fp32 partials
//   bwd_dkdv_reduce  adds each long bucket's partials to dK / dV in chunk
//              order
//   bwd_dq_combine  dq = sum of a row's slot partials in slot order
// No atomics touch the arithmetic: every result is bitwise reproducible.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kBwdThreads = 256;
constexpr int kBwdRow = 136;      // LDS row of Q / dO for one MFMA row: 128 bf16 + 8 pad
constexpr int kBwdWindow = 8192;  // query rows per edge-list window
constexpr int kDkvChunk = 256;    // edges per bwd_dkdv workgroup (64 quads)
static_assert(kBwdWindow <= 65536, "bwd_dkdv keeps rows of the window as 16-bit numbers");
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
  const int32_t* chunk_start;
  int32_t* edges;
  float* delta;
  int32_t* dkv_chunk;  // [nbuckets + 1] exclusive prefix of the buckets' bwd_dkdv chunks
  int32_t* dkv_part;   // [nbuckets + 1] exclusive prefix of the partial slots (buckets of > 1 chunk)
  float* part_dkv;     // [slots][2][128 keys][128 dims]: a chunk's dK (unscaled) and dV
  bf16* part_dq;     // [window rows, G, topk, 16, 128]: each edge's block contribution to dq (unscaled)
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

// dk = dv = 0 over the key rows of the buckets without an edge in the first
// window: one workgroup per bucket (sequence, group, block), 128 rows of the
// group's 128 dims.
__global__ __launch_bounds__(256) void bwd_zero(BwdKernelArgs a) {
  const int nbk = a.batch * a.G * a.nb_max;
  const int bucket = blockIdx.x;
  if (bucket >= nbk || a.offsets[bucket + 1] > a.offsets[bucket]) return;
  const int c = bucket % a.nb_max;
  const int g = (bucket / a.nb_max) % a.G;
  const int b = bucket / (a.nb_max * a.G);
  const int64_t kb0 = a.cu_k[b];
  const int N = a.cu_k[b + 1] - a.cu_k[b];
  const int64_t rs = (int64_t)a.G * kHeadDim;
  for (int u = threadIdx.x; u < kBlock * kHeadDim / 4; u += 256) {
    const int kk = c * kBlock + u / (kHeadDim / 4), d = 4 * (u % (kHeadDim / 4));
    if (kk >= N) continue;
    const int64_t off = (kb0 + kk) * rs + g * kHeadDim + d;
    *reinterpret_cast<f32x4*>(a.dk + off) = f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(a.dv + off) = f32x4{0.f, 0.f, 0.f, 0.f};
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

// Chunk starts and partial slots of bwd_dkdv, one workgroup: thread i scans
// a contiguous range of buckets, then the 1024 range sums are scanned in LDS.
__global__ __launch_bounds__(1024) void bwd_dkv_scan(BwdKernelArgs a, int nbk) {
  __shared__ int s_c[1024];
  __shared__ int s_p[1024];
  const int tid = threadIdx.x;
  const int seg = (nbk + 1023) / 1024;
  const int lo = min(tid * seg, nbk), hi = min(lo + seg, nbk);
  int sc = 0, sp = 0;
  for (int j = lo; j < hi; ++j) {
    const int ch = (a.offsets[j + 1] - a.offsets[j] + kDkvChunk - 1) / kDkvChunk;
    sc += ch;
    sp += ch > 1 ? ch : 0;
  }
  s_c[tid] = sc;
  s_p[tid] = sp;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int vc = tid >= off ? s_c[tid - off] : 0;
    const int vp = tid >= off ? s_p[tid - off] : 0;
    __syncthreads();
    s_c[tid] += vc;
    s_p[tid] += vp;
    __syncthreads();
  }
  int oc = s_c[tid] - sc, op = s_p[tid] - sp;
  for (int j = lo; j < hi; ++j) {
    const int ch = (a.offsets[j + 1] - a.offsets[j] + kDkvChunk - 1) / kDkvChunk;
    a.dkv_chunk[j] = oc;
    a.dkv_part[j] = op;
    oc += ch;
    op += ch > 1 ? ch : 0;
  }
  if (tid == 1023) {
    a.dkv_chunk[nbk] = s_c[1023];
    a.dkv_part[nbk] = s_p[1023];
  }
}

// One quad of edges (4 queries x 16 heads = 64 MFMA rows).  Its Q and dO are
// staged in LDS row-major, one tile each, rows of kBwdRow bf16 (256 bytes of
// data and a 16-byte pad slot, so 16-byte reads of 32 rows at one column
// spread over the banks), by direct buffer-to-LDS loads: a tile is 64 x 17
// slots of 16 bytes, filled by 17 loads of 64 consecutive slots (lane i slot
// i); a pad slot receives a copy of its row's first slot.  S = Q K^T and
// dP = dO V^T read the tiles row-major; dV += P^T dO and dK += dS^T Q read
// them transposed (lds_read_tr4), so no second copy is staged.
constexpr int kQuadRows = 64;
constexpr int kRowSlots = kBwdRow * 2 / 16;               // 17 slots of 16 bytes per row
constexpr int kTileRuns = kQuadRows * kRowSlots / kWave;  // 17 loads of 64 slots per tile
constexpr int kQuadRuns = 2 * kTileRuns;                  // Q and dO
constexpr int kDkvThreads = 512;  // bwd_dkdv: two waves per key tile of 32 keys, two per SIMD
constexpr int kDkvWaves = kDkvThreads / kWave;
constexpr int kRunsPerWave = (kQuadRuns + kDkvWaves - 1) / kDkvWaves;
static_assert(kQuadRows * kRowSlots % kWave == 0, "a tile is a whole number of 64-slot loads");

// Tile row of MFMA row m = 16 s + 4 k + e: 16 s + 4 e + k (a 4 x 4 transpose
// inside each block of 16 rows; its own inverse).  A 272-byte row shifts the
// LDS banks by 4 (of 64), so the four MFMA rows 4 k .. 4 k + 3 that a
// transposed read gathers, four tile rows apart, start 16 banks apart and,
// with the second 16-dim half of the 32 lanes read together 8 banks further
// on, the 32 lanes' 8-byte pieces fill distinct banks; 16 consecutive MFMA
// rows of a 16-byte row-major read are still 16 distinct tile rows of the
// block.  Consecutive rows made the transposed reads conflict (44% of LDS
// cycles; 21% with the rows only two apart).
__device__ __forceinline__ int bwd_tile_row(int m) {
  return (m & ~15) | ((m & 3) << 2) | ((m >> 2) & 3);
}
__device__ __forceinline__ int bwd_mfma_row(int p) { return bwd_tile_row(p); }

// One staging buffer.  The kernel keeps two as separate LDS objects and
// alternates them in an unrolled loop, so the compiler can see that the
// tile being read is never the one the staging loads are filling (with one
// array indexed by the buffer number it waits for those loads first).
struct BwdTile {
  bf16 rm[2][kQuadRows * kBwdRow];  // [Q, dO]
  float lse[kQuadRows];             // per MFMA row, log2 units (read 4 at a time)
  float delta[kQuadRows];
  int pos[4];
};

// A lane's part of a quad's staging loads (the same for every quad of the
// chunk but for the quad's query rows), kept in LDS rather than registers:
// for its run u, the query of the quad (0..3, bits 30..31) whose row the
// lane's slot belongs to, and the byte offset of the slot inside that
// query's row of heads (bits 0..29).  Slots of heads past R read the group's
// first head (finite values; those MFMA rows get probability 0).
__device__ __forceinline__ void bwd_dma_plan(uint32_t* plan, int wave, int lane, int g, int R) {
#pragma unroll
  for (int u = 0; u < kRunsPerWave; ++u) {
    const int run = wave + kDkvWaves * u;
    const int slot = (run % kTileRuns) * kWave + lane;
    const int row = bwd_mfma_row(slot / kRowSlots), c = slot % kRowSlots;
    const int h = row & 15;
    const uint32_t cst = (uint32_t)(((g * R + (h < R ? h : 0)) * kHeadDim + 8 * (c < 16 ? c : 0)) * 2);
    plan[u * kWave + lane] = cst | ((uint32_t)(row >> 4) << 30);
  }
}

// Issue the staging loads of quad qi into tile T (nothing waits for them
// here).  The quad's four query rows and the lane's plan are read from LDS
// at once, before any load (a staging load writes LDS, so a read after it
// could wait for it).  A missing query (past the chunk's n edges) reads the first row of
// the window: finite values whose MFMA rows get probability 0.
__device__ __forceinline__ void bwd_issue_quad(BwdTile& T, const uint32_t* plan, const uint32_t* codes, int qi, int n,
                                               int wave, int lane, const bf16* win_q, const bf16* win_g,
                                               int win_bytes, uint32_t row_bytes) {
  const u32x4 cc = *reinterpret_cast<const u32x4*>(codes + 4 * qi);  // edges 4 qi .. 4 qi + 3
  uint32_t pk[kRunsPerWave];
#pragma unroll
  for (int u = 0; u < kRunsPerWave; ++u) pk[u] = plan[u * kWave + lane];
  uint32_t rq[4] = {cc.x >> 4, cc.y >> 4, cc.z >> 4, cc.w >> 4};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (4 * qi + j >= n) rq[j] = 0;
#pragma unroll
  for (int u = 0; u < kRunsPerWave; ++u) {
    const int run = wave + kDkvWaves * u;
    if (run < kQuadRuns) {
      const uint32_t jq = pk[u] >> 30;
      const uint32_t t = jq == 0 ? rq[0] : jq == 1 ? rq[1] : jq == 2 ? rq[2] : rq[3];
      const int tsr = run / kTileRuns;
      lds_load16(tsr ? win_g : win_q, win_bytes, (int)(t * row_bytes + (pk[u] & 0x3fffffffu)),
                 &T.rm[tsr][(run % kTileRuns) * kWave * 8]);
    }
  }
}

// lse, delta of the quad's 64 MFMA rows (threads 0..63) and the positions of
// its 4 queries (threads 64..67), loaded into registers while the previous
// quad is computed and stored after it.
struct QuadAux {
  float lse, delta;
  int pos;
  bool ok;
};

__device__ __forceinline__ void bwd_load_aux(const BwdKernelArgs& a, QuadAux& x, const uint32_t* codes, int qi,
                                             int n, int g, int R, int N, int M, int64_t q0) {
  const int tid = threadIdx.x;
  const int e = 4 * qi;
  if (tid < kQuadRows) {
    const int jq = tid >> 4, h = tid & 15;
    x.ok = e + jq < n && h < R;
    const int64_t t = a.row_lo + (x.ok ? (codes[e + jq] >> 4) : 0);
    const int64_t rh = t * a.Hq + g * R + (x.ok ? h : 0);
    x.lse = a.lse[rh];
    x.delta = a.delta[rh];
  } else if (tid < kQuadRows + 4) {
    const int jq = tid - kQuadRows;
    const bool ok = e + jq < n;
    const int64_t t = a.row_lo + (ok ? (codes[e + jq] >> 4) : 0);
    x.pos = ok ? (int)((int64_t)N - M + (t - q0)) : -1;
  }
}

__device__ __forceinline__ void bwd_store_aux(BwdTile& T, const QuadAux& x) {
  const int tid = threadIdx.x;
  if (tid < kQuadRows) {
    // a missing MFMA row gets lse = +inf, so its probabilities are exactly 0
    T.lse[tid] = x.ok ? x.lse * kLog2e : __builtin_inff();
    T.delta[tid] = x.ok ? x.delta : 0.f;
  } else if (tid < kQuadRows + 4) {
    T.pos[tid - kQuadRows] = x.pos;
  }
}

// One staged quad against a key tile of 32 keys, by the tile's two waves.
// Wave A (keeps the keys' K rows as MFMA operands) computes S = Q K^T over
// the quad's 64 rows, P = exp(S - lse) (0 where the key is past the query),
// hands P to wave B through LDS (fp32, each lane its own 16 values per half)
// and accumulates dV += P^T dO; wave B (keeps the V rows) computes
// dP = dO V^T, dS = P (dP - delta) and accumulates dK += dS^T Q.  The two
// share a SIMD, so one's arithmetic runs while the other waits.  S, dP, P
// and dS are the same numbers in the same order as a single wave computing
// all four products.
struct BwdXch {
  float p[kBlock / 32][2 * 16][kWave];  // [key tile][half * 16 + C register][lane]
};

// S (A) or dP (B) of the quad's 64 rows: two halves of 32 MFMA rows, 8 k-steps
// each, the halves' MFMAs alternating (each accumulator sums its k-steps in
// order, and consecutive MFMAs do not depend on each other) with operands
// read from LDS two steps ahead.
__device__ __forceinline__ void bwd_first_product(const bf16* tile, const bf16x8 (&kv)[kHeadDim / 16], int col,
                                                  int a32, f32x16 (&acc)[2]) {
  constexpr int kKs = kHeadDim / 16;
  const int arow0 = bwd_tile_row(col) * kBwdRow + 8 * a32;  // MFMA row col (+ 32 for the second half)
  // step st: half st % 2, k-step st / 2
  auto aofs = [&](int st) { return arow0 + (st & 1) * 32 * kBwdRow + 16 * (st >> 1); };
  bf16x8 op[3];
  op[0] = *reinterpret_cast<const bf16x8*>(&tile[aofs(0)]);
  op[1] = *reinterpret_cast<const bf16x8*>(&tile[aofs(1)]);
  acc[0] = acc[1] = f32x16{};
#pragma unroll
  for (int st = 0; st < 2 * kKs; ++st) {
    if (st + 2 < 2 * kKs) op[(st + 2) % 3] = *reinterpret_cast<const bf16x8*>(&tile[aofs(st + 2)]);
    acc[st & 1] = mma32(op[st % 3], kv[st >> 1], acc[st & 1]);
  }
}

// acc[dt] += X^T Y over the quad's 64 rows: A operands x (P or dS, k-step s4
// = rows 16 s4 .. +15 in the slots of the C layout: slot i of lane half a32
// is row 16 s4 + 4 a32 + i (i < 4) or 16 s4 + 8 + 4 a32 + i - 4), B operands
// read transposed from the row-major tile (dO or Q): two reads per step,
// MFMA rows 16 s4 + 4 a32 .. +3 and 8 rows further, dims 32 dt + col; in
// tile rows that is 16 s4 + 4 e + a32 (+ 2) for the lane's e (tr_off holds
// the lane's tile row 4 e + a32 and column 16 (lane / 16 % 2) + 4 q).
// The four dim tiles' MFMAs alternate (each accumulator still sums its
// k-steps in order 0..3); operands are read two steps ahead.
__device__ __forceinline__ void bwd_second_product(const bf16* tile, const bf16x8 (&x)[4], int tr_off,
                                                   f32x16 (&acc)[kHeadDim / 32]) {
  constexpr int kDt = kHeadDim / 32;
  // step st: dim tile st % kDt, k-step st / kDt
  auto opnd = [&](int st) {
    const bf16* p = tile + tr_off + 16 * (st / kDt) * kBwdRow + 32 * (st % kDt);
    const bf16x4 lo = lds_read_tr4(p), hi = lds_read_tr4(p + 2 * kBwdRow);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  constexpr int kSteps = 4 * kDt;
  bf16x8 b[3];
  b[0] = opnd(0);
  b[1] = opnd(1);
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    if (st + 2 < kSteps) b[(st + 2) % 3] = opnd(st + 2);
    acc[st % kDt] = mma32(x[st / kDt], b[st % 3], acc[st % kDt]);
  }
}

// dS of a quad, key-major for the dQ product: [key][MFMA row], rows of kDsRow
// bf16.  96 elements (48 dwords, 16 of the 64 banks back) put the four keys a
// transposed read gathers on distinct banks; within a key row, the 8-byte
// unit of MFMA rows 4 u .. 4 u + 3 is stored at unit u ^ ((key / 4) % 8), so
// the writes of 32 keys at one unit also spread over all banks (without it
// they fell on 4 bank groups, 8-way).  The four keys of a read share the XOR.
// Both the writes and the transposed reads take the minimum two cycles per
// 512 bytes (a model of the 64 banks; 64 or 80 elements would take four).
constexpr int kDsRow = 96;
struct BwdDsT {
  bf16 ds[kBlock * kDsRow];
};
__device__ __forceinline__ int bwd_ds_off(int key, int row4) {  // row4: first of 4 MFMA rows, a multiple of 4
  return key * kDsRow + 4 * ((row4 >> 2) ^ ((key >> 2) & 7));
}

// A quad's dQ, staged in LDS by the B waves (each 32 of the 128 dims of all
// 64 MFMA rows) and stored to the partials by the A waves, one edge (16 heads
// x 128 dims, 4 KB contiguous in the partials) each: whole rows, so every
// store writes 1 KB of whole cache lines (the C layout would scatter 16-byte
// pieces of 32 rows per store).  Rows of 136 bf16 (272 bytes) keep both the
// 8-byte writes of 32 rows and the 16-byte reads of 4 rows free of bank
// conflicts.
struct BwdDqStage {
  bf16 q[kQuadRows * kBwdRow];
};

// Quad qi's dQ^T over the block's 128 keys for dims 32 dt .. +31: two 32 x 32
// tiles, MFMA rows 0..31 and 32..63, their MFMAs alternating; A operands K^T
// of those dims (registers, k-step ks = keys 16 ks .. +15, lane half a32
// holding keys 16 ks + 8 a32 .. +7), B operands dS^T read transposed from the
// key-major tile two steps ahead.  The result goes to the staging tile.
__device__ __forceinline__ void bwd_dq_tiles(const BwdDsT& D, BwdDqStage& Q, const bf16x8 (&kt)[kHeadDim / 16], int dt,
                                             int lane) {
  const int a32 = lane >> 5;
  // lane 16 g + 4 e + q of a transposed read: key 16 ks + 8 (g / 2) + e (+ 4),
  // MFMA rows rb + 16 (g % 2) + 4 q .. +3
  const int gq = lane >> 4;
  const int key0 = 8 * (gq >> 1) + ((lane & 15) >> 2), row4 = 16 * (gq & 1) + 4 * (lane & 3);
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  constexpr int kKs = kHeadDim / 16;
  // step st: row tile st % 2 (rb = 32 (st % 2)), k-step st / 2
  auto opnd = [&](int st) {
    const int ks = st >> 1, rb = 32 * (st & 1);
    const bf16x4 lo = lds_read_tr4(D.ds + bwd_ds_off(16 * ks + key0, rb + row4));
    const bf16x4 hi = lds_read_tr4(D.ds + bwd_ds_off(16 * ks + key0 + 4, rb + row4));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  bf16x8 bq[3];
  bq[0] = opnd(0);
  bq[1] = opnd(1);
#pragma unroll
  for (int st = 0; st < 2 * kKs; ++st) {
    if (st + 2 < 2 * kKs) bq[(st + 2) % 3] = opnd(st + 2);
    acc[st & 1] = mma32(kt[st >> 1], bq[st % 3], acc[st & 1]);
  }
  // C layout: column = MFMA row 32 t + lane % 32, rows = dims 32 dt + 8 j + 4 a32 + i
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      lds_store8(&Q.q[(32 * t + (lane & 31)) * kBwdRow + 32 * dt + 8 * j + 4 * a32],
                 bf16x4{bf16(acc[t][4 * j]), bf16(acc[t][4 * j + 1]), bf16(acc[t][4 * j + 2]), bf16(acc[t][4 * j + 3])});
}

// Edge e's rows of the staged dQ (MFMA rows 16 jq .. 16 jq + 15, jq = e % 4)
// to the bf16 partial of its selection slot (unscaled, like the forward's
// partial outputs; bwd_dq_combine sums a row's slots in order): four stores
// of 64 lanes x 16 bytes, heads 4 i .. 4 i + 3.  The stores go through a
// buffer that spans the edge's R heads only, so the hardware drops those of
// heads past R, and all of them for a missing edge (e >= n): the wave always
// issues exactly four stores, which lets the end of a step wait for its
// earlier loads without waiting for these.
constexpr int kDqStores = 4;
__device__ __forceinline__ void bwd_dq_store(const BwdKernelArgs& a, const BwdDqStage& Q, const uint32_t* codes, int e,
                                             int n, int lane, int g, int R) {
  const bool ok = e < n;
  const uint32_t cd = __builtin_amdgcn_readfirstlane(ok ? codes[e] : 0u);
  const int64_t slot = ((int64_t)(cd >> 4) * a.G + g) * a.topk + (cd & 15);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(a.part_dq + slot * 16 * kHeadDim, 0,
                                                                     ok ? R * kHeadDim * 2 : 0, 0x00020000);
  const bf16* src = Q.q + (16 * (e & 3) + (lane >> 4)) * kBwdRow + 8 * (lane & 15);
#pragma unroll
  for (int i = 0; i < kDqStores; ++i) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + 4 * i * kBwdRow);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (4 * i + (lane >> 4)) * kHeadDim * 2 + 16 * (lane & 15), 0, 0);
  }
}

__global__ __launch_bounds__(kDkvThreads, 1) void bwd_dkdv(BwdKernelArgs a) {
  __shared__ __attribute__((aligned(16))) BwdTile T0;
  __shared__ __attribute__((aligned(16))) BwdTile T1;
  __shared__ __attribute__((aligned(16))) BwdXch X;
  __shared__ __attribute__((aligned(16))) BwdDsT D;
  __shared__ __attribute__((aligned(16))) uint32_t codes[kDkvChunk];
  __shared__ __attribute__((aligned(16))) BwdDqStage Q;
  __shared__ uint32_t plan[kDkvWaves][kRunsPerWave * kWave];
  static_assert(sizeof(T0.rm) >= (size_t)kBlock * kBwdRow * sizeof(bf16), "the K tile of the set-up fits a staging tile");
  const int nbk = a.batch * a.G * a.nb_max;
  const int w = blockIdx.x;
  if (w >= a.dkv_chunk[nbk]) return;
  const int bucket = bwd_find(a.dkv_chunk, nbk, w);
  const int chunk = w - a.dkv_chunk[bucket];
  const int nchunks = a.dkv_chunk[bucket + 1] - a.dkv_chunk[bucket];
  const int c = bucket % a.nb_max;
  const int g = (bucket / a.nb_max) % a.G;
  const int b = bucket / (a.nb_max * a.G);
  const int e_lo = a.offsets[bucket] + chunk * kDkvChunk;
  const int n = min(kDkvChunk, a.offsets[bucket + 1] - e_lo);
  if (n <= 0) return;
  const int64_t kb0 = a.cu_k[b];
  const int N = a.cu_k[b + 1] - a.cu_k[b];
  const int64_t q0 = a.cu_q[b];
  const int M = a.cu_q[b + 1] - a.cu_q[b];
  const int R = a.Hq / a.G;
  const int64_t rs = (int64_t)a.G * kHeadDim;
  const int tid = threadIdx.x;

  // ---- the chunk's edge codes, (row in window) << 4 | selection slot (the
  // bucket's list is sorted, so the order in which edges are summed is fixed)
  for (int i = tid; i < n; i += kDkvThreads) codes[i] = (uint32_t)a.edges[e_lo + i];

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kt = wave & 3;          // key tile: keys 32 kt .. 32 kt + 31 of the block
  const bool role_b = wave >= 4;    // A: S, P, dV (K rows); B: dP, dS, dK (V rows)
  const int lane = lane_id();
  const int col = lane & 31;  // MFMA row of A / column of B and C
  const int a32 = lane >> 5;
  // staging: buffer resources over the window's rows of Q and dO (a window
  // holds at most kBwdWindow rows of at most 256 heads: offsets fit 32 bits)
  const int64_t win_rows = min((int64_t)kBwdWindow, (int64_t)a.cu_q[a.batch] - a.row_lo);
  const uint32_t row_bytes = (uint32_t)a.Hq * kHeadDim * 2;
  const int win_bytes = (int)(win_rows * row_bytes);
  const bf16* win_q = a.q + a.row_lo * a.Hq * kHeadDim;
  const bf16* win_g = a.dout + a.row_lo * a.Hq * kHeadDim;
  bwd_dma_plan(plan[wave], wave, lane, g, R);
  // transposed reads: this lane's MFMA row 4 a32 + e (tile row 4 e + a32) and
  // column 16 (lane / 16 % 2) + 4 q inside a 16-row k-step (lane = 16 (2 a32
  // + lane / 16 % 2) + 4 e + q)
  const int tr_off = (4 * ((lane & 15) >> 2) + a32) * kBwdRow + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // this tile's 32 keys: K (wave A) or V (wave B) rows as the B operands of
  // the first product (column = key, 8 dims per k-step half); rows past the
  // sequence end clamp to its last row and are masked (key > every p)
  const int key_seq = c * kBlock + 32 * kt + col;
  const int64_t krow = kb0 + (key_seq < N ? key_seq : N - 1);
  const bf16* kvsrc = role_b ? a.v : a.k;
  bf16x8 kvf[kHeadDim / 16];
#pragma unroll
  for (int ks = 0; ks < kHeadDim / 16; ++ks) kvf[ks] = load8(kvsrc + krow * rs + g * kHeadDim + 16 * ks + 8 * a32);
  f32x16 acc[kHeadDim / 32];  // dV (A) or dK (B, unscaled)
#pragma unroll
  for (int dt = 0; dt < kHeadDim / 32; ++dt) acc[dt] = f32x16{};

  // ---- K^T fragments of the dQ product (wave B: the dQ^T tiles of dims 32 kt,
  // both row halves): the block's K rows staged row-major in T0 for the
  // set-up, then read transposed: dims 32 kt + lane % 32, keys 16 ks + 8
  // (lane / 32) .. +7 (rows past the sequence end clamp to its last row;
  // their dS are 0)
  bf16x8 ktf[kHeadDim / 16];
  {
    bf16* kt_lds = &T0.rm[0][0];
#pragma unroll
    for (int u = 0; u < kBlock * kHeadDim / 8 / kDkvThreads; ++u) {
      const int piece = tid + u * kDkvThreads;
      const int row = piece >> 4, cc = (piece & 15) * 8;
      const int64_t key = min(c * kBlock + row, N - 1);
      *reinterpret_cast<bf16x8*>(kt_lds + row * kBwdRow + cc) = load8(a.k + (kb0 + key) * rs + g * kHeadDim + cc);
    }
    lds_barrier();
    const int gq = lane >> 4;
    const bf16* src = kt_lds + (8 * (gq >> 1) + ((lane & 15) >> 2)) * kBwdRow + 32 * kt + 16 * (gq & 1) +
                      4 * (lane & 3);
    if (role_b) {
#pragma unroll
      for (int ks = 0; ks < kHeadDim / 16; ++ks) {
        const bf16x4 lo = lds_read_tr4(src + 16 * ks * kBwdRow), hi = lds_read_tr4(src + (16 * ks + 4) * kBwdRow);
        ktf[ks] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
  }

  // Quads alternate between the two tiles: the staging loads of quad qi + 1
  // are issued before quad qi is computed and waited for after it.  Quad
  // qi - 1's dQ (its dS tile is complete) is computed by the B waves before
  // their dP, while the A waves compute S, so the two waves' MFMAs share the
  // SIMD's pipe, and the A waves' P runs beside the B waves' dP.
  const int nquads = (n + 3) / 4;
  QuadAux x;
  lds_barrier();  // the codes and the plan are written; the K tile is read
  bwd_issue_quad(T0, plan[wave], codes, 0, n, wave, lane, win_q, win_g, win_bytes, row_bytes);
  bwd_load_aux(a, x, codes, 0, n, g, R, N, M, q0);
  bwd_store_aux(T0, x);
  vmem_wait_all();
  lds_barrier();
  const float sl2 = a.scale_log2;
  auto step = [&](BwdTile& cur, BwdTile& nxt, int qi) {
    const bool more = qi + 1 < nquads;
    if (more) {
      // the lse / delta loads first: waiting for them later then does not
      // wait for the staging loads issued after them
      bwd_load_aux(a, x, codes, qi + 1, n, g, R, N, M, q0);
      bwd_issue_quad(nxt, plan[wave], codes, qi + 1, n, wave, lane, win_q, win_g, win_bytes, row_bytes);
    }
    if (role_b && qi > 0) bwd_dq_tiles(D, Q, ktf, kt, lane);
    f32x16 f[2];  // S (A) or dP (B), halves of 32 rows
    bwd_first_product(cur.rm[role_b ? 1 : 0], kvf, col, a32, f);
    bf16x8 xa[4];  // P (A) or dS (B) as the A operands of the second product
    if (!role_b) {
      // C layout: this lane's key, rows 32 rh + 8 (r / 4) + 4 a32 + r % 4;
      // rows 16 j .. 16 j + 15 belong to query j of the quad
#pragma unroll
      for (int rh = 0; rh < 2; ++rh) {
        const bool live0 = key_seq <= cur.pos[2 * rh], live1 = key_seq <= cur.pos[2 * rh + 1];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 ls = *reinterpret_cast<const f32x4*>(&cur.lse[32 * rh + 8 * q4 + 4 * a32]);
          const bool live = q4 < 2 ? live0 : live1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * q4 + i;
            const float pv = live ? __builtin_amdgcn_exp2f(f[rh][r] * sl2 - ls[i]) : 0.f;
            X.p[kt][16 * rh + r][lane] = pv;
            xa[2 * rh + (r >> 3)][r & 7] = bf16(pv);
          }
        }
      }
    }
    lds_barrier();  // P and quad qi - 1's dQ are in LDS; the B waves are done with its dS tile
    if (role_b) {
#pragma unroll
      for (int rh = 0; rh < 2; ++rh)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 dl = *reinterpret_cast<const f32x4*>(&cur.delta[32 * rh + 8 * q4 + 4 * a32]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * q4 + i;
            const float ds = X.p[kt][16 * rh + r][lane] * (f[rh][r] - dl[i]);
            xa[2 * rh + (r >> 3)][r & 7] = bf16(ds);
          }
          // dS^T for the dQ product: this lane's key, rows 32 rh + 8 q4 + 4 a32 .. +3
          const bf16x8& v = xa[2 * rh + (q4 >> 1)];
          const int o = 4 * (q4 & 1);
          lds_store8(&D.ds[bwd_ds_off(32 * kt + col, 32 * rh + 8 * q4 + 4 * a32)], bf16x4{v[o], v[o + 1], v[o + 2], v[o + 3]});
        }
    }
    bwd_second_product(cur.rm[role_b ? 0 : 1], xa, tr_off, acc);
    if (more) bwd_store_aux(nxt, x);  // before the dQ stores: its wait for the lse / delta loads then excludes them
    if (!role_b && qi > 0) bwd_dq_store(a, Q, codes, 4 * (qi - 1) + kt, n, lane, g, R);
    // quad qi + 1 is in LDS (an A wave's four dQ stores, issued last, may
    // still be in flight)
    if (!role_b && qi > 0) vmem_wait_all_but<kDqStores>(); else vmem_wait_all();
    lds_barrier();  // and quad qi's dS tile is complete; the dQ stage is read
  };
  for (int qi = 0; qi < nquads; qi += 2) {
    step(T0, T1, qi);
    if (qi + 1 < nquads) step(T1, T0, qi + 1);
  }
  if (role_b) bwd_dq_tiles(D, Q, ktf, kt, lane);
  lds_barrier();
  if (!role_b) bwd_dq_store(a, Q, codes, 4 * (nquads - 1) + kt, n, lane, g, R);

  // ---- lane column d = 32 dt + col, rows = keys 8 (r / 4) + 4 a32 + r % 4 of
  // the tile's 32.  A bucket's only chunk adds this window's contribution to
  // dV (wave A) / dK (wave B); the chunks of a longer bucket write partials
  // for bwd_dkdv_reduce.
  const float osc = role_b ? a.scale : 1.f;
  if (nchunks == 1) {
    // the first window writes its blocks' rows outright; later ones add, all
    // loads issued (branch-free: rows past the sequence end read its last
    // row) before the first store
    float* dst = role_b ? a.dk : a.dv;
    const bool add = a.row_lo != 0;
    float old[kHeadDim / 32][16];
    if (add) {
#pragma unroll
      for (int dt = 0; dt < kHeadDim / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = c * kBlock + 32 * kt + 8 * (r >> 2) + 4 * a32 + (r & 3);
          old[dt][r] = dst[(kb0 + (kk < N ? kk : N - 1)) * rs + g * kHeadDim + 32 * dt + col];
        }
    }
#pragma unroll
    for (int dt = 0; dt < kHeadDim / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = c * kBlock + 32 * kt + 8 * (r >> 2) + 4 * a32 + (r & 3);
        if (kk >= N) continue;
        const float xv = acc[dt][r] * osc;
        dst[(kb0 + kk) * rs + g * kHeadDim + 32 * dt + col] = add ? old[dt][r] + xv : xv;
      }
  } else {
    // partial: [dK (unscaled) | dV] of the chunk
    float* part = a.part_dkv + (int64_t)(a.dkv_part[bucket] + chunk) * (2 * kBlock * kHeadDim) +
                  (role_b ? 0 : kBlock * kHeadDim);
#pragma unroll
    for (int dt = 0; dt < kHeadDim / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kt + 8 * (r >> 2) + 4 * a32 + (r & 3);
        part[key * kHeadDim + 32 * dt + col] = acc[dt][r];
      }
  }
}

// dK += scale * (sum of the chunk partials), dV += sum of the partials, for
// each bucket of more than one chunk, the chunks summed in order: four
// workgroups per bucket, each a quarter of the partial; a thread's four
// chunk loads are issued together before their in-order sum.
constexpr int kReduceSplit = 4;

__global__ __launch_bounds__(256) void bwd_dkdv_reduce(BwdKernelArgs a) {
  const int nbk = a.batch * a.G * a.nb_max;
  const int bucket = blockIdx.x / kReduceSplit;
  const int quarter = blockIdx.x % kReduceSplit;
  if (bucket >= nbk) return;
  const int nchunks = a.dkv_chunk[bucket + 1] - a.dkv_chunk[bucket];
  if (nchunks <= 1) return;
  const int c = bucket % a.nb_max;
  const int g = (bucket / a.nb_max) % a.G;
  const int b = bucket / (a.nb_max * a.G);
  const int64_t kb0 = a.cu_k[b];
  const int N = a.cu_k[b + 1] - a.cu_k[b];
  const int64_t rs = (int64_t)a.G * kHeadDim;
  constexpr int64_t kSlot = 2 * kBlock * kHeadDim;  // floats of one partial
  const f32x4* p0 = reinterpret_cast<const f32x4*>(a.part_dkv + (int64_t)a.dkv_part[bucket] * kSlot);
  constexpr int kPer = (int)(kSlot / 4) / kReduceSplit;  // float4 units of this workgroup
  for (int u = quarter * kPer + threadIdx.x; u < (quarter + 1) * kPer; u += 256) {
    f32x4 acc = p0[u];
    int k = 1;
    for (; k + 4 <= nchunks; k += 4) {
      const f32x4 x0 = p0[(int64_t)k * (kSlot / 4) + u], x1 = p0[(int64_t)(k + 1) * (kSlot / 4) + u];
      const f32x4 x2 = p0[(int64_t)(k + 2) * (kSlot / 4) + u], x3 = p0[(int64_t)(k + 3) * (kSlot / 4) + u];
      acc += x0;
      acc += x1;
      acc += x2;
      acc += x3;
    }
    for (; k < nchunks; ++k) acc += p0[(int64_t)k * (kSlot / 4) + u];
    const int e = 4 * u;
    const bool is_v = e >= kBlock * kHeadDim;
    const int key = (e % (kBlock * kHeadDim)) / kHeadDim, d = e % kHeadDim;
    const int kk = c * kBlock + key;
    if (kk >= N) continue;
    float* dst = (is_v ? a.dv : a.dk) + (kb0 + kk) * rs + g * kHeadDim + d;
    const f32x4 add = is_v ? acc : acc * a.scale;
    if (a.row_lo == 0) *reinterpret_cast<f32x4*>(dst) = add;  // the first window writes outright
    else *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<f32x4*>(dst) + add;
  }
}

// ---------------------------------------------------------------- dQ
// KV-outer, one workgroup per chunk of <= kEdgeChunk edges of one bucket (the
// chunks of the forward's schedule).  K is staged row-major (A operand of
// S^T = K Q^T) and transposed (B operand of dQ = dS K), V row-major (A operand
// of dP^T = V dO^T).  Each wave runs pairs of edges (2 queries x 16 heads =
// 32 MFMA columns) tile by tile over 32 keys: S^T and dP^T, then dS, whose
// registers (column = the lane's (query, head), 8 keys per k-step) are
// directly the A operand of dQ += dS K.  Each edge writes its block's dQ
// contribution (bf16) to the partial slot of its selection entry; a
// fixed-order fp32 sum over the slots follows.
// Validity of the entries of one selection row: attended when the id names a
// block at or before the local block and does not repeat an earlier entry.
__device__ __forceinline__ unsigned bwd_row_mask(const int32_t* sel, int topk, int64_t local, int nb_max) {
  int cc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) cc[i] = i < topk ? sel[i] : -1;
  unsigned mask = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    bool ok = cc[i] >= 0 && cc[i] <= local && cc[i] < nb_max;
#pragma unroll
    for (int j = 0; j < i; ++j) ok = ok && (cc[j] != cc[i]);
    mask |= ok ? (1u << i) : 0u;
  }
  return mask;
}

// dq = scale * sum over the row's selection slots (in slot order) of the
// partials: one wave per (row, group).
__global__ __launch_bounds__(256) void bwd_dq_combine(BwdKernelArgs a, int64_t row_hi) {
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (row_hi - a.row_lo) * a.G) return;
  const int64_t trel = item / a.G;
  const int g = (int)(item % a.G);
  const int64_t t = a.row_lo + trel;
  if (t >= a.cu_q[a.batch]) return;
  const int lane = lane_id();
  const int R = a.Hq / a.G;
  // lane: dims 8 (lane % 16) .. +7 of heads lane / 16 + 4 j, j < nj, so each
  // load (fixed j) reads 1 KB of a slot's partial and each store writes 512
  // contiguous bytes of dq per head
  const int hl = lane >> 4, d0 = 8 * (lane & 15);
  const int nj = (R + 3) / 4;  // quads of heads that hold heads < R
  const int bq = bwd_find(a.cu_q, a.batch, t);
  const int64_t p = (int64_t)(a.cu_k[bq + 1] - a.cu_k[bq]) - (a.cu_q[bq + 1] - a.cu_q[bq]) + (t - a.cu_q[bq]);
  const unsigned mask = p >= 0 ? bwd_row_mask(a.block_idx + (t * a.G + g) * a.topk, a.topk, p / kBlock, a.nb_max)
                               : 0u;
  const int64_t slot0 = (trel * a.G + g) * a.topk;
  f32x4 acc[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < a.topk; ++i) {
    if (!((mask >> i) & 1u)) continue;
    const bf16* src = a.part_dq + ((slot0 + i) * 16 + hl) * kHeadDim + d0;
    bf16x8 v8[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < nj) v8[j] = load8(src + 4 * j * kHeadDim);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < nj) {
        acc[j][0] += f32x4{(float)v8[j][0], (float)v8[j][1], (float)v8[j][2], (float)v8[j][3]};
        acc[j][1] += f32x4{(float)v8[j][4], (float)v8[j][5], (float)v8[j][6], (float)v8[j][7]};
      }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * j + hl;
    if (h >= R) continue;
    float* dst = a.dq + (t * a.Hq + g * R + h) * kHeadDim + d0;
    *reinterpret_cast<f32x4*>(dst) = acc[j][0] * a.scale;
    *reinterpret_cast<f32x4*>(dst + 4) = acc[j][1] * a.scale;
  }
}

BwdPlan plan_bwd(int batch, int max_q_len, int max_kv_len, int Hq, int G, int topk) {
  BwdPlan pl;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  pl.nb_max = (max_kv_len + kBlock - 1) / kBlock;
  pl.nbuckets = batch * G * pl.nb_max;
  pl.rows_bound = (int64_t)batch * max_q_len;
  const int64_t win = kBwdWindow;
  pl.window = pl.rows_bound < win ? pl.rows_bound : win;
  const size_t nbk = (size_t)pl.nbuckets;
  size_t off = 0;
  pl.counts_off = off;  off += al(nbk * 4);
  pl.offsets_off = off; off += al((nbk + 1) * 4);
  pl.chunks_off = off;  off += al((nbk + 1) * 4);
  pl.cursor_off = off;  off += al(nbk * 4);
  pl.edges_off = off;   off += al((size_t)pl.window * G * topk * 4);
  pl.delta_off = off;   off += al((size_t)pl.rows_bound * Hq * 4);
  pl.dkv_chunk_off = off; off += al((nbk + 1) * 4);
  pl.dkv_part_off = off;  off += al((nbk + 1) * 4);
  // a bucket of n > kDkvChunk edges takes ceil(n / kDkvChunk) < 2 n / kDkvChunk slots
  const size_t slots = 2 * (size_t)pl.window * G * topk / kDkvChunk + 1;
  pl.part_dkv_off = off;  off += al(slots * 2 * kBlock * kHeadDim * sizeof(float));
  pl.part_dq_off = off; off += al((size_t)pl.window * G * topk * 16 * kHeadDim * sizeof(bf16));
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
  a.chunk_start = chunks;
  a.edges = reinterpret_cast<int32_t*>(w + pl.edges_off);
  a.delta = reinterpret_cast<float*>(w + pl.delta_off);
  a.dkv_chunk = reinterpret_cast<int32_t*>(w + pl.dkv_chunk_off);
  a.dkv_part = reinterpret_cast<int32_t*>(w + pl.dkv_part_off);
  a.part_dkv = reinterpret_cast<float*>(w + pl.part_dkv_off);
  a.part_dq = reinterpret_cast<bf16*>(w + pl.part_dq_off);
  a.dq = x.dq;
  a.dk = x.dk;
  a.dv = x.dv;

  hipLaunchKernelGGL(bwd_delta, dim3((unsigned)((pl.rows_bound * a.Hq + 7) / 8)), dim3(256), 0, st, a);
  for (int64_t r0 = 0; r0 < pl.rows_bound; r0 += pl.window) {
    const int64_t r1 = r0 + pl.window < pl.rows_bound ? r0 + pl.window : pl.rows_bound;
    hipError_t e = build_edge_lists(x.fwd, pl.nb_max, r0, r1, counts, offsets, chunks, nullptr, cursor, a.edges, true, st);
    if (e != hipSuccess) return e;
    a.row_lo = r0;
    if (r0 == 0) hipLaunchKernelGGL(bwd_zero, dim3((unsigned)pl.nbuckets), dim3(256), 0, st, a);
    const int64_t entries = (r1 - r0) * a.G * a.topk;
    hipLaunchKernelGGL(bwd_dkv_scan, dim3(1), dim3(1024), 0, st, a, pl.nbuckets);
    // chunks of kDkvChunk edges: at most entries / kDkvChunk + one partial chunk per bucket
    const int64_t ub_kv = entries / kDkvChunk + (entries < pl.nbuckets ? entries : pl.nbuckets) + 1;
    hipLaunchKernelGGL(bwd_dkdv, dim3((unsigned)ub_kv), dim3(kDkvThreads), 0, st, a);
    hipLaunchKernelGGL(bwd_dkdv_reduce, dim3((unsigned)pl.nbuckets * kReduceSplit), dim3(256), 0, st, a);
    hipLaunchKernelGGL(bwd_dq_combine, dim3((unsigned)(((r1 - r0) * a.G + 3) / 4)), dim3(256), 0, st, a, r1);
  }
  return hipGetLastError();
}

}  // namespace msa
