// index_topk.hip -- MSA index branch on gfx950: score, block max-pool, top-k.
//
// Method: "MiniMax Sparse Attention: let each query pick its own blocks",
// section "The mechanism, precisely" and the paper's Figure 1 there (index
// query head per group, one shared index key head, Q_idx K_idx^T, block max
// pooling, top-k blocks, local block always kept).  Selection is on raw
// scores with no softmax ("exp-free" top-k in the atlas record's kernel list).
//
// Prefill path (two kernels):
//   idx_scan_prefill  one workgroup per (sequence, query block, query slice,
//                     key chunk), or per mirror pair of them when a call has
//                     two rounds of those.  Its columns are the (query, group) pairs of
//                     one query block -- all queries of a block scan the same
//                     earlier blocks, so no causal mask is ever needed.  Each
//                     key block (128 x d_idx) is staged in LDS once and shared
//                     by 8 waves; scores come from 32x32 MFMA tiles oriented
//                     keys x columns, so a column's 128 scores sit in two lanes
//                     (16 registers x 4 tiles each) and the block max is a
//                     register max plus one lane swap.  The pooled score of
//                     every (row, group, earlier block) is written to the
//                     workspace as fp32, [rows, G, score_stride], in aligned
//                     64-byte runs of 16 consecutive blocks.  The top-k is not
//                     kept inside the GEMM: a per-lane sorted list there costs
//                     the whole wave an insertion whenever any of its 64 lanes
//                     takes a block, which is nearly every block.
//   idx_select_prefill one wave per (row, group): 64-bit selection keys
//                     (order-preserving score bits, inverted block id, so the
//                     lower id wins ties) are read back in rounds of 1024; the
//                     16th largest of the lane maxima (a bitwise search
//                     counted by ballots), or the 16th best kept from earlier
//                     rounds if larger, is a threshold; the few keys at or
//                     above it are compacted (lane offsets from one ballot
//                     per bit of the lanes' counts) and ranked exactly;
//                     the best k-1 and the local block are written ascending,
//                     -1 padded.
// Decode path (two kernels):
//   idx_decode_scores streams the index-key cache once: the earlier blocks of
//                     all sequences are one flat range scored grid-stride by
//                     waves (16x16 MFMA, keys x groups), one fp32 per (group,
//                     block).
//   idx_decode_select one workgroup per (sequence, group): a threshold from
//                     the per-thread maxima of 64-bit selection keys, then an
//                     exact rank of the few keys that reach it.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

// --------------------------------------------------------------------------
// Prefill scan
// --------------------------------------------------------------------------
constexpr int kScanThreads = 512;  // 8 waves; each owns 64 columns (two 32-wide tiles)

template <typename T, int DI>
struct ScanLds {
  // One key block in LDS: rows of kChunksPerRow 16-byte chunks plus one chunk
  // of padding, so 16-byte reads of 32 rows at the same column spread over
  // the banks.  It is written by direct global-to-LDS loads, each filling 64
  // consecutive 16-byte slots (lane i slot i), so the padding slots are
  // written too (with a copy of the row's first chunk) and the buffer is a
  // whole number of such runs.
  static constexpr int kChunksPerRow = DI * (int)sizeof(T) / 16;
  static constexpr int kRowSlots = kChunksPerRow + 1;
  static constexpr int kRowBytes = kRowSlots * 16;
  static constexpr int kRuns = (kBlock * kRowSlots + kWave - 1) / kWave;  // 64-slot loads per block
  static constexpr int kBufBytes = kRuns * kWave * 16;
};

// Operands of the scan's 32x32 MFMA per element type: a lane feeds kLaneK
// consecutive contraction elements of its row (one fragment) and one MFMA
// contracts kStep elements (lanes l and l + 32 cover the two halves).
template <typename T> struct ScanMma;
template <> struct ScanMma<bf16> {
  using frag = bf16x8;
  static constexpr int kStep = 16, kLaneK = 8;
  static __device__ __forceinline__ frag load(const bf16* p) { return load8(p); }
  static __device__ __forceinline__ frag zero() { return zero8<bf16>(); }
  static __device__ __forceinline__ f32x16 mma(const frag& a, const frag& b, f32x16 c) { return mma32(a, b, c); }
};
template <> struct ScanMma<float> {
  using frag = f32x8;
  static constexpr int kStep = 16, kLaneK = 8;
  static __device__ __forceinline__ frag load(const float* p) { return load8(p); }
  static __device__ __forceinline__ frag zero() { return zero8<float>(); }
  static __device__ __forceinline__ f32x16 mma(const frag& a, const frag& b, f32x16 c) { return mma32(a, b, c); }
};
template <> struct ScanMma<fp8e4m3> {
  using frag = i32x8;
  static constexpr int kStep = 64, kLaneK = 32;
  static __device__ __forceinline__ frag load(const fp8e4m3* p) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(p), hi = *reinterpret_cast<const u32x4*>(p + 16);
    return frag{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  static __device__ __forceinline__ frag zero() { return frag{0, 0, 0, 0, 0, 0, 0, 0}; }
  static __device__ __forceinline__ f32x16 mma(const frag& a, const frag& b, f32x16 c) { return mma32_fp8(a, b, c); }
};

template <typename T, int DI>
__global__ __launch_bounds__(kScanThreads, 1) void idx_scan_prefill(
    const T* __restrict__ q_idx, const T* __restrict__ k_idx, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int G, int qw, int nsub, int max_qblocks, int chunk,
    int max_chunks, int nb_stride, int n_items, float* __restrict__ scores) {
  using L = ScanLds<T, DI>;
  using Mm = ScanMma<T>;
  constexpr int KS = DI / Mm::kStep;  // MFMA contraction steps
  // three LDS buffers where they fit beside nothing else (all but fp32 with
  // d_idx 128); the next key tile's fragments are read ahead, except for fp32,
  // whose fragments would not fit beside the query fragments in registers
  constexpr int kRing = 3 * L::kBufBytes <= 112 * 1024 ? 3 : 2;
  constexpr bool kPrefetch = sizeof(T) < 4;
  // block scores of the current group of 16 blocks, per wave [block % 16][lane]
  // (in LDS where it fits, else in registers)
  constexpr bool kSbLds = kRing * L::kBufBytes + 16 * kScanThreads * 4 <= 128 * 1024;
  __shared__ __attribute__((aligned(16))) char lds[kRing * L::kBufBytes];
  __shared__ float s_sb[kSbLds ? kScanThreads / kWave : 1][16][kWave];

  // The plan may pair items: item k and its mirror n_items - 1 - k on one
  // workgroup, one after the other.  With the heaviest query blocks first
  // in each key chunk, a mirror pair sums to about the same work everywhere
  // (for one causal sequence cut into two chunks, a full first chunk plus an
  // empty last one, or a short first chunk plus a long last one), so one
  // round of workgroups does a call that would otherwise take one and a half.
  const int n_pass = n_items > (int)gridDim.x ? 2 : 1;
  for (int pass = 0; pass < n_pass; ++pass) {
    if (pass == 1) {
      if (n_items - 1 - (int)blockIdx.x == (int)blockIdx.x) break;  // the middle item of an odd count
      __syncthreads();  // every wave is done with the ring buffers and the score stage
    }
    // Decode the workgroup: query block fastest (latest, i.e. heaviest, first),
    // then query slice, then key chunk, then sequence.  Workgroups are handed
    // to the 8 XCDs in turn by id, and each XCD runs its own share on its own
    // CUs, so neighbouring ids must carry similar work: with the key chunk
    // fastest and 2 or 4 chunks, an XCD received one chunk index only (all
    // full chunks on some XCDs, all short last chunks on others).
    int bid = pass == 0 ? (int)blockIdx.x : n_items - 1 - (int)blockIdx.x;
    const int slot = max_qblocks - 1 - (bid % max_qblocks);  bid /= max_qblocks;
    const int sub = bid % nsub;       bid /= nsub;
    const int ch = bid % max_chunks;
    const int b = bid / max_chunks;

    const int q0 = cu_q[b], M = cu_q[b + 1] - q0;
    const int k0 = cu_k[b], N = cu_k[b + 1] - k0;
    if (M <= 0 || N <= 0) continue;
    const int pfirst = N - M > 0 ? N - M : 0;  // first position that has keys
    const int c = pfirst / kBlock + slot;      // this workgroup's query block
    if (c * kBlock >= N) continue;
    const int plo = max(c * kBlock, pfirst) + sub * qw;
    const int phi = min(min((c + 1) * kBlock, N), plo + qw);
    if (plo >= phi) continue;
    const int s_lo = ch * chunk;
    const int s_hi = min(s_lo + chunk, c);  // scan earlier blocks only
    if (s_lo >= s_hi) continue;

    const int ncols = (phi - plo) * G;
    const int64_t row0 = (int64_t)(plo - (N - M)) + q0;  // first query row
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = lane_id();
    const int col_base = wave * 64;
    const bool active = col_base < ncols;
    // This lane's column after the block-max swap, and its row of block scores.
    // The scores of 16 consecutive blocks are gathered in registers (newest
    // last) and written as one 64-byte run: chunks start at multiples of 16
    // blocks and rows are 16-byte aligned, so every full group is aligned.
    const int col_mine = col_base + lane;
    const bool col_ok = col_mine < ncols;
    float* srow = scores + (row0 * G + (col_ok ? col_mine : 0)) * (int64_t)nb_stride;
    float sbuf[kSbLds ? 1 : 16];
#pragma unroll
    for (int j = 0; j < (kSbLds ? 1 : 16); ++j) sbuf[j] = 0.f;

    // B operand (Q^T): columns col_base + 32*j + lane%32, contraction slots
    // kStep*ks + kLaneK*(lane/32) .. +kLaneK-1.
    typename Mm::frag qf[2][KS];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = col_base + 32 * j + (lane & 31);
      const bool ok = col < ncols;
      const T* qp = q_idx + (row0 * G + (ok ? col : 0)) * DI + Mm::kLaneK * (lane >> 5);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[j][ks] = ok ? Mm::load(qp + Mm::kStep * ks) : Mm::zero();
    }

    // Key blocks are staged into LDS in 16-byte pieces (coalesced global reads
    // that write LDS directly, no register round trip) through a ring of kRing
    // buffers: block s + kRing - 1 is requested while block s is scored, and
    // the wait and barrier at the end of the step make it visible.  With three
    // buffers, block s + 1 is already in LDS while block s is scored, so the
    // key fragments of its first tile are read before the step's barrier and
    // the MFMAs of one block follow those of the previous without a gap.
    const char* kseq = reinterpret_cast<const char*>(k_idx + (int64_t)k0 * DI);
    constexpr int64_t kBlockBytes = (int64_t)kBlock * DI * sizeof(T);
    // Block `blk` into ring buffer `ring`: run u (of kRuns) fills slots
    // 64 u .. 64 u + 63, lane i slot 64 u + i; wave w does runs w, w + 8, ...
    // A slot's byte offset in the block (its row's chunk, or the row's first
    // chunk for a padding slot) does not depend on the block.
    constexpr int kRunsPerWave = (L::kRuns + kScanThreads / kWave - 1) / (kScanThreads / kWave);
    int src_off[kRunsPerWave];
#pragma unroll
    for (int u = 0; u < kRunsPerWave; ++u) {
      const int sl = (u * (kScanThreads / kWave) + wave) * kWave + lane;
      const int row = min(sl / L::kRowSlots, kBlock - 1);
      const int chunk = sl % L::kRowSlots;
      src_off[u] = row * (L::kChunksPerRow * 16) + (chunk < L::kChunksPerRow ? chunk : 0) * 16;
    }
    auto fetch = [&](int blk, int ring) {
      const char* src = kseq + blk * kBlockBytes;
#pragma unroll
      for (int u = 0; u < kRunsPerWave; ++u) {
        const int run = u * (kScanThreads / kWave) + wave;
        if (run < L::kRuns)
          lds_load16(src, (int)kBlockBytes, src_off[u], lds + ring * L::kBufBytes + run * kWave * 16);
      }
    };
#pragma unroll
    for (int pre = 0; pre < kRing - 1; ++pre)
      if (s_lo + pre < s_hi) fetch(s_lo + pre, pre);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // A operand (K rows): this lane's fragment of key tile kt, step ks, of ring
    // buffer r: row 32 kt + lane % 32, elements kStep ks + kLaneK (lane / 32) ..
    constexpr int kStepBytes = Mm::kStep * (int)sizeof(T);
    const int frag_off = (lane & 31) * L::kRowBytes + Mm::kLaneK * (lane >> 5) * (int)sizeof(T);
    auto kfrag = [&](int ring, int kt, int ks) {
      return *reinterpret_cast<const typename Mm::frag*>(lds + ring * L::kBufBytes + 32 * kt * L::kRowBytes + frag_off +
                                                         kStepBytes * ks);
    };
    typename Mm::frag kf[kPrefetch ? 2 : 1][KS];
    // kf[0]: tile 0 of the first block (later blocks' first tiles are read
    // during the tile before, with three buffers)
    if (kPrefetch && active) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[0][ks] = kfrag(0, 0, ks);
    }
    // A block's score: lane l < 32 owns column l of tile 0, lane l >= 32 column
    // l - 32 of tile 1; each needs the other half-wave's partial max of its own
    // column.  The scores of 16 consecutive blocks are stored together.
    auto finish = [&](int sb, float a0, float a1) {
      const float send = lane < 32 ? a1 : a0;
      const float recv = xchg_halves_f(send);
      const float v = fmaxf(lane < 32 ? a0 : a1, recv);
      if constexpr (kSbLds) {
        s_sb[wave][sb & 15][lane] = v;
        if ((sb & 15) == 15 && col_ok) {
          f32x4* dst = reinterpret_cast<f32x4*>(srow + (sb - 15));
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dst[q] = f32x4{s_sb[wave][4 * q][lane], s_sb[wave][4 * q + 1][lane], s_sb[wave][4 * q + 2][lane],
                           s_sb[wave][4 * q + 3][lane]};
        }
      } else {
#pragma unroll
        for (int j = 0; j < 15; ++j) sbuf[j] = sbuf[j + 1];
        sbuf[15] = v;
        if ((sb & 15) == 15 && col_ok) {
          f32x4* dst = reinterpret_cast<f32x4*>(srow + (sb - 15));
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[q] = f32x4{sbuf[4 * q], sbuf[4 * q + 1], sbuf[4 * q + 2], sbuf[4 * q + 3]};
        }
      }
    };
    // With the fragments read ahead (kPrefetch), two accumulator sets persist
    // across blocks: tile kt's scores are max-pooled during the second half of
    // tile kt + 1's MFMAs (its results are complete by then), the last tile of
    // block s - 1 during tile 0 of block s, and block s - 1's score is finished
    // after that tile.  So the MFMA pipe never waits for the pooling, and the
    // score stores have a whole block to complete before the wait at its end.
    static_assert((kBlock / 32) % 2 == 0, "the last tile of a block must land in acc[1]");
    f32x16 acc[2][2];
    float pm0 = -__builtin_inff(), pm1 = -__builtin_inff();  // block s - 1 over tiles 0 .. 2
    if constexpr (kPrefetch) {
#pragma unroll
      for (int r = 0; r < 16; ++r) { acc[1][0][r] = -__builtin_inff(); acc[1][1][r] = -__builtin_inff(); }
    }
    int ring = 0;  // ring buffer of block s
    for (int s = s_lo; s < s_hi; ++s) {
      const int ring_next = ring + 1 == kRing ? 0 : ring + 1;
      // the buffer of block s - 1, which nothing reads any more
      if (s + kRing - 1 < s_hi) fetch(s + kRing - 1, ring == 0 ? kRing - 1 : ring - 1);
      if (active) {
        if (kPrefetch && kRing == 2 && s > s_lo) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) kf[0][ks] = kfrag(ring, 0, ks);
        }
        float m0 = -__builtin_inff(), m1 = -__builtin_inff();
        if constexpr (kPrefetch) {
          // the pooling runs in the last kPool steps of a tile (at least one)
          constexpr int kPool = KS / 2 > 0 ? KS / 2 : 1;
          constexpr int kRowsPerStep = (16 + kPool - 1) / kPool;
#pragma unroll
          for (int kt = 0; kt < kBlock / 32; ++kt) {
            const int cur = kt & 1;
            // the next tile's fragments are read between this tile's MFMAs
            // (the next ring buffer's first tile is read even after the last
            // block: in bounds, and then unused)
            const bool pf = kt + 1 < kBlock / 32 || kRing == 3;
            const int pr = kt + 1 < kBlock / 32 ? ring : ring_next;
            const int pk = kt + 1 < kBlock / 32 ? kt + 1 : 0;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              acc[cur][0] = Mm::mma(kf[cur][ks], qf[0][ks], ks == 0 ? f32x16{} : acc[cur][0]);
              acc[cur][1] = Mm::mma(kf[cur][ks], qf[1][ks], ks == 0 ? f32x16{} : acc[cur][1]);
              if (pf) kf[cur ^ 1][ks] = kfrag(pr, pk, ks);
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMAs
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
              const int h = ks - (KS - kPool);
              if (h >= 0) {
                // tile kt - 1 of this block, or the last tile of the previous one
                float& a0 = kt > 0 ? m0 : pm0;
                float& a1 = kt > 0 ? m1 : pm1;
#pragma unroll
                for (int r = h * kRowsPerStep; r < (h + 1) * kRowsPerStep && r < 16; ++r) {
                  a0 = fmaxf(a0, acc[cur ^ 1][0][r]);
                  a1 = fmaxf(a1, acc[cur ^ 1][1][r]);
                }
                __builtin_amdgcn_sched_group_barrier(0x002, kRowsPerStep, 0);  // the pooling
              }
              // keep the next tile's fragment reads in k-step order: left free,
              // the compiler issued k-step 0's last, so the next tile's first
              // MFMA waited for the most recent read
              __builtin_amdgcn_sched_barrier(0);
            }
            if (kt == 0 && s > s_lo) finish(s - 1, pm0, pm1);
            // keep each tile's MFMAs within its own step: the next tile's
            // MFMAs would otherwise be pulled up behind their fragment reads
            __builtin_amdgcn_sched_barrier(0);
          }
          pm0 = m0;
          pm1 = m1;
        } else {
#pragma unroll
          for (int kt = 0; kt < kBlock / 32; ++kt) {
            f32x16 acc0 = {}, acc1 = {};
            // one fragment at a time: with all of a tile's fp32 fragments
            // held at once beside the query fragments, registers spilled
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              const typename Mm::frag kv = kfrag(ring, kt, ks);
              acc0 = Mm::mma(kv, qf[0][ks], acc0);
              acc1 = Mm::mma(kv, qf[1][ks], acc1);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) { m0 = fmaxf(m0, acc0[r]); m1 = fmaxf(m1, acc1[r]); }
          }
          finish(s, m0, m1);
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // block s + kRing - 1 is in LDS
      if constexpr (kPrefetch && kRing == 3) {
        // every wave has read block s (its buffer is refilled next); the KS
        // reads of block s + 1's first tile, the last LDS operations issued,
        // may stay in flight (LDS operations complete in order)
        asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(KS) : "memory");
      } else {
        __syncthreads();
      }
      ring = ring_next;
    }
    if constexpr (kPrefetch) {
      // the last block's last tile
      if (active) {
#pragma unroll
        for (int r = 0; r < 16; ++r) { pm0 = fmaxf(pm0, acc[1][0][r]); pm1 = fmaxf(pm1, acc[1][1][r]); }
        finish(s_hi - 1, pm0, pm1);
      }
    }
    // a trailing partial group (only at the end of a query block's last chunk)
    const int n_tail = s_hi & 15;
    if (active && col_ok && n_tail != 0) {
      const int g0 = s_hi - n_tail;
      if constexpr (kSbLds) {
        for (int j = 0; j < n_tail; ++j) srow[g0 + j] = s_sb[wave][j][lane];
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = i - (16 - n_tail);
          if (j >= 0) srow[g0 + j] = sbuf[i];
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// Prefill merge: one wave per (query row, group)
// --------------------------------------------------------------------------
__device__ __forceinline__ int find_seq(const int32_t* cu, int batch, int64_t row) {
  int lo = 0, hi = batch;  // invariant: cu[lo] <= row < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

constexpr int kPreRound = 16 * kWave;     // blocks per selection round (16 keys per lane)
constexpr int kPreCand = 16 * 16 + 16;    // candidate bound per round (see below)

// Number of lanes whose predicate holds: one 64-bit population count of the
// ballot.  The empty asm hands the count on as an opaque 32-bit scalar, so
// the comparison that follows stays a scalar 32-bit one (seen as a 64-bit
// value it is compared on the vector unit).
__device__ __forceinline__ int wave_count(bool pred) {
  int c = (int)__builtin_popcountll(__ballot(pred));
  asm volatile("" : "+s"(c));
  return c;
}

// A th such that at least kth of the lanes' xh are >= th: a bitwise binary
// search from the top bit, counted by ballots, for the largest such th (0 when
// fewer than kth lanes hold a nonzero xh).  It stops early once exactly kth
// lanes reach th: those are then the kth largest, and th is below every one
// of them, which is all a threshold needs (it happens as soon as th passes
// the (kth+1)-th largest, typically half-way down the bits).
__device__ __forceinline__ uint32_t wave_kth_hi(uint32_t xh, int kth) {
  uint32_t th = 0;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t t = th | (1u << b);
    const int c = wave_count(xh >= t);
    if (c >= kth) th = t;
    if (c == kth) break;
  }
  return th;
}

// Continues wave_kth_hi on the full 64-bit keys x (one per lane, high words
// xh) when more than kth lanes reach its th: among keys whose high word
// equals th only the low `lo_bits` bits vary (selection keys hold
// 0xffffffff - id with id < 2^lo_bits), so the bits above are set at once
// and the rest are searched.  The result r has at least kth keys >= r and,
// keys being distinct, at most kth.
__device__ __forceinline__ uint64_t wave_kth_lo(uint64_t x, uint32_t th, int kth, int lo_bits) {
  uint32_t tl = lo_bits >= 32 ? 0u : (0xffffffffu << lo_bits);
  for (int b = lo_bits - 1; b >= 0; --b) {
    const uint64_t t = ((uint64_t)th << 32) | (tl | (1u << b));
    if (wave_count(x >= t) >= kth) tl |= 1u << b;
  }
  return ((uint64_t)th << 32) | tl;
}

// One selection round over the blocks r0 .. r0 + 64 NU - 1 of a row (block
// r0 + lane + 64 u in key u of a lane; ids >= local give the empty key 0):
//   1. lane maxima of the round's keys; T = the threshold of their 16th
//      largest (wave_kth_hi on the high words, wave_kth_lo on ties), raised
//      to best[15] if that is larger (taken at once when fewer than 16 lanes
//      reach best[15], as the 16th largest maximum is then below it), and
//      to 1 (keys of real blocks are nonzero).  At least 16 keys of the round
//      and the previous best are >= T, so every member of their top 16 is.
//      Only lanes whose maximum reaches T hold such keys, and there are at
//      most 16 of them: either exactly 16 lanes reach the high word of T, or
//      T is the exact 16th largest maximum (keys are distinct), or fewer than
//      16 lanes hold any key.  So there are at most 16 * 16 + 16 candidates;
//   2. candidates are compacted into LDS lane by lane: each lane counts its
//      keys >= T (and lanes < 16 the previous best[lane]), the lane offsets
//      are an exclusive prefix sum of those counts built from one ballot per
//      count bit, and every key is stored unconditionally (keys below T to a
//      discard slot of the lane's own), so no scalar instruction is spent per
//      key; the candidates are ranked exactly (keys are distinct); ranks
//      0..15 become the new best.
// NU is the round's number of 64-block slices rounded up to a power of two,
// so the loops have no per-slice branches.
template <int NU>
__device__ __forceinline__ void sel_round(const float* __restrict__ sc, int r0, int local, int lo_bits, int lane,
                                          uint64_t* cand, uint64_t* best) {
  float v[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) v[u] = sc[min(r0 + lane + kWave * u, local - 1)];
  uint64_t k[NU];
  uint32_t mxh = 0;  // high word of the lane's largest key
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int c = r0 + lane + kWave * u;
    k[u] = c < local ? sel_key(v[u], c) : 0;
    mxh = max(mxh, (uint32_t)(k[u] >> 32));
  }
  // best[15] is the same for every lane: read it as a scalar
  const uint64_t b15l = best[15];
  const uint64_t b15 = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b15l >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b15l);
  uint64_t T = b15;
  // Later rounds: when fewer than 16 lanes hold a key >= best[15], the 16th
  // largest lane maximum is below it, so T = best[15] without the search
  // (usually so once a full round has been seen).
  bool search = true;
  if (b15 != 0) {
    bool reach = false;
#pragma unroll
    for (int u = 0; u < NU; ++u) reach = reach || k[u] >= b15;
    search = wave_count(reach) >= 16;
  }
  if (search) {
    const uint32_t th = wave_kth_hi(mxh, 16);
    uint64_t t_round = (uint64_t)th << 32;
    if (wave_count(mxh >= th) > 16) {
      // high words tie at th: search the low bits of the exact lane maxima
      uint64_t mx = 0;
#pragma unroll
      for (int u = 0; u < NU; ++u) mx = k[u] > mx ? k[u] : mx;
      t_round = wave_kth_lo(mx, th, 16, lo_bits);
    }
    T = t_round > b15 ? t_round : b15;
  }
  T = T > 1 ? T : 1;
  const uint64_t x = lane < 16 ? best[lane] : 0;
  int cnt = x >= T ? 1 : 0;
#pragma unroll
  for (int u = 0; u < NU; ++u) cnt += k[u] >= T ? 1 : 0;
  // exclusive prefix of cnt (<= NU + 1) over the lanes, one ballot per bit
  constexpr int kBits = NU >= 16 ? 5 : NU >= 8 ? 4 : NU >= 4 ? 3 : 2;
  int off = 0;
#pragma unroll
  for (int j = 0; j < kBits; ++j) {
    const uint64_t m = __ballot((cnt >> j) & 1);
    off += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0)) << j;
  }
  int n = __builtin_amdgcn_readlane(off + cnt, kWave - 1);
  uint64_t* discard = cand + kPreCand + 4 + lane;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const bool take = k[u] >= T;
    *(take ? cand + min(off, kPreCand - 1) : discard) = k[u];  // off < kPreCand (bound above)
    off += take ? 1 : 0;
  }
  *(x >= T ? cand + min(off, kPreCand - 1) : discard) = x;
  n = min(n, kPreCand);
  if (lane < 4) cand[n + lane] = 0;  // pads the rank loop to a multiple of 4
  // exact ranks of the candidates, 64 at a time (usually one pass), 4
  // candidates per LDS read pair
  for (int i0 = 0; i0 < n; i0 += kWave) {
    const bool has = i0 + lane < n;
    const uint64_t mine = has ? cand[i0 + lane] : 0;
    int rank = 0;
    for (int j = 0; j < n; j += 4) {
      const u64x2 c01 = *reinterpret_cast<const u64x2*>(cand + j);
      const u64x2 c23 = *reinterpret_cast<const u64x2*>(cand + j + 2);
      rank += (c01.x > mine ? 1 : 0) + (c01.y > mine ? 1 : 0) + (c23.x > mine ? 1 : 0) + (c23.y > mine ? 1 : 0);
    }
    if (has && rank < 16) best[rank] = mine;
  }
  if (lane < 16 && lane >= n) best[lane] = 0;
}

// One wave per (query row, group).  The scan left the row's block scores in
// `scores`; rounds of 1024 earlier blocks (16 per lane) update the 16 best
// selection keys (per-wave LDS, `best`, see sel_round).  The best topk - 1
// plus the local block are written ascending.
__global__ __launch_bounds__(256) void idx_select_prefill(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch, int64_t rows_bound, int G,
    int topk, int nb_stride, const float* __restrict__ scores, int32_t* __restrict__ block_idx) {
  // candidates, 4 zero keys that pad the rank loop, and one discard slot per lane
  constexpr int kCandSlots = kPreCand + 4 + kWave;
  __shared__ __attribute__((aligned(16))) uint64_t s_cand[4][kCandSlots];
  __shared__ uint64_t s_best[4][16];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = lane_id();
  // (row, group) items fit 31 bits (the launcher refuses more), so the item
  // arithmetic is 32-bit; a power-of-two group count divides by a shift
  const int rg = (int)blockIdx.x * 4 + wave;
  if (rg >= (int)(rows_bound * G)) return;
  const int row = (G & (G - 1)) == 0 ? rg >> __builtin_ctz((unsigned)G) : rg / G;
  if (row >= cu_q[batch]) return;
  const int b = find_seq(cu_q, batch, row);
  const int M = cu_q[b + 1] - cu_q[b], N = cu_k[b + 1] - cu_k[b];
  const int p = N - M + (row - cu_q[b]);
  int32_t* out = block_idx + (int64_t)rg * topk;
  if (p < 0) {
    if (lane < topk) out[lane] = -1;
    return;
  }
  const int local = (int)(p / kBlock);
  const float* sc = scores + rg * (int64_t)nb_stride;
  uint64_t* cand = s_cand[wave];
  uint64_t* best = s_best[wave];
  if (lane < 16) best[lane] = 0;
  const int lo_bits = local > 1 ? 32 - __clz(local - 1) : 0;  // bits of the largest earlier id
  for (int r0 = 0; r0 < local; r0 += kPreRound) {
    const int nu = (local - r0 + kWave - 1) / kWave;  // slices holding blocks (wave-uniform)
    if (nu > 8) sel_round<16>(sc, r0, local, lo_bits, lane, cand, best);
    else if (nu > 4) sel_round<8>(sc, r0, local, lo_bits, lane, cand, best);
    else if (nu > 2) sel_round<4>(sc, r0, local, lo_bits, lane, cand, best);
    else if (nu > 1) sel_round<2>(sc, r0, local, lo_bits, lane, cand, best);
    else sel_round<1>(sc, r0, local, lo_bits, lane, cand, best);
  }
  const int found = min(local, topk - 1);
  const uint64_t mk = lane < 16 ? best[lane] : 0;
  const int mine = (lane < found && mk != 0) ? sel_key_id(mk) : -1;
  write_selection(mine, found, local, topk, out);
}

// --------------------------------------------------------------------------
// Decode: stream the index-key cache once, one fp32 score per (group, block)
// --------------------------------------------------------------------------
// Earlier blocks of sequence b that the decode scan scores (0 unless the
// sequence has exactly one query row and a non-empty context).
__device__ __forceinline__ int dec_blocks(const int32_t* cu_q, const int32_t* cu_k, int b) {
  const int N = cu_k[b + 1] - cu_k[b];
  return (cu_q[b + 1] - cu_q[b] == 1 && N > 0) ? (N - 1) / kBlock : 0;
}

// Earlier-block counts per sequence as exclusive prefix sums, for batches too
// large for the scan's LDS copy (one thread).
__global__ __launch_bounds__(256) void idx_decode_prefix(const int32_t* __restrict__ cu_q,
                                                         const int32_t* __restrict__ cu_k, int batch,
                                                         int32_t* __restrict__ blk_off) {
  if (threadIdx.x != 0) return;
  int acc = 0;
  for (int b = 0; b < batch; ++b) {
    blk_off[b] = acc;
    acc += dec_blocks(cu_q, cu_k, b);
  }
  blk_off[batch] = acc;
}

// Batches below this size keep the block offsets in LDS, computed by every
// scan workgroup itself (no prefix kernel; the per-block sequence search is an
// LDS binary search).
constexpr int kDecLdsSeq = 1024;

// The earlier blocks of all sequences form one flat range; wave w scores
// blocks w, w + W, w + 2W, ... so the waves running at any moment read
// neighbouring 32 KB runs of the cache (copy-like DRAM locality).  Each block
// is scored for all groups at once: 16x16 MFMA, keys x groups.
template <typename T, int DI, bool kLdsOff>
__global__ __launch_bounds__(256) void idx_decode_scores(
    const T* __restrict__ q_idx, const T* __restrict__ k_idx, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, const int32_t* __restrict__ blk_off_g, int batch, int G, int nb_max,
    float* __restrict__ scores) {
  constexpr int DS = DI / 32;  // 32-wide contraction steps of the 16x16 MFMA
  __shared__ int32_t s_off[kLdsOff ? kDecLdsSeq : 1];
  __shared__ int32_t s_part[kLdsOff ? 256 : 1];
  const int32_t* blk_off = blk_off_g;
  if constexpr (kLdsOff) {
    // thread i counts sequences 4i .. 4i+3; inclusive scan of the 256 sums
    int cnt[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 4 * (int)threadIdx.x + i;
      cnt[i] = b < batch ? dec_blocks(cu_q, cu_k, b) : 0;
      sum += cnt[i];
    }
    s_part[threadIdx.x] = sum;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = threadIdx.x >= (unsigned)off ? s_part[threadIdx.x - off] : 0;
      __syncthreads();
      s_part[threadIdx.x] += v;
      __syncthreads();
    }
    int acc = s_part[threadIdx.x] - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 4 * (int)threadIdx.x + i;
      if (b <= batch) s_off[b] = acc;  // batch < kDecLdsSeq: the total lands in s_off[batch]
      acc += cnt[i];
    }
    __syncthreads();
    blk_off = s_off;
  }
  const int lane = lane_id();
  const int nwaves = gridDim.x * 4;
  const int total = blk_off[batch];
  const int gcol = lane & 15;
  // Workgroups are dispatched round-robin over the 8 XCDs (grid a multiple of
  // 8): in every sweep XCD x takes one contiguous range of blocks, so the
  // 128-byte lines of block scores are written whole from one L2.
  const int per_xcd = (gridDim.x >> 3) * 4;
  const int first = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3) * 4 + (int)(threadIdx.x / kWave);
  // A wave visits its blocks in increasing order, so each block's sequence
  // is found by stepping forward from the previous one (one or two offsets
  // read per block instead of a binary search's chain of dependent reads).
  int bseq = 0;
  auto locate = [&](int gb) {
    while (blk_off[bseq + 1] <= gb) ++bseq;  // blk_off[batch] = total > gb ends it
    return bseq;
  };
  if constexpr (sizeof(T) == 1) {
    // fp8: lane l takes the 16-byte pieces 16 (l/16) + 64 u (u < NL) of its
    // key row, so the four lane groups of a row read 64 contiguous bytes per
    // load (pieces 32 bytes apart made both loads touch both halves of the
    // 128-byte row); MFMA (u, half) contracts bytes 8 half .. 8 half + 7 of
    // piece u across the four lane groups, the index query using the same
    // bytes.  A
    // block's loads are half the size of bf16's, so the wave keeps two blocks
    // in flight: the next block is located and its loads issued before the
    // current block's MFMAs (a block in flight per wave left the scan at 5.8
    // against the bf16 scan's 6.0 TB/s).
    constexpr int NL = DI / 64;  // 16-byte pieces per lane
    struct Blk {
      u32x4 a[kBlock / 16][NL];
      u32x4 qv[NL];
      int b, c;
    };
    auto issue = [&](int gb, Blk& B) {
      B.b = locate(gb);
      B.c = gb - blk_off[B.b];
      const uint8_t* qp =
          reinterpret_cast<const uint8_t*>(q_idx) + ((int64_t)cu_q[B.b] * G + gcol) * DI + 16 * (lane >> 4);
#pragma unroll
      for (int u = 0; u < NL; ++u)
        B.qv[u] = gcol < G ? *reinterpret_cast<const u32x4*>(qp + 64 * u) : u32x4{0u, 0u, 0u, 0u};
      const uint8_t* kb = reinterpret_cast<const uint8_t*>(k_idx) +
                          ((int64_t)cu_k[B.b] + (int64_t)B.c * kBlock + (lane & 15)) * DI + 16 * (lane >> 4);
#pragma unroll
      for (int kt = 0; kt < kBlock / 16; ++kt)
#pragma unroll
        for (int u = 0; u < NL; ++u) B.a[kt][u] = *reinterpret_cast<const u32x4*>(kb + (int64_t)kt * 16 * DI + 64 * u);
    };
    auto finish = [&](const Blk& B) {
      float m = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < kBlock / 16; ++kt) {
        f32x4 acc = {};
#pragma unroll
        for (int u = 0; u < NL; ++u) {
          acc = mma16_fp8((long)(((uint64_t)B.a[kt][u].y << 32) | B.a[kt][u].x),
                          (long)(((uint64_t)B.qv[u].y << 32) | B.qv[u].x), acc);
          acc = mma16_fp8((long)(((uint64_t)B.a[kt][u].w << 32) | B.a[kt][u].z),
                          (long)(((uint64_t)B.qv[u].w << 32) | B.qv[u].z), acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, acc[r]);
      }
      m = fmaxf(m, shfl_xor_f(m, 16));
      m = fmaxf(m, shfl_xor_f(m, 32));
      if (lane < G) scores[((int64_t)B.b * G + lane) * nb_max + B.c] = m;
    };
    Blk P0, P1;
    int gb = first;
    if (gb < total) issue(gb, P0);
    while (gb < total) {
      const int g1 = gb + nwaves;
      if (g1 < total) issue(g1, P1);
      __builtin_amdgcn_sched_barrier(0);  // the next block's loads go out before these MFMAs
      finish(P0);
      if (g1 >= total) break;
      const int g2 = g1 + nwaves;
      if (g2 < total) issue(g2, P0);
      __builtin_amdgcn_sched_barrier(0);
      finish(P1);
      gb = g2;
    }
  } else {
  for (int gb = first; gb < total; gb += nwaves) {
    const int b = locate(gb);
    const int c = gb - blk_off[b];
    const int q0 = cu_q[b];
    float m = -__builtin_inff();
    {
      // B operand: columns are the groups (lane%16 < G), slots 32*ds + 8*(lane/16).
      frag8<T> qf[DS];
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        qf[ds] = gcol < G ? load8(q_idx + ((int64_t)q0 * G + gcol) * DI + 32 * ds + 8 * (lane >> 4))
                          : zero8<T>();
      const T* kb = k_idx + ((int64_t)cu_k[b] + (int64_t)c * kBlock + (lane & 15)) * DI + 8 * (lane >> 4);
      frag8<T> a[kBlock / 16][DS];
#pragma unroll
      for (int kt = 0; kt < kBlock / 16; ++kt)
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) a[kt][ds] = load8(kb + (int64_t)kt * 16 * DI + 32 * ds);
      // keep the whole block's loads in flight together before the MFMAs (the
      // scheduler would otherwise interleave them and starve the memory system)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kt = 0; kt < kBlock / 16; ++kt) {
        f32x4 acc = {};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) acc = mma16(a[kt][ds], qf[ds], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, acc[r]);
      }
    }
    m = fmaxf(m, shfl_xor_f(m, 16));
    m = fmaxf(m, shfl_xor_f(m, 32));
    if (lane < G) scores[((int64_t)b * G + lane) * nb_max + c] = m;
  }
  }
}

constexpr int kSelThreads = 1024;                     // 16 waves
constexpr int kSelPer = 8;                            // keys per thread per round
constexpr int kSelRound = kSelThreads * kSelPer;      // 8192 blocks per round
constexpr int kSelCand = 16 * kSelPer + 16;           // candidate bound per round (see below)

// Sort a lane's 16 keys descending (bitonic sorting network).
__device__ __forceinline__ void key_sort16(uint64_t (&kl)[16]) {
#pragma unroll
  for (int k = 2; k <= 16; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int l = i ^ j;
        if (l > i) {
          const uint64_t x = kl[i], y = kl[l];
          const bool sw = ((i & k) == 0) ? (x < y) : (x > y);
          kl[i] = sw ? y : x;
          kl[l] = sw ? x : y;
        }
      }
}

// One workgroup per (sequence, group), over rounds of 8192 earlier blocks.
// A round keeps the 16 best selection keys seen so far (s_best) up to date:
//   1. each thread forms the keys of its 8 blocks; its largest goes to LDS;
//   2. wave 0 finds T, the 16th largest of the 1024 thread maxima (a sort of
//      16 per lane, then butterfly merges), raised to s_best[15] if larger.
//      At least 16 keys of the round's blocks and the previous best are >= T,
//      so every member of their top 16 is >= T; and only the 16 threads
//      whose maximum reaches T hold keys >= T, so there are at most
//      16 * 8 + 16 candidates;
//   3. the candidates are gathered in LDS and ranked by wave 0 (keys are
//      distinct, so ranks are too); ranks 0..15 become the new s_best.
// The key carries the score bits and the id, so no score is fetched back.
__global__ __launch_bounds__(kSelThreads) void idx_decode_select(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int G, int topk, int nb_max,
    const float* __restrict__ scores, int32_t* __restrict__ block_idx) {
  __shared__ uint64_t s_max[kSelThreads];
  __shared__ uint64_t s_cand[kSelCand];
  __shared__ uint64_t s_best[16];
  __shared__ uint64_t s_T;
  __shared__ int s_n;
  const int b = blockIdx.x / G, g = blockIdx.x % G;
  const int q0 = cu_q[b];
  if (cu_q[b + 1] - q0 != 1) return;
  const int N = cu_k[b + 1] - cu_k[b];
  int32_t* out = block_idx + ((int64_t)q0 * G + g) * topk;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  if (N <= 0) {
    if (wave == 0 && lane < topk) out[lane] = -1;
    return;
  }
  const int local = (N - 1) / kBlock;
  const float* sc = scores + ((int64_t)b * G + g) * nb_max;
  if (threadIdx.x < 16) s_best[threadIdx.x] = 0;

  for (int r0 = 0; r0 < local; r0 += kSelRound) {
    uint64_t k8[kSelPer];
    float v[kSelPer];
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
      const int c = r0 + (int)threadIdx.x + u * kSelThreads;
      v[u] = c < local ? sc[c] : 0.0f;
    }
    uint64_t mx = 0;
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
      const int c = r0 + (int)threadIdx.x + u * kSelThreads;
      k8[u] = c < local ? sel_key(v[u], c) : 0;
      mx = k8[u] > mx ? k8[u] : mx;
    }
    s_max[threadIdx.x] = mx;
    if (threadIdx.x == 0) s_n = 0;
    __syncthreads();
    if (wave == 0) {
      uint64_t kl[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) kl[j] = s_max[j * kWave + lane];
      key_sort16(kl);
#pragma unroll
      for (int m = 1; m < kWave; m <<= 1) key_merge_xor(kl, m);
      if (lane == 0) s_T = kl[15] > s_best[15] ? kl[15] : s_best[15];
    }
    __syncthreads();
    const uint64_t T = s_T;
#pragma unroll
    for (int u = 0; u < kSelPer; ++u)
      if (k8[u] != 0 && k8[u] >= T) {
        const int slot = atomicAdd(&s_n, 1);
        if (slot < kSelCand) s_cand[slot] = k8[u];  // always true (bound above)
      }
    if (threadIdx.x < 16) {
      const uint64_t x = s_best[threadIdx.x];
      if (x != 0 && x >= T) {
        const int slot = atomicAdd(&s_n, 1);
        if (slot < kSelCand) s_cand[slot] = x;
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int n = min(s_n, kSelCand);
      uint64_t mine[3];
      int rank[3];
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        mine[i] = lane + kWave * i < n ? s_cand[lane + kWave * i] : 0;
        rank[i] = 0;
      }
      for (int j = 0; j < n; ++j) {
        const uint64_t x = s_cand[j];
#pragma unroll
        for (int i = 0; i < 3; ++i) rank[i] += x > mine[i] ? 1 : 0;
      }
#pragma unroll
      for (int i = 0; i < 3; ++i)
        if (lane + kWave * i < n && rank[i] < 16) s_best[rank[i]] = mine[i];
      if (lane < 16 && lane >= n) s_best[lane] = 0;
    }
    __syncthreads();
  }
  if (wave != 0) return;
  // s_best holds the best min(local, 16) earlier blocks, descending
  const int found = min(local, topk - 1);
  const uint64_t mk = lane < 16 ? s_best[lane] : 0;
  const int mine = (lane < found && mk != 0) ? sel_key_id(mk) : -1;
  write_selection(mine, found, local, topk, out);
}

// --------------------------------------------------------------------------
// Launchers
// --------------------------------------------------------------------------
template <typename T, int DI>
static hipError_t launch_index_prefill(const IndexPlan& pl, const void* q_idx, const void* k_idx,
                                       const int32_t* cu_q, const int32_t* cu_k, int batch, int G,
                                       int topk, int32_t* block_idx, char* ws, hipStream_t st) {
  float* scores = reinterpret_cast<float*>(ws);
  if (pl.scan_wgs > 0) {
    const int64_t grid = pl.scan_pair ? (pl.scan_wgs + 1) / 2 : pl.scan_wgs;
    hipLaunchKernelGGL((idx_scan_prefill<T, DI>), dim3((unsigned)grid), dim3(kScanThreads), 0, st,
                       static_cast<const T*>(q_idx), static_cast<const T*>(k_idx), cu_q, cu_k, G,
                       pl.qw, pl.nsub, pl.max_qblocks, pl.chunk, pl.max_chunks, pl.score_stride, (int)pl.scan_wgs,
                       scores);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t items = pl.rows_bound * G;
  if (items >= INT32_MAX) return hipErrorInvalidValue;  // the selection's item indices are 32-bit
  hipLaunchKernelGGL(idx_select_prefill, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st, cu_q, cu_k,
                     batch, pl.rows_bound, G, topk, pl.score_stride, scores, block_idx);
  return hipGetLastError();
}

template <typename T, int DI>
static hipError_t launch_index_decode(const IndexPlan& pl, const void* q_idx, const void* k_idx,
                                      const int32_t* cu_q, const int32_t* cu_k, int batch, int G,
                                      int topk, int32_t* block_idx, char* ws, hipStream_t st) {
  float* scores = reinterpret_cast<float*>(ws);
  int32_t* blk_off = reinterpret_cast<int32_t*>(ws + pl.score_bytes);
  if (batch < kDecLdsSeq) {
    hipLaunchKernelGGL((idx_decode_scores<T, DI, true>), dim3((unsigned)pl.dec_wgs), dim3(256), 0, st,
                       static_cast<const T*>(q_idx), static_cast<const T*>(k_idx), cu_q, cu_k, nullptr, batch,
                       G, pl.nb_max, scores);
  } else {
    hipLaunchKernelGGL(idx_decode_prefix, dim3(1), dim3(256), 0, st, cu_q, cu_k, batch, blk_off);
    hipLaunchKernelGGL((idx_decode_scores<T, DI, false>), dim3((unsigned)pl.dec_wgs), dim3(256), 0, st,
                       static_cast<const T*>(q_idx), static_cast<const T*>(k_idx), cu_q, cu_k, blk_off, batch,
                       G, pl.nb_max, scores);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(idx_decode_select, dim3((unsigned)(batch * G)), dim3(kSelThreads), 0, st, cu_q, cu_k, G,
                     topk, pl.nb_max, scores, block_idx);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_index_t(const IndexPlan& pl, int DI, const void* q_idx, const void* k_idx,
                                 const int32_t* cu_q, const int32_t* cu_k, int batch, int G, int topk,
                                 int32_t* block_idx, char* w, hipStream_t st) {
  if (pl.decode)
    return DI == 64 ? launch_index_decode<T, 64>(pl, q_idx, k_idx, cu_q, cu_k, batch, G, topk, block_idx, w, st)
                    : launch_index_decode<T, 128>(pl, q_idx, k_idx, cu_q, cu_k, batch, G, topk, block_idx, w, st);
  return DI == 64 ? launch_index_prefill<T, 64>(pl, q_idx, k_idx, cu_q, cu_k, batch, G, topk, block_idx, w, st)
                  : launch_index_prefill<T, 128>(pl, q_idx, k_idx, cu_q, cu_k, batch, G, topk, block_idx, w, st);
}

// dtype: 0 fp32, 1 bf16, 2 fp8 E4M3
hipError_t launch_index_topk(const IndexPlan& pl, int dtype, int DI, const void* q_idx, const void* k_idx,
                             const int32_t* cu_q, const int32_t* cu_k, int batch, int G, int topk,
                             int32_t* block_idx, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  if (dtype == 0) return launch_index_t<float>(pl, DI, q_idx, k_idx, cu_q, cu_k, batch, G, topk, block_idx, w, st);
  if (dtype == 2)
    return launch_index_t<fp8e4m3>(pl, DI, q_idx, k_idx, cu_q, cu_k, batch, G, topk, block_idx, w, st);
  return launch_index_t<bf16>(pl, DI, q_idx, k_idx, cu_q, cu_k, batch, G, topk, block_idx, w, st);
}

}  // namespace msa
