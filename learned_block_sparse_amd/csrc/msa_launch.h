// msa_launch.h -- host-side work plans and kernel launchers (internal).
//
// A plan is a pure function of the host-visible sizes, so the workspace size
// query and the launch always agree.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

struct IndexPlan {
  bool decode = false;
  int nb_max = 0;            // ceil(max_kv_len / 128)
  int64_t rows_bound = 0;    // batch * max_q_len
  // prefill scan
  int qw = 0;                // queries per workgroup slice (columns = qw * G <= 512)
  int nsub = 0;              // slices per query block
  int max_qblocks = 0;       // query blocks per sequence (upper bound)
  int chunk = 1;             // key blocks per scan workgroup
  int max_chunks = 1;        // key chunks per query block
  int64_t scan_wgs = 0;      // scan items (query block, slice, key chunk, sequence)
  bool scan_pair = false;    // two mirror items per workgroup (when there are enough of them)
  int score_stride = 0;      // floats per (row, group) of prefill block scores
  // decode scan
  int dec_wgs = 0;           // workgroups (4 waves) of the grid-stride decode scan
  size_t score_bytes = 0;    // block scores: prefill [rows, G, nb_max], decode [batch, G, nb_max]
  size_t workspace_bytes = 0;
};

struct AttnPlan {
  int nsplit = 1;            // chunks per selection (query-outer schedule)
  int bps = 16;              // selected blocks per chunk
  int64_t rows_bound = 0;    // query rows (upper bound)
  size_t part_o_bytes = 0;   // [rows, Hq, nsplit, D] fp32
  size_t part_lse_bytes = 0; // [rows, Hq, nsplit] fp32
  // KV-outer schedule (prefill, bf16): per-block edge lists and per-slot partials
  bool kvouter = false;
  int nb_max = 0;
  int64_t kvo_window = 0;    // query rows per window
  int kvo_nbuckets = 0;      // batch * G * nb_max
  size_t kvo_counts_off = 0, kvo_offsets_off = 0, kvo_chunks_off = 0, kvo_cursor_off = 0;
  size_t kvo_edges_off = 0, kvo_part_o_off = 0, kvo_part_lse_off = 0;
  size_t kvo_cbucket_off = 0;  // bucket of each edge chunk
  size_t workspace_bytes = 0;
};

IndexPlan plan_index(int batch, int max_q_len, int max_kv_len, int G);
AttnPlan plan_attn(int batch, int max_q_len, int max_kv_len, int Hq, int G, int D, int topk, int num_splits);

hipError_t launch_index_topk(const IndexPlan& pl, int dtype, int DI, const void* q_idx, const void* k_idx,
                             const int32_t* cu_q, const int32_t* cu_k, int batch, int G, int topk,
                             int32_t* block_idx, void* ws, hipStream_t st);

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_idx;
  const int32_t* cu_q;        // prefill: query row offsets; null for decode (row b = sequence b)
  const int32_t* cu_k;        // prefill: key row offsets; null for decode
  const int64_t* k_offsets;   // decode: first cache row per sequence
  const int32_t* k_lens;      // decode: context length per sequence
  int batch;
  int Hq, Hkv, topk;
  float scale;
  void* out;
  float* lse;
  float* block_lse = nullptr;  // [rows, Hq, topk]: LSE of each selection slot's block, or null
};

// dtype: element type of q and out (0 fp32, 1 bf16); kv_dtype: of K and V
// (equal to dtype, or 2 = E4M3 with bf16 q/out)
hipError_t launch_sparse_attn(const AttnPlan& pl, int dtype, int kv_dtype, const AttnArgs& a, void* ws,
                              hipStream_t st);
hipError_t launch_attn_kvouter(const AttnPlan& pl, bool kv_e4m3, const AttnArgs& a, void* ws, hipStream_t st);
size_t kvo_part_slot_bytes();
int kvo_window_rows();

// Edges per workgroup chunk of the KV-outer schedules (chunk_start counts
// chunks of this many edges).
constexpr int kEdgeChunk = 64;

// Per-(sequence, group, block) lists of the selection entries of query rows
// [row_lo, row_hi) (at most 8192 rows): each entry is ((row - row_lo) << 4 |
// selection slot), the entries of bucket i are edges[offsets[i] ..
// offsets[i + 1]), ascending when `sorted`, else in the order the placing
// atomics handed out.  counts, chunk_start and cursor are scratch of
// batch * G * nb_max (+1) ints each; chunk_bucket (or null) receives the
// bucket of every chunk of kEdgeChunk edges.
hipError_t build_edge_lists(const AttnArgs& x, int nb_max, int64_t row_lo, int64_t row_hi, int32_t* counts,
                            int32_t* offsets, int32_t* chunk_start, int32_t* chunk_bucket, int32_t* cursor,
                            int32_t* edges, bool sorted, hipStream_t st);

// Backward of the main branch (bf16 inputs, fp32 gradients).
struct BwdPlan {
  int nb_max = 0;
  int nbuckets = 0;
  int64_t rows_bound = 0;
  int64_t window = 0;        // query rows per edge-list window
  size_t counts_off = 0, offsets_off = 0, chunks_off = 0, cursor_off = 0, edges_off = 0, delta_off = 0;
  size_t dkv_chunk_off = 0;  // [nbuckets + 1] int32: bwd_dkdv chunk starts
  size_t dkv_part_off = 0;   // [nbuckets + 1] int32: partial-slot starts of multi-chunk buckets
  size_t part_dkv_off = 0;   // [slots][2][128][128] fp32 chunk partials of dK, dV
  size_t part_dq_off = 0;    // [window rows, G, topk, 16, 128] bf16
  size_t workspace_bytes = 0;
};
BwdPlan plan_bwd(int batch, int max_q_len, int max_kv_len, int Hq, int G, int topk);
struct BwdArgs {
  AttnArgs fwd;               // q, k, v, block_idx, cu_q, cu_k, sizes, scale (out/lse unused)
  const void* o;              // forward output [Tq, Hq, D]
  const void* dout;           // gradient of the output [Tq, Hq, D]
  const float* lse;           // forward LSE [Tq, Hq]
  float* dq;                  // [Tq, Hq, D]
  float* dk;                  // [Tk, Hkv, D]
  float* dv;                  // [Tk, Hkv, D]
};
hipError_t launch_sparse_attn_bwd(const BwdPlan& pl, const BwdArgs& a, void* ws, hipStream_t st);

// KL alignment loss of the index branch.
struct KlPlan {
  int nb_max = 0;
  int nbuckets = 0;
  int64_t rows_bound = 0;
  int64_t window = 0;        // query rows per edge-list window
  size_t counts_off = 0, offsets_off = 0, chunks_off = 0, cursor_off = 0, edges_off = 0;
  size_t cbucket_off = 0;                    // bucket of each edge chunk
  size_t s_off = 0, j_off = 0, pos_off = 0;  // per selection slot of a window: score, argmax, edge position
  size_t key_off = 0, ds_off = 0;            // per edge-list position: edge key, dS
  size_t workspace_bytes = 0;
};
KlPlan plan_kl(int batch, int max_q_len, int max_kv_len, int G, int topk);
struct KlLaunch {
  AttnArgs attn;              // block_idx, cu_q, cu_k, batch, Hq, Hkv (= G), topk
  const void* q_idx;          // [Tq, G, DI]
  const void* k_idx;          // [Tk, DI]
  const float* lse;           // [Tq, Hq] from the attention call
  const float* block_lse;     // [Tq, Hq, topk] from the attention call
  float* loss;                // [Tq, G]
  float* dq_idx;              // [Tq, G, DI]
  float* dk_idx;              // [Tk, DI]
};
hipError_t launch_index_kl(const KlPlan& pl, int dtype, int DI, const KlLaunch& x, void* ws, hipStream_t st);

// Index front-end: projection + RMS norm + RoPE (no workspace).
struct FrontendLaunch {
  const void* x;              // [T, d_model]
  const void* w_q;            // [G*DI, d_model]
  const void* w_k;            // [DI, d_model]
  const float* gain_q;        // [DI]
  const float* gain_k;        // [DI]
  const int32_t* cu_q;
  const int32_t* cu_k;
  int batch, G, DI, d_model, rope_dim;
  int64_t total;              // T
  float theta, eps;
  bool in_f32, out_f32;
  void* q_out;                // [T, G, DI]
  void* k_out;                // key rows at cu_k[b] + p
};
hipError_t launch_index_frontend(const FrontendLaunch& f, hipStream_t st);
struct FrontendBwdPlan {
  int64_t tiles = 0;         // 128-token tiles of the recompute kernel
  int64_t tp = 0;            // tiles * 128
  int mrows = 0;             // (G+1) * DI
  int splits = 1;            // token ranges of the weight-gradient GEMM
  int chunks_per_split = 1;  // 64-token chunks per range
  size_t dy_off = 0, gain_off = 0, dw_off = 0;
  size_t workspace_bytes = 0;
};
FrontendBwdPlan plan_index_frontend_bwd(int64_t total, int d_model, int G, int DI);
hipError_t launch_index_frontend_bwd(const FrontendBwdPlan& pl, const FrontendLaunch& f, const float* dq,
                                     const float* dk, float* dw_q, float* dw_k, float* dgain_q, float* dgain_k,
                                     void* ws, hipStream_t st);

}  // namespace msa
