// msa_api.hip -- the C ABI declared in include/msa.h: argument checks, work
// plans and dispatch to the HIP kernels.  The library allocates no device
// memory; scratch comes from the caller's workspace.
#include "msa.h"
#include "msa_device.h"
#include "msa_launch.h"

#include <math.h>

#include <mutex>

namespace msa {

static constexpr size_t kAlign = 256;
static size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Scan workgroups aimed at per launch: one per CU of the MI355X (256 CUs;
// a scan workgroup takes a whole CU), so each CU runs one long chunk of key
// blocks and pays the workgroup's start-up (query fragments, first staging)
// once.  Measured on the 128K prefill: 6.68 ms of index calls per step at
// 256, 7.07 at 512, 8.57 at 384 (one and a half rounds), 7.27 at 1024.
static constexpr int64_t kScanTargetWgs = 256;
// Decode scan: waves aimed at per launch.
static constexpr int64_t kDecodeTargetWaves = 8192;
// Attention: work items (waves) aimed at before splitting selections.
static constexpr int64_t kAttnTargetWaves = 8192;
// Attention: (query, group) items from which the KV-outer schedule is used.
static constexpr int64_t kKvoMinItems = 4096;

IndexPlan plan_index(int batch, int max_q_len, int max_kv_len, int G) {
  IndexPlan pl;
  pl.nb_max = (int)ceil_div(max_kv_len, kBlock);
  pl.rows_bound = (int64_t)batch * max_q_len;
  pl.decode = (max_q_len == 1);
  if (pl.decode) {
    // grid-stride waves over all earlier blocks: enough to fill the GPU, no
    // more than there are blocks
    const int64_t total_blocks = (int64_t)batch * pl.nb_max;
    int64_t waves = total_blocks < kDecodeTargetWaves ? total_blocks : kDecodeTargetWaves;
    if (waves < 4) waves = 4;
    pl.dec_wgs = (int)ceil_div(ceil_div(waves, 4), 8) * 8;  // a multiple of the 8 XCDs
    pl.score_bytes = align_up((size_t)batch * G * pl.nb_max * sizeof(float));
    pl.workspace_bytes = pl.score_bytes + align_up((size_t)(batch + 1) * sizeof(int32_t));
    return pl;
  }
  pl.qw = 512 / G < kBlock ? 512 / G : kBlock;
  pl.nsub = (int)ceil_div(kBlock, pl.qw);
  int64_t qb = ceil_div(max_q_len, kBlock) + 1;
  if (qb > pl.nb_max) qb = pl.nb_max;
  pl.max_qblocks = (int)qb;
  const int64_t c_max = pl.nb_max - 1;  // most earlier blocks any query scans
  if (c_max <= 0) {
    pl.chunk = 1;
    pl.max_chunks = 1;
    pl.scan_wgs = 0;
  } else {
    // Work estimate: query blocks c_max-qb+1 .. c_max, each scanning c blocks.
    const int64_t c_first = c_max - qb + 1 > 0 ? c_max - qb + 1 : 0;
    const int64_t work = (int64_t)batch * pl.nsub * (c_first + c_max) * (c_max - c_first + 1) / 2;
    // a multiple of 16 blocks: the scan writes its block scores in aligned groups of 16
    int64_t chunk = ceil_div(ceil_div(work, kScanTargetWgs), 16) * 16;
    pl.chunk = (int)chunk;
    pl.max_chunks = (int)ceil_div(c_max, chunk);
    pl.scan_wgs = (int64_t)batch * pl.max_qblocks * pl.nsub * pl.max_chunks;
    // at least two rounds of workgroups: pair mirror items, one round of equal work
    pl.scan_pair = pl.scan_wgs >= 2 * kScanTargetWgs;
  }
  // block scores [rows, G, score_stride] fp32 (rows padded to 16 bytes),
  // written by the scan, read by the selection
  pl.score_stride = (int)ceil_div(pl.nb_max, 4) * 4;
  pl.score_bytes = pl.scan_wgs > 0 ? align_up((size_t)pl.rows_bound * G * pl.score_stride * sizeof(float)) : 0;
  pl.workspace_bytes = pl.score_bytes;
  return pl;
}

AttnPlan plan_attn(int batch, int max_q_len, int max_kv_len, int Hq, int G, int D, int topk, int num_splits) {
  AttnPlan pl;
  const int64_t rows = (int64_t)batch * max_q_len;
  pl.rows_bound = rows;
  pl.nb_max = (int)ceil_div(max_kv_len, kBlock);
  if (max_q_len > 1 && num_splits == 0 && rows * G >= kKvoMinItems) {
    // KV-outer: each selected K/V block is staged once and shared by every
    // query that picked it; partial outputs per selection slot.
    pl.kvouter = true;
    pl.kvo_window = rows < kvo_window_rows() ? rows : kvo_window_rows();
    pl.kvo_nbuckets = (int)((int64_t)batch * G * pl.nb_max);
    const size_t nbk = (size_t)pl.kvo_nbuckets;
    const size_t slots = (size_t)pl.kvo_window * G * topk;
    size_t off = 0;
    pl.kvo_counts_off = off;  off += align_up(nbk * 4);
    pl.kvo_offsets_off = off; off += align_up((nbk + 1) * 4);
    pl.kvo_chunks_off = off;  off += align_up((nbk + 1) * 4);
    pl.kvo_cursor_off = off;  off += align_up(nbk * 4);
    pl.kvo_edges_off = off;   off += align_up(slots * 4);
    // chunks of <= kEdgeChunk edges: at most slots / kEdgeChunk full ones plus one partial per bucket
    pl.kvo_cbucket_off = off; off += align_up((slots / kEdgeChunk + (slots < nbk ? slots : nbk) + 1) * 4);
    pl.kvo_part_o_off = off;  off += align_up(slots * kvo_part_slot_bytes());
    pl.kvo_part_lse_off = off; off += align_up(slots * 16 * sizeof(float));
    pl.workspace_bytes = off;
    return pl;
  }
  int ns = num_splits;
  if (ns <= 0) {
    const int64_t items = rows * G;
    ns = (int)ceil_div(kAttnTargetWaves, items > 0 ? items : 1);
  }
  if (ns < 1) ns = 1;
  if (ns > topk) ns = topk;
  pl.bps = (int)ceil_div(topk, ns);
  pl.nsplit = (int)ceil_div(topk, pl.bps);
  if (pl.nsplit > 1) {
    pl.part_o_bytes = align_up((size_t)rows * Hq * pl.nsplit * D * sizeof(float));
    pl.part_lse_bytes = align_up((size_t)rows * Hq * pl.nsplit * sizeof(float));
  }
  pl.workspace_bytes = pl.part_o_bytes + pl.part_lse_bytes;
  return pl;
}

}  // namespace msa

using namespace msa;

static thread_local int g_last_hip_error = 0;

// Scratch of msa_index_topk_noalloc: a file-scope device array, so that call
// needs no allocation.  Every GPU the library runs on holds its own copy, at
// its own address, until the process ends.  In host code the array's name is
// not a device address: the per-device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[MSA_NOALLOC_SCRATCH_BYTES];
static constexpr int kMaxDevices = 64;
static void* g_scratch_addr[kMaxDevices];
static std::mutex g_scratch_mu;

static msa_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return MSA_OK;
  g_last_hip_error = (int)e;
  return MSA_ERR_HIP;
}

static bool dtype_ok(msa_dtype_t d) { return d == MSA_F32 || d == MSA_BF16 || d == MSA_FP8_E4M3; }

extern "C" {

const char* msa_status_string(msa_status_t status) {
  switch (status) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
  }
  return "MSA_ERR_UNKNOWN";
}

int msa_last_hip_error(void) { return g_last_hip_error; }

size_t msa_index_topk_workspace_size(int batch, int max_q_len, int max_kv_len, int num_groups,
                                     int block_size, int topk) {
  if (batch <= 0 || max_q_len <= 0 || max_kv_len <= 0 || num_groups <= 0 || block_size != kBlock ||
      topk <= 0)
    return 0;
  return plan_index(batch, max_q_len, max_kv_len, num_groups).workspace_bytes;
}

msa_status_t msa_index_topk(const void* q_idx, const void* k_idx, msa_dtype_t dtype,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                            int max_q_len, int max_kv_len, int num_groups, int index_dim,
                            int block_size, int topk, int32_t* block_idx, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (!q_idx || !k_idx || !cu_seqlens_q || !cu_seqlens_k || !block_idx) return MSA_ERR_INVALID_ARG;
  if (batch <= 0 || max_q_len <= 0 || max_kv_len <= 0 || num_groups <= 0 || index_dim <= 0 ||
      block_size <= 0 || topk <= 0 || !dtype_ok(dtype))
    return MSA_ERR_INVALID_ARG;
  if (block_size != kBlock || (index_dim != 64 && index_dim != 128) || topk > 16 || num_groups > 16)
    return MSA_ERR_UNSUPPORTED;
  const IndexPlan pl = plan_index(batch, max_q_len, max_kv_len, num_groups);
  if (pl.workspace_bytes > 0 && (!workspace || workspace_bytes < pl.workspace_bytes)) return MSA_ERR_WORKSPACE;
  return hip_status(launch_index_topk(pl, (int)dtype, index_dim, q_idx, k_idx, cu_seqlens_q, cu_seqlens_k,
                                      batch, num_groups, topk, block_idx, workspace, stream));
}

msa_status_t msa_index_topk_noalloc(const void* q_idx, const void* k_idx, msa_dtype_t dtype,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                                    int max_q_len, int max_kv_len, int num_groups, int index_dim,
                                    int block_size, int topk, int32_t* block_idx, hipStream_t stream) {
  if (!q_idx || !k_idx || !cu_seqlens_q || !cu_seqlens_k || !block_idx) return MSA_ERR_INVALID_ARG;
  if (batch <= 0 || max_q_len <= 0 || max_kv_len <= 0 || num_groups <= 0 || index_dim <= 0 ||
      block_size <= 0 || topk <= 0 || !dtype_ok(dtype))
    return MSA_ERR_INVALID_ARG;
  if (block_size != kBlock || (index_dim != 64 && index_dim != 128) || topk > 16 || num_groups > 16)
    return MSA_ERR_UNSUPPORTED;
  const IndexPlan pl = plan_index(batch, max_q_len, max_kv_len, num_groups);
  if (pl.workspace_bytes > (size_t)MSA_NOALLOC_SCRATCH_BYTES) return MSA_ERR_WORKSPACE;
  // the scratch of the device the stream runs on, which must be the current one
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (stream != nullptr) {
    int sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return hip_status(e);
    if (sdev != dev) return MSA_ERR_INVALID_ARG;
  }
  if (dev < 0 || dev >= kMaxDevices) return MSA_ERR_UNSUPPORTED;
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_addr[dev] == nullptr) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e);
      if (addr == nullptr) return hip_status(hipErrorInvalidSymbol);
      g_scratch_addr[dev] = addr;
    }
    ws = g_scratch_addr[dev];
  }
  // Nothing in the scratch has to start at zero: the scans write every block
  // score (and the decode block offsets) before the selection reads it.
  return hip_status(launch_index_topk(pl, (int)dtype, index_dim, q_idx, k_idx, cu_seqlens_q, cu_seqlens_k,
                                      batch, num_groups, topk, block_idx, ws, stream));
}

size_t msa_sparse_attn_workspace_size(int batch, int max_q_len, int max_kv_len, int num_heads,
                                      int num_kv_heads, int head_dim, int topk, int num_splits) {
  if (batch <= 0 || max_q_len <= 0 || max_kv_len <= 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || topk <= 0 || num_splits < 0)
    return 0;
  return plan_attn(batch, max_q_len, max_kv_len, num_heads, num_kv_heads, head_dim, topk, num_splits)
      .workspace_bytes;
}

static msa_status_t check_attn(const void* q, const void* k, const void* v, msa_dtype_t dtype,
                               msa_dtype_t kv_dtype, const int32_t* block_idx, const void* out, int batch,
                               int num_heads, int num_kv_heads, int head_dim, int block_size, int topk,
                               int num_splits) {
  if (!q || !k || !v || !block_idx || !out) return MSA_ERR_INVALID_ARG;
  if (batch <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || topk <= 0 ||
      num_splits < 0 || !dtype_ok(dtype) || !dtype_ok(kv_dtype))
    return MSA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return MSA_ERR_INVALID_ARG;
  if (block_size != kBlock || head_dim != kHeadDim || topk > 16 || num_heads / num_kv_heads > 16 ||
      num_kv_heads > 16)
    return MSA_ERR_UNSUPPORTED;
  // element types: q/out fp32 or bf16; K/V of the same type, or E4M3 under bf16 q/out
  const bool same = (dtype == MSA_F32 || dtype == MSA_BF16) && kv_dtype == dtype;
  const bool kv8 = dtype == MSA_BF16 && kv_dtype == MSA_FP8_E4M3;
  if (!same && !kv8) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

static float resolve_scale(float s, int head_dim) {
  return s > 0.f ? s : 1.0f / sqrtf((float)head_dim);
}

msa_status_t msa_sparse_attn_prefill_ex(const void* q, const void* k, const void* v, msa_dtype_t dtype,
                                        msa_dtype_t kv_dtype, const int32_t* block_idx,
                                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                                        int max_q_len, int max_kv_len, int num_heads, int num_kv_heads,
                                        int head_dim, int block_size, int topk, float softmax_scale,
                                        int num_splits, void* out, float* lse, float* block_lse,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  msa_status_t st = check_attn(q, k, v, dtype, kv_dtype, block_idx, out, batch, num_heads, num_kv_heads,
                               head_dim, block_size, topk, num_splits);
  if (st != MSA_OK) return st;
  if (!cu_seqlens_q || !cu_seqlens_k || max_q_len <= 0 || max_kv_len <= 0) return MSA_ERR_INVALID_ARG;
  const AttnPlan pl = plan_attn(batch, max_q_len, max_kv_len, num_heads, num_kv_heads, head_dim, topk, num_splits);
  if (pl.workspace_bytes > 0 && (!workspace || workspace_bytes < pl.workspace_bytes)) return MSA_ERR_WORKSPACE;
  AttnArgs a{q, k, v, block_idx, cu_seqlens_q, cu_seqlens_k, nullptr, nullptr, batch, num_heads, num_kv_heads,
             topk, resolve_scale(softmax_scale, head_dim), out, lse, block_lse};
  return hip_status(launch_sparse_attn(pl, (int)dtype, (int)kv_dtype, a, workspace, stream));
}

msa_status_t msa_sparse_attn_prefill(const void* q, const void* k, const void* v, msa_dtype_t dtype,
                                     const int32_t* block_idx, const int32_t* cu_seqlens_q,
                                     const int32_t* cu_seqlens_k, int batch, int max_q_len,
                                     int max_kv_len, int num_heads, int num_kv_heads, int head_dim,
                                     int block_size, int topk, float softmax_scale, int num_splits,
                                     void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  return msa_sparse_attn_prefill_ex(q, k, v, dtype, dtype, block_idx, cu_seqlens_q, cu_seqlens_k, batch,
                                    max_q_len, max_kv_len, num_heads, num_kv_heads, head_dim, block_size, topk,
                                    softmax_scale, num_splits, out, lse, nullptr, workspace, workspace_bytes,
                                    stream);
}

msa_status_t msa_sparse_attn_decode_ex(const void* q, const void* k_cache, const void* v_cache,
                                       msa_dtype_t dtype, msa_dtype_t kv_dtype, const int32_t* block_idx,
                                       const int64_t* cache_offsets, const int32_t* ctx_lens, int batch,
                                       int max_ctx, int num_heads, int num_kv_heads, int head_dim,
                                       int block_size, int topk, float softmax_scale, int num_splits,
                                       void* out, float* lse, float* block_lse, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  msa_status_t st = check_attn(q, k_cache, v_cache, dtype, kv_dtype, block_idx, out, batch, num_heads,
                               num_kv_heads, head_dim, block_size, topk, num_splits);
  if (st != MSA_OK) return st;
  if (!cache_offsets || !ctx_lens || max_ctx <= 0) return MSA_ERR_INVALID_ARG;
  const AttnPlan pl = plan_attn(batch, 1, max_ctx, num_heads, num_kv_heads, head_dim, topk, num_splits);
  if (pl.workspace_bytes > 0 && (!workspace || workspace_bytes < pl.workspace_bytes)) return MSA_ERR_WORKSPACE;
  AttnArgs a{q, k_cache, v_cache, block_idx, nullptr, nullptr, cache_offsets, ctx_lens, batch, num_heads,
             num_kv_heads, topk, resolve_scale(softmax_scale, head_dim), out, lse, block_lse};
  return hip_status(launch_sparse_attn(pl, (int)dtype, (int)kv_dtype, a, workspace, stream));
}

msa_status_t msa_sparse_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                    msa_dtype_t dtype, const int32_t* block_idx,
                                    const int64_t* cache_offsets, const int32_t* ctx_lens,
                                    int batch, int max_ctx, int num_heads, int num_kv_heads,
                                    int head_dim, int block_size, int topk, float softmax_scale,
                                    int num_splits, void* out, float* lse, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  return msa_sparse_attn_decode_ex(q, k_cache, v_cache, dtype, dtype, block_idx, cache_offsets, ctx_lens, batch,
                                   max_ctx, num_heads, num_kv_heads, head_dim, block_size, topk, softmax_scale,
                                   num_splits, out, lse, nullptr, workspace, workspace_bytes, stream);
}

size_t msa_sparse_attn_backward_workspace_size(int batch, int max_q_len, int max_kv_len, int num_heads,
                                               int num_kv_heads, int head_dim, int topk) {
  if (batch <= 0 || max_q_len <= 0 || max_kv_len <= 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || topk <= 0)
    return 0;
  return plan_bwd(batch, max_q_len, max_kv_len, num_heads, num_kv_heads, topk).workspace_bytes;
}

msa_status_t msa_sparse_attn_backward(const void* q, const void* k, const void* v, const void* out,
                                      const void* dout, const float* lse, msa_dtype_t dtype,
                                      const int32_t* block_idx, const int32_t* cu_seqlens_q,
                                      const int32_t* cu_seqlens_k, int batch, int max_q_len, int max_kv_len,
                                      int num_heads, int num_kv_heads, int head_dim, int block_size, int topk,
                                      float softmax_scale, float* dq, float* dk, float* dv, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  msa_status_t st = check_attn(q, k, v, dtype, dtype, block_idx, out, batch, num_heads, num_kv_heads, head_dim,
                               block_size, topk, 0);
  if (st != MSA_OK) return st;
  if (!dout || !lse || !dq || !dk || !dv || !cu_seqlens_q || !cu_seqlens_k || max_q_len <= 0 ||
      max_kv_len <= 0)
    return MSA_ERR_INVALID_ARG;
  if (dtype != MSA_BF16) return MSA_ERR_UNSUPPORTED;  // the backward kernels take bf16 inputs
  const BwdPlan pl = plan_bwd(batch, max_q_len, max_kv_len, num_heads, num_kv_heads, topk);
  if (!workspace || workspace_bytes < pl.workspace_bytes) return MSA_ERR_WORKSPACE;
  BwdArgs a;
  a.fwd = AttnArgs{q, k, v, block_idx, cu_seqlens_q, cu_seqlens_k, nullptr, nullptr, batch, num_heads,
                   num_kv_heads, topk, resolve_scale(softmax_scale, head_dim), nullptr, nullptr};
  a.o = out;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  return hip_status(launch_sparse_attn_bwd(pl, a, workspace, stream));
}

size_t msa_index_kl_workspace_size(int batch, int max_q_len, int max_kv_len, int num_groups, int topk) {
  if (batch <= 0 || max_q_len <= 0 || max_kv_len <= 0 || num_groups <= 0 || topk <= 0) return 0;
  return plan_kl(batch, max_q_len, max_kv_len, num_groups, topk).workspace_bytes;
}

msa_status_t msa_index_kl_backward(const void* q_idx, const void* k_idx, msa_dtype_t dtype,
                                   const int32_t* block_idx, const float* lse, const float* block_lse,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                                   int max_q_len, int max_kv_len, int num_heads, int num_groups, int index_dim,
                                   int block_size, int topk, float* loss, float* dq_idx, float* dk_idx,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q_idx || !k_idx || !block_idx || !lse || !block_lse || !cu_seqlens_q || !cu_seqlens_k || !loss ||
      !dq_idx || !dk_idx)
    return MSA_ERR_INVALID_ARG;
  if (batch <= 0 || max_q_len <= 0 || max_kv_len <= 0 || num_heads <= 0 || num_groups <= 0 || index_dim <= 0 ||
      block_size <= 0 || topk <= 0 || !dtype_ok(dtype) || num_heads % num_groups != 0)
    return MSA_ERR_INVALID_ARG;
  if (block_size != kBlock || (index_dim != 64 && index_dim != 128) || topk > 16 || num_groups > 16 ||
      num_heads / num_groups > 16 || (dtype != MSA_F32 && dtype != MSA_BF16))
    return MSA_ERR_UNSUPPORTED;
  const KlPlan pl = plan_kl(batch, max_q_len, max_kv_len, num_groups, topk);
  if (!workspace || workspace_bytes < pl.workspace_bytes) return MSA_ERR_WORKSPACE;
  KlLaunch x;
  x.attn = AttnArgs{nullptr, nullptr, nullptr, block_idx, cu_seqlens_q, cu_seqlens_k, nullptr, nullptr, batch,
                    num_heads, num_groups, topk, 0.f, nullptr, nullptr};
  x.q_idx = q_idx;
  x.k_idx = k_idx;
  x.lse = lse;
  x.block_lse = block_lse;
  x.loss = loss;
  x.dq_idx = dq_idx;
  x.dk_idx = dk_idx;
  return hip_status(launch_index_kl(pl, (int)dtype, index_dim, x, workspace, stream));
}

msa_status_t msa_index_frontend(const void* x, const void* w_q, const void* w_k, msa_dtype_t dtype,
                                const float* q_norm_weight, const float* k_norm_weight,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                                int64_t total_q, int d_model, int num_groups, int index_dim, int rope_dim,
                                float rope_theta, float norm_eps, void* q_idx, void* k_idx,
                                msa_dtype_t out_dtype, hipStream_t stream) {
  // token-indexed buffers may be null when there are no tokens
  if (!w_q || !w_k || !q_norm_weight || !k_norm_weight || !cu_seqlens_q || !cu_seqlens_k ||
      (total_q > 0 && (!x || !q_idx || !k_idx)))
    return MSA_ERR_INVALID_ARG;
  if (batch <= 0 || total_q < 0 || d_model <= 0 || num_groups <= 0 || index_dim <= 0 || rope_dim < 0 ||
      rope_dim > index_dim || !(rope_theta > 0.f) || !(norm_eps >= 0.f) || !dtype_ok(dtype) ||
      !dtype_ok(out_dtype))
    return MSA_ERR_INVALID_ARG;
  if ((dtype != MSA_F32 && dtype != MSA_BF16) || (out_dtype != MSA_F32 && out_dtype != MSA_BF16) ||
      (index_dim != 64 && index_dim != 128) || d_model % 64 != 0 || rope_dim % 64 != 0 || num_groups > 65535)
    return MSA_ERR_UNSUPPORTED;
  FrontendLaunch f;
  f.x = x;
  f.w_q = w_q;
  f.w_k = w_k;
  f.gain_q = q_norm_weight;
  f.gain_k = k_norm_weight;
  f.cu_q = cu_seqlens_q;
  f.cu_k = cu_seqlens_k;
  f.batch = batch;
  f.G = num_groups;
  f.DI = index_dim;
  f.d_model = d_model;
  f.rope_dim = rope_dim;
  f.total = total_q;
  f.theta = rope_theta;
  f.eps = norm_eps;
  f.in_f32 = dtype == MSA_F32;
  f.out_f32 = out_dtype == MSA_F32;
  f.q_out = q_idx;
  f.k_out = k_idx;
  return hip_status(launch_index_frontend(f, stream));
}

size_t msa_index_frontend_backward_workspace_size(int64_t total_q, int d_model, int num_groups, int index_dim) {
  if (total_q < 0 || d_model <= 0 || num_groups <= 0 || (index_dim != 64 && index_dim != 128) || d_model % 64 != 0)
    return 0;
  return plan_index_frontend_bwd(total_q, d_model, num_groups, index_dim).workspace_bytes;
}

msa_status_t msa_index_frontend_backward(const void* x, const void* w_q, const void* w_k, msa_dtype_t dtype,
                                         const float* q_norm_weight, const float* k_norm_weight,
                                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                                         int64_t total_q, int d_model, int num_groups, int index_dim, int rope_dim,
                                         float rope_theta, float norm_eps, const float* dq_idx, const float* dk_idx,
                                         float* dw_q, float* dw_k, float* dq_norm_weight, float* dk_norm_weight,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  // token-indexed buffers may be null when there are no tokens
  if (!w_q || !w_k || !q_norm_weight || !k_norm_weight || !cu_seqlens_q || !cu_seqlens_k || !dw_q || !dw_k ||
      !dq_norm_weight || !dk_norm_weight || (total_q > 0 && (!x || !dq_idx || !dk_idx)))
    return MSA_ERR_INVALID_ARG;
  if (batch <= 0 || total_q < 0 || d_model <= 0 || num_groups <= 0 || index_dim <= 0 || rope_dim < 0 ||
      rope_dim > index_dim || !(rope_theta > 0.f) || !(norm_eps >= 0.f) || !dtype_ok(dtype))
    return MSA_ERR_INVALID_ARG;
  if (dtype != MSA_BF16 || (index_dim != 64 && index_dim != 128) || d_model % 64 != 0 || rope_dim % 64 != 0 ||
      num_groups > 65535)
    return MSA_ERR_UNSUPPORTED;
  const FrontendBwdPlan pl = plan_index_frontend_bwd(total_q, d_model, num_groups, index_dim);
  if (pl.workspace_bytes > 0 && (!workspace || workspace_bytes < pl.workspace_bytes)) return MSA_ERR_WORKSPACE;
  FrontendLaunch f;
  f.x = x;
  f.w_q = w_q;
  f.w_k = w_k;
  f.gain_q = q_norm_weight;
  f.gain_k = k_norm_weight;
  f.cu_q = cu_seqlens_q;
  f.cu_k = cu_seqlens_k;
  f.batch = batch;
  f.G = num_groups;
  f.DI = index_dim;
  f.d_model = d_model;
  f.rope_dim = rope_dim;
  f.total = total_q;
  f.theta = rope_theta;
  f.eps = norm_eps;
  f.in_f32 = false;
  f.out_f32 = true;
  f.q_out = nullptr;
  f.k_out = nullptr;
  return hip_status(launch_index_frontend_bwd(pl, f, dq_idx, dk_idx, dw_q, dw_k, dq_norm_weight, dk_norm_weight,
                                              workspace, stream));
}

}  // extern "C"
