// Host-side launch descriptors shared by the C ABI and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355attn {

// Launch log. With MI355ATTN_LOG set in the environment to anything but "" or
// "0", every kernel launch prints one line to stderr ("mi355attn: " then the
// kernel, its grid and block and the problem's shape). The variable is read
// once per process, at the first launch; logging never changes what runs.
bool launch_log_on();
void launch_log(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
#define MI355_LOG(...)                                              \
  do {                                                              \
    if (::mi355attn::launch_log_on()) ::mi355attn::launch_log(__VA_ARGS__); \
  } while (0)

inline const char* dtype_name(int dt) { return dt == 0 ? "bf16" : "fp16"; }

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  int dtype;
  // Packed variable-length batch (cu_q != nullptr): q/o [total_q, Hq, d],
  // k/v [total_k, Hkv, d], lse [Hq, total_q]; Nq / Nk are the largest lengths.
  const int* cu_q = nullptr;
  const int* cu_k = nullptr;
  int total_q = 0, total_k = 0;
  // Token-major layouts (cu_q set, or uniform_len > 0): row strides in
  // elements of q, of k / v and of o, row r of head h at base + r*stride + h*d.
  int q_stride = 0, kv_stride = 0, o_stride = 0;
  int uniform_len = 0;
  // Local attention (local = true): key j allowed for row i iff
  // i + off - window_left <= j <= i + off + window_right, a negative bound
  // meaning none (off = Nk - Nq); causal is ignored then.
  bool local = false;
  int window_left = -1, window_right = -1;
};

struct SplitArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int* seq_lens;
  float* part_o;
  float* part_lse;
  int B, Hq, Hkv, max_len, d, chunk;
  float scale;
  int dtype;
  // Paged caches (block_table != nullptr): k_cache / v_cache are
  // [num_pages, page_size, Hkv, d] and max_len is max_pages * page_size.
  const int* block_table = nullptr;
  int page_size = 0, max_pages = 0, num_pages = 0;
  // One pass (chunk >= max_len): final O [B, Hq, d] (dtype) and LSE [B, Hq].
  void* o_final = nullptr;
  float* lse_final = nullptr;
  // Combine fused into the split kernel (counters != nullptr): one int32 per
  // (sequence, kv-head) [B, Hkv], zero on entry and left zero; the partials go
  // to part_o / part_lse and the final result to o_final / lse_final.
  int* counters = nullptr;
};

struct CombineArgs {
  const float* part_o;
  const float* part_lse;
  const int* seq_lens;
  void* o;
  float* lse;
  int B, Hq, max_chunks, d, chunk;
  int dtype;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  int dtype;
  // attn_bwd_ds: the stored dS^T in blocks of 64 keys x 128 rows
  // (ds_row_blocks = bwd_ds_row_blocks(Nq)).
  void* ds = nullptr;
  int ds_row_blocks = 0;
};

// Number of workgroups the forward launch uses (for the grid-size check).
int64_t fwd_grid_blocks(int B, int Hq, int Nq);
// Upper bound on the split kernel's work items (sequence, chunk, kv-head); the
// kernel indexes them with 32-bit integers.
int64_t split_work_items(int B, int Hkv, int max_len, int chunk);
// Chunk length attn_decode uses for this shape (max_len: one pass).
int decode_chunk_policy(int B, int Hkv, int max_len);

// Largest grid of the three backward launches.
int64_t bwd_grid_blocks(int B, int Hq, int Hkv, int Nq, int Nk);

// Floats of the library's fixed backward scratch on each GPU (attn_bwd_noalloc:
// one per query row, so B * Hq * Nq must not exceed it).
constexpr int64_t kBwdScratchFloats = int64_t(1) << 22;

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
// launch_bwd with a.delta replaced by the fixed scratch of the current device.
hipError_t launch_bwd_ds(const BwdArgs& a, hipStream_t stream);
// Row blocks of the stored dS^T and its bytes per (batch, head).
int64_t bwd_ds_row_blocks(int Nq);
int64_t bwd_ds_bytes_per_head(int Nq, int Nk);
int64_t bwd_ds_grid_blocks(int B, int Hq, int Nq);
hipError_t launch_bwd_noalloc(const BwdArgs& a, hipStream_t stream);
hipError_t launch_split(const SplitArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

}  // namespace mi355attn
