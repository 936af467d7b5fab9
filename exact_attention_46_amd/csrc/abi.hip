// C ABI of the attention library: argument checks, then one launch per call.
// Every check runs before any HIP call, so a rejected call has no side effect.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/mi355attn.h"
#include "launch.hpp"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool head_dim_ok(int d) { return d == 64 || d == 128; }
bool dtype_ok(int dt) { return dt == MI355ATTN_BF16 || dt == MI355ATTN_FP16; }
bool scale_ok(float s) { return isfinite(s) && s > 0.f; }

constexpr int64_t kMaxGrid = 0x7fffffff;
// Longest sequence: keeps the kernels' 32-bit per-head byte offsets and row
// index arithmetic exact (2^23 rows x 256 bytes = 2 GiB per head).
constexpr int kMaxSeq = 1 << 23;

int from_hip(hipError_t e) { return e == hipSuccess ? MI355ATTN_OK : MI355ATTN_ERR_HIP; }

}  // namespace

namespace mi355attn {

bool launch_log_on() {
  // C++ initialises a function-local static once, even under concurrent first calls.
  static const bool on = [] {
    const char* e = getenv("MI355ATTN_LOG");
    return e != nullptr && e[0] != '\0' && strcmp(e, "0") != 0;
  }();
  return on;
}

void launch_log(const char* fmt, ...) {
  char line[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(line, sizeof line, fmt, ap);
  va_end(ap);
  fprintf(stderr, "mi355attn: %s\n", line);
}

}  // namespace mi355attn

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                        int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return MI355ATTN_ERR_NULL_PTR;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return MI355ATTN_ERR_BAD_SHAPE;
  if (Hq % Hkv != 0 || Nq > kMaxSeq || Nk > kMaxSeq) return MI355ATTN_ERR_BAD_SHAPE;
  if (!head_dim_ok(d) || !dtype_ok(dtype)) return MI355ATTN_ERR_UNSUPPORTED;
  if (!scale_ok(scale) || (causal != 0 && causal != 1)) return MI355ATTN_ERR_BAD_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return MI355ATTN_ERR_MISALIGNED;
  if (mi355attn::fwd_grid_blocks(B, Hq, Nq) > kMaxGrid || (int64_t)B * Hq > kMaxGrid)
    return MI355ATTN_ERR_BAD_SHAPE;
  mi355attn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype};
  return from_hip(mi355attn::launch_fwd(a, static_cast<hipStream_t>(stream)));
}

extern "C" int attn_fwd_qkvpacked(const void* qkv, void* o, float* lse, int B, int N, int H,
                                  int d, float scale, int causal, int dtype, void* stream) {
  if (!qkv || !o || !lse) return MI355ATTN_ERR_NULL_PTR;
  if (B <= 0 || N <= 0 || H <= 0 || d <= 0) return MI355ATTN_ERR_BAD_SHAPE;
  if (N > kMaxSeq || (int64_t)3 * H * d * 2 * 256 > 0xffffffffLL) return MI355ATTN_ERR_BAD_SHAPE;
  if (!head_dim_ok(d) || !dtype_ok(dtype)) return MI355ATTN_ERR_UNSUPPORTED;
  if (!scale_ok(scale) || (causal != 0 && causal != 1)) return MI355ATTN_ERR_BAD_ARG;
  if (!aligned(qkv, 16) || !aligned(o, 16) || !aligned(lse, 4)) return MI355ATTN_ERR_MISALIGNED;
  if (mi355attn::fwd_grid_blocks(B, H, N) > kMaxGrid || (int64_t)B * H > kMaxGrid)
    return MI355ATTN_ERR_BAD_SHAPE;
  const uint16_t* base = static_cast<const uint16_t*>(qkv);
  const int64_t hd = (int64_t)H * d;
  mi355attn::FwdArgs a{base, base + hd, base + 2 * hd, o, lse, B, H, H, N, N, d, scale, causal,
                       dtype};
  a.q_stride = a.kv_stride = 3 * H * d;
  a.o_stride = H * d;
  a.uniform_len = N;
  a.total_q = a.total_k = B * N;
  return from_hip(mi355attn::launch_fwd(a, static_cast<hipStream_t>(stream)));
}

extern "C" int attn_fwd_local(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                              int window_left, int window_right, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return MI355ATTN_ERR_NULL_PTR;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return MI355ATTN_ERR_BAD_SHAPE;
  if (Hq % Hkv != 0 || Nq > kMaxSeq || Nk > kMaxSeq) return MI355ATTN_ERR_BAD_SHAPE;
  if (!head_dim_ok(d) || !dtype_ok(dtype)) return MI355ATTN_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return MI355ATTN_ERR_BAD_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return MI355ATTN_ERR_MISALIGNED;
  if (mi355attn::fwd_grid_blocks(B, Hq, Nq) > kMaxGrid || (int64_t)B * Hq > kMaxGrid)
    return MI355ATTN_ERR_BAD_SHAPE;
  // Bounds beyond the key range are no bounds (keeps the kernel's int arithmetic small).
  const int wl = window_left < 0 || window_left >= kMaxSeq * 2 ? -1 : window_left;
  const int wr = window_right < 0 || window_right >= kMaxSeq * 2 ? -1 : window_right;
  mi355attn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, 0, dtype};
  a.local = true;
  a.window_left = wl;
  a.window_right = wr;
  return from_hip(mi355attn::launch_fwd(a, static_cast<hipStream_t>(stream)));
}

namespace {

// Checks shared by attn_bwd and attn_bwd_noalloc (delta excepted).
int bwd_status(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
               int Nk, int d, float scale, int causal, int dtype) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return MI355ATTN_ERR_NULL_PTR;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return MI355ATTN_ERR_BAD_SHAPE;
  if (Hq % Hkv != 0 || Nq > kMaxSeq || Nk > kMaxSeq) return MI355ATTN_ERR_BAD_SHAPE;
  if (!head_dim_ok(d) || !dtype_ok(dtype)) return MI355ATTN_ERR_UNSUPPORTED;
  if (!scale_ok(scale) || (causal != 0 && causal != 1)) return MI355ATTN_ERR_BAD_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4))
    return MI355ATTN_ERR_MISALIGNED;
  if (mi355attn::bwd_grid_blocks(B, Hq, Hkv, Nq, Nk) > kMaxGrid) return MI355ATTN_ERR_BAD_SHAPE;
  return MI355ATTN_OK;
}

}  // namespace

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, float* delta, void* dq, void* dk,
                        void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                        int causal, int dtype, void* stream) {
  if (!delta) return MI355ATTN_ERR_NULL_PTR;
  const int st = bwd_status(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale,
                            causal, dtype);
  if (st != MI355ATTN_OK) return st;
  if (!aligned(delta, 4)) return MI355ATTN_ERR_MISALIGNED;
  mi355attn::BwdArgs a{q, k, v, o, dout, lse, delta, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale,
                       causal, dtype};
  return from_hip(mi355attn::launch_bwd(a, static_cast<hipStream_t>(stream)));
}

namespace {

// Bytes of the stored dS^T for attn_bwd_ds (-1 when the shape is out of range).
int64_t bwd_ds_bytes(int B, int Hq, int Nq, int Nk) {
  if (B <= 0 || Hq <= 0 || Nq <= 0 || Nk <= 0 || Nq > kMaxSeq || Nk > kMaxSeq) return -1;
  const int64_t per_head = mi355attn::bwd_ds_bytes_per_head(Nq, Nk);
  if (per_head > (INT64_MAX / 2) / ((int64_t)B * Hq)) return -1;
  return (int64_t)B * Hq * per_head;
}

}  // namespace

extern "C" long long attn_bwd_ds_workspace(int B, int Hq, int Nq, int Nk) {
  const int64_t n = bwd_ds_bytes(B, Hq, Nq, Nk);
  return n < 0 ? (long long)MI355ATTN_ERR_BAD_SHAPE : (long long)n;
}

extern "C" int attn_bwd_ds(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, float* delta, void* ds,
                           long long ds_bytes, void* dq, void* dk, void* dv, int B, int Hq,
                           int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype,
                           void* stream) {
  if (!delta || !ds) return MI355ATTN_ERR_NULL_PTR;
  const int st = bwd_status(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale,
                            causal, dtype);
  if (st != MI355ATTN_OK) return st;
  if (!aligned(delta, 4) || !aligned(ds, 256)) return MI355ATTN_ERR_MISALIGNED;
  const int64_t need = bwd_ds_bytes(B, Hq, Nq, Nk);
  if (need < 0) return MI355ATTN_ERR_BAD_SHAPE;
  if (ds_bytes < need) return MI355ATTN_ERR_BAD_ARG;
  if (mi355attn::bwd_ds_grid_blocks(B, Hq, Nq) > kMaxGrid) return MI355ATTN_ERR_BAD_SHAPE;
  mi355attn::BwdArgs a{q, k, v, o, dout, lse, delta, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale,
                       causal, dtype};
  a.ds = ds;
  a.ds_row_blocks = (int)mi355attn::bwd_ds_row_blocks(Nq);
  return from_hip(mi355attn::launch_bwd_ds(a, static_cast<hipStream_t>(stream)));
}

extern "C" int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                                int causal, int dtype, void* stream) {
  const int st = bwd_status(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale,
                            causal, dtype);
  if (st != MI355ATTN_OK) return st;
  if ((int64_t)B * Hq * Nq > mi355attn::kBwdScratchFloats) return MI355ATTN_ERR_SCRATCH;
  mi355attn::BwdArgs a{q, k, v, o, dout, lse, nullptr, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale,
                       causal, dtype};
  return from_hip(mi355attn::launch_bwd_noalloc(a, static_cast<hipStream_t>(stream)));
}

extern "C" int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                               const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq,
                               int Hkv, int total_q, int total_k, int max_seqlen_q, int d,
                               float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return MI355ATTN_ERR_NULL_PTR;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || total_q <= 0 || total_k <= 0 || max_seqlen_q <= 0 ||
      d <= 0)
    return MI355ATTN_ERR_BAD_SHAPE;
  if (Hq % Hkv != 0 || max_seqlen_q > kMaxSeq) return MI355ATTN_ERR_BAD_SHAPE;
  if (!head_dim_ok(d) || !dtype_ok(dtype)) return MI355ATTN_ERR_UNSUPPORTED;
  if (!scale_ok(scale) || (causal != 0 && causal != 1)) return MI355ATTN_ERR_BAD_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return MI355ATTN_ERR_MISALIGNED;
  if (mi355attn::fwd_grid_blocks(B, Hq, max_seqlen_q) > kMaxGrid || (int64_t)B * Hq > kMaxGrid)
    return MI355ATTN_ERR_BAD_SHAPE;
  mi355attn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, max_seqlen_q, max_seqlen_q, d, scale, causal,
                       dtype, cu_seqlens_q, cu_seqlens_k, total_q, total_k};
  a.q_stride = Hq * d;
  a.kv_stride = Hkv * d;
  a.o_stride = Hq * d;
  return from_hip(mi355attn::launch_fwd(a, static_cast<hipStream_t>(stream)));
}

extern "C" int attn_decode_split(const void* q, const void* k_cache, const void* v_cache,
                                 const int* seq_lens, float* part_o, float* part_lse, int B,
                                 int Hq, int Hkv, int max_len, int d, int chunk, float scale,
                                 int dtype, void* stream) {
  if (!q || !k_cache || !v_cache || !seq_lens || !part_o || !part_lse)
    return MI355ATTN_ERR_NULL_PTR;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_len <= 0 || d <= 0 || chunk <= 0)
    return MI355ATTN_ERR_BAD_SHAPE;
  if (Hq % Hkv != 0 || max_len > kMaxSeq) return MI355ATTN_ERR_BAD_SHAPE;
  if (!head_dim_ok(d) || !dtype_ok(dtype) || Hq / Hkv > 32) return MI355ATTN_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return MI355ATTN_ERR_BAD_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(part_o, 16) ||
      !aligned(part_lse, 4) || !aligned(seq_lens, 4))
    return MI355ATTN_ERR_MISALIGNED;
  if (mi355attn::split_work_items(B, Hkv, max_len, chunk) > kMaxGrid ||
      (int64_t)B * Hq * (((int64_t)max_len + chunk - 1) / chunk) > ((int64_t)1 << 40))
    return MI355ATTN_ERR_BAD_SHAPE;
  mi355attn::SplitArgs a{q, k_cache, v_cache, seq_lens, part_o, part_lse, B, Hq, Hkv, max_len,
                         d, chunk, scale, dtype};
  return from_hip(mi355attn::launch_split(a, static_cast<hipStream_t>(stream)));
}

extern "C" int attn_decode_split_paged(const void* q, const void* k_pages, const void* v_pages,
                                       const int* block_table, const int* seq_lens,
                                       float* part_o, float* part_lse, int B, int Hq, int Hkv,
                                       int num_pages, int page_size, int max_pages, int d,
                                       int chunk, float scale, int dtype, void* stream) {
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !part_o || !part_lse)
    return MI355ATTN_ERR_NULL_PTR;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || num_pages <= 0 || page_size <= 0 || max_pages <= 0 ||
      d <= 0 || chunk <= 0)
    return MI355ATTN_ERR_BAD_SHAPE;
  if (Hq % Hkv != 0 || (int64_t)max_pages * page_size > kMaxSeq) return MI355ATTN_ERR_BAD_SHAPE;
  if (!head_dim_ok(d) || !dtype_ok(dtype) || Hq / Hkv > 32) return MI355ATTN_ERR_UNSUPPORTED;
  // Every 1 KiB load of a tile (4 rows at d = 128, 8 at d = 64, starting at a
  // multiple of that count when chunk and page_size are multiples of 16) stays
  // inside one page, and the chunk of a work item may span at most 16 pages.
  const int item_pages = chunk % page_size == 0 ? chunk / page_size
                                                : (chunk + page_size - 2) / page_size + 1;
  if (page_size % 16 != 0 || chunk % 16 != 0 || item_pages > 16)
    return MI355ATTN_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return MI355ATTN_ERR_BAD_ARG;
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(part_o, 16) ||
      !aligned(part_lse, 4) || !aligned(seq_lens, 4) || !aligned(block_table, 4))
    return MI355ATTN_ERR_MISALIGNED;
  const int max_len = max_pages * page_size;
  if (mi355attn::split_work_items(B, Hkv, max_len, chunk) > kMaxGrid ||
      (int64_t)B * Hq * (((int64_t)max_len + chunk - 1) / chunk) > ((int64_t)1 << 40) ||
      (int64_t)B * max_pages > kMaxGrid)
    return MI355ATTN_ERR_BAD_SHAPE;
  mi355attn::SplitArgs a{q, k_pages, v_pages, seq_lens, part_o, part_lse, B, Hq, Hkv, max_len,
                         d, chunk, scale, dtype, block_table, page_size, max_pages, num_pages};
  return from_hip(mi355attn::launch_split(a, static_cast<hipStream_t>(stream)));
}

namespace {

// Shared checks of attn_decode and attn_decode_workspace (everything but pointers).
int decode_shape_status(int B, int Hq, int Hkv, int max_len, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_len <= 0 || d <= 0) return MI355ATTN_ERR_BAD_SHAPE;
  if (Hq % Hkv != 0 || max_len > kMaxSeq) return MI355ATTN_ERR_BAD_SHAPE;
  if (!head_dim_ok(d) || Hq / Hkv > 32) return MI355ATTN_ERR_UNSUPPORTED;
  return MI355ATTN_OK;
}

int64_t decode_workspace_floats(int B, int Hq, int Hkv, int max_len, int d, int* chunk_out) {
  const int chunk = mi355attn::decode_chunk_policy(B, Hkv, max_len);
  if (chunk_out) *chunk_out = chunk;
  if (chunk >= max_len) return 0;
  const int64_t C = ((int64_t)max_len + chunk - 1) / chunk;
  return (int64_t)B * Hq * C * (d + 1);
}

}  // namespace

extern "C" long long attn_decode_workspace(int B, int Hq, int Hkv, int max_len, int d) {
  const int st = decode_shape_status(B, Hq, Hkv, max_len, d);
  if (st != MI355ATTN_OK) return st;
  return decode_workspace_floats(B, Hq, Hkv, max_len, d, nullptr);
}

extern "C" int attn_decode(const void* q, const void* k_cache, const void* v_cache,
                           const int* seq_lens, void* o, float* lse, float* workspace,
                           long long workspace_floats, int B, int Hq, int Hkv, int max_len, int d,
                           float scale, int dtype, void* stream) {
  if (!q || !k_cache || !v_cache || !seq_lens || !o || !lse) return MI355ATTN_ERR_NULL_PTR;
  const int st = decode_shape_status(B, Hq, Hkv, max_len, d);
  if (st != MI355ATTN_OK) return st;
  if (!dtype_ok(dtype)) return MI355ATTN_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return MI355ATTN_ERR_BAD_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(seq_lens, 4) || !aligned(workspace, 16))
    return MI355ATTN_ERR_MISALIGNED;
  int chunk = 0;
  const int64_t need = decode_workspace_floats(B, Hq, Hkv, max_len, d, &chunk);
  if (need > 0 && (!workspace || workspace_floats < need)) return MI355ATTN_ERR_BAD_ARG;
  if (mi355attn::split_work_items(B, Hkv, max_len, chunk) > kMaxGrid) return MI355ATTN_ERR_BAD_SHAPE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (need == 0) {  // one chunk per sequence: the split kernel writes the result
    mi355attn::SplitArgs a{q, k_cache, v_cache, seq_lens, nullptr, nullptr, B, Hq, Hkv, max_len,
                           d, chunk, scale, dtype};
    a.o_final = o;
    a.lse_final = lse;
    return from_hip(mi355attn::launch_split(a, s));
  }
  const int C = (int)(((int64_t)max_len + chunk - 1) / chunk);
  float* part_o = workspace;
  float* part_lse = workspace + (int64_t)B * Hq * C * d;
  mi355attn::SplitArgs a{q, k_cache, v_cache, seq_lens, part_o, part_lse, B, Hq, Hkv, max_len,
                         d, chunk, scale, dtype};
  const int rc = from_hip(mi355attn::launch_split(a, s));
  if (rc != MI355ATTN_OK) return rc;
  mi355attn::CombineArgs c{part_o, part_lse, seq_lens, o, lse, B, Hq, C, d, chunk, dtype};
  return from_hip(mi355attn::launch_combine(c, s));
}

namespace {

// Workspace of the fused decode, in 4-byte words: the counters [B, Hkv] (int32),
// then part_lse [B, Hq, C], then part_o [B, Hq, C, d], each region starting on
// a 256-byte boundary. Returns a negative status for a shape the fused decode
// rejects.
int64_t fused_layout(int B, int Hq, int Hkv, int max_len, int d, int chunk, int64_t* lse_off,
                     int64_t* o_off) {
  const int st = decode_shape_status(B, Hq, Hkv, max_len, d);
  if (st != MI355ATTN_OK) return st;
  if (chunk <= 0) return MI355ATTN_ERR_BAD_SHAPE;
  const int64_t C = ((int64_t)max_len + chunk - 1) / chunk;
  // One (sequence, kv-head) pair's partials are addressed with 32-bit byte
  // offsets from its first partial.
  if ((int64_t)(Hq / Hkv) * C * d * 4 >= ((int64_t)1 << 32)) return MI355ATTN_ERR_UNSUPPORTED;
  if (mi355attn::split_work_items(B, Hkv, max_len, chunk) > kMaxGrid ||
      (int64_t)B * Hq * C > ((int64_t)1 << 40))
    return MI355ATTN_ERR_BAD_SHAPE;
  auto up = [](int64_t n) { return (n + 63) / 64 * 64; };
  const int64_t l0 = up((int64_t)B * Hkv);
  const int64_t o0 = l0 + up((int64_t)B * Hq * C);
  if (lse_off) *lse_off = l0;
  if (o_off) *o_off = o0;
  return o0 + (int64_t)B * Hq * C * d;
}

int fused_args_status(const void* q, const void* k, const void* v, const int* seq_lens, void* o,
                      float* lse, float* workspace, long long workspace_floats, int64_t need,
                      float scale, int dtype) {
  if (!q || !k || !v || !seq_lens || !o || !lse || !workspace) return MI355ATTN_ERR_NULL_PTR;
  if (need < 0) return (int)need;
  if (!dtype_ok(dtype)) return MI355ATTN_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return MI355ATTN_ERR_BAD_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(seq_lens, 4) || !aligned(workspace, 256))
    return MI355ATTN_ERR_MISALIGNED;
  if (workspace_floats < need) return MI355ATTN_ERR_BAD_ARG;
  return MI355ATTN_OK;
}

}  // namespace

extern "C" long long attn_decode_fused_workspace(int B, int Hq, int Hkv, int max_len, int d,
                                                 int chunk) {
  return fused_layout(B, Hq, Hkv, max_len, d, chunk, nullptr, nullptr);
}

extern "C" int attn_decode_fused(const void* q, const void* k_cache, const void* v_cache,
                                 const int* seq_lens, void* o, float* lse, float* workspace,
                                 long long workspace_floats, int B, int Hq, int Hkv, int max_len,
                                 int d, int chunk, float scale, int dtype, void* stream) {
  int64_t l0 = 0, o0 = 0;
  const int64_t need = fused_layout(B, Hq, Hkv, max_len, d, chunk, &l0, &o0);
  const int st = fused_args_status(q, k_cache, v_cache, seq_lens, o, lse, workspace,
                                   workspace_floats, need, scale, dtype);
  if (st != MI355ATTN_OK) return st;
  mi355attn::SplitArgs a{q, k_cache, v_cache, seq_lens, workspace + o0, workspace + l0, B, Hq,
                         Hkv, max_len, d, chunk, scale, dtype};
  a.o_final = o;
  a.lse_final = lse;
  a.counters = reinterpret_cast<int*>(workspace);
  return from_hip(mi355attn::launch_split(a, static_cast<hipStream_t>(stream)));
}

extern "C" int attn_decode_fused_paged(const void* q, const void* k_pages, const void* v_pages,
                                       const int* block_table, const int* seq_lens, void* o,
                                       float* lse, float* workspace, long long workspace_floats,
                                       int B, int Hq, int Hkv, int num_pages, int page_size,
                                       int max_pages, int d, int chunk, float scale, int dtype,
                                       void* stream) {
  if (!block_table) return MI355ATTN_ERR_NULL_PTR;
  if (num_pages <= 0 || page_size <= 0 || max_pages <= 0) return MI355ATTN_ERR_BAD_SHAPE;
  if ((int64_t)max_pages * page_size > kMaxSeq || (int64_t)B * max_pages > kMaxGrid)
    return MI355ATTN_ERR_BAD_SHAPE;
  const int max_len = max_pages * page_size;
  int64_t l0 = 0, o0 = 0;
  const int64_t need = fused_layout(B, Hq, Hkv, max_len, d, chunk, &l0, &o0);
  const int st = fused_args_status(q, k_pages, v_pages, seq_lens, o, lse, workspace,
                                   workspace_floats, need, scale, dtype);
  if (st != MI355ATTN_OK) return st;
  const int item_pages = chunk % page_size == 0 ? chunk / page_size
                                                : (chunk + page_size - 2) / page_size + 1;
  if (page_size % 16 != 0 || chunk % 16 != 0 || item_pages > 16)
    return MI355ATTN_ERR_UNSUPPORTED;
  if (!aligned(block_table, 4)) return MI355ATTN_ERR_MISALIGNED;
  mi355attn::SplitArgs a{q, k_pages, v_pages, seq_lens, workspace + o0, workspace + l0, B, Hq,
                         Hkv, max_len, d, chunk, scale, dtype, block_table, page_size,
                         max_pages, num_pages};
  a.o_final = o;
  a.lse_final = lse;
  a.counters = reinterpret_cast<int*>(workspace);
  return from_hip(mi355attn::launch_split(a, static_cast<hipStream_t>(stream)));
}

extern "C" int attn_decode_combine(const float* part_o, const float* part_lse,
                                   const int* seq_lens, void* o, float* lse, int B, int Hq,
                                   int max_chunks, int d, int chunk, int dtype, void* stream) {
  if (!part_o || !part_lse || !seq_lens || !o || !lse) return MI355ATTN_ERR_NULL_PTR;
  if (B <= 0 || Hq <= 0 || max_chunks <= 0 || d <= 0 || chunk <= 0) return MI355ATTN_ERR_BAD_SHAPE;
  if (!head_dim_ok(d) || !dtype_ok(dtype)) return MI355ATTN_ERR_UNSUPPORTED;
  if (!aligned(part_o, 16) || !aligned(part_lse, 4) || !aligned(seq_lens, 4) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return MI355ATTN_ERR_MISALIGNED;
  if (((int64_t)B * Hq + 3) / 4 > kMaxGrid) return MI355ATTN_ERR_BAD_SHAPE;
  mi355attn::CombineArgs a{part_o, part_lse, seq_lens, o, lse, B, Hq, max_chunks, d, chunk, dtype};
  return from_hip(mi355attn::launch_combine(a, static_cast<hipStream_t>(stream)));
}

extern "C" const char* attn_status_str(int status) {
  switch (status) {
    case MI355ATTN_OK: return "ok";
    case MI355ATTN_ERR_NULL_PTR: return "a required pointer is NULL";
    case MI355ATTN_ERR_BAD_SHAPE: return "bad shape: a size <= 0, Hq % Hkv != 0, or grid too large";
    case MI355ATTN_ERR_UNSUPPORTED: return "unsupported: head dim, dtype or Hq/Hkv not supported";
    case MI355ATTN_ERR_MISALIGNED: return "misaligned pointer (16 bytes for tensors, 4 for lse/lens)";
    case MI355ATTN_ERR_BAD_ARG: return "bad argument: scale must be finite and > 0, causal 0 or 1";
    case MI355ATTN_ERR_HIP: return "the HIP runtime reported an error at launch";
    case MI355ATTN_ERR_SCRATCH:
      return "the problem needs more than the library's fixed scratch (attn_bwd_noalloc: "
             "B * Hq * Nq above 4194304)";
    default: return "unknown status";
  }
}
