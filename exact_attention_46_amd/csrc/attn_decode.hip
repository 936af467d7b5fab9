// Split-KV ("flash decoding") decode for gfx950.
//
// attn_decode_split. Work item = (sequence b, chunk c, kv-head g): the exact
// attention of the R = Hq / Hkv query heads that share kv-head g (grouped-query
// attention, head h reads kv-head floor(h * Hkv / Hq)) over the keys of chunk
// c, normalised within the chunk, with its LSE. The R heads are the columns of
// one 32-column MFMA tile, so every K/V byte of the chunk is read from HBM once
// for all R heads, and K is never read twice (unlike a two-pass max-then-sum
// decode).
//
// Each wave owns whole items: it walks the items w, w + W, w + 2W, ... of the
// list of valid items (chunk slots past the end of a sequence are not in the
// list; item i is kv-head i % Hkv of the (i / Hkv)-th chunk of the list). The
// list holds the chunks of all sequences in order or, with at most 64
// sequences and at least eight items per wave, their full chunks in order and
// then each sequence's shorter last chunk, longest first (see the kernel).
// Since a wave visits its items in increasing order, it finds the sequences of
// its full chunks with a cursor that only moves forward, reading seq_lens with
// scalar loads, and a short chunk by its rank among the lanes of the wave;
// no workspace is needed.
//
// A wave streams its items' K and V in 32-key tiles straight from HBM into
// its own two-stage LDS ring (buffer loads to LDS, non-temporal, zero-filled
// past L_b), one tile ahead of the tile it computes, across item boundaries
// too; the R query rows of the next item follow the same way into a Q slot of
// the wave. No wave ever waits for another, and a wave waits only for the
// tile it is about to use: vector-memory operations of a wave complete in
// issue order, so "at most N outstanding" with N = the loads issued after the
// tile (plus the partial-result stores issued after it) means the tile has
// landed. Because completion is in order, a store also holds back every load
// issued after it until it is acknowledged; an item's output therefore waits
// in registers and is stored one iteration later, after every load that
// iteration issues, which gives the stores two tiles' time.
//
// Per tile: S^T[32 keys x 32 cols] = K Q^T (8 MFMAs 32x32x16), the running
// max / sum update of the online softmax (the OnlineSoftmaxState of the
// rustytorch "flash_attention_forward.cu" page, with the lazy rescale and the
// two row sums of the forward kernel), O^T += V^T P^T (8 MFMAs, V^T through
// transposing LDS reads). At the end of an item the wave writes O_c (fp32)
// and LSE_c for its R heads.
//
// attn_decode_combine: one wave per (b, h) merges the chunk partials with the
// rescaling combine of the aprender-gpu "flash_decoding/reduce_kernel.rs" page
// (global max of the chunk LSEs, weights exp(LSE_c - M), normalised weighted
// sum), skipping chunks whose LSE is -inf.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace mi355attn {

constexpr int kSplitWaves = 4;        // waves per workgroup (one workgroup per CU)
constexpr int kSplitThreads = 64 * kSplitWaves;
constexpr int kSplitBN = 32;          // keys per tile
constexpr int kSplitMaxGroup = 32;    // query heads per kv-head (the MFMA's columns)
constexpr float kSplitTau = 8.0f;     // lazy-rescale threshold, log2 units

template <int D>
struct SplitLayout {
  static constexpr int kRow = D * 2;
  static constexpr int kChunks = D / 8;
  static constexpr int kRowsPerLoad = 64 / kChunks;           // rows per 1 KB load
  static constexpr int kLoads = kSplitBN / kRowsPerLoad;      // loads per tile and tensor
  static constexpr int kTile = kSplitBN * kRow;               // bytes of a K or V tile
  static constexpr int kStage = 2 * kTile;                    // K then V
  static constexpr int kQ = kSplitMaxGroup * kRow;            // Q rows of one group
  static constexpr int kWave = 2 * kStage + kQ;               // two stages + the Q slot
  static constexpr int kLds = kSplitWaves * kWave;
  // Vector-memory stores at the end of an item, per wave: four 16-byte stores
  // per 32 columns of O_c, and one for LSE_c.
  static constexpr int kItemStores = 4 * (D / 32) + 1;
};
static_assert(SplitLayout<128>::kLds <= 160 * 1024, "LDS budget of a gfx950 workgroup");

// Chunk swizzles as in the forward kernel (conflict-free MFMA operand reads).
template <int D>
__device__ __forceinline__ int dk_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int dv_swz(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

__device__ __forceinline__ int clamp_len(const int* seq_lens, int b, int max_len) {
  const int L = seq_lens[b];
  return L < 0 ? 0 : (L > max_len ? max_len : L);
}

// Number of chunk slots of sequence b that hold keys.
__device__ __forceinline__ int chunks_of(const int* seq_lens, int b, int max_len, int chunk) {
  return (int)(((int64_t)clamp_len(seq_lens, b, max_len) + chunk - 1) / chunk);
}

__device__ __forceinline__ int total_chunks(const int* seq_lens, int B, int max_len, int chunk,
                                            int lane) {
  int t = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    int n = b < B ? chunks_of(seq_lens, b, max_len, chunk) : 0;
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) n += __shfl_xor(n, sh, 64);
    t += n;
  }
  return t;
}

// Paged caches: the chunk of one work item spans at most this many pages (the
// C ABI checks it), whose physical numbers the wave keeps in scalar registers.
constexpr int kMaxItemPages = 16;

// Where the keys of a sequence live. Contiguous: [B, Hkv, max_len, d]. Paged:
// [num_pages, page_size, Hkv, d] with block_table [B, max_pages]; logical key j
// of sequence b is row j % page_size of page block_table[b][j / page_size].
struct PagedKV {
  const int* block_table;
  int page_size, max_pages, num_pages;
};

// Cache policy of the partial results in the fused form: device scope (sc1:
// the store is complete only once it is visible to every XCD's L2, and the load
// reads the value that is visible at device scope, not a line an XCD's L2 may
// still hold) and streamed (nt).
constexpr int kDeviceScopeNt = 18;  // sc1 | nt
constexpr int kDeviceScope = 16;    // sc1

// FINAL: every sequence fits one chunk (chunk >= max_len), so each item's
// normalised output is the final one: it is written rounded to the input dtype
// into o [B, Hq, d] and its LSE into lse [B, Hq], and no combine is needed
// (sequences of length 0 get O = 0, LSE = -inf).
//
// FUSED: the combine runs inside this kernel. Every (sequence, kv-head) pair
// has a counter (caller's workspace, zero between calls). An item of a
// sequence with more than one chunk stores its partial result with
// device-scope stores; once those are known to be complete (counted waits,
// two iterations later) the wave adds one to the pair's counter, and the wave
// whose addition completes the count (the last of the pair's chunks to finish)
// reads every partial of the pair back with device-scope loads, merges them
// with the rescaling combine and writes o and lse, then sets the counter back
// to zero. Nothing waits on another wave. A sequence of one chunk writes its
// final output directly, as in FINAL.
template <int DT, int D, bool PAGED, bool FINAL, bool FUSED>
__global__ void __launch_bounds__(kSplitThreads, 1)
attn_decode_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                         const uint16_t* __restrict__ vc, const int* __restrict__ seq_lens,
                         float* __restrict__ part_o, float* __restrict__ part_lse, int B, int Hq,
                         int Hkv, int max_len, int chunk, int C, float scale, PagedKV pk,
                         uint16_t* __restrict__ o_fin, float* __restrict__ lse_fin,
                         int* __restrict__ counters) {
  static_assert(!(FINAL && FUSED), "one output mode");
  using Lay = SplitLayout<D>;
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  constexpr int ROW = Lay::kRow;
  constexpr int NL = Lay::kLoads;
  constexpr int NS = Lay::kItemStores;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[Lay::kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int half = lane >> 5;
  const int R = Hq / Hkv;
  const int gwave = blockIdx.x * kSplitWaves + wave;
  const int nwaves = gridDim.x * kSplitWaves;

  if constexpr (FINAL || FUSED) {
    // Empty sequences: O = 0, LSE = -inf (no item covers them).
    for (int64_t i = (int64_t)blockIdx.x * kSplitThreads + tid; i < (int64_t)B * Hq;
         i += (int64_t)gridDim.x * kSplitThreads) {
      if (chunks_of(seq_lens, (int)(i / Hq), max_len, chunk) == 0) {
        lse_fin[i] = -INFINITY;
        for (int t = 0; t < D; t += 8)
          *reinterpret_cast<u32x4_t*>(o_fin + i * D + t) = (u32x4_t){0u, 0u, 0u, 0u};
      }
    }
  } else {
    // Chunk slots past the end of a sequence: LSE = -inf (O is not written).
    for (int64_t i = (int64_t)blockIdx.x * kSplitThreads + tid; i < (int64_t)B * Hq * C;
         i += (int64_t)gridDim.x * kSplitThreads) {
      const int cc = (int)(i % C);
      const int bb = (int)(i / ((int64_t)Hq * C));
      if (cc >= chunks_of(seq_lens, bb, max_len, chunk)) part_lse[i] = -INFINITY;
    }
  }

  const int n_items =
      __builtin_amdgcn_readfirstlane(total_chunks(seq_lens, B, max_len, chunk, lane) * Hkv);
  unsigned char* ring = smem + wave * Lay::kWave;
  unsigned char* qslot = ring + 2 * Lay::kStage;

  // DMA offsets of this lane inside a tile (relative to the tile's first row):
  // load i covers rows i*RPL .. +RPL-1; lane p fills physical chunk p % C of
  // row p / C, i.e. loads logical chunk (p % C) ^ swz(row).
  // Paged caches: each load gets a buffer resource of its own, based at its
  // first row inside its page; lane offsets then step by the page row stride.
  const uint32_t pstride = PAGED ? (uint32_t)Hkv * ROW : (uint32_t)ROW;  // bytes between rows
  uint32_t koff[NL], voff[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int row = i * Lay::kRowsPerLoad + lane / Lay::kChunks;
    const int pc = lane % Lay::kChunks;
    const uint32_t rbase = PAGED ? (uint32_t)(lane / Lay::kChunks) * pstride : (uint32_t)row * ROW;
    koff[i] = rbase + (uint32_t)((pc ^ dk_swz<D>(row)) * 16);
    voff[i] = rbase + (uint32_t)((pc ^ dv_swz<D>(row)) * 16);
  }
  // Operand read offsets, as in the forward kernel.
  const int kx = dk_swz<D>(r32);
  const int vkk = (lane & 15) >> 2, va = lane & 3;
  const int vrow0 = 4 * half + vkk;
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * va;
  uint32_t vop[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int col = 32 * db + vcol;
    vop[db] = (uint32_t)(vrow0 * ROW + (((col >> 3) ^ dv_swz<D>(vrow0)) * 16) + (col & 7) * 2);
  }
  // Q^T operand: column r32 is query head g*R + r32. Columns r32 >= R repeat
  // head g*R; their results are never written.
  const uint32_t qop = (uint32_t)((r32 < R ? r32 : 0) * ROW + half * DS * 16);

  // Item order. With at most 64 sequences (one per lane) and at least eight
  // items per wave, the full chunks of all sequences come first, in sequence
  // order, and the last, shorter chunk of each sequence after them, longest
  // first (ties by sequence): the waves then take the short items in the last
  // rounds, which evens out their work (on the 64-sequence decode workload at
  // 512-key chunks the largest per-wave tile count falls from 1.065 to 1.019
  // times the mean, and the split kernel runs 1.7 % faster; with fewer items
  // per wave a whole item is a large part of a wave's work either way, and
  // this order measured 2 % slower at 2048-key chunks). Lane b holds sequence
  // b's length, its full-chunk count and the rank of its short chunk.
  // Otherwise every valid chunk in sequence order.
  const bool by_size = B <= 64 && n_items >= 8 * nwaves;
  int lane_len = 0, lane_full = 0, lane_rank = 0, n_full = 0;
  if (by_size) {
    lane_len = lane < B ? clamp_len(seq_lens, lane, max_len) : 0;
    lane_full = lane_len / chunk;
    const int rem = lane_len - lane_full * chunk;
    for (int j = 0; j < B; ++j) {
      const int rj = __builtin_amdgcn_readlane(rem, j);
      lane_rank += (rj > rem || (rj == rem && j < lane)) && rj > 0 ? 1 : 0;
    }
    if (rem == 0) lane_rank = 64;  // no short chunk
    int f = lane_full;
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) f += __shfl_xor(f, sh, 64);
    n_full = __builtin_amdgcn_readfirstlane(f);
  }

  // Sequence cursor of this wave (wave-uniform): sequence cb, whose first
  // chunk (full chunk, when ordered by size) is number cbase of that list,
  // with cn of them and length cl_len.
  int cb = 0;
  int cl_len = clamp_len(seq_lens, 0, max_len);
  int cn = by_size ? cl_len / chunk : (cl_len + chunk - 1) / chunk;
  int cbase = 0;

  // A work position: item, tile inside the item, and the item's geometry.
  struct Pos {
    int item, tile, b, g, c, L, n_tiles;
    int nc;                   // chunks of sequence b
    int lp0;                  // paged: first logical page of the chunk
    int pg[PAGED ? kMaxItemPages : 1];  // paged: physical pages of the chunk's pages
  };
  auto locate = [&](int item, Pos& p) -> bool {
    p.item = item;
    p.tile = 0;
    if (item >= n_items) return false;
    const int idx = item / Hkv;
    p.g = item - idx * Hkv;
    if (by_size && idx >= n_full) {
      // the short chunk of rank idx - n_full
      const int rk = idx - n_full;
      const uint64_t m = __ballot(lane_rank == rk);
      const int sb = (int)__builtin_ctzll(m);  // m != 0: rk < the number of short chunks
      p.b = sb;
      p.c = __builtin_amdgcn_readlane(lane_full, sb);
      p.L = __builtin_amdgcn_readlane(lane_len, sb);
      p.nc = p.c + 1;
    } else {
      while (idx >= cbase + cn) {  // terminates: idx < the number of chunks in the list
        cbase += cn;
        ++cb;
        cl_len = clamp_len(seq_lens, cb, max_len);
        cn = by_size ? cl_len / chunk : (cl_len + chunk - 1) / chunk;
      }
      p.b = cb;
      p.c = idx - cbase;
      p.L = cl_len;
      p.nc = (cl_len + chunk - 1) / chunk;
    }
    const int lo = p.c * chunk;
    const int hi = min(p.L, lo + chunk);
    p.n_tiles = (hi - lo + kSplitBN - 1) / kSplitBN;
    if constexpr (PAGED) {
      // Scalar loads of the block-table entries of this chunk (indices clamped
      // into the sequence's row of the table; entries past the chunk are
      // never used).
      p.lp0 = lo / pk.page_size;
      const int* row = pk.block_table + (int64_t)p.b * pk.max_pages;
#pragma unroll
      for (int k = 0; k < kMaxItemPages; ++k) p.pg[k] = row[min(p.lp0 + k, pk.max_pages - 1)];
    }
    return true;
  };
  auto issue_kv = [&](const Pos& p, int stage) {
    const int r0 = p.c * chunk + p.tile * kSplitBN;  // < L for every issued tile
    unsigned char* kt = ring + stage * Lay::kStage;
    unsigned char* vt = kt + Lay::kTile;
    if constexpr (PAGED) {
      // Load i covers logical rows r0 + i*RPL .. +RPL-1, all inside one page
      // (RPL divides the page size). Rows at or past L, and pages outside
      // [0, num_pages), read as zeros. The tile's 32 rows span at most two
      // pages (page size >= 16), whose physical numbers are looked up once.
      const int lp_a = r0 / pk.page_size, lp_b = (r0 + kSplitBN - 1) / pk.page_size;
      int phys_a = p.pg[0], phys_b = p.pg[0];
#pragma unroll
      for (int k = 1; k < kMaxItemPages; ++k) {
        phys_a = (lp_a - p.lp0 == k) ? p.pg[k] : phys_a;
        phys_b = (lp_b - p.lp0 == k) ? p.pg[k] : phys_b;
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int ri = r0 + i * Lay::kRowsPerLoad;
        const int lp = ri / pk.page_size;
        const int phys = lp == lp_a ? phys_a : phys_b;
        int rows = min(p.L - ri, Lay::kRowsPerLoad);
        if (phys < 0 || phys >= pk.num_pages) rows = 0;
        if (rows < 0) rows = 0;
        const int64_t base =
            (((int64_t)(rows > 0 ? phys : 0) * pk.page_size + (ri - lp * pk.page_size)) * Hkv +
             p.g) * (int64_t)D;
        const uint32_t bytes = rows > 0 ? (uint32_t)(rows - 1) * pstride + ROW : 0u;
        buf_load16_lds<kNonTemporal>(make_rsrc(kc + base, bytes), kt + i * 1024, koff[i]);
        buf_load16_lds<kNonTemporal>(make_rsrc(vc + base, bytes), vt + i * 1024, voff[i]);
      }
    } else {
      const int64_t head = ((int64_t)p.b * Hkv + p.g) * (int64_t)max_len + r0;
      const uint32_t valid = (uint32_t)(p.L - r0) * ROW;  // rows past L read as zero
      const auto rk = make_rsrc(kc + head * D, valid);
      const auto rv = make_rsrc(vc + head * D, valid);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        buf_load16_lds<kNonTemporal>(rk, kt + i * 1024, koff[i]);
        buf_load16_lds<kNonTemporal>(rv, vt + i * 1024, voff[i]);
      }
    }
  };
  // The R query rows of item p (contiguous in q) into the Q slot, row-major.
  auto issue_q = [&](const Pos& p) {
    const uint32_t bytes = (uint32_t)(R * ROW);
    const auto rq = make_rsrc(q + ((int64_t)p.b * Hq + (int64_t)p.g * R) * D, bytes);
    for (uint32_t off = 0; off < bytes; off += 1024)
      buf_load16_lds(rq, qslot + off, off + (uint32_t)lane * 16);
  };

  const float cl = scale * kLog2e;
  u32x4_t qf[DS];
  float m_used = -INFINITY, l_part = 0.f, lr_part = 0.f;
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16_t){};

  Pos cur, nxt;
  bool have = locate(gwave, cur);
  if (have) {
    issue_kv(cur, 0);
    issue_q(cur);
  }
  int stage = 0;
  bool stores_out = false;  // the previous iteration issued an item's stores
  // An item's output waits in registers for one iteration and is stored after
  // the next tile's loads have landed (see the header).
  bool pend = false;
  f32x16_t opend[DB];
  float* pend_dst = part_o;
  uint16_t* pend_fin = o_fin;
  float* pend_lse = FINAL ? lse_fin : part_lse;
  float pend_lse_val = 0.f;
  // Fused form: whether the pending output is final (a one-chunk sequence),
  // else its pair (sequence, kv-head), the sequence's chunk count and its chunk.
  bool pend_final = FINAL;
  int pend_b = 0, pend_g = 0, pend_nc = 0, pend_c = 0;
  // Byte offsets, relative to the first partial of a pair, of this lane's head
  // (column r32) in part_o and part_lse; a pair's partials span R*C*D*4 bytes
  // (below 2^32, checked by the C ABI).
  const uint32_t lane_po = (uint32_t)(r32 < R ? r32 : 0) * (uint32_t)C * (uint32_t)(D * 4);
  const uint32_t lane_pl = (uint32_t)(r32 < R ? r32 : 0) * (uint32_t)C * 4u;
  auto pair_rsrc_o = [&](int b, int g) {
    return make_rsrc(part_o + ((int64_t)b * Hq + (int64_t)g * R) * C * D,
                     (uint32_t)R * (uint32_t)C * (uint32_t)(D * 4));
  };
  auto pair_rsrc_l = [&](int b, int g) {
    return make_rsrc(part_lse + ((int64_t)b * Hq + (int64_t)g * R) * C,
                     (uint32_t)R * (uint32_t)C * 4u);
  };
  // Exactly NS vector-memory stores (lanes 0 and 32 always take part).
  auto store_pending = [&]() {
    if (r32 < R) {
      if (FINAL || (FUSED && pend_final)) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int d0 = db * 32 + 8 * gq + 4 * half;
            *reinterpret_cast<u32x2_t*>(pend_fin + d0) =
                (u32x2_t){pack2<DT>(opend[db][4 * gq + 0], opend[db][4 * gq + 1]),
                          pack2<DT>(opend[db][4 * gq + 2], opend[db][4 * gq + 3])};
          }
        if (half == 0) __builtin_nontemporal_store(pend_lse_val, pend_lse);
      } else if constexpr (FUSED) {
        const auto ro = pair_rsrc_o(pend_b, pend_g);
        const auto rl = pair_rsrc_l(pend_b, pend_g);
        const uint32_t cb = (uint32_t)pend_c * (uint32_t)(D * 4);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int d0 = db * 32 + 8 * gq + 4 * half;
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4_t, (f32x4_t){opend[db][4 * gq + 0], opend[db][4 * gq + 1],
                                                      opend[db][4 * gq + 2], opend[db][4 * gq + 3]}),
                ro, lane_po + cb + (uint32_t)d0 * 4u, 0, kDeviceScopeNt);
          }
        if (half == 0)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pend_lse_val), rl,
                                                lane_pl + (uint32_t)pend_c * 4u, 0, kDeviceScopeNt);
      } else {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int d0 = db * 32 + 8 * gq + 4 * half;
            // The combine reads the partials once, later: stream them past
            // the caches instead of holding KV lines' space for them.
            __builtin_nontemporal_store((f32x4_t){opend[db][4 * gq + 0], opend[db][4 * gq + 1],
                                                  opend[db][4 * gq + 2], opend[db][4 * gq + 3]},
                                        reinterpret_cast<f32x4_t*>(pend_dst + d0));
          }
        if (half == 0) __builtin_nontemporal_store(pend_lse_val, pend_lse);
      }
    }
    pend = false;
  };

  // Fused form: the merge of pair (b, g) by the wave that completed its count.
  // Lanes take (head r, 4 consecutive d values) pieces, up to two each per
  // round (128 pieces: all of them at R * d <= 512), and read the pair's nc
  // chunk LSEs and partial outputs with device-scope loads, 16 chunks per
  // batch of loads in flight, in one pass with a running maximum (the rescaling
  // combine of the aprender-gpu reduce kernel done online): M = max LSE_c,
  // w_c = exp(LSE_c - M), O = sum w_c O_c / sum w_c (rounded to the dtype),
  // LSE = M + log sum w_c; chunks with LSE = -inf carry no weight. Then the
  // counter is set back to zero for the next call.
  auto merge = [&](int b, int g, int nc) {
    constexpr int CPH = D / 4;  // 16-byte pieces per head
    constexpr int MB = 16;      // chunks per batch of loads
    const auto ro = pair_rsrc_o(b, g);
    const auto rl = pair_rsrc_l(b, g);
    const int64_t row0 = (int64_t)b * Hq + (int64_t)g * R;
    for (int p0 = 0; p0 < R * CPH; p0 += 128) {
      uint32_t vl[2], vo[2];
      int rr[2], c4[2];
      bool on[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int pp = p0 + 64 * u + lane;
        on[u] = pp < R * CPH;
        rr[u] = on[u] ? pp / CPH : 0;
        c4[u] = pp % CPH;
        vl[u] = (uint32_t)rr[u] * (uint32_t)C * 4u;
        vo[u] = (uint32_t)rr[u] * (uint32_t)C * (uint32_t)(D * 4) + (uint32_t)c4[u] * 16u;
      }
      float M[2] = {-INFINITY, -INFINITY}, wsum[2] = {0.f, 0.f};
      f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      for (int c0 = 0; c0 < nc; c0 += MB) {
        float lc[2][MB];
        f32x4_t x[2][MB];
#pragma unroll
        for (int j = 0; j < MB; ++j)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int c = min(c0 + j, nc - 1);
            lc[u][j] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(rl, vl[u], c * 4, kDeviceScope));
            x[u][j] = __builtin_bit_cast(
                f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ro, vo[u], c * (D * 4), kDeviceScope));
          }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float mb = M[u];
#pragma unroll
          for (int j = 0; j < MB; ++j)
            if (c0 + j < nc) mb = fmaxf(mb, lc[u][j]);
          if (mb == -INFINITY) continue;
          const float alpha = M[u] == -INFINITY ? 0.f : fast_exp2((M[u] - mb) * kLog2e);
          acc[u] *= alpha;
          wsum[u] *= alpha;
          M[u] = mb;
#pragma unroll
          for (int j = 0; j < MB; ++j) {
            // the batch's clamped repeats past nc, and empty chunks: no weight
            const float w = (c0 + j >= nc || lc[u][j] == -INFINITY)
                                ? 0.f : fast_exp2((lc[u][j] - mb) * kLog2e);
            acc[u] += w * x[u][j];
            wsum[u] += w;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (!on[u]) continue;
        const float inv = wsum[u] > 0.f ? 1.f / wsum[u] : 0.f;
        *reinterpret_cast<u32x2_t*>(o_fin + (row0 + rr[u]) * D + 4 * c4[u]) =
            (u32x2_t){pack2<DT>(acc[u][0] * inv, acc[u][1] * inv),
                      pack2<DT>(acc[u][2] * inv, acc[u][3] * inv)};
        if (c4[u] == 0)
          lse_fin[row0 + rr[u]] = wsum[u] > 0.f ? M[u] + kLn2 * fast_log2(wsum[u]) : -INFINITY;
      }
    }
    if (lane == 0)
      __hip_atomic_store(counters + (int64_t)b * Hkv + g, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  };
  // Fused form, pipeline of the counter additions. A pair's partials are
  // stored last in iteration s; the wait of iteration s+2 finds them complete
  // (every later wait leaves fewer operations in flight than were issued after
  // them). At the top of iteration s+3, before that iteration's loads, the
  // wave adds one to the pair's counter and waits for the old count (a full
  // wait, but at a point where the only loads in flight are those of the tile
  // it is about to use); the wave that completes the count merges. Slots: the
  // pairs (b * Hkv + g, chunk count) stored one, two and three iterations ago.
  bool s1 = false, s2 = false, s3 = false;
  int s1_p = 0, s1_nc = 0, s2_p = 0, s2_nc = 0, s3_p = 0, s3_nc = 0;
  auto count_top = [&]() {
    if (s3) {
      int old = 0;
      if (lane == 0)
        old = __hip_atomic_fetch_add(counters + s3_p, 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
      if (__builtin_amdgcn_readfirstlane(old) == s3_nc - 1) merge(s3_p / Hkv, s3_p % Hkv, s3_nc);
    }
    s3 = s2, s3_p = s2_p, s3_nc = s2_nc;
    s2 = s1, s2_p = s1_p, s2_nc = s1_nc;
    s1 = false;
  };

  while (have) {
    if constexpr (FUSED) count_top();
    // The next position (next tile of this item, or the first tile of the
    // wave's next item) goes out before this tile's products. Then wait for
    // this tile (and, at an item's first tile, its Q rows): everything but the
    // 2*NL loads just issued and the item-end stores the previous iteration
    // issued last (after all of its loads).
    nxt = cur;
    bool have_next;
    if (cur.tile + 1 < cur.n_tiles) {
      nxt.tile = cur.tile + 1;
      have_next = true;
    } else {
      have_next = locate(cur.item + nwaves, nxt);
    }
    if (have_next) {
      issue_kv(nxt, stage ^ 1);
      if (stores_out)
        wait_vmcnt<2 * NL + NS>();
      else
        wait_vmcnt<2 * NL>();
    } else {
      wait_all_memory();
    }
    if (cur.tile == 0) {
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        qf[ds] = *reinterpret_cast<const u32x4_t*>(qslot + qop + ds * 16);
      // The slot is free once these reads are done; the next item's rows
      // may then be fetched into it.
      wait_lgkmcnt0();
    }
    if (have_next && nxt.tile == 0) issue_q(nxt);
    // The previous item's output goes out last, after every load this
    // iteration issues (the next tile and, when this tile is the last of its
    // item, the next item's Q rows): the wait of the next iteration then only
    // has to leave these NS stores and the 2*NL loads issued after them in
    // flight, and everything older (the tile and the Q rows it will use) is
    // known to have landed.
    stores_out = false;
    if (pend) {
      if (FUSED && !pend_final) s1 = true, s1_p = pend_b * Hkv + pend_g, s1_nc = pend_nc;
      store_pending();
      stores_out = true;
    }

    const unsigned char* kt = ring + stage * Lay::kStage;
    const unsigned char* vt = kt + Lay::kTile;

    // V^T operands of both 16-key steps: vtr[4 * db + 2 * ks + h] holds the
    // rows 8h .. 8h+7 of step ks for column block db (read as one group now,
    // so that their latency hides behind the K reads).
    u32x2_t vtr[4 * DB];
    {
      uint32_t vbase[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) vbase[db] = lds_addr(vt) + vop[db];
      if constexpr (DB == 4)
        lds_read_tr16_x16<8 * ROW>(vtr, vbase);
      else
        lds_read_tr16_x8<8 * ROW>(vtr, vbase);
    }

    f32x16_t s = (f32x16_t){};
    const unsigned char* krow = kt + r32 * ROW;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      u32x4_t a = *reinterpret_cast<const u32x4_t*>(krow + (((half * DS + ds) ^ kx) << 4));
      s = mfma32x32x16<DT>(a, qf[ds], s);
    }
    // Keys at or past the chunk end: element e holds key
    // lo + 32*tile + 4*half + 8*(e/4) + e%4, whose offset is at most 27.
    const int lo = cur.c * chunk;
    const int hi = min(cur.L, lo + chunk);
    const int lim = hi - 1 - (lo + cur.tile * kSplitBN + 4 * half);
    if (lim < 27) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = (8 * (e >> 2) + (e & 3) > lim) ? -INFINITY : s[e];
    }
    float mx = s[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
    mx = max_with_partner32(mx);
    const float m_tile = mx * cl;
    const bool grow = m_tile > m_used + kSplitTau;
    if (__any(grow)) {
      const float m_new = grow ? m_tile : m_used;
      const float alpha = grow ? fast_exp2(m_used - m_new) : 1.f;
      m_used = m_new;
      l_part *= alpha;
      lr_part *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    }
    const float neg_m = (m_used == -INFINITY) ? 0.f : -m_used;
    float p[16];
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = fast_exp2(__builtin_fmaf(s[e], cl, neg_m));
      lsum += p[e];
    }
    l_part += lsum;
    u32x4_t pf[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      pf[j] = (u32x4_t){pack2<DT>(p[8 * j + 0], p[8 * j + 1]), pack2<DT>(p[8 * j + 2], p[8 * j + 3]),
                        pack2<DT>(p[8 * j + 4], p[8 * j + 5]), pack2<DT>(p[8 * j + 6], p[8 * j + 7])};
    float lrsum = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) lrsum = add_pair<DT>(pf[j][w], lrsum);
    lr_part += lrsum;
    // O^T += V^T P^T, two 16-key steps (see the forward kernel for the slots).
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2_t a_lo = vtr[4 * db + 2 * ks];
        const u32x2_t a_hi = vtr[4 * db + 2 * ks + 1];
        const u32x4_t a = {a_lo[0], a_lo[1], a_hi[0], a_hi[1]};
        oacc[db] = mfma32x32x16<DT>(a, pf[ks], oacc[db]);
      }
    }

    if (cur.tile + 1 == cur.n_tiles) {
      // End of the item: O_c = O^T / l_rounded, LSE_c = ln2 * (m + log2 l),
      // held until the next iteration (at most one item's output is pending:
      // it was stored at the top of this iteration).
      const float l_row = sum_with_partner32(l_part);
      const float lr_row = sum_with_partner32(lr_part);
      const int64_t row = (int64_t)cur.b * Hq + (int64_t)cur.g * R + (r32 < R ? r32 : 0);
      const bool empty = !(l_row > 0.f);
      const float inv = empty ? 0.f : 1.f / lr_row;
      if constexpr (FUSED) {
        pend_final = cur.nc == 1;
        pend_b = cur.b, pend_g = cur.g, pend_nc = cur.nc, pend_c = cur.c;
      }
      if (FINAL || (FUSED && cur.nc == 1)) {
        pend_fin = o_fin + row * D;
        pend_lse = lse_fin + row;
      } else if constexpr (!FUSED) {
        pend_dst = part_o + (row * C + cur.c) * D;
        pend_lse = part_lse + row * C + cur.c;
      }
      pend_lse_val = empty ? -INFINITY : kLn2 * (m_used + fast_log2(l_row));
#pragma unroll
      for (int db = 0; db < DB; ++db) opend[db] = oacc[db] * inv;
      pend = true;
      m_used = -INFINITY;
      l_part = 0.f;
      lr_part = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = (f32x16_t){};
    }
    // This wave's reads of the stage must be complete before the loads of the
    // tile after next are issued into it.
    wait_lgkmcnt0();
    __builtin_amdgcn_wave_barrier();
    cur = nxt;
    have = have_next;
    stage ^= 1;
  }
  if constexpr (FUSED) {
    // Drain: once every store is complete, the remaining counter additions
    // (each result waited for before it is used).
    wait_all_memory();  // every partial store complete
    for (int k = 0; k < 3; ++k) count_top();  // the pairs of slots s3, s2 and s1, in turn
    if (pend) {  // the wave's last item (its slot is free now)
      if (!pend_final) s1 = true, s1_p = pend_b * Hkv + pend_g, s1_nc = pend_nc;
      store_pending();
      wait_all_memory();
      for (int k = 0; k < 3; ++k) count_top();
    }
  } else {
    if (pend) store_pending();
  }
}

template <int DT, int D>
__global__ void __launch_bounds__(256)
attn_decode_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                           const int* __restrict__ seq_lens, uint16_t* __restrict__ o,
                           float* __restrict__ lse, int B, int Hq, int C, int chunk) {
  // One wave per (b, h) row. A chunk's partial row is read by LPC lanes, 16
  // bytes (4 d values) each, so one load instruction covers CPI chunks and U of
  // them are in flight at once; the CPI lane groups' sums are added at the end.
  constexpr int LPC = D / 4, CPI = 64 / LPC, U = 8;
  __shared__ float wts[4][64];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;  // (b, h) pair
  if (row >= (int64_t)B * Hq) return;
  const int b = (int)(row / Hq);
  int L = seq_lens[b];
  L = L < 0 ? 0 : L;
  int nc = (int)(((int64_t)L + chunk - 1) / chunk);
  nc = nc > C ? C : nc;
  const float* pl = part_lse + row * C;
  const float* po = part_o + row * C * D;
  const int sub = lane / LPC, dl = (lane % LPC) * 4;

  // Global maximum of the chunk LSEs, lanes over chunks.
  float M = -INFINITY;
  for (int cc = lane; cc < nc; cc += 64) M = fmaxf(M, pl[cc]);
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) M = fmaxf(M, __shfl_xor(M, sh, 64));

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int c0 = 0; c0 < nc; c0 += 64) {
      // Weights of up to 64 chunks, one per lane, shared through LDS.
      const int cc = c0 + lane;
      const float lc = cc < nc ? pl[cc] : -INFINITY;
      const float w = lc == -INFINITY ? 0.f : fast_exp2((lc - M) * kLog2e);
      wts[wv][lane] = w;
      float ws = w;
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) ws += __shfl_xor(ws, sh, 64);
      wsum += ws;
      wait_lgkmcnt0();
      __builtin_amdgcn_wave_barrier();
      const int n = min(64, nc - c0);
      for (int j = 0; j < n; j += CPI * U) {
        f32x4_t x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = j + u * CPI + sub;
          x[u] = c < n ? *reinterpret_cast<const f32x4_t*>(po + (int64_t)(c0 + c) * D + dl)
                       : (f32x4_t){0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = j + u * CPI + sub;
          const float wc = c < n ? wts[wv][c] : 0.f;
          acc += wc * x[u];
        }
      }
      wait_lgkmcnt0();
      __builtin_amdgcn_wave_barrier();
    }
  }
#pragma unroll
  for (int sh = LPC; sh < 64; sh <<= 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], sh, 64);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (sub == 0)
    *reinterpret_cast<u32x2_t*>(o + row * D + dl) =
        (u32x2_t){pack2<DT>(acc[0] * inv, acc[1] * inv), pack2<DT>(acc[2] * inv, acc[3] * inv)};
  if (lane == 0) lse[row] = wsum > 0.f ? M + kLn2 * fast_log2(wsum) : -INFINITY;
}

int64_t split_work_items(int B, int Hkv, int max_len, int chunk) {
  return (int64_t)B * Hkv * (((int64_t)max_len + chunk - 1) / chunk);
}

static int device_cus() {
  // Queried once per device (the value never changes); the cache is atomic so
  // concurrent first calls from several host threads are well defined.
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Chunk length for attn_decode: enough work items (about eight per resident
// wave when every sequence had max_len keys) to balance sequences of unequal
// length, without chunks so short that the partials and the combine dominate
// (measured on gfx950: 2048-key chunks stream the 64-sequence, L ~ U[512, 32768]
// decode at 6.5 TB/s against 6.0 with 512). Returns max_len (one pass, no
// combine) when that many (sequence, kv-head) items already fill the waves.
int decode_chunk_policy(int B, int Hkv, int max_len) {
  const int64_t waves = (int64_t)device_cus() * kSplitWaves;
  if (max_len <= 2048 && (int64_t)B * Hkv >= waves) return max_len;
  int64_t c = (int64_t)B * Hkv * max_len / (8 * waves);
  int chunk = 256;
  while (chunk < 2048 && 2 * chunk <= c) chunk *= 2;
  return max_len <= chunk ? max_len : chunk;
}

template <int DT, int D>
static hipError_t launch_split_t(const SplitArgs& a, hipStream_t stream) {
  const int max_len = a.block_table ? a.max_pages * a.page_size : a.max_len;
  const int C = (int)(((int64_t)max_len + a.chunk - 1) / a.chunk);
  const PagedKV pk{a.block_table, a.page_size, a.max_pages, a.num_pages};
  uint16_t* o_fin = (uint16_t*)a.o_final;
  MI355_LOG("attn_decode_split_kernel<%s,%d,%s%s> grid=%d block=%d B=%d Hq=%d Hkv=%d max_len=%d "
            "chunk=%d chunks=%d page_size=%d scale=%g stream=%p",
            dtype_name(DT), D, a.block_table ? "paged" : "padded",
            a.counters ? ",fused" : a.o_final ? ",one-pass" : "", device_cus(), kSplitThreads,
            a.B, a.Hq, a.Hkv, max_len, a.chunk, C, a.page_size, (double)a.scale, (void*)stream);
#define MI355_SPLIT_LAUNCH(P, FIN, FU)                                                           \
  hipLaunchKernelGGL((attn_decode_split_kernel<DT, D, P, FIN, FU>), dim3((unsigned)device_cus()), \
                     dim3(kSplitThreads), 0, stream, (const uint16_t*)a.q,                       \
                     (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.seq_lens,         \
                     a.part_o, a.part_lse, a.B, a.Hq, a.Hkv, max_len, a.chunk, C, a.scale, pk,   \
                     o_fin, a.lse_final, a.counters)
  if (a.counters) {
    if (a.block_table)
      MI355_SPLIT_LAUNCH(true, false, true);
    else
      MI355_SPLIT_LAUNCH(false, false, true);
  } else if (a.block_table) {
    MI355_SPLIT_LAUNCH(true, false, false);
  } else if (a.o_final) {
    MI355_SPLIT_LAUNCH(false, true, false);
  } else {
    MI355_SPLIT_LAUNCH(false, false, false);
  }
#undef MI355_SPLIT_LAUNCH
  return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_combine_t(const CombineArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.Hq;
  const int64_t blocks = (rows + 3) / 4;
  MI355_LOG("attn_decode_combine_kernel<%s,%d> grid=%lld block=256 B=%d Hq=%d chunks=%d chunk=%d "
            "stream=%p",
            dtype_name(DT), D, (long long)blocks, a.B, a.Hq, a.max_chunks, a.chunk, (void*)stream);
  hipLaunchKernelGGL((attn_decode_combine_kernel<DT, D>), dim3((unsigned)blocks), dim3(256), 0,
                     stream, a.part_o, a.part_lse, a.seq_lens, (uint16_t*)a.o, a.lse, a.B, a.Hq,
                     a.max_chunks, a.chunk);
  return hipGetLastError();
}

hipError_t launch_split(const SplitArgs& a, hipStream_t stream) {
  if (a.dtype == kBF16 && a.d == 128) return launch_split_t<kBF16, 128>(a, stream);
  if (a.dtype == kBF16 && a.d == 64) return launch_split_t<kBF16, 64>(a, stream);
  if (a.dtype == kFP16 && a.d == 128) return launch_split_t<kFP16, 128>(a, stream);
  if (a.dtype == kFP16 && a.d == 64) return launch_split_t<kFP16, 64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.dtype == kBF16 && a.d == 128) return launch_combine_t<kBF16, 128>(a, stream);
  if (a.dtype == kBF16 && a.d == 64) return launch_combine_t<kBF16, 64>(a, stream);
  if (a.dtype == kFP16 && a.d == 128) return launch_combine_t<kFP16, 128>(a, stream);
  if (a.dtype == kFP16 && a.d == 64) return launch_combine_t<kFP16, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace mi355attn
