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
// list; the list is the prefix sum of ceil(L_b / chunk), computed by every wave
// from seq_lens with ballots, so no workspace is needed). A wave streams its
// items' K and V in 32-key tiles straight from HBM into its own two-stage LDS
// ring (buffer loads to LDS, zero-filled past L_b), one tile ahead of the tile
// it computes, across item boundaries too. No wave ever waits for another.
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
#include "common.hpp"
#include "launch.hpp"

namespace mi355attn {

constexpr int kSplitWaves = 4;        // waves per workgroup (one workgroup per CU)
constexpr int kSplitThreads = 64 * kSplitWaves;
constexpr int kSplitBN = 32;          // keys per tile
constexpr float kSplitTau = 8.0f;     // lazy-rescale threshold, log2 units

template <int D>
struct SplitLayout {
  static constexpr int kRow = D * 2;
  static constexpr int kChunks = D / 8;
  static constexpr int kRowsPerLoad = 64 / kChunks;           // rows per 1 KB load
  static constexpr int kLoads = kSplitBN / kRowsPerLoad;      // loads per tile and tensor
  static constexpr int kTile = kSplitBN * kRow;               // bytes of a K or V tile
  static constexpr int kStage = 2 * kTile;                    // K then V
  static constexpr int kWave = 2 * kStage;                    // two stages per wave
  static constexpr int kLds = kSplitWaves * kWave;
};

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

// Maps compact chunk index `idx` (the chunks of all sequences in order) to
// (b, c), scanning the sequences 64 at a time with one lane per sequence.
// Must be called by the whole wave; the result is the same in every lane.
__device__ __forceinline__ void locate_chunk(const int* seq_lens, int B, int max_len, int chunk,
                                             int idx, int lane, int& b_out, int& c_out) {
  int base = 0;  // chunks of the sequences before this group of 64
  b_out = B;
  c_out = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const int n = b < B ? chunks_of(seq_lens, b, max_len, chunk) : 0;
    int incl = n;  // inclusive prefix sum across the 64 lanes
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const int y = __shfl_up(incl, sh, 64);
      if (lane >= sh) incl += y;
    }
    const int total = __shfl(incl, 63, 64);
    if (idx < base + total) {
      // the sequence is the first lane whose inclusive prefix exceeds idx - base
      const int lb = __popcll(__ballot(incl <= idx - base));
      b_out = b0 + lb;
      c_out = idx - base - __shfl(incl - n, lb, 64);
      return;
    }
    base += total;
  }
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

template <int DT, int D>
__global__ void __launch_bounds__(kSplitThreads, 1)
attn_decode_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                         const uint16_t* __restrict__ vc, const int* __restrict__ seq_lens,
                         float* __restrict__ part_o, float* __restrict__ part_lse, int B, int Hq,
                         int Hkv, int max_len, int chunk, int C, float scale) {
  using Lay = SplitLayout<D>;
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  constexpr int ROW = Lay::kRow;
  constexpr int NL = Lay::kLoads;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[Lay::kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int half = lane >> 5;
  const int R = Hq / Hkv;
  const int gwave = blockIdx.x * kSplitWaves + wave;
  const int nwaves = gridDim.x * kSplitWaves;

  // Chunk slots past the end of a sequence: LSE = -inf (O is not written).
  for (int64_t i = (int64_t)blockIdx.x * kSplitThreads + tid; i < (int64_t)B * Hq * C;
       i += (int64_t)gridDim.x * kSplitThreads) {
    const int cc = (int)(i % C);
    const int bb = (int)(i / ((int64_t)Hq * C));
    if (cc >= chunks_of(seq_lens, bb, max_len, chunk)) part_lse[i] = -INFINITY;
  }

  const int n_items = total_chunks(seq_lens, B, max_len, chunk, lane) * Hkv;
  unsigned char* ring = smem + wave * Lay::kWave;

  // DMA offsets of this lane inside a tile (relative to the tile's first row):
  // load i covers rows i*RPL .. +RPL-1; lane p fills physical chunk p % C of
  // row p / C, i.e. loads logical chunk (p % C) ^ swz(row).
  uint32_t koff[NL], voff[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int row = i * Lay::kRowsPerLoad + lane / Lay::kChunks;
    const int pc = lane % Lay::kChunks;
    koff[i] = (uint32_t)row * ROW + (uint32_t)((pc ^ dk_swz<D>(row)) * 16);
    voff[i] = (uint32_t)row * ROW + (uint32_t)((pc ^ dv_swz<D>(row)) * 16);
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

  // A work position: item, tile inside the item, and the item's geometry.
  struct Pos {
    int item, tile, b, g, c, L, n_tiles;
  };
  auto locate = [&](int item, Pos& p) -> bool {
    p.item = item;
    p.tile = 0;
    if (item >= n_items) return false;
    p.g = item % Hkv;
    locate_chunk(seq_lens, B, max_len, chunk, item / Hkv, lane, p.b, p.c);
    p.L = clamp_len(seq_lens, p.b, max_len);
    const int lo = p.c * chunk;
    const int hi = min(p.L, lo + chunk);
    p.n_tiles = (hi - lo + kSplitBN - 1) / kSplitBN;
    return true;
  };
  auto issue = [&](const Pos& p, int stage) {
    const int r0 = p.c * chunk + p.tile * kSplitBN;  // < L for every issued tile
    const int64_t head = ((int64_t)p.b * Hkv + p.g) * (int64_t)max_len + r0;
    const uint32_t valid = (uint32_t)(p.L - r0) * ROW;  // rows past L read as zero
    const auto rk = make_rsrc(kc + head * D, valid);
    const auto rv = make_rsrc(vc + head * D, valid);
    unsigned char* kt = ring + stage * Lay::kStage;
    unsigned char* vt = kt + Lay::kTile;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      buf_load16_lds(rk, kt + i * 1024, koff[i]);
      buf_load16_lds(rv, vt + i * 1024, voff[i]);
    }
  };

  const float cl = scale * kLog2e;
  u32x4_t qf[DS];
  float m_used = -INFINITY, l_part = 0.f, lr_part = 0.f;
  f32x16_t oacc[DB];
  auto begin_item = [&](const Pos& p) {
    // Q^T operand: column r32 is query head g*R + r32 (zero for r32 >= R).
    const int rr = r32 < R ? r32 : 0;
    const uint16_t* qrow = q + ((int64_t)p.b * Hq + (int64_t)p.g * R + rr) * D;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const u32x4_t x = reinterpret_cast<const u32x4_t*>(qrow)[half * DS + ds];
      qf[ds] = r32 < R ? x : (u32x4_t){0u, 0u, 0u, 0u};
    }
    m_used = -INFINITY;
    l_part = 0.f;
    lr_part = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = (f32x16_t){};
  };

  Pos cur, nxt;
  bool have = locate(gwave, cur);
  if (have) {
    issue(cur, 0);
    begin_item(cur);
  }
  int stage = 0;

  while (have) {
    // The next position (next tile of this item, or the first tile of the
    // wave's next item) goes out before this tile's products; then wait for
    // the current tile only (the 2*NL newest loads may stay in flight).
    nxt = cur;
    bool have_next;
    if (cur.tile + 1 < cur.n_tiles) {
      nxt.tile = cur.tile + 1;
      have_next = true;
    } else {
      have_next = locate(cur.item + nwaves, nxt);
    }
    if (have_next) {
      issue(nxt, stage ^ 1);
      wait_vmcnt<2 * NL>();
    } else {
      wait_all_memory();
    }

    const unsigned char* kt = ring + stage * Lay::kStage;
    const unsigned char* vt = kt + Lay::kTile;

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
        const unsigned char* p0 = vt + vop[db] + ks * 16 * ROW;
        const u32x2_t a_lo = lds_read_tr16(p0);
        const u32x2_t a_hi = lds_read_tr16(p0 + 8 * ROW);
        const u32x4_t a = {a_lo[0], a_lo[1], a_hi[0], a_hi[1]};
        oacc[db] = mfma32x32x16<DT>(a, pf[ks], oacc[db]);
      }
    }

    if (cur.tile + 1 == cur.n_tiles) {
      // End of the item: O_c = O^T / l_rounded, LSE_c = ln2 * (m + log2 l).
      const float l_row = sum_with_partner32(l_part);
      const float lr_row = sum_with_partner32(lr_part);
      if (r32 < R) {
        const int64_t row = (int64_t)cur.b * Hq + (int64_t)cur.g * R + r32;
        const bool empty = !(l_row > 0.f);
        const float inv = empty ? 0.f : 1.f / lr_row;
        float* dst = part_o + (row * C + cur.c) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int d0 = db * 32 + 8 * gq + 4 * half;
            *reinterpret_cast<f32x4_t*>(dst + d0) =
                (f32x4_t){oacc[db][4 * gq + 0] * inv, oacc[db][4 * gq + 1] * inv,
                          oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv};
          }
        if (half == 0)
          part_lse[row * C + cur.c] = empty ? -INFINITY : kLn2 * (m_used + fast_log2(l_row));
      }
      if (have_next) begin_item(nxt);
    }
    // This wave's reads of the stage must be complete before the loads of the
    // tile after next are issued into it.
    wait_lgkmcnt0();
    __builtin_amdgcn_wave_barrier();
    cur = nxt;
    have = have_next;
    stage ^= 1;
  }
}

template <int DT, int D>
__global__ void __launch_bounds__(256)
attn_decode_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                           const int* __restrict__ seq_lens, uint16_t* __restrict__ o,
                           float* __restrict__ lse, int B, int Hq, int C, int chunk) {
  constexpr int PER = D / 64;  // d values per lane
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

  // Global maximum of the chunk LSEs, lanes over chunks.
  float M = -INFINITY;
  for (int cc = lane; cc < nc; cc += 64) M = fmaxf(M, pl[cc]);
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) M = fmaxf(M, __shfl_xor(M, sh, 64));

  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
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
      int j = 0;
      for (; j + 4 <= n; j += 4) {  // four independent loads in flight
        float x[4][PER];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < PER; ++i) x[u][i] = po[(int64_t)(c0 + j + u) * D + lane * PER + i];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < PER; ++i) acc[i] += wts[wv][j + u] * x[u][i];
      }
      for (; j < n; ++j)
#pragma unroll
        for (int i = 0; i < PER; ++i)
          acc[i] += wts[wv][j] * po[(int64_t)(c0 + j) * D + lane * PER + i];
      wait_lgkmcnt0();
      __builtin_amdgcn_wave_barrier();
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  uint16_t* orow = o + row * D + lane * PER;
  if constexpr (PER == 2) {
    *reinterpret_cast<uint32_t*>(orow) = pack2<DT>(acc[0] * inv, acc[1] * inv);
  } else {
    const uint32_t w = pack2<DT>(acc[0] * inv, 0.f);
    *orow = (uint16_t)(w & 0xffffu);
  }
  if (lane == 0) lse[row] = wsum > 0.f ? M + kLn2 * fast_log2(wsum) : -INFINITY;
}

int64_t split_work_items(int B, int Hkv, int max_len, int chunk) {
  return (int64_t)B * Hkv * (((int64_t)max_len + chunk - 1) / chunk);
}

static int device_cus() {
  // Queried once per device (the value never changes).
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int DT, int D>
static hipError_t launch_split_t(const SplitArgs& a, hipStream_t stream) {
  const int C = (int)(((int64_t)a.max_len + a.chunk - 1) / a.chunk);
  hipLaunchKernelGGL((attn_decode_split_kernel<DT, D>), dim3((unsigned)device_cus()),
                     dim3(kSplitThreads), 0, stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.seq_lens, a.part_o,
                     a.part_lse, a.B, a.Hq, a.Hkv, a.max_len, a.chunk, C, a.scale);
  return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_combine_t(const CombineArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.Hq;
  const int64_t blocks = (rows + 3) / 4;
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
