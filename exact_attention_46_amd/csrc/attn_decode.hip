// Split-KV ("flash decoding") decode for gfx950.
//
// attn_decode_split: one workgroup per (sequence b, kv-head g, chunk c). The
// R = Hq / Hkv query heads that share kv-head g (grouped-query attention, head
// h reads kv-head floor(h * Hkv / Hq)) are the columns of one 32-column MFMA
// tile, so every K/V byte of the chunk is read from HBM once and serves all R
// heads; K is never read twice (unlike a two-pass max-then-sum decode). The 4
// waves take interleaved 32-key tiles of the chunk, each with its own running
// max / sum (the online-softmax state of the rustytorch
// "flash_attention_forward.cu" page), and are merged at the end with the same
// algebra as the combine below; the chunk emits its normalised O_c (fp32) and
// LSE_c.
//
// attn_decode_combine: one wave per (b, h) merges the chunk partials with the
// rescaling combine of the aprender-gpu "flash_decoding/reduce_kernel.rs" page
// (global max of the chunk LSEs, weights exp(LSE_c - M), normalised weighted
// sum), skipping chunks whose LSE is -inf.
#include "common.hpp"
#include "launch.hpp"

namespace mi355attn {

constexpr int kSplitThreads = 256;
constexpr int kSplitWaves = 4;
constexpr int kSplitBN = 32;         // keys per wave tile
constexpr float kSplitTau = 8.0f;    // lazy-rescale threshold, log2 units

template <int D>
struct SplitLayout {
  static constexpr int kChunks = D / 8;            // 16-byte chunks per key row
  static constexpr int kKeysPerLane = D / 16;      // consecutive key rows per lane
  static constexpr int kKPitch = D * 2 + 16;
  static constexpr int kKBytes = kSplitBN * kKPitch;
  static constexpr int kVPitch = kSplitBN * 2 + 16;
  static constexpr int kVBytes = D * kVPitch;
  static constexpr int kWaveBytes = kKBytes + kVBytes;
  static constexpr int kLds = kSplitWaves * kWaveBytes;
  // The merge of the 4 waves reuses the same LDS: per wave 32 columns x D
  // floats of O plus 32 (m, l, l_rounded, pad) quadruples.
  static constexpr int kMergeBytes = kSplitWaves * (32 * D + 128) * 4;
  static_assert(kMergeBytes <= kLds, "merge area must fit in the staging LDS");
};

// Key position inside the 32-key V^T tile row: bits 2 and 3 of the offset in
// each 16-key group swapped, so the 8 keys one MFMA lane-half consumes per
// 16-key step are contiguous.
__device__ __forceinline__ int vt_pos32(int key) {
  int o = key & 15;
  return (key & ~15) | ((o & 4) << 1) | ((o & 8) >> 1) | (o & 3);
}

// Byte offset of (row d, key position pos) in the V^T tile; the 16-byte slot
// index is XOR-ed with (d >> 3) & 3 so that the staging writes of rows
// d = 8c + e (one slot, many c) spread over the LDS banks.
template <int PITCH>
__device__ __forceinline__ int vt_off32(int d, int pos) {
  const int slot = (pos >> 3) ^ ((d >> 3) & 3);
  return d * PITCH + slot * 16 + (pos & 7) * 2;
}

template <int DT, int D>
__global__ void __launch_bounds__(kSplitThreads, 2)
attn_decode_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                         const uint16_t* __restrict__ vc, const int* __restrict__ seq_lens,
                         float* __restrict__ part_o, float* __restrict__ part_lse, int Hq,
                         int Hkv, int max_len, int chunk, int C, float scale) {
  using Lay = SplitLayout<D>;
  constexpr int KPL = Lay::kKeysPerLane;
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(16))) unsigned char smem[Lay::kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31;
  const int half = lane >> 5;

  const int c = blockIdx.x % C;
  const int g = (blockIdx.x / C) % Hkv;
  const int b = blockIdx.x / (C * Hkv);
  const int R = Hq / Hkv;

  int L = seq_lens[b];
  L = L < 0 ? 0 : (L > max_len ? max_len : L);
  const int64_t lo = (int64_t)c * chunk;
  float* lse_out = part_lse + ((int64_t)b * Hq + (int64_t)g * R) * C + c;
  if (lo >= L) {
    // Chunk slot past the end of the sequence: no keys, LSE = -inf.
    if (tid < R) lse_out[(int64_t)tid * C] = -INFINITY;
    return;
  }
  const int64_t hi = min((int64_t)L, lo + chunk);
  const int n_keys = (int)(hi - lo);
  const int n_tiles = (n_keys + kSplitBN - 1) / kSplitBN;
  const int iters = (n_tiles + kSplitWaves - 1) / kSplitWaves;

  // Buffer resources cover only the L valid rows of this (b, g): cache rows
  // past the end of the sequence read as zero and are never fetched.
  const uint16_t* kg = kc + ((int64_t)b * Hkv + g) * (int64_t)max_len * D;
  const uint16_t* vg = vc + ((int64_t)b * Hkv + g) * (int64_t)max_len * D;
  const auto rk = make_rsrc(kg, (uint32_t)L * (D * 2));
  const auto rv = make_rsrc(vg, (uint32_t)L * (D * 2));

  // Q^T operand: column r32 is query head g*R + r32 (zero for r32 >= R).
  u32x4_t qf[DS];
  {
    const bool ok = r32 < R;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
        q + ((int64_t)b * Hq + (int64_t)g * R + (ok ? r32 : 0)) * D);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      u32x4_t x = src[half * DS + ds];
      qf[ds] = ok ? x : (u32x4_t){0u, 0u, 0u, 0u};
    }
  }

  // Staging: lane covers 16-byte chunk st_c of the consecutive key rows
  // st_a*KPL .. st_a*KPL+KPL-1 (each load instruction reads whole 256-byte rows).
  const int st_c = lane % Lay::kChunks;
  const int st_a = lane / Lay::kChunks;
  u32x4_t kreg[KPL], vreg[KPL];
  unsigned char* kt = smem + wave * Lay::kWaveBytes;
  unsigned char* vt = kt + Lay::kKBytes;

  const uint32_t st_off = (uint32_t)(st_a * KPL) * (D * 2) + st_c * 16;
  auto gload = [&](int tile) {
    // Rows at or past the chunk end belong to the next chunk (or lie past L):
    // they are loaded but masked out of the scores; the values are finite.
    const uint32_t base = (uint32_t)(lo + (int64_t)tile * kSplitBN) * (D * 2) + st_off;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      kreg[i] = buf_load16(rk, base + i * (D * 2));
      vreg[i] = buf_load16(rv, base + i * (D * 2));
    }
  };

  auto lds_store = [&]() {
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      *reinterpret_cast<u32x4_t*>(kt + (st_a * KPL + i) * Lay::kKPitch + st_c * 16) = kreg[i];
    // V^T: for each d of the chunk, groups of 4 consecutive keys side by side.
#pragma unroll
    for (int g4 = 0; g4 < KPL / 4; ++g4) {
      const int pos = vt_pos32(st_a * KPL + 4 * g4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint32_t w0, w1;
        if (e & 1) {
          w0 = hi_halves(vreg[4 * g4 + 0][w], vreg[4 * g4 + 1][w]);
          w1 = hi_halves(vreg[4 * g4 + 2][w], vreg[4 * g4 + 3][w]);
        } else {
          w0 = lo_halves(vreg[4 * g4 + 0][w], vreg[4 * g4 + 1][w]);
          w1 = lo_halves(vreg[4 * g4 + 2][w], vreg[4 * g4 + 3][w]);
        }
        *reinterpret_cast<u32x2_t*>(vt + vt_off32<Lay::kVPitch>(st_c * 8 + e, pos)) =
            (u32x2_t){w0, w1};
      }
    }
  };

  const float cl = scale * kLog2e;
  float m_used = -INFINITY;
  float l_part = 0.f;   // row sum of the unrounded P (for the LSE)
  float lr_part = 0.f;  // row sum of the rounded P fed to the MFMA (normalises O)
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16_t){};

  int tile = wave;
  gload(tile);
  for (int it = 0; it < iters; ++it, tile += kSplitWaves) {
    __syncthreads();  // previous readers of this wave's LDS are done
    lds_store();
    __syncthreads();
    // Unconditional prefetch (the last iteration re-reads its own tile) keeps
    // every buffer load provably complete at the store above.
    gload(it + 1 < iters ? tile + kSplitWaves : tile);
    if (tile < n_tiles) {
      f32x16_t s = (f32x16_t){};
      const unsigned char* krow = kt + r32 * Lay::kKPitch + half * DS * 16;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        u32x4_t a = *reinterpret_cast<const u32x4_t*>(krow + ds * 16);
        s = mfma32x32x16<DT>(a, qf[ds], s);
      }
      const int64_t k0 = lo + (int64_t)tile * kSplitBN;
      if (k0 + kSplitBN > hi) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t key = k0 + 8 * (e >> 2) + 4 * half + (e & 3);
          s[e] = key >= hi ? -INFINITY : s[e];
        }
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
      for (int j = 0; j < 2; ++j) {
        pf[j] = (u32x4_t){pack2<DT>(p[8 * j + 0], p[8 * j + 1]), pack2<DT>(p[8 * j + 2], p[8 * j + 3]),
                          pack2<DT>(p[8 * j + 4], p[8 * j + 5]), pack2<DT>(p[8 * j + 6], p[8 * j + 7])};
      }
      float lrsum = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int w = 0; w < 4; ++w) lrsum = add_pair<DT>(pf[j][w], lrsum);
      lr_part += lrsum;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int vr = db * 32 + r32;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          u32x4_t a =
              *reinterpret_cast<const u32x4_t*>(vt + vt_off32<Lay::kVPitch>(vr, 16 * ks + 8 * half));
          oacc[db] = mfma32x32x16<DT>(a, pf[ks], oacc[db]);
        }
      }
    }
  }

  // ---- merge the 4 waves: each publishes (m, l, l_rounded) and its
  // unnormalised O^T; O_c = sum_w a_w O_w / sum_w a_w lr_w and
  // LSE_c = ln2 * (M + log2 sum_w a_w l_w) with a_w = 2^(m_w - M).
  const float l_row = sum_with_partner32(l_part);
  const float lr_row = sum_with_partner32(lr_part);
  __syncthreads();  // all waves are done with the staging LDS
  float* mo = reinterpret_cast<float*>(smem);                  // [wave][32][D]
  float* ml = mo + kSplitWaves * 32 * D;                        // [wave][32][4]
  if (r32 < R) {
    float* dst = mo + ((int64_t)wave * 32 + r32) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) dst[db * 32 + 8 * (e >> 2) + 4 * half + (e & 3)] = oacc[db][e];
    if (half == 0) {
      ml[(wave * 32 + r32) * 4 + 0] = m_used;
      ml[(wave * 32 + r32) * 4 + 1] = l_row;
      ml[(wave * 32 + r32) * 4 + 2] = lr_row;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < R * D; idx += kSplitThreads) {
    const int r = idx / D, dd = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) M = fmaxf(M, ml[(w * 32 + r) * 4]);
    float num = 0.f, den = 0.f, den_r = 0.f;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
      const float mw = ml[(w * 32 + r) * 4];
      const float wt = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
      den += wt * ml[(w * 32 + r) * 4 + 1];
      den_r += wt * ml[(w * 32 + r) * 4 + 2];
      num += wt * mo[((int64_t)w * 32 + r) * D + dd];
    }
    const int64_t row = (int64_t)b * Hq + (int64_t)g * R + r;
    part_o[(row * C + c) * D + dd] = den > 0.f ? num / den_r : 0.f;
    if (dd == 0) part_lse[row * C + c] = den > 0.f ? kLn2 * (M + fast_log2(den)) : -INFINITY;
  }
}

template <int DT, int D>
__global__ void __launch_bounds__(256)
attn_decode_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                           const int* __restrict__ seq_lens, uint16_t* __restrict__ o,
                           float* __restrict__ lse, int B, int Hq, int C, int chunk) {
  constexpr int PER = D / 64;  // d values per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b, h) pair
  if (row >= (int64_t)B * Hq) return;
  const int b = (int)(row / Hq);
  int L = seq_lens[b];
  L = L < 0 ? 0 : L;
  int nc = (int)(((int64_t)L + chunk - 1) / chunk);
  nc = nc > C ? C : nc;
  const float* pl = part_lse + row * C;
  const float* po = part_o + row * C * D;

  float M = -INFINITY;
  for (int cc = lane; cc < nc; cc += 64) M = fmaxf(M, pl[cc]);
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) M = fmaxf(M, __shfl_xor(M, sh, 64));

  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int cc = 0; cc < nc; ++cc) {
      const float lc = pl[cc];
      if (lc == -INFINITY) continue;
      const float w = fast_exp2((lc - M) * kLog2e);
      wsum += w;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += w * po[(int64_t)cc * D + lane * PER + i];
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

int64_t split_grid_blocks(int B, int Hkv, int max_len, int chunk) {
  const int64_t C = ((int64_t)max_len + chunk - 1) / chunk;
  return (int64_t)B * Hkv * C;
}

template <int DT, int D>
static hipError_t launch_split_t(const SplitArgs& a, hipStream_t stream) {
  const int C = (int)(((int64_t)a.max_len + a.chunk - 1) / a.chunk);
  const int64_t blocks = split_grid_blocks(a.B, a.Hkv, a.max_len, a.chunk);
  hipLaunchKernelGGL((attn_decode_split_kernel<DT, D>), dim3((unsigned)blocks),
                     dim3(kSplitThreads), 0, stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.seq_lens, a.part_o,
                     a.part_lse, a.Hq, a.Hkv, a.max_len, a.chunk, C, a.scale);
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
