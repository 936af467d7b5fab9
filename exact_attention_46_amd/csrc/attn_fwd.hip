// Exact attention forward for gfx950: O = softmax(scale * Q K^T + causal mask) V
// plus LSE, computed tile by tile with the online-softmax rescale (the algorithm
// in the module documentation of the abaddon "attention.rs" page; the running
// max / sum state and its LSE follow OnlineSoftmaxState on the rustytorch
// "flash_attention_forward.cu" page).
//
// Work decomposition
//   one workgroup = 4 waves = 128 query rows of one (batch, head); each wave owns
//   32 query rows for the whole pass. K/V tiles of 64 keys stream through
//   double-buffered LDS and are shared by the 4 waves.
//
// Per wave and K/V tile (both products on 32x32x16 MFMA, fp32 accumulate):
//   S^T[64 keys x 32 rows] = K_tile * Q_w^T      A = K from LDS, B = Q^T in VGPRs
//   P^T = exp2(S^T * scale*log2e - m)            in registers, no data movement:
//                                                the S^T accumulator already has
//                                                the B-operand lane layout
//   O^T[d x 32 rows] += V_tile^T * P^T           A = V^T from LDS, B = P^T
// Computing the transposed products puts one query row per lane (and its
// partner lane l ^ 32), so the row max needs a single cross-lane exchange, the
// row sum none until the end, and the rescale of O is a per-lane scalar.
//
// Lazy rescale: the running maximum m used in the exponent is only moved when
// the row maximum grows by more than kTau (log2 units), so P <= 2^kTau and O is
// rescaled rarely. The result is the same quantity: O = sum 2^(u-m) v / sum
// 2^(u-m) for any fixed m, and LSE = ln2 * (m + log2 sum 2^(u-m)).
//
// Two row sums are kept: the sum of the unrounded fp32 P (for the LSE) and the
// sum of the 16-bit P values that actually enter the P V product (to normalise
// O). With the latter the weights applied to V sum to exactly one, so the
// rounding of a dominant P cancels instead of scaling its V row.
#include "common.hpp"
#include "launch.hpp"

namespace mi355attn {

constexpr int kFwdBM = 128;     // query rows per workgroup
constexpr int kFwdBN = 64;      // keys per K/V tile
constexpr int kFwdThreads = 256;
constexpr float kTau = 8.0f;    // lazy-rescale threshold, log2 units

template <int D>
struct FwdLayout {
  static constexpr int kChunks = D / 8;                 // 16-byte chunks per row
  static constexpr int kKeysPerThread = D / 32;         // rows each thread stages
  static constexpr int kKPitch = D * 2 + 16;            // K tile row pitch, bytes
  static constexpr int kKBytes = kFwdBN * kKPitch;
  static constexpr int kVPitch = kFwdBN * 2 + 16;       // V^T tile row pitch, bytes
  static constexpr int kVBytes = D * kVPitch;
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kLds = 2 * kStage;
};

// Position of key offset o (0..15) inside its 16-key group of the V^T tile:
// bits 2 and 3 swapped, so the eight keys an MFMA lane-half needs for one
// 16-key step are contiguous (see the P^T operand layout below).
__device__ __forceinline__ int vt_pos(int key) {
  int o = key & 15;
  return (key & ~15) | ((o & 4) << 1) | ((o & 8) >> 1) | (o & 3);
}

// Maps the linear workgroup id to (batch*head unit, query tile). Heaviest causal
// tiles first; when the units split evenly over the 8 XCDs (workgroups are
// dispatched round-robin over XCDs) every XCD gets a contiguous block of units,
// whole GQA groups included, so K/V reuse stays inside one L2.
__device__ __forceinline__ void fwd_tile_of(int L, int units, int nqt, int group, int causal,
                                            int& unit, int& qtile) {
  int rank;
  if (units % 8 == 0 && (units / 8) % group == 0) {
    const int upx = units / 8;
    const int x = L % 8, s = L / 8;
    rank = s / upx;
    unit = x * upx + s % upx;
  } else {
    rank = L / units;
    unit = L % units;
  }
  qtile = causal ? (nqt - 1 - rank) : rank;
}

template <int DT, int D, bool CAUSAL>
__global__ void __launch_bounds__(kFwdThreads, 2)
attn_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                float* __restrict__ lse, int B, int Hq, int Hkv, int Nq, int Nk, float scale) {
  using Lay = FwdLayout<D>;
  constexpr int KPT = Lay::kKeysPerThread;
  constexpr int DS = D / 16;   // MFMA k-steps over d
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) unsigned char smem[Lay::kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31;
  const int half = lane >> 5;

  const int nqt = (Nq + kFwdBM - 1) / kFwdBM;
  const int group = Hq / Hkv;
  int unit, qtile;
  fwd_tile_of(blockIdx.x, B * Hq, nqt, group, CAUSAL ? 1 : 0, unit, qtile);
  const int b = unit / Hq;
  const int h = unit % Hq;
  const int g = h / group;  // == floor(h * Hkv / Hq) since Hq % Hkv == 0

  const int64_t off = (int64_t)Nk - Nq;  // bottom-right causal alignment
  const int q0 = qtile * kFwdBM;
  const int qw0 = q0 + wave * 32;        // first query row of this wave
  const int my_row = qw0 + r32;

  const uint16_t* qh = q + ((int64_t)b * Hq + h) * (int64_t)Nq * D;
  const uint16_t* kh = k + ((int64_t)b * Hkv + g) * (int64_t)Nk * D;
  const uint16_t* vh = v + ((int64_t)b * Hkv + g) * (int64_t)Nk * D;

  // Keys this workgroup can see: [0, kv_end).
  int64_t kv_end = Nk;
  if (CAUSAL) {
    int64_t last_row = (int64_t)min(q0 + kFwdBM, Nq) - 1;
    kv_end = last_row + off + 1;
    if (kv_end < 0) kv_end = 0;
    if (kv_end > Nk) kv_end = Nk;
  }
  const int n_tiles = (int)((kv_end + kFwdBN - 1) / kFwdBN);

  // ---- Q^T operand: lane holds row my_row, d-chunk (half * DS + ds) for step ds.
  u32x4_t qf[DS];
  {
    const bool ok = my_row < Nq;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(qh + (int64_t)(ok ? my_row : 0) * D);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      u32x4_t x = src[half * DS + ds];
      qf[ds] = ok ? x : (u32x4_t){0u, 0u, 0u, 0u};
    }
  }

  // ---- K/V staging: thread covers chunk c of rows a*KPT .. a*KPT+KPT-1.
  const int st_c = tid % Lay::kChunks;
  const int st_a = tid / Lay::kChunks;
  u32x4_t kreg[KPT], vreg[KPT];

  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int64_t key = (int64_t)t * kFwdBN + st_a * KPT + i;
      if (key < Nk) {
        kreg[i] = *reinterpret_cast<const u32x4_t*>(kh + key * D + st_c * 8);
        vreg[i] = *reinterpret_cast<const u32x4_t*>(vh + key * D + st_c * 8);
      } else {
        kreg[i] = (u32x4_t){0u, 0u, 0u, 0u};
        vreg[i] = (u32x4_t){0u, 0u, 0u, 0u};
      }
    }
  };

  auto lds_store = [&](int buf) {
    unsigned char* kt = smem + buf * Lay::kStage;
    unsigned char* vt = kt + Lay::kKBytes;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      *reinterpret_cast<u32x4_t*>(kt + (st_a * KPT + i) * Lay::kKPitch + st_c * 16) = kreg[i];
    }
    // V^T: for each of the 8 d values of the chunk, the KPT keys side by side.
    const int pos = vt_pos(st_a * KPT);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int dd = st_c * 8 + e;
      unsigned char* dst = vt + dd * Lay::kVPitch + pos * 2;
      if constexpr (KPT == 4) {
        uint32_t w0, w1;
        if (e & 1) {
          w0 = hi_halves(vreg[0][e >> 1], vreg[1][e >> 1]);
          w1 = hi_halves(vreg[2][e >> 1], vreg[3][e >> 1]);
        } else {
          w0 = lo_halves(vreg[0][e >> 1], vreg[1][e >> 1]);
          w1 = lo_halves(vreg[2][e >> 1], vreg[3][e >> 1]);
        }
        *reinterpret_cast<u32x2_t*>(dst) = (u32x2_t){w0, w1};
      } else {
        uint32_t w0 = (e & 1) ? hi_halves(vreg[0][e >> 1], vreg[1][e >> 1])
                              : lo_halves(vreg[0][e >> 1], vreg[1][e >> 1]);
        *reinterpret_cast<uint32_t*>(dst) = w0;
      }
    }
  };

  // ---- per-row state (identical in lanes l and l ^ 32)
  const float c = scale * kLog2e;
  float m_used = -INFINITY;  // exponent offset, log2 units
  float l_part = 0.f;        // this lane's share of the row sum (unrounded P)
  float lr_part = 0.f;       // the same over the rounded P fed to the MFMA
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16_t){};

  const int64_t row_kmax = CAUSAL ? (int64_t)my_row + off : (int64_t)Nk - 1;
  const bool wave_rows_valid = qw0 < Nq;
  const int64_t wave_last_row = (int64_t)min(qw0 + 31, Nq - 1);

  if (n_tiles > 0) {
    gload(0);
    lds_store(0);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) gload(t + 1);

    const int64_t k0 = (int64_t)t * kFwdBN;
    const bool active =
        wave_rows_valid && (!CAUSAL || k0 <= wave_last_row + off);
    if (active) {
      const unsigned char* kt = smem + buf * Lay::kStage;
      const unsigned char* vt = kt + Lay::kKBytes;

      // S^T = K * Q^T for two 32-key blocks.
      f32x16_t s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = (f32x16_t){};
        const unsigned char* krow = kt + (kb * 32 + r32) * Lay::kKPitch + half * DS * 16;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          u32x4_t a = *reinterpret_cast<const u32x4_t*>(krow + ds * 16);
          s[kb] = mfma32x32x16<DT>(a, qf[ds], s[kb]);
        }
      }

      // Mask keys past the end and (causal) keys after the row's limit.
      const bool need_mask =
          (k0 + kFwdBN > Nk) || (CAUSAL && k0 + kFwdBN - 1 > (int64_t)qw0 + off);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int64_t key = k0 + kb * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
            const bool dead = (key >= Nk) || (key > row_kmax);
            s[kb][e] = dead ? -INFINITY : s[kb][e];
          }
        }
      }

      // Row maximum of this tile (raw scores; scale > 0 keeps the order).
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
      mx = max_with_partner32(mx);
      const float m_tile = mx * c;

      const bool grow = m_tile > m_used + kTau;
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

      // P^T = exp2(s * c - m); the row sum uses the unrounded values.
      u32x4_t pf[4];
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float p[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          p[e] = fast_exp2(__builtin_fmaf(s[kb][e], c, neg_m));
          lsum += p[e];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          pf[kb * 2 + j] = (u32x4_t){pack2<DT>(p[8 * j + 0], p[8 * j + 1]),
                                     pack2<DT>(p[8 * j + 2], p[8 * j + 3]),
                                     pack2<DT>(p[8 * j + 4], p[8 * j + 5]),
                                     pack2<DT>(p[8 * j + 6], p[8 * j + 7])};
        }
      }
      l_part += lsum;
      float lrsum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int w = 0; w < 4; ++w) lrsum = add_pair<DT>(pf[j][w], lrsum);
      lr_part += lrsum;

      // O^T += V^T * P^T: 16-key steps; lane-half `half` reads the 8 keys
      // 16*ks + {8*(m/4) + 4*half + m%4}, stored contiguously at 16*ks + 8*half.
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const unsigned char* vrow = vt + (db * 32 + r32) * Lay::kVPitch + half * 16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          u32x4_t a = *reinterpret_cast<const u32x4_t*>(vrow + ks * 32);
          oacc[db] = mfma32x32x16<DT>(a, pf[ks], oacc[db]);
        }
      }
    }

    if (t + 1 < n_tiles) lds_store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l).
  const float l_row = sum_with_partner32(l_part);
  const float lr_row = sum_with_partner32(lr_part);
  if (my_row < Nq) {
    const bool empty = !(l_row > 0.f);
    const float inv = empty ? 0.f : 1.f / lr_row;
    uint16_t* orow = o + (((int64_t)b * Hq + h) * (int64_t)Nq + my_row) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = db * 32 + 8 * gq + 4 * half;
        u32x2_t w = {pack2<DT>(oacc[db][4 * gq + 0] * inv, oacc[db][4 * gq + 1] * inv),
                     pack2<DT>(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv)};
        *reinterpret_cast<u32x2_t*>(orow + d0) = w;
      }
    }
    if (half == 0) {
      float out = empty ? -INFINITY : kLn2 * (m_used + fast_log2(l_row));
      lse[((int64_t)b * Hq + h) * (int64_t)Nq + my_row] = out;
    }
  }
}

template <int DT, int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.Nq + kFwdBM - 1) / kFwdBM;
  const int64_t blocks = (int64_t)a.B * a.Hq * nqt;
  hipLaunchKernelGGL((attn_fwd_kernel<DT, D, CAUSAL>), dim3((unsigned)blocks), dim3(kFwdThreads),
                     0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale);
  return hipGetLastError();
}

int64_t fwd_grid_blocks(int B, int Hq, int Nq) {
  return (int64_t)B * Hq * ((Nq + kFwdBM - 1) / kFwdBM);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
#define MI355_FWD_CASE(DTV, DV)                                                 \
  if (a.dtype == DTV && a.d == DV) {                                            \
    return a.causal ? launch_fwd_t<DTV, DV, true>(a, stream)                    \
                    : launch_fwd_t<DTV, DV, false>(a, stream);                  \
  }
  MI355_FWD_CASE(kBF16, 128)
  MI355_FWD_CASE(kBF16, 64)
  MI355_FWD_CASE(kFP16, 128)
  MI355_FWD_CASE(kFP16, 64)
#undef MI355_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace mi355attn
