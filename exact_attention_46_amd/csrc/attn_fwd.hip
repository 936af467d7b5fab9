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
//
// Global reads go through raw buffer resources sized to the valid rows, so the
// rows of a ragged last tile (and the Q rows past Nq) read as zero with no
// per-row branch; K/V tiles are prefetched into registers one tile ahead and
// written to LDS after the current tile's products.
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
  static constexpr int kKPitch = D * 2 + 16;            // K tile row pitch, bytes
  static constexpr int kKBytes = kFwdBN * kKPitch;
  static constexpr int kVPitch = kFwdBN * 2 + 16;       // V^T tile row pitch, bytes
  static constexpr int kVBytes = D * kVPitch;
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kLds = 2 * kStage;
  // Staging roles: threads [0, 128) stage K, threads [128, 128 + D) stage V.
  static constexpr int kKRowsPerThread = kFwdBN * kChunks / 128;  // D/16
  static constexpr int kVThreads = 8 * (D / 8);                   // 8 slots x D/8 blocks
};

// V^T tile: row d holds the 64 keys of the tile in 8 slots of 16 bytes. Slot s
// = 2*grp + hh holds the keys 16*grp + {4*hh + 0..3, 8 + 4*hh + 0..3}: exactly
// the 8 k-slots that MFMA lane-half hh consumes in the 16-key step grp (see the
// P^T operand layout), so every MFMA A-operand is one 16-byte read.
__device__ __forceinline__ int vslot_key(int s, int m) {
  return 16 * (s >> 1) + 8 * (m >> 2) + 4 * (s & 1) + (m & 3);
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
  constexpr int DS = D / 16;   // MFMA k-steps over d
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  constexpr int ROW = D * 2;   // bytes per row
  __shared__ __attribute__((aligned(16))) unsigned char smem[Lay::kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index through readfirstlane: a scalar, so everything derived
  // from it (rows of the wave, staging role) is known to be wave-uniform.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int half = lane >> 5;

  const int nqt = (Nq + kFwdBM - 1) / kFwdBM;
  const int group = Hq / Hkv;
  int unit, qtile;
  fwd_tile_of(blockIdx.x, B * Hq, nqt, group, CAUSAL ? 1 : 0, unit, qtile);
  const int b = unit / Hq;
  const int h = unit % Hq;
  const int g = h / group;  // == floor(h * Hkv / Hq) since Hq % Hkv == 0

  const int off = Nk - Nq;  // bottom-right causal alignment
  const int q0 = qtile * kFwdBM;
  const int qw0 = q0 + wave * 32;  // first query row of this wave
  const int my_row = qw0 + r32;

  const uint16_t* qh = q + ((int64_t)b * Hq + h) * (int64_t)Nq * D;
  const uint16_t* kh = k + ((int64_t)b * Hkv + g) * (int64_t)Nk * D;
  const uint16_t* vh = v + ((int64_t)b * Hkv + g) * (int64_t)Nk * D;
  const auto rq = make_rsrc(qh, (uint32_t)Nq * ROW);
  const auto rk = make_rsrc(kh, (uint32_t)Nk * ROW);
  const auto rv = make_rsrc(vh, (uint32_t)Nk * ROW);

  // Keys this workgroup can see: [0, kv_end).
  int kv_end = Nk;
  if (CAUSAL) {
    kv_end = min(q0 + kFwdBM, Nq) - 1 + off + 1;
    kv_end = max(0, min(kv_end, Nk));
  }
  const int n_tiles = (kv_end + kFwdBN - 1) / kFwdBN;

  // ---- Q^T operand: lane holds row my_row, d-chunk (half * DS + ds) for step ds
  // (rows past Nq read as zero).
  u32x4_t qf[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds)
    qf[ds] = buf_load16(rq, (uint32_t)my_row * ROW + (half * DS + ds) * 16);

  // ---- K/V staging, in two wave-uniform roles (measured on gfx950: 16-byte
  // LDS writes whose 8- or 16-lane groups cover contiguous 128/256-byte runs
  // are conflict-free at any row stride).
  //  K role (threads 0..127): chunk kc of the consecutive rows ka*KR .. +KR-1,
  //    one whole 256-byte row per 16 lanes and write instruction.
  //  V role (threads 128..): V^T slot vs of d-block vd (d = 8*vd .. +7): loads
  //    the slot's 8 key rows (16 bytes each), transposes the 8x8 block in
  //    registers and writes 8 whole slots (rows d = 8*vd + e).
  constexpr int KR = Lay::kKRowsPerThread;
  const bool k_role = wave < 2;
  const bool v_role = !k_role && wave < 2 + Lay::kVThreads / 64;
  const int kc = tid % Lay::kChunks;
  const int ka = (tid & 127) / Lay::kChunks;
  const int vs = (tid - 128) & 7;
  const int vd = ((tid - 128) >> 3) & (D / 8 - 1);
  uint32_t st_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    st_off[i] = k_role ? (uint32_t)(ka * KR + (i % KR)) * ROW + kc * 16
                       : (uint32_t)vslot_key(vs, i) * ROW + vd * 16;
  u32x4_t sreg[8];

  auto gload = [&](int t) {
    const uint32_t base = (uint32_t)t * (kFwdBN * ROW);
    if (k_role) {
#pragma unroll
      for (int i = 0; i < KR; ++i) sreg[i] = buf_load16(rk, base + st_off[i]);
    } else if (v_role) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sreg[i] = buf_load16(rv, base + st_off[i]);
    }
  };

  auto lds_store = [&](int buf) {
    unsigned char* kt = smem + buf * Lay::kStage;
    unsigned char* vt = kt + Lay::kKBytes;
    if (k_role) {
#pragma unroll
      for (int i = 0; i < KR; ++i)
        *reinterpret_cast<u32x4_t*>(kt + (ka * KR + i) * Lay::kKPitch + kc * 16) = sreg[i];
    } else if (v_role) {
      // Row e of the block: element e of each of the 8 keys, two keys per dword.
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        u32x4_t out;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          out[j] = (e & 1) ? hi_halves(sreg[2 * j][w], sreg[2 * j + 1][w])
                           : lo_halves(sreg[2 * j][w], sreg[2 * j + 1][w]);
        *reinterpret_cast<u32x4_t*>(vt + (vd * 8 + e) * Lay::kVPitch + vs * 16) = out;
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

  // Largest key index this row may see (may be negative: then nothing).
  const int row_kmax = CAUSAL ? min(my_row + off, Nk - 1) : Nk - 1;
  const bool wave_rows_valid = qw0 < Nq;
  const int wave_last_row = min(qw0 + 31, Nq - 1);

  // The prologue and every iteration load and store unconditionally (the
  // prefetch index is clamped to the last tile, an L2 hit), so every buffer
  // load is provably complete at the loop head and the products of a tile never
  // wait on the next tile's prefetch. All loads are in bounds or read as zero.
  gload(0);
  lds_store(0);
  wait_all_memory();
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    gload(min(t + 1, n_tiles - 1));

    const int k0 = t * kFwdBN;
    const bool active = wave_rows_valid && (!CAUSAL || k0 <= wave_last_row + off);
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
      // Element e of block kb holds key k0 + 32*kb + 4*half + 8*(e/4) + e%4.
      const bool need_mask = (k0 + kFwdBN > Nk) || (CAUSAL && k0 + kFwdBN - 1 > qw0 + off);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int lim = row_kmax - (k0 + kb * 32 + 4 * half);
#pragma unroll
          for (int e = 0; e < 16; ++e)
            s[kb][e] = (8 * (e >> 2) + (e & 3) > lim) ? -INFINITY : s[kb][e];
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
      // V^T rows d = db*32 + r32, slot 2*ks + half.
      const unsigned char* vbase = vt + r32 * Lay::kVPitch + half * 16;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          u32x4_t a = *reinterpret_cast<const u32x4_t*>(vbase + db * 32 * Lay::kVPitch + ks * 32);
          oacc[db] = mfma32x32x16<DT>(a, pf[ks], oacc[db]);
        }
      }
    }

    lds_store(buf ^ 1);
    wait_all_memory();
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l_rounded, LSE = ln2 * (m + log2 l).
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
