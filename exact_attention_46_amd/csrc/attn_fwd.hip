// Exact attention forward for gfx950: O = softmax(scale * Q K^T + causal mask) V
// plus LSE, computed tile by tile with the online-softmax rescale (the algorithm
// in the module documentation of the abaddon "attention.rs" page; the running
// max / sum state and its LSE follow OnlineSoftmaxState on the rustytorch
// "flash_attention_forward.cu" page).
//
// Work decomposition
//   one workgroup = 8 waves = 256 query rows of one (batch, head); each wave owns
//   32 query rows for the whole pass. K/V tiles of 64 keys stream through LDS
//   (two K and two V buffers) and are shared by the 8 waves.
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
// Memory path. K and V tiles go from HBM straight into LDS with buffer loads
// (no VGPR staging): each wave moves 1 KB per instruction, the buffer resource
// of a tile covers only its valid rows, so the rows of a ragged last tile land
// as zeros. Both tiles are stored row-major without padding; the 16-byte chunk
// index inside a row is XOR-swizzled by a function of the row so that the MFMA
// operand reads are conflict-free (measured on gfx950). K operands are 16-byte
// reads; V^T operands come from two ds_read_b64_tr_b16 per MFMA, whose
// 16-lane transpose turns row-major V into the key-major A-operand layout.
//
// Two-phase schedule. The two waves that share a SIMD (waves w and w + 4) take
// opposite roles: while one issues its matrix products the other runs its
// softmax on the vector ALU, and a barrier between the phases swaps them. An
// exponential issued by the same wave between its own MFMAs stalls the matrix
// pipe (measured on gfx950), while one from the partner wave does not. Per
// tile t, wave group A does [S(t+1) = K(t+1) Q^T, O += P(t) V(t)] | barrier |
// [softmax of S(t+1)], group B does [softmax of S(t)] | barrier |
// [S(t+1), O += P(t) V(t)]; in both orders the rescale of O for a tile follows
// the P V of the tile before it. Iteration t also loads K(t+2) and V(t+1) (into
// the buffers K(t) and V(t-1) left) and ends with a barrier that publishes
// them. Each product runs as one dependent MFMA chain per accumulator block
// (all steps of S block 0, then block 1; all key steps of each O block), 2-3%
// faster on gfx950 than interleaving the blocks.
#include <climits>

#include "common.hpp"
#include "launch.hpp"

namespace mi355attn {

constexpr int kFwdBM = 256;     // query rows per workgroup
constexpr int kFwdBN = 64;      // keys per K/V tile
constexpr int kFwdWaves = 8;
constexpr int kFwdThreads = 64 * kFwdWaves;
constexpr float kTau = 8.0f;    // lazy-rescale threshold, log2 units

template <int D>
struct FwdLayout {
  static constexpr int kRow = D * 2;                 // bytes per row
  static constexpr int kChunks = D / 8;              // 16-byte chunks per row
  static constexpr int kRowsPerLoad = 64 / kChunks;  // rows one wave load covers
  static constexpr int kLoadsPerWave = kFwdBN / kRowsPerLoad / kFwdWaves;  // per tensor
  static constexpr int kTile = kFwdBN * kRow;        // bytes of one K or V tile
  static constexpr int kQWave = 32 * kRow;           // one wave's Q rows
  static constexpr int kQLoads = 32 / kRowsPerLoad;  // loads per wave for them
  static constexpr int kLds = 4 * kTile + kFwdWaves * kQWave;  // K, V (two each), Q
  // Local attention: two K/V rings (one per 128-row half), Q straight to registers.
  static constexpr int kLdsLocal = 8 * kTile;
};
static_assert(FwdLayout<128>::kLds <= 160 * 1024 && FwdLayout<128>::kLdsLocal <= 160 * 1024,
              "LDS of a gfx950 workgroup");

// Chunk swizzles (chunk index XOR f(row)), chosen against the LDS bank layout
// (64 four-byte banks; a 256-byte window is one bank row):
//  K: 32 lanes read 16 bytes of rows r..r+31 at one logical chunk; 16
//     consecutive rows must hit 16 distinct 16-byte bank groups.
//  V: each 32-lane half of a transposing read covers 4 consecutive rows x 64
//     bytes; the 4 rows must land on 4 disjoint 64-byte bank groups.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// Maps the linear workgroup id to (batch*head unit, query tile). Workgroups are
// dispatched round-robin over the 8 XCDs, each with its own L2. When the units
// split evenly, every XCD gets a contiguous block of units (whole GQA groups
// included) and walks it kFwdL2Units units at a time, all query tiles of those
// units before the next ones, heaviest causal tiles first within them: the
// workgroups resident on an XCD then share the K/V of a few heads, which stay
// in its L2 (measured on gfx950 at B=4 H=32 N=2048: 2 units at a time -10 %,
// 8 -1.5 %, 16 -3 % against 4; at N = 8192 and 32768 within 0.3 %).
constexpr int kFwdL2Units = 4;  // 4 heads' K and V (1 MiB each at N = 2048) fill one 4 MB L2

// Packed variable-length batches (spread = true) take the plain order instead:
// consecutive workgroups, which land on consecutive XCDs, take consecutive
// units, so every XCD gets the same share of every sequence (a contiguous block
// of units per XCD would hand whole long sequences to a few XCDs); all query
// tiles of a unit still land on one XCD when the unit count is a multiple of 8.
// Token-major batches of equal lengths (packed QKV) keep the contiguous order.
__device__ __forceinline__ void fwd_tile_of(int L, int units, int nqt, int group, int causal,
                                            bool spread, int& unit, int& qtile) {
  constexpr int G = kFwdL2Units;
  int rank;
  if (spread) {
    rank = L / units;
    unit = L % units;
  } else if (units % 8 == 0 && (units / 8) % G == 0 && G % group == 0) {
    const int upx = units / 8;
    const int x = L % 8, s = L / 8;
    const int grp = s / (G * nqt), r = s % (G * nqt);
    rank = r / G;
    unit = x * upx + grp * G + r % G;
  } else if (units % 8 == 0 && (units / 8) % group == 0) {
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

// Token-major batches. With cu_q: packed variable-length sequences, sequence b
// owns token rows [cu_q[b], cu_q[b+1]) of q / o and [cu_k[b], cu_k[b+1]) of k / v
// (offsets clamped into the tensors), lse is [Hq, total_q]. Without (uniform_len
// > 0): sequence b owns rows [b*uniform_len, (b+1)*uniform_len) of all of them,
// lse is [B, Hq, uniform_len]. Row r of head h of q sits at q + r*q_stride + h*d
// (k, v: kv_stride; o: o_stride); e.g. a packed [B, N, 3, H, d] qkv tensor is
// q = qkv, k = qkv + H*d, v = qkv + 2*H*d with q_stride = kv_stride = 3*H*d.
struct VarLen {
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  int q_stride, kv_stride, o_stride;
  int uniform_len;
};

// Local (sliding-window) attention: key j is allowed for query row i iff
// i + off - left <= j <= i + off + right (off = Nk - Nq); a negative bound is
// no bound on that side, so (left, right) = (-1, 0) is the causal mask.
struct Window {
  int left, right;
};

// The 16-bit value at half `hi` of a dword, widened to fp32.
template <int DT>
__device__ __forceinline__ float widen16(uint32_t w, int hi) {
  const uint32_t h = hi ? (w >> 16) : (w & 0xffffu);
  if constexpr (DT == kBF16)
    return __uint_as_float(h << 16);
  else
    return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}

// VARLEN = false: dense [B, H, N, d] tensors of Nq / Nk rows per head.
// VARLEN = true: packed batches (see VarLen); Nq / Nk are then the largest
// sequence lengths, which size the grid, and each workgroup takes its
// sequence's own lengths (workgroups past the end of a sequence exit).
// LOCAL = true: the mask is the window `win` (CAUSAL is false then); each
// workgroup walks only the key tiles its rows' windows touch, and each wave
// only the range of them its own rows touch.
// SPLIT (with LOCAL only): the two-halves form below, for narrow windows.
template <int DT, int D, bool CAUSAL, bool VARLEN, bool LOCAL, bool SPLIT = false>
__global__ void __launch_bounds__(kFwdThreads, 1)
attn_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                float* __restrict__ lse, int B, int Hq, int Hkv, int Nq, int Nk, float scale,
                VarLen vl, Window win) {
  using Lay = FwdLayout<D>;
  constexpr int DS = D / 16;   // MFMA k-steps over d
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  constexpr int ROW = Lay::kRow;
  static_assert(LOCAL || !SPLIT, "the two-halves form is for local attention");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SPLIT ? Lay::kLdsLocal : Lay::kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index through readfirstlane: a scalar, so everything derived
  // from it is known to be wave-uniform.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int half = lane >> 5;

  const int nqt = (Nq + kFwdBM - 1) / kFwdBM;
  const int group = Hq / Hkv;
  int unit, qtile;
  fwd_tile_of(blockIdx.x, B * Hq, nqt, group, CAUSAL ? 1 : 0, VARLEN && vl.cu_q != nullptr, unit,
              qtile);
  const int b = unit / Hq;
  const int h = unit % Hq;
  const int g = h / group;  // == floor(h * Hkv / Hq) since Hq % Hkv == 0
  const int q0 = qtile * kFwdBM;

  // Row strides (elements) and this sequence's first rows.
  constexpr int QS_DENSE = D;
  const int QS = VARLEN ? vl.q_stride : QS_DENSE;   // q
  const int KS = VARLEN ? vl.kv_stride : QS_DENSE;  // k / v
  const int OS = VARLEN ? vl.o_stride : QS_DENSE;   // o
  int64_t q_row0 = 0, k_row0 = 0;
  if constexpr (VARLEN) {
    if (vl.cu_q) {
      const int qs = min(max(vl.cu_q[b], 0), vl.total_q);
      const int qe = min(max(vl.cu_q[b + 1], qs), vl.total_q);
      const int ks = min(max(vl.cu_k[b], 0), vl.total_k);
      const int ke = min(max(vl.cu_k[b + 1], ks), vl.total_k);
      q_row0 = qs;
      k_row0 = ks;
      Nq = min(qe - qs, Nq);  // rows past the grid's largest length are not computed
      Nk = ke - ks;
    } else {
      q_row0 = k_row0 = (int64_t)b * vl.uniform_len;
    }
    if (q0 >= Nq) return;  // the whole workgroup: this sequence is shorter
  }

  const int off = Nk - Nq;  // bottom-right causal alignment
  // Role and rows: waves w and w + 4 share a SIMD; w < 4 is group A, the
  // others group B. The partners own adjacent 32-row blocks, so their causal
  // work is nearly equal.
  const int role_b = wave >> 2;
  const int qw0 = q0 + (2 * (wave & 3) + role_b) * 32;  // first query row of this wave
  const int my_row = qw0 + r32;

  const uint16_t* qh = VARLEN ? q + q_row0 * QS + (int64_t)h * D : q + ((int64_t)b * Hq + h) * (int64_t)Nq * D;
  const uint16_t* kh = VARLEN ? k + k_row0 * KS + (int64_t)g * D : k + ((int64_t)b * Hkv + g) * (int64_t)Nk * D;
  const uint16_t* vh = VARLEN ? v + k_row0 * KS + (int64_t)g * D : v + ((int64_t)b * Hkv + g) * (int64_t)Nk * D;
  // Q rows of this workgroup. Dense: the head's rows, addressed from row 0.
  // Packed: based at row q0, ranging over the rows below Nq (strided rows).
  const int q_rows = min(kFwdBM, Nq - q0);
  const auto rq = VARLEN ? make_rsrc(qh + (int64_t)q0 * QS, (uint32_t)(q_rows - 1) * QS * 2 + ROW)
                         : make_rsrc(qh, (uint32_t)Nq * ROW);

  // Tile-sharing group: the whole workgroup, or (SPLIT) one of two halves of 4
  // waves and 128 rows (waves 0, 4, 1, 5 and 2, 6, 3, 7: each half holds both
  // roles on two SIMDs) with a K/V ring of its own. A sliding window's key range
  // grows with the rows that share it; halving them cuts the keys walked per
  // row for a 512-key window from 768 to 640, at the price of two rings of
  // loads per iteration (worth it for narrow windows only).
  constexpr int G_WAVES = SPLIT ? 4 : kFwdWaves;
  constexpr int G_ROWS = 32 * G_WAVES;
  const int grp = SPLIT ? ((wave & 3) >> 1) : 0;
  const int wig = SPLIT ? 2 * (wave & 1) + role_b : wave;  // wave index inside the group
  // Keys a group with first row gq0 can see: its tiles [gt0, gn).
  auto group_tiles = [&](int gq0, int& gt0, int& gn) {
    int kv_end = Nk, kv_begin = 0;
    if (CAUSAL) kv_end = max(0, min(Nk, min(gq0 + G_ROWS, Nq) - 1 + off + 1));
    if constexpr (LOCAL) {
      if (win.right >= 0) kv_end = max(0, min(Nk, min(gq0 + G_ROWS, Nq) - 1 + off + win.right + 1));
      if (win.left >= 0) kv_begin = max(0, gq0 + off - win.left);
      if (gq0 >= Nq) kv_end = 0;  // a half past the last row reads nothing
      if (kv_begin > kv_end) kv_begin = kv_end;
    }
    gt0 = LOCAL ? kv_begin / kFwdBN : 0;
    gn = max(gt0, (kv_end + kFwdBN - 1) / kFwdBN);
  };
  int t0, n_tiles;
  group_tiles(q0 + G_ROWS * grp, t0, n_tiles);
  // Iterations of the tile loop: the larger count of the groups (all waves
  // pass the same barriers; a group past its last tile only waits).
  int n_iter = n_tiles - t0;
  if constexpr (SPLIT) {
    int o0, on;
    group_tiles(q0 + G_ROWS * (1 - grp), o0, on);
    n_iter = max(n_iter, on - o0);
  }

  // ---- Q: the wave's 32 rows go HBM -> its own LDS block once, swizzled like
  // K (rows past Nq land as zeros); the Q^T operand of each product is read
  // from there (lane: row r32, d-chunk half * DS + ds), which keeps the
  // registers for the accumulators.
  // SPLIT: no Q block (Q goes straight to registers); the epilogue stages O in
  // the group's ring instead, free after the last tile.
  unsigned char* qslot = SPLIT ? smem + grp * 4 * Lay::kTile + wig * Lay::kQWave
                               : smem + 4 * Lay::kTile + wave * Lay::kQWave;
  auto issue_q = [&]() {
#pragma unroll
    for (int i = 0; i < Lay::kQLoads; ++i) {
      const int row = i * Lay::kRowsPerLoad + lane / Lay::kChunks;
      const int pc = lane % Lay::kChunks;
      const uint32_t src = VARLEN ? (uint32_t)(qw0 - q0 + row) * QS * 2 + (uint32_t)((pc ^ k_swz<D>(row)) * 16)
                                  : (uint32_t)(qw0 + row) * ROW + (uint32_t)((pc ^ k_swz<D>(row)) * 16);
      buf_load16_lds(rq, qslot + i * 1024, src);
    }
  };

  // ---- tile loads: load i of wave w covers tile rows (w*LPW + i)*RPL ..
  // +RPL-1; lane p fills physical chunk p % C of row p / C, i.e. it loads
  // logical chunk (p % C) ^ swz(row). Offsets are relative to the tile's first
  // row, whose address is carried by the per-tile buffer resource.
  constexpr int RPL = Lay::kRowsPerLoad;
  constexpr int LPW = kFwdBN / RPL / G_WAVES;  // loads per wave and tensor
  uint32_t koff[LPW], voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = (wig * LPW + i) * RPL + lane / Lay::kChunks;
    const int pc = lane % Lay::kChunks;
    const uint32_t rb = (uint32_t)row * (uint32_t)KS * 2;  // == row * ROW when dense
    koff[i] = rb + (uint32_t)((pc ^ k_swz<D>(row)) * 16);
    voff[i] = rb + (uint32_t)((pc ^ v_swz<D>(row)) * 16);
  }
  // Bytes a tile's buffer resource covers: its rows below Nk (rows past them
  // read as zeros).
  auto tile_bytes = [&](int r0) -> uint32_t {
    if constexpr (VARLEN)
      return (uint32_t)(min(kFwdBN, Nk - r0) - 1) * (uint32_t)KS * 2 + ROW;
    else
      return (uint32_t)(Nk - r0) * ROW;
  };
  // LDS: K buffers at [0, 2*kTile), V buffers at [2*kTile, 4*kTile) (of the
  // group's ring: SPLIT has two).
  unsigned char* kbuf = smem + (SPLIT ? grp * 4 * Lay::kTile : 0);
  unsigned char* vbuf = kbuf + 2 * Lay::kTile;
  auto issue_k = [&](int t) {
    const int r0 = t * kFwdBN;  // < Nk for every tile that is issued
    const auto rk = make_rsrc(kh + (int64_t)r0 * KS, tile_bytes(r0));
    unsigned char* dst = kbuf + (t & 1) * Lay::kTile;
#pragma unroll
    for (int i = 0; i < LPW; ++i) buf_load16_lds(rk, dst + (wig * LPW + i) * 1024, koff[i]);
  };
  auto issue_v = [&](int t) {
    const int r0 = t * kFwdBN;
    const auto rv = make_rsrc(vh + (int64_t)r0 * KS, tile_bytes(r0));
    unsigned char* dst = vbuf + (t & 1) * Lay::kTile;
#pragma unroll
    for (int i = 0; i < LPW; ++i) buf_load16_lds(rv, dst + (wig * LPW + i) * 1024, voff[i]);
  };

  // ---- per-lane LDS operand offsets (relative to the tile base)
  // K: row 32*kb + r32, logical chunk half*DS + ds, physical chunk ^ k_swz(r32).
  const int kx = k_swz<D>(r32);
  // V (transposing read): in each 16-lane group, source lane j = 4*kk + a
  // addresses row 16*ks + 4*half + kk (+8 for the second read) at column
  // d = 32*db + 16*((lane >> 4) & 1) + 4*a. The swizzle of those rows equals
  // v_swz(4*half + kk) for every ks and for the +8 rows.
  const int vkk = (lane & 15) >> 2, va = lane & 3;
  const int vrow0 = 4 * half + vkk;
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * va;
  uint32_t vop[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int col = 32 * db + vcol;
    vop[db] = (uint32_t)(vrow0 * ROW + (((col >> 3) ^ v_swz<D>(vrow0)) * 16) + (col & 7) * 2);
  }

  // ---- per-row state (identical in lanes l and l ^ 32)
  const float c = scale * kLog2e;
  float m_used = -INFINITY;  // exponent offset, log2 units
  float l_part = 0.f;        // this lane's share of the row sum (unrounded P)
  float lr_part = 0.f;       // the same over the rounded P fed to the MFMA
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16_t){};

  // Largest key index this row may see (may be negative: then nothing).
  int row_kmax = CAUSAL ? min(my_row + off, Nk - 1) : Nk - 1;
  int row_kmin = 0;  // LOCAL: smallest key index this row may see
  if constexpr (LOCAL) {
    if (win.right >= 0) row_kmax = min(my_row + off + win.right, Nk - 1);
    row_kmin = win.left >= 0 ? my_row + off - win.left : INT_MIN / 2;
  }
  const bool wave_rows_valid = qw0 < Nq;
  const int wave_last_row = min(qw0 + 31, Nq - 1);

  u32x4_t qf[DS];  // Q^T operands, read from the wave's LDS block after the prologue

  // Operand reads run a few products ahead of the MFMAs that use them, in a
  // fixed order (each step is closed by a scheduling barrier), so that an
  // MFMA finds its operands in registers instead of waiting for LDS.
  constexpr int VA = 3;  // V^T products read ahead
  const unsigned char* vbase_t;  // V tile of the P V being prefetched
  u32x2_t vlo[VA + 1], vhi[VA + 1];
  // V^T operand of product i of P V (column block db = i / 4, step ks = i % 4).
  auto read_v = [&](int i) {
    const int ks = i % 4, db = i / 4, slot = i % (VA + 1);
    const unsigned char* p0 = vbase_t + vop[db] + ks * 16 * ROW;
    vlo[slot] = lds_read_tr16_staged((const lds_s16x4_t*)p0);
    vhi[slot] = lds_read_tr16_staged((const lds_s16x4_t*)(p0 + 8 * ROW));
  };

  // S^T(t) = K(t) * Q^T for two 32-key blocks; with_v: the first V^T operands
  // of the P V of tile tv are read during the last steps.
  auto qk = [&](int t, f32x16_t* s, bool with_v, int tv) {
    const unsigned char* kt = kbuf + (t & 1) * Lay::kTile;
    vbase_t = vbuf + (tv & 1) * Lay::kTile;
    s[0] = (f32x16_t){};
    s[1] = (f32x16_t){};
    constexpr int KR = 4;  // K operand reads ahead
    u32x4_t kr[KR];
    // product j: key block kb = j / DS, step ds = j % DS
    auto read_k = [&](int j) {
      const int kb = j / DS, ds = j % DS;
      const int chunk = ((half * DS + ds) ^ kx) << 4;
      kr[j % KR] = *reinterpret_cast<const u32x4_t*>(kt + (32 * kb + r32) * ROW + chunk);
    };
#pragma unroll
    for (int j = 0; j < KR; ++j) read_k(j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 2 * DS; ++j) {
      const int kb = j / DS, ds = j % DS;
      s[kb] = mfma32x32x16<DT>(kr[j % KR], qf[ds], s[kb]);
      if (j + KR < 2 * DS) {
        read_k(j + KR);
      } else if (with_v) {
        const int i = j + KR - 2 * DS;  // 0 .. KR-1
        if (i < VA) read_v(i);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Masks S^T(t), takes its row maximum and moves the exponent offset m
  // (rescaling O and the sums) when the maximum outgrew it; then
  // P^T = exp2(s * c - m) into the 16-bit B operands pf (the row sum uses the
  // unrounded values, the second sum the rounded ones).
  auto softmax = [&](int t, f32x16_t* s, u32x4_t* pf) {
    const int k0 = t * kFwdBN;
    // Mask keys past the end and (causal) keys after the row's limit.
    // Element e of block kb holds key k0 + 32*kb + 4*half + 8*(e/4) + e%4.
    bool need_mask = (k0 + kFwdBN > Nk) || (CAUSAL && k0 + kFwdBN - 1 > qw0 + off);
    if constexpr (LOCAL)
      need_mask = need_mask || (win.right >= 0 && k0 + kFwdBN - 1 > qw0 + off + win.right) ||
                  (win.left >= 0 && k0 < wave_last_row + off - win.left);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int lim = row_kmax - (k0 + kb * 32 + 4 * half);
        const int lim_lo = row_kmin - (k0 + kb * 32 + 4 * half);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int ke = 8 * (e >> 2) + (e & 3);
          const bool out = LOCAL ? (ke > lim || ke < lim_lo) : (ke > lim);
          s[kb][e] = out ? -INFINITY : s[kb][e];
        }
      }
    }

    // Row maximum of this tile (raw scores; scale > 0 keeps the order): one
    // chain of three-way maxima per 32-key block, two new values per step.
    float mb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x16_t& x = s[kb];
      float r = fmaxf(fmaxf(x[0], x[1]), x[2]);
#pragma unroll
      for (int e = 3; e + 1 < 16; e += 2) r = fmaxf(fmaxf(r, x[e]), x[e + 1]);
      mb[kb] = fmaxf(r, x[15]);
    }
    float mx = max_with_partner32(fmaxf(mb[0], mb[1]));
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

    // Both row sums in four independent partial sums each (the unrounded
    // ones start from the first four values).
    float ls[4], lrs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = fast_exp2(__builtin_fmaf(s[kb][e], c, neg_m));
        if (kb == 0 && e < 4)
          ls[e] = p[e];
        else
          ls[e & 3] += p[e];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        pf[kb * 2 + j] = (u32x4_t){pack2<DT>(p[8 * j + 0], p[8 * j + 1]),
                                   pack2<DT>(p[8 * j + 2], p[8 * j + 3]),
                                   pack2<DT>(p[8 * j + 4], p[8 * j + 5]),
                                   pack2<DT>(p[8 * j + 6], p[8 * j + 7])};
#pragma unroll
        for (int w = 0; w < 4; ++w) lrs[w] = add_pair<DT>(pf[kb * 2 + j][w], lrs[w]);
      }
    }
    l_part += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    lr_part += (lrs[0] + lrs[1]) + (lrs[2] + lrs[3]);
  };

  // O^T += V(t)^T * P^T. For step ks the lane-half `half` needs, in k-slot m,
  // key 16*ks + 8*(m/4) + 4*half + m%4: the first transposing read gives slots
  // 0..3 (rows 16*ks + 4*half + 0..3), the second slots 4..7 (8 rows further).
  // prefetched: the first VA products' operands were read during S^T.
  auto pv = [&](int t, const u32x4_t* pf, bool prefetched) {
    vbase_t = vbuf + (t & 1) * Lay::kTile;
    constexpr int NP = 4 * DB;
    if (!prefetched) {
#pragma unroll
      for (int i = 0; i < VA; ++i) read_v(i);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int slot = i % (VA + 1);
      if (i + VA < NP) read_v(i + VA);
      const u32x4_t a = {vlo[slot][0], vlo[slot][1], vhi[slot][0], vhi[slot][1]};
      oacc[i / 4] = mfma32x32x16<DT>(a, pf[i % 4], oacc[i / 4]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Tiles active for this wave (some row may see a key of tile t) form the
  // range [a_lo, n_act) (a prefix, a_lo = 0, unless LOCAL).
  int n_act = 0;
  int a_lo = 0;
  if (wave_rows_valid) {
    n_act = n_tiles;
    if (CAUSAL) {
      const int last_key = wave_last_row + off;  // keys up to here are visible
      n_act = last_key < 0 ? 0 : min(n_tiles, last_key / kFwdBN + 1);
    }
    if constexpr (LOCAL) {
      int hi = Nk, lo = 0;
      if (win.right >= 0) hi = max(0, min(Nk, wave_last_row + off + win.right + 1));
      if (win.left >= 0) lo = max(0, qw0 + off - win.left);
      n_act = hi > lo ? (hi + kFwdBN - 1) / kFwdBN : t0;
      a_lo = hi > lo ? lo / kFwdBN : t0;
    }
  }
  auto active = [&](int t) -> bool { return (LOCAL ? t >= a_lo : true) && t < n_act; };

  // Prologue: K(0), V(0), K(1) and the wave's Q rows in flight; S(0) once they
  // land; group A also takes the softmax of S(0). The barrier after that frees
  // K(0)'s buffer. Each group then runs its own copy of the loop (one code path
  // per role keeps the register allocation of each to what that role needs);
  // both pass the same barriers.
  f32x16_t st[2];  // S of the next tile to take through the softmax
  u32x4_t pf[4];   // P of the next tile to multiply with V
  if (n_tiles > t0) {
    issue_k(t0);
    issue_v(t0);
  }
  if (n_tiles > t0 + 1) issue_k(t0 + 1);
  if constexpr (SPLIT) {
    // Q^T operands straight from memory (rows past Nq read as zeros).
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qf[ds] = buf_load16(rq, (uint32_t)(qw0 + r32) * ROW + (uint32_t)((half * DS + ds) * 16));
  } else {
    issue_q();
  }
  wait_all_memory();
  __syncthreads();
  // Q^T operand in registers: lane holds row r32, d-chunk half * DS + ds.
  if constexpr (!SPLIT) {
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qf[ds] = *reinterpret_cast<const u32x4_t*>(qslot + r32 * ROW + (((half * DS + ds) ^ kx) << 4));
  }
  auto loads = [&](int t) {
    if (t + 2 < n_tiles) issue_k(t + 2);
    if (t + 1 < n_tiles) issue_v(t + 1);
  };
  // The barrier between the two phases only keeps the partners in step; no
  // data crosses it, so it carries no memory fence (a fence would wait for the
  // tile loads still in flight).
  auto phase_barrier = []() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // The matrix phase of tile t: S(t+1) when tile t+1 is active, P V of tile t
  // when tile t is. The wave raises its issue priority for it, so that when
  // both waves of a SIMD have an instruction ready the next MFMA of the chain
  // goes first and the softmax of the partner fills the cycles in between
  // (1.5-2% faster on gfx950 across causal and non-causal shapes).
  auto matrix_phase = [&](int t) {
    const bool act = active(t), act_next = active(t + 1);
    __builtin_amdgcn_s_setprio(1);
    if (act_next) qk(t + 1, st, act, t);
    if (act) pv(t, pf, act_next);
    __builtin_amdgcn_s_setprio(0);
  };
  if (!role_b) {
    if (active(t0)) {
      qk(t0, st, false, t0);
      softmax(t0, st, pf);
    }
    __syncthreads();
    for (int t = t0; t < t0 + n_iter; ++t) {
      loads(t);
      matrix_phase(t);
      phase_barrier();
      if (active(t + 1)) softmax(t + 1, st, pf);
      wait_all_memory();
      __syncthreads();
    }
  } else {
    if (active(t0)) qk(t0, st, false, t0);
    __syncthreads();
    for (int t = t0; t < t0 + n_iter; ++t) {
      loads(t);
      if (active(t)) softmax(t, st, pf);
      phase_barrier();
      matrix_phase(t);
      wait_all_memory();
      __syncthreads();
    }
  }

  // ---- epilogue: O = O^T / l_rounded, LSE = ln2 * (m + log2 l).
  const float l_row = sum_with_partner32(l_part);
  const float lr_row = sum_with_partner32(lr_part);
  const bool empty = !(l_row > 0.f);
  float inv = empty ? 0.f : 1.f / lr_row;
  if constexpr (CAUSAL || LOCAL) {
    // A masked key has P = 0, but the products still form 0 * Inf or
    // 0 * NaN = NaN from its V row in every row of the wave. A wave whose
    // accumulators are all finite took no such value (and the common case
    // ends here); otherwise its rows are recomputed key by key over each row's
    // allowed keys only (Q from the wave's LDS block, K and V from memory,
    // P = exp2(s * c - m) with the final offset m, fp32, into the same
    // accumulators), so an Inf or NaN in V reaches exactly the rows that
    // attend to its key. Only input holding Inf or NaN gets there.
    bool fin = true;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        fin = fin && ((__float_as_uint(oacc[db][e]) & 0x7f800000u) != 0x7f800000u);
    if (!__all(fin) && wave_rows_valid) {
      int j_lo = 0, j_hi = Nk - 1;
      if constexpr (CAUSAL) j_hi = min(Nk - 1, wave_last_row + off);
      if constexpr (LOCAL) {
        if (win.right >= 0) j_hi = min(Nk - 1, wave_last_row + off + win.right);
        if (win.left >= 0) j_lo = max(0, qw0 + off - win.left);
      }
      const float neg_m = (m_used == -INFINITY) ? 0.f : -m_used;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = (f32x16_t){};
      const unsigned char* qrow = qslot + r32 * ROW;
#pragma unroll 1
      for (int j = j_lo; j <= j_hi; ++j) {
        // this lane's half of q.k (d-chunks half*DS .. +DS-1), then its partner's
        const uint16_t* kr = kh + (int64_t)j * KS + half * (D / 2);
        float part = 0.f;
        auto dot8 = [&](const u32x4_t& qq, const u32x4_t& kk) {
#pragma unroll
          for (int w = 0; w < 4; ++w)
            part = __builtin_fmaf(widen16<DT>(qq[w], 0), widen16<DT>(kk[w], 0),
                                  __builtin_fmaf(widen16<DT>(qq[w], 1), widen16<DT>(kk[w], 1), part));
        };
        if constexpr (SPLIT) {  // Q is in registers (this form keeps no Q block)
#pragma unroll
          for (int ds = 0; ds < DS; ++ds)
            dot8(qf[ds], *reinterpret_cast<const u32x4_t*>(kr + 8 * ds));
        } else {
#pragma unroll 2
          for (int ds = 0; ds < DS; ++ds)
            dot8(*reinterpret_cast<const u32x4_t*>(qrow + (((half * DS + ds) ^ kx) << 4)),
                 *reinterpret_cast<const u32x4_t*>(kr + 8 * ds));
        }
        const float sdot = sum_with_partner32(part);
        bool allowed = my_row < Nq && j <= row_kmax;
        if constexpr (LOCAL) allowed = allowed && j >= row_kmin;
        if (allowed) {
          const float p = fast_exp2(__builtin_fmaf(sdot, c, neg_m));
          const uint16_t* vr = vh + (int64_t)j * KS + 4 * half;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const u32x2_t w2 = *reinterpret_cast<const u32x2_t*>(vr + 32 * db + 8 * gq);
#pragma unroll
              for (int cc = 0; cc < 4; ++cc)
                oacc[db][4 * gq + cc] += p * widen16<DT>(w2[cc >> 1], cc & 1);
            }
        }
      }
      inv = empty ? 0.f : 1.f / l_row;  // these P were not rounded
    }
  }
  // O^T (lane: row r32, d = 32 db + 8 gq + 4 half + 0..3) goes row-major
  // through the wave's Q block in LDS (free since the prologue; 32 rows x ROW
  // bytes), 16-byte chunk c of row r stored at chunk c ^ (r mod chunks per
  // row) so that neither side has bank conflicts; the rows then leave in
  // whole-row stores of 16 bytes per lane (4 rows per store at d = 128), not
  // written through the caches. Scattered 8-byte stores straight from the
  // accumulators cost 4% of the kernel on gfx950.
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RPS = 64 / CPR;  // rows per store
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      u32x2_t w = {pack2<DT>(oacc[db][4 * gq + 0] * inv, oacc[db][4 * gq + 1] * inv),
                   pack2<DT>(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv)};
      const int chunk = (4 * db + gq) ^ (r32 & (CPR - 1));
      *reinterpret_cast<u32x2_t*>(qslot + r32 * ROW + chunk * 16 + half * 8) = w;
    }
  }
  wait_lgkmcnt0();
  uint16_t* otile = VARLEN ? o + (q_row0 + qw0) * OS + (int64_t)h * D
                           : o + (((int64_t)b * Hq + h) * (int64_t)Nq + qw0) * D;
  const int cl = lane % CPR, rl = lane / CPR;
#pragma unroll
  for (int s0 = 0; s0 < 32; s0 += RPS) {
    const int r = s0 + rl;
    const u32x4_t val = *reinterpret_cast<const u32x4_t*>(qslot + r * ROW + ((cl ^ (r & (CPR - 1))) << 4));
    if (qw0 + r < Nq)
      __builtin_nontemporal_store(val, reinterpret_cast<u32x4_t*>(otile + (int64_t)r * OS + cl * 8));
  }
  if (my_row < Nq && half == 0) {
    const float out = empty ? -INFINITY : kLn2 * (m_used + fast_log2(l_row));
    if constexpr (VARLEN) {
      if (vl.cu_q)
        lse[(int64_t)h * vl.total_q + q_row0 + my_row] = out;
      else
        lse[((int64_t)b * Hq + h) * (int64_t)Nq + my_row] = out;
    }
    else
      lse[((int64_t)b * Hq + h) * (int64_t)Nq + my_row] = out;
  }
}

// The two-halves form of local attention: both window bounds set and a window
// of at most 1024 keys (measured on gfx950 at N = 2048, d = 128: +5 % at 512
// keys back, -8 % at 2048, where both halves load nearly the same tiles).
static bool local_split(int left, int right) {
  return left >= 0 && right >= 0 && (int64_t)left + right <= 1024;
}

template <int DT, int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.Nq + kFwdBM - 1) / kFwdBM;
  const int64_t blocks = (int64_t)a.B * a.Hq * nqt;
  const VarLen vl{a.cu_q, a.cu_k, a.total_q, a.total_k, a.q_stride, a.kv_stride, a.o_stride,
                  a.uniform_len};
  const Window win{a.window_left, a.window_right};
  const bool halves = a.local && local_split(a.window_left, a.window_right);
  MI355_LOG("attn_fwd_kernel<%s,%d,%s> grid=%lld block=%d B=%d Hq=%d Hkv=%d Nq=%d Nk=%d "
            "window=(%d,%d) total_q=%d total_k=%d scale=%g stream=%p",
            dtype_name(DT), D,
            halves ? "local,two-halves" : a.local ? "local" : a.cu_q ? (CAUSAL ? "causal,varlen" : "varlen")
            : a.uniform_len > 0 ? (CAUSAL ? "causal,token-major" : "token-major")
            : (CAUSAL ? "causal" : "full"),
            (long long)blocks, kFwdThreads, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.window_left,
            a.window_right, a.total_q, a.total_k, (double)a.scale, (void*)stream);
  if (halves) {
    hipLaunchKernelGGL((attn_fwd_kernel<DT, D, false, false, true, true>), dim3((unsigned)blocks),
                       dim3(kFwdThreads), 0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
                       a.scale, vl, win);
  } else if (a.local) {
    hipLaunchKernelGGL((attn_fwd_kernel<DT, D, false, false, true>), dim3((unsigned)blocks),
                       dim3(kFwdThreads), 0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
                       a.scale, vl, win);
  } else if (a.cu_q || a.uniform_len > 0) {
    hipLaunchKernelGGL((attn_fwd_kernel<DT, D, CAUSAL, true, false>), dim3((unsigned)blocks),
                       dim3(kFwdThreads), 0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
                       a.scale, vl, win);
  } else {
    hipLaunchKernelGGL((attn_fwd_kernel<DT, D, CAUSAL, false, false>), dim3((unsigned)blocks),
                       dim3(kFwdThreads), 0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
                       a.scale, vl, win);
  }
  return hipGetLastError();
}

int64_t fwd_grid_blocks(int B, int Hq, int Nq) {
  return (int64_t)B * Hq * ((Nq + kFwdBM - 1) / kFwdBM);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
#define MI355_FWD_CASE(DTV, DV)                                                 \
  if (a.dtype == DTV && a.d == DV) {                                            \
    return a.causal && !a.local ? launch_fwd_t<DTV, DV, true>(a, stream)        \
                                : launch_fwd_t<DTV, DV, false>(a, stream);      \
  }
  MI355_FWD_CASE(kBF16, 128)
  MI355_FWD_CASE(kBF16, 64)
  MI355_FWD_CASE(kFP16, 128)
  MI355_FWD_CASE(kFP16, 64)
#undef MI355_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace mi355attn
