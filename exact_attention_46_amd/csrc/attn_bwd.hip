// Exact attention backward for gfx950: the gradients dQ, dK, dV of
// L = sum(dO * O) for O = softmax(scale * Q K^T + causal mask) V, recomputing the
// probabilities from the forward's per-row LSE instead of storing them (the
// backward of the flash-attention page's kernel and the attention_backward of
// the llm.c page compute the same quantities):
//   D_i   = sum_t dO_it O_it
//   P_ij  = exp(scale * q_i.k_j - LSE_i)          (0 for masked keys)
//   dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - D_i)
//   dV_j  = sum_i P_ij dO_i,   dK_j = scale sum_i dS_ij q_i,   dQ_i = scale sum_j dS_ij k_j
// dK and dV of kv-head g sum over the query heads that read it (GQA).
//
// Two kernels on one stream, no atomics (the result is deterministic):
//  * attn_bwd_dkdv_kernel: one workgroup of 8 waves per (batch, kv-head, 128
//    keys). Two waves own each 32 keys: the first keeps their K rows in
//    registers, computes S = Q K^T and P and accumulates dV^T += dO^T P; the
//    second keeps their V rows, computes dP = dO V^T, takes P from the first
//    through LDS, forms dS = P (dP - D) and accumulates dK^T += Q^T dS (32x32x16
//    MFMA, fp32 accumulate). Each wave holds one operand block and one
//    accumulator, so it fits in 256 registers and two waves share each SIMD.
//    The workgroup walks 64-row steps of Q and dO (every query head of the
//    group), staged in LDS with their LSE and D in a three-slot ring, in two
//    phases per step in which the two waves of a SIMD take opposite roles: one
//    issues products while the other forms P or dS (the schedule is described
//    at the kernel). The S / dP accumulators hold one key per lane and 16 rows
//    per lane, which is the B-operand layout of the next products, so P and dS
//    enter them as they are (rounded to the input dtype), with dO^T and Q^T
//    read from the staged tiles by transposing LDS reads.
//  * attn_bwd_dq_kernel: one workgroup of 8 waves per 256 query rows of one
//    (batch, head); each wave keeps its 32 rows of Q and dO in registers and
//    walks the 32-key blocks of K and V staged in LDS (64-key tiles, three
//    slots deep): S^T = K Q^T, dP^T = V dO^T (one query row per lane), dS^T,
//    then dQ^T += K^T dS^T with K^T from transposing reads, with every A
//    operand read four products ahead. The two waves of a SIMD alternate: one
//    issues a block's products while the other forms its dS (the schedule is
//    described at the kernel). It runs first and also computes D for its rows
//    (from their dO and O rows, each lane pair summing half of d), which the
//    dK/dV kernel then reads. One workgroup per CU, two waves per SIMD.
// The dK/dV and dQ kernels both recompute S and dP (7 matrix products in all
// instead of 5), which is what removes the atomics on dQ.
#include <type_traits>

#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace mi355attn {

typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;

// An LDS pointer from a 32-bit LDS byte address.
template <typename T>
__device__ __forceinline__ T* lds_ptr(uint32_t addr) {
  return (T*)(size_t)addr;
}

// 16-byte LDS read of a tile staged with buffer loads to LDS (restrict-scoped
// for the same reason as lds_read_tr16_staged: no wait for the loads still in
// flight, which write other bytes).
__device__ __forceinline__ u32x4_t lds_read16_staged(const lds_u32x4_t* __restrict__ p) {
  return *p;
}

constexpr int kDkdvWaves = 8;                  // dK/dV workgroup: 4 key blocks x 2 roles
constexpr int kDkdvThreads = 64 * kDkdvWaves;
constexpr int kBwdKeysWG = 32 * (kDkdvWaves / 2);  // keys per dK/dV workgroup
constexpr int kBwdQT = 64;                  // query rows per dK/dV step
constexpr int kBwdKT = 64;                  // keys per dQ step

// LDS tiles are row-major with the 16-byte chunk index XOR-swizzled by a
// function of the row, and each is read both as rows (16-byte reads of one
// logical chunk from 16 consecutive rows: the swizzle must be a bijection on
// any 16 consecutive rows) and transposed (each 32-lane half of a
// ds_read_b64_tr_b16 covers 4 chunks c0..c0+3 of an aligned group of 4 rows:
// within such a group the swizzle's low two bits must be constant and its high
// two bits distinct). At d = 128, 4 (r & 3) + ((r >> 2) & 3) meets both (the
// row-only swizzle r & 15 of the forward's K tile cost the backward 5e7 bank
// conflict cycles per dK/dV launch at B=4, H=32, N=2048, d=128).
template <int D>
__device__ __forceinline__ int bwd_swz(int row) {
  return D == 128 ? 4 * (row & 3) + ((row >> 2) & 3) : ((row >> 1) & 7);
}

// Stages rows [r0, r0 + ROWS) of a [*, D] row-major tensor (rows >= n read as
// zero) into an LDS tile: all threads of the workgroup take part, each load
// moves 1 KiB.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void stage_rows(const uint16_t* base, int r0, int n, unsigned char* tile,
                                           int tid) {
  constexpr int ROW = D * 2, CH = D / 8, RPL = 64 / CH;
  constexpr int LOADS = ROWS / RPL;  // 1 KiB loads for the tile
  static_assert(LOADS % NW == 0, "loads split evenly over the waves");
  const int wave = tid >> 6, lane = tid & 63;
  const int rows_valid = n - r0;  // > 0 for every staged tile
  const auto rs = make_rsrc(base + (int64_t)r0 * D, (uint32_t)rows_valid * ROW);
#pragma unroll
  for (int i = 0; i < LOADS / NW; ++i) {
    const int ld = wave * (LOADS / NW) + i;
    const int row = ld * RPL + lane / CH;
    const int pc = lane % CH;
    buf_load16_lds(rs, tile + ld * 1024, (uint32_t)row * ROW + (uint32_t)((pc ^ bwd_swz<D>(row)) << 4));
  }
}

// Stages 64 consecutive floats src[r0 .. r0+63] (entries at or past n read as
// zero) into LDS with one 4-byte-per-lane load of the calling wave.
__device__ __forceinline__ void stage_floats64(const float* src, int r0, int n, float* dst,
                                               int lane) {
  const auto rs = make_rsrc(src + r0, (uint32_t)max(0, n - r0) * 4u);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 4,
                                           (uint32_t)lane * 4u, 0, 0, 0);
}

// A-operand row read of a staged tile: row r, logical 16-byte chunk c.
template <int D>
__device__ __forceinline__ u32x4_t tile_row16(const unsigned char* tile, int r, int c) {
  return *reinterpret_cast<const u32x4_t*>(tile + r * (D * 2) + ((c ^ bwd_swz<D>(r)) << 4));
}

// Transposed A operand of step ks (16 tile rows 16ks..16ks+15) for output
// block db (32 columns of d): lane l supplies d index 32db + l%32 and, in
// k-slot m, tile row 16ks + 8(m/4) + 4(l/32) + m%4 -- the slot order of the
// accumulator rows of S / dP, so P and dS serve as B operands unchanged.
// Within each 16-lane group, source lane 4kk + a addresses row 4half + kk
// (+8 for the second read) at columns 32db + 16((l>>4)&1) + 4a.
template <int D>
__device__ __forceinline__ u32x4_t tile_tr(const unsigned char* tile, int ks, int db, int lane) {
  constexpr int ROW = D * 2;
  const int half = lane >> 5, kk = (lane & 15) >> 2, a = lane & 3;
  const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * a;
  const int r1 = 16 * ks + 4 * half + kk, r2 = r1 + 8;
  const unsigned char* p1 = tile + r1 * ROW + (((col >> 3) ^ bwd_swz<D>(r1)) << 4) + (col & 7) * 2;
  const unsigned char* p2 = tile + r2 * ROW + (((col >> 3) ^ bwd_swz<D>(r2)) << 4) + (col & 7) * 2;
  const u32x2_t lo = lds_read_tr16_staged((const lds_s16x4_t*)p1);
  const u32x2_t hi = lds_read_tr16_staged((const lds_s16x4_t*)p2);
  return (u32x4_t){lo[0], lo[1], hi[0], hi[1]};
}

// Workgroup L's (unit, block) pair. Consecutive workgroups go to the 8 XCDs in
// turn, so with units % 8 == 0 each XCD is given a contiguous range of units
// and walks the blocks of one unit after another: the workgroups resident on
// an XCD share the staged rows of a few units in its L2 (spreading a unit's
// blocks over all XCDs makes every L2 fetch every unit).
__device__ __forceinline__ void bwd_block_of(int L, int units, int per_unit, int& unit, int& idx) {
  if (units % 8 == 0) {
    const int x = L % 8, s = L / 8;
    unit = x * (units / 8) + s / per_unit;
    idx = s % per_unit;
  } else {
    unit = L / per_unit;
    idx = L % per_unit;
  }
}

// Workgroup L's (unit, rank) for the gradient kernels: as bwd_block_of, each
// XCD is given a contiguous range of units, but walks it G units at a time
// with the blocks of those units in rank order across them (every unit's
// causally heaviest block first), so that the list the dispatcher deals out
// to the XCD's CUs goes from heavy to light within each group instead of
// within each unit; the rows the group's workgroups share (K and V, or Q and
// dO) stay in the XCD's L2. Group sizes measured best on B=4, H=32, N=2048,
// d=128 causal (against 1, 2, 4, 8, 16 units): 8 for the recomputing dK/dV
// and dQ kernels, 2 for the dK/dV kernel that also stores dS, 4 for the dQ
// kernel that reads it.
constexpr int kDkdvGroup = 8, kDkdvDsGroup = 2, kDqGroup = 8, kDqDsGroup = 4;
template <int G>
__device__ __forceinline__ void bwd_group_order(int L, int units, int per_unit, int& unit, int& rank) {
  if (G > 1 && units % 8 == 0 && (units / 8) % G == 0) {
    const int x = L % 8, s = L / 8;
    const int grp = s / (G * per_unit), r = s % (G * per_unit);
    unit = x * (units / 8) + grp * G + r % G;
    rank = r / G;
  } else {
    bwd_block_of(L, units, per_unit, unit, rank);
  }
}

// acc + a.x b.x + a.y b.y for two packed pairs of the input dtype (products exact
// in fp32).
template <int DT>
__device__ __forceinline__ float dot2_acc(uint32_t a, uint32_t b, float acc) {
  if constexpr (DT == kBF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  acc, false);
  }
}

// ---------------------------------------------------------------- dK, dV

// Barriers of a dK/dV iteration. phase_barrier<VM>: the wave first waits until
// at most VM of its vector-memory operations are outstanding (the newest ones:
// completion is in order, so everything issued before them has landed) and
// for all of its LDS operations; the barrier then publishes the stage loads
// and the LDS stores of every wave. lds_barrier waits for this wave's LDS
// operations only; bare_barrier waits for nothing (each wave has consumed what
// it read). The compiler fences keep memory accesses on their side.
template <int VM>
__device__ __forceinline__ void phase_barrier() {
  wait_vmcnt_lgkmcnt0<VM>();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void lds_barrier() {
  wait_lgkmcnt0();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void bare_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

template <int V>
using ic = std::integral_constant<int, V>;

// Stored dS^T (attn_bwd_ds): blocks of kDsKeys keys x kDsRows query rows, one
// per (batch * Hq + head, 128-row block, 64-key tile) in that order, each
// kDsBlock bytes contiguous, key-major inside (a key's 128 rows are 256
// contiguous bytes); the dQ kernel streams the key tiles of its row blocks.
constexpr int kDsKeys = 64;
constexpr int kDsRows = 128;
constexpr int kDsBlock = kDsKeys * kDsRows * 2;
static_assert(kDsKeys == kBwdKT && kBwdKeysWG % kDsKeys == 0 &&
                  kDsRows % kBwdQT == 0,
              "a dK/dV wave's step and a dQ tile each fall in one block");

// STORE_DS: the second role also stores its dS (rounded to the input dtype) to
// ds_t in the blocked layout above (ds_row_blocks = ceil(Nq / kDsRows)), for
// attn_bwd_dq_ds_kernel. Every (key, row) pair with the key allowed for the row
// is written (rows >= Nq and keys >= Nk of a block as zeros); pairs of rows the
// workgroup's steps do not reach are causally masked and left as they were.
//
// Schedule. Step j is one 64-row tile of Q and dO (with its LSE and D) in LDS
// ring slot j % 3. Iteration j has two phases, and in each the two waves of a
// SIMD take opposite roles, one issuing matrix products while the other runs
// element-wise work (as in the forward):
//   phase 1: first role  P(j) = exp(scale S(j) - LSE) -> exchange buffer
//            second role dK^T += Q(j-1)^T dS(j-1), dP(j) = dO(j) V^T
//   phase 2: first role  dV^T += dO(j)^T P(j), S(j+1) = Q(j+1) K^T
//            second role dS(j) = P(j) (dP(j) - D)
// After the barrier between the phases each wave issues its part of stage
// j+2's loads (into the slot of step j-1, whose last reader was dK(j-1)); they
// have the next two phases to land and are waited for at the next iteration's
// phase barrier. The first-role S(0) runs before iteration 0, and iteration
// n_steps only finishes dK.
template <int DT, int D, bool CAUSAL, bool STORE_DS = false>
__global__ void __launch_bounds__(kDkdvThreads, 2)
attn_bwd_dkdv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                     const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                     const float* __restrict__ lse, const float* __restrict__ delta,
                     uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int B, int Hq, int Hkv,
                     int Nq, int Nk, float scale, uint16_t* __restrict__ ds_t,
                     int ds_row_blocks) {
  constexpr int DS = D / 16, DB = D / 32, ROW = D * 2;
  constexpr int TILE = kBwdQT * ROW;
  constexpr int XCHG = kBwdKeysWG * kBwdQT * 4;     // P of one step (fp32)
  // LDS: the P exchange, the LSE and D rows of three ring slots, then the Q
  // tiles and the dO tiles of the three slots. The exchange and the rows are
  // addressed with immediate offsets (which reach 64 KiB), the tiles through
  // per-lane bases (below).
  constexpr int XCHG_AT = 0, LD_AT = XCHG;
  constexpr int Q_AT = LD_AT + ((3 * 2 * kBwdQT * 4 + 1023) / 1024) * 1024;
  constexpr int DO_AT = Q_AT + 3 * TILE;
  // Loads per second-role wave of one stage (the second-role waves issue all
  // of them, in their element-wise phase): Q and dO rows; waves 4 and 5 also
  // load LSE / D.
  constexpr int ROW_LOADS = kBwdQT / (64 / (D / 8)) / (kDkdvWaves / 2);
  static_assert(ROW_LOADS >= 1 && DO_AT + 3 * TILE <= 160 * 1024, "stage ring of a gfx950 workgroup");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[DO_AT + 3 * TILE];
  float* const xchg = reinterpret_cast<float*>(smem + XCHG_AT);
  auto q_tile = [&](int sl) { return smem + Q_AT + sl * TILE; };
  auto do_tile = [&](int sl) { return smem + DO_AT + sl * TILE; };
  auto lse_rows = [&](int sl) { return reinterpret_cast<float*>(smem + LD_AT) + sl * 2 * kBwdQT; };
  auto d_rows = [&](int sl) { return lse_rows(sl) + kBwdQT; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Waves kb and kb + 4 (which share a SIMD) own the same 32 keys. The first
  // keeps their K rows and computes S, P and dV; the second keeps their V rows
  // and computes dP, dS (with the first's P, through LDS) and dK.
  const int kb = wave & 3;
  const bool second = wave >= 4;
  const int r32 = lane & 31, half = lane >> 5;
  const int nkt = (Nk + kBwdKeysWG - 1) / kBwdKeysWG;
  // b * Hkv + g and its key block; the causally heaviest (first) blocks of a
  // unit go first.
  int unit, kt;
  bwd_group_order<STORE_DS ? kDkdvDsGroup : kDkdvGroup>(blockIdx.x, B * Hkv, nkt, unit, kt);
  const int b = unit / Hkv, g = unit % Hkv;
  const int group = Hq / Hkv;
  const int off = Nk - Nq;  // bottom-right causal alignment
  const int k0 = kt * kBwdKeysWG;
  const int kw0 = k0 + 32 * kb;   // first key of this wave
  const int my_key = kw0 + r32;   // this lane's key (column of S / dP)

  // K rows (first role) or V rows (second role) of the wave's keys as B
  // operands: lane key r32, chunk half*DS + ds (keys >= Nk read as zero).
  const int64_t kvoff = ((int64_t)b * Hkv + g) * (int64_t)Nk * D;
  u32x4_t bf[DS];
  {
    const int valid = __builtin_amdgcn_readfirstlane(max(0, min(32, Nk - kw0)));
    const auto rs = make_rsrc((second ? v : k) + kvoff + (int64_t)kw0 * D, (uint32_t)valid * ROW);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      bf[ds] = buf_load16(rs, (uint32_t)r32 * ROW + (uint32_t)((half * DS + ds) << 4));
  }
  // dV^T (first role) or dK^T (second role): d x this wave's 32 keys.
  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = (f32x16_t){};
  // S (first role) or dP (second role) of a step: 64 rows x 32 keys in two
  // 32-row blocks, one key per lane; and P (first role) or dS (second role)
  // packed to 16 bits in the B-operand layout of the dV / dK products.
  f32x16_t sp[2];
  u32x4_t pk[2][2];
  const float c = scale * kLog2e;
  // This lane's P values of row block rb in the exchange buffer: four 16-byte
  // pieces, each piece of the 64 lanes contiguous.
  auto xchg_at = [&](int rb, int part) {
    return reinterpret_cast<f32x4_t*>(xchg + (((kb * 2 + rb) * 4 + part) * 64 + lane) * 4);
  };

  // Steps: every query head of the group, its 64-row tiles from the first one
  // whose rows may see a key of this workgroup (i >= k0 - off when causal).
  const int r_begin = CAUSAL ? max(0, k0 - off) : 0;
  const int t_begin = r_begin / kBwdQT;
  const int t_end = (Nq + kBwdQT - 1) / kBwdQT;
  const int per_head = max(0, t_end - t_begin);
  const int n_steps = group * per_head;
  auto step_row0 = [&](int i) { return (t_begin + i % per_head) * kBwdQT; };
  // Stage of step i into ring slot SL (== i % 3), issued by the second-role
  // waves: Q and dO rows, LSE (wave 4) and D (wave 5).
  auto issue = [&](auto slot_c, int i) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    const int h = g * group + i / per_head;
    const int r0 = step_row0(i);
    const int64_t qoff = ((int64_t)b * Hq + h) * (int64_t)Nq;
    const int rtid = tid - 64 * (kDkdvWaves / 2);  // thread index within the role
    stage_rows<D, kBwdQT, kDkdvWaves / 2>(q + qoff * D, r0, Nq, q_tile(SL), rtid);
    stage_rows<D, kBwdQT, kDkdvWaves / 2>(dout + qoff * D, r0, Nq, do_tile(SL), rtid);
    if (wave == 4) stage_floats64(lse + qoff, r0, Nq, lse_rows(SL), lane);
    if (wave == 5) stage_floats64(delta + qoff, r0, Nq, d_rows(SL), lane);
  };
  // The LSE rows of a stage, scaled in place to -LSE * log2(e) (the exponent
  // offset of P = exp2(scale log2(e) S - LSE log2(e))) by wave 4 once they have
  // landed, so that P takes one multiply-add per element.
  auto scale_lse = [&](int sl) {
    float* l = lse_rows(sl) + lane;
    *l = -*l * kLog2e;
  };
  // Whether any (row, key) pair of the step at r0 and this wave's keys is
  // masked: rows past Nq, keys past Nk, or (causal) a key after some row's
  // diagonal.
  auto needs_mask = [&](int r0) {
    return r0 + kBwdQT > Nq || kw0 + 32 > Nk || (CAUSAL && kw0 + 31 > r0 + off);
  };

  // Per-lane LDS byte addresses of the operand reads, each including the base
  // of the kind of tile it reads (the first role reads Q as rows and dO
  // transposed, the second the reverse); a ring slot, row block or k-step adds
  // a compile-time offset below 64 KiB, which the reads take as their
  // immediate. The empty asm keeps the compiler from folding those offsets
  // into the addresses (which would need a register per slot).
  // rows: row r32 (+32 rb) at logical chunk half*DS + ds;
  // transposed: rows 4half + kk (+8 for the second read) at columns
  // 32db + 16((lane >> 4) & 1) + 4a (as tile_tr).
  uint32_t row_a[DS], tr_a[DB][2];
  {
    const uint32_t base = lds_addr(smem);
    const uint32_t fam_rows = base + (second ? DO_AT : Q_AT);
    const uint32_t fam_tr = base + (second ? Q_AT : DO_AT);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      row_a[ds] = fam_rows + (uint32_t)(r32 * ROW + (((half * DS + ds) ^ bwd_swz<D>(r32)) << 4));
      asm volatile("" : "+v"(row_a[ds]));
    }
    const int kk = (lane & 15) >> 2, a4 = lane & 3;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int r = 4 * half + kk + 8 * w;
        const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * a4;
        tr_a[db][w] = fam_tr + (uint32_t)(r * ROW + (((col >> 3) ^ bwd_swz<D>(r)) << 4) + (col & 7) * 2);
        asm volatile("" : "+v"(tr_a[db][w]));
      }
  }

  // One matrix phase: N1 products into acc (block db = n / 4, k-step n % 4 =
  // 2 rb + ks: A = the transposed tile in slot TRS, B = pk[rb][ks]), then N2
  // products into sp (block rb = m / DS, step ds = m % DS: A = rows of the
  // tile in slot RWS, B = bf[ds]). Each accumulator block is one dependent
  // chain; A operands are read RA products ahead.
  auto chain = [&](auto n1_c, auto n2_c, auto trs_c, auto rws_c) __attribute__((always_inline)) {
    constexpr int N1 = decltype(n1_c)::value, N2 = decltype(n2_c)::value, NP = N1 + N2;
    constexpr uint32_t TRS = decltype(trs_c)::value * TILE, RWS = decltype(rws_c)::value * TILE;
    constexpr int RA = 4;
    u32x4_t ring[RA];
    auto read_a = [&](int n) {
      if (n < N1) {
        const int db = n / 4, kstep = n % 4;
        const uint32_t o = TRS + (uint32_t)(16 * kstep * ROW);
        const u32x2_t lo = lds_read_tr16_staged(lds_ptr<const lds_s16x4_t>(tr_a[db][0] + o));
        const u32x2_t hi = lds_read_tr16_staged(lds_ptr<const lds_s16x4_t>(tr_a[db][1] + o));
        ring[n % RA] = (u32x4_t){lo[0], lo[1], hi[0], hi[1]};
      } else {
        const int m = n - N1, rb = m / DS, ds = m % DS;
        ring[n % RA] = lds_read16_staged(lds_ptr<const lds_u32x4_t>(row_a[ds] + RWS + (uint32_t)(32 * rb * ROW)));
      }
    };
#pragma unroll
    for (int n = 0; n < RA && n < NP; ++n) read_a(n);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < NP; ++n) {
      if (n < N1) {
        const int db = n / 4, rb = (n % 4) / 2, ks = n % 2;
        acc[db] = mfma32x32x16<DT>(ring[n % RA], pk[rb][ks], acc[db]);
      } else {
        const int m = n - N1, rb = m / DS, ds = m % DS;
        sp[rb] = mfma32x32x16<DT>(ring[n % RA], bf[ds], ds == 0 ? (f32x16_t){} : sp[rb]);
      }
      if (n + RA < NP) read_a(n + RA);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // First role, phase 1: P(j) = exp(scale S(j) - LSE) (0 where masked) from
  // sp, stored for the partner and packed into pk for dV. All LDS reads of the
  // phase go out first and the exchange stores last: interleaved, each group
  // of rows would wait for a whole LDS round trip (the stores and the reads
  // share the wait counter).
  auto make_p = [&](auto slot_c, int j) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    const int r0 = step_row0(j);
    const bool masked = needs_mask(r0);
    const float* slse = lse_rows(SL);
    // this lane's rows 32rb + 8gq + 4half + 0..3
    f32x4_t l4[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        l4[rb][gq] = *reinterpret_cast<const f32x4_t*>(slse + 32 * rb + 8 * gq + 4 * half);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        sp[rb][e] = fast_exp2(__builtin_fmaf(sp[rb][e], c, l4[rb][e / 4][e % 4]));
    if (masked) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = r0 + 32 * rb + 8 * (e / 4) + 4 * half + e % 4;
          const bool ok = row < Nq && my_key < Nk && (!CAUSAL || my_key <= row + off);
          sp[rb][e] = ok ? sp[rb][e] : 0.f;
        }
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        *xchg_at(rb, gq) = (f32x4_t){sp[rb][4 * gq], sp[rb][4 * gq + 1], sp[rb][4 * gq + 2], sp[rb][4 * gq + 3]};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        pk[rb][ks] = (u32x4_t){pack2<DT>(sp[rb][8 * ks + 0], sp[rb][8 * ks + 1]), pack2<DT>(sp[rb][8 * ks + 2], sp[rb][8 * ks + 3]),
                               pack2<DT>(sp[rb][8 * ks + 4], sp[rb][8 * ks + 5]), pack2<DT>(sp[rb][8 * ks + 6], sp[rb][8 * ks + 7])};
    }
  };

  // Second role, phase 2: dS(j) = P(j) (dP(j) - D) with the partner's P (same
  // lane and slot layout as dP) into pk for dK (and, STORE_DS, to ds_t). The
  // P and D reads of a row block go out together before its arithmetic.
  auto make_ds = [&](auto slot_c, int j) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    const float* sdl = d_rows(SL);
    // The dS^T block of this wave's keys and the step's rows (a wave whose
    // keys all lie past Nk has no block: its resource is empty).
    __amdgpu_buffer_rsrc_t rds;
    uint32_t ds_lane = 0;
    if constexpr (STORE_DS) {
      const int h = g * group + j / per_head;
      const int r0 = step_row0(j);
      const int nkb = (Nk + kDsKeys - 1) / kDsKeys;
      const int64_t blk = (((int64_t)b * Hq + h) * ds_row_blocks + r0 / kDsRows) * nkb + kw0 / kDsKeys;
      rds = make_rsrc(ds_t + blk * (kDsBlock / 2), kw0 < Nk ? (uint32_t)kDsBlock : 0u);
      ds_lane = (uint32_t)((kw0 % kDsKeys + r32) * kDsRows + r0 % kDsRows + 8 * half) * 2u;
    } else {
      (void)j;
    }
#pragma unroll
    for (int rb = 0; rb < kBwdQT / 32; ++rb) {
      f32x4_t d4[4], p4[4];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        d4[gq] = *reinterpret_cast<const f32x4_t*>(sdl + 32 * rb + 8 * gq + 4 * half);
        p4[gq] = *xchg_at(rb, gq);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) sp[rb][e] = p4[e / 4][e % 4] * (sp[rb][e] - d4[e / 4][e % 4]);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        pk[rb][ks] = (u32x4_t){pack2<DT>(sp[rb][8 * ks + 0], sp[rb][8 * ks + 1]),
                               pack2<DT>(sp[rb][8 * ks + 2], sp[rb][8 * ks + 3]),
                               pack2<DT>(sp[rb][8 * ks + 4], sp[rb][8 * ks + 5]),
                               pack2<DT>(sp[rb][8 * ks + 6], sp[rb][8 * ks + 7])};
      if constexpr (STORE_DS) {
        // pk[rb][ks] holds rows 32rb + 16ks + 8j + 4half + 0..3 in words 2j,
        // 2j+1. Swapping the j = 1 pieces of the low half with the j = 0
        // pieces of the high half leaves rows 32rb + 16ks + 8half + 0..7 in
        // each lane: one 16-byte store.
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const auto w0 = __builtin_amdgcn_permlane32_swap(pk[rb][ks][0], pk[rb][ks][2], false, false);
          const auto w1 = __builtin_amdgcn_permlane32_swap(pk[rb][ks][1], pk[rb][ks][3], false, false);
          __builtin_amdgcn_raw_buffer_store_b128((u32x4_t){w0[0], w1[0], w0[1], w1[1]}, rds,
                                                 ds_lane + (uint32_t)(32 * rb + 16 * ks) * 2u, 0,
                                                 0);
        }
      }
    }
  };
  // Stores of make_ds per step: they follow the next stage's loads in issue
  // order and may stay in flight across the next phase barrier.
  constexpr int DS_STORES = STORE_DS ? 2 * (kBwdQT / 32) : 0;

  // Iteration j of each role (SL == j % 3); both roles pass the same two
  // barriers. The steady-state iterations (FULL) take both products of their
  // matrix phase; the first and last iterations of a role take one, and are
  // compiled apart from the hot loop so that its register assignment is one.
  // First role: FULL for j < n_steps - 1 (dV(j) and S(j+1)); j = n_steps - 1
  // takes dV only, j = n_steps only passes the barriers.
  auto iter_first = [&](auto slot_c, int j, auto full_c) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr int NX = (SL + 1) % 3, PV = (SL + 2) % 3;
    make_p(slot_c, j);
    phase_barrier<0>();  // the exchange stores are complete
    __builtin_amdgcn_s_setprio(1);
    if constexpr (decltype(full_c)::value)
      chain(ic<4 * DB>{}, ic<2 * DS>{}, ic<SL>{}, ic<NX>{});
    else
      chain(ic<4 * DB>{}, ic<0>{}, ic<SL>{}, ic<NX>{});
    __builtin_amdgcn_s_setprio(0);
    bare_barrier();
  };
  // Second role: j = 0 takes dP(0) only, FULL for 0 < j < n_steps (dK(j-1)
  // and dP(j)), j = n_steps takes dK(n_steps - 1) only.
  // KIND: 0 first, 1 full, 2 last.
  auto iter_second = [&](auto slot_c, int j, auto kind_c) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr int NX = (SL + 1) % 3, PV = (SL + 2) % 3;
    constexpr int KIND = decltype(kind_c)::value;
    __builtin_amdgcn_s_setprio(1);
    if constexpr (KIND == 0)
      chain(ic<0>{}, ic<2 * DS>{}, ic<PV>{}, ic<SL>{});
    else if constexpr (KIND == 1)
      chain(ic<4 * DB>{}, ic<2 * DS>{}, ic<PV>{}, ic<SL>{});
    else
      chain(ic<4 * DB>{}, ic<0>{}, ic<PV>{}, ic<SL>{});
    __builtin_amdgcn_s_setprio(0);
    // stage j+1 landed; the dS stores of step j-1 (issued after it) may not have
    if constexpr (DS_STORES > 0 && KIND != 0)
      phase_barrier<DS_STORES>();
    else
      phase_barrier<0>();
    if (j + 2 < n_steps) issue(ic<PV>{}, j + 2);
    if (wave == 4 && j + 1 < n_steps) scale_lse(NX);
    if constexpr (KIND != 2) make_ds(slot_c, j);
    bare_barrier();
  };

  if (n_steps > 0) {
    // Stages 0 and 1 in flight; stage 0 landed and published, its LSE scaled
    // (and published); S(0).
    if (second) {
      issue(ic<0>{}, 0);
      if (n_steps > 1) issue(ic<1>{}, 1);
    }
    if (second && n_steps > 1) {
      if (wave == 4 || wave == 5)
        phase_barrier<2 * ROW_LOADS + 1>();
      else
        phase_barrier<2 * ROW_LOADS>();
    } else {
      phase_barrier<0>();
    }
    if (wave == 4) scale_lse(0);
    lds_barrier();
    if (!second) {
      __builtin_amdgcn_s_setprio(1);
      chain(ic<0>{}, ic<2 * DS>{}, ic<0>{}, ic<0>{});
      __builtin_amdgcn_s_setprio(0);
      const int full = n_steps - 1;  // iterations 0 .. n_steps - 2
      int j = 0;
      for (; j + 3 <= full; j += 3) {
        iter_first(ic<0>{}, j, std::true_type{});
        iter_first(ic<1>{}, j + 1, std::true_type{});
        iter_first(ic<2>{}, j + 2, std::true_type{});
      }
      if (j < full) iter_first(ic<0>{}, j++, std::true_type{});
      if (j < full) iter_first(ic<1>{}, j++, std::true_type{});
      // j == n_steps - 1: dV only
      if (j % 3 == 0)
        iter_first(ic<0>{}, j, std::false_type{});
      else if (j % 3 == 1)
        iter_first(ic<1>{}, j, std::false_type{});
      else
        iter_first(ic<2>{}, j, std::false_type{});
      // j == n_steps: the second role finishes dK
      phase_barrier<0>();
      bare_barrier();
    } else {
      iter_second(ic<0>{}, 0, ic<0>{});
      int j = 1;
      for (; j + 3 <= n_steps; j += 3) {
        iter_second(ic<1>{}, j, ic<1>{});
        iter_second(ic<2>{}, j + 1, ic<1>{});
        iter_second(ic<0>{}, j + 2, ic<1>{});
      }
      if (j < n_steps) iter_second(ic<1>{}, j++, ic<1>{});
      if (j < n_steps) iter_second(ic<2>{}, j++, ic<1>{});
      // j == n_steps: dK only
      if (j % 3 == 0)
        iter_second(ic<0>{}, j, ic<2>{});
      else if (j % 3 == 1)
        iter_second(ic<1>{}, j, ic<2>{});
      else
        iter_second(ic<2>{}, j, ic<2>{});
    }
  }

  // dV = (dV^T)^T, dK = scale * (dK^T)^T: lane key r32, d = 32db + 8(e/4) + 4half + e%4.
  if (my_key < Nk) {
    const float f = second ? scale : 1.f;
    uint16_t* po = (second ? dk : dv) + kvoff + (int64_t)my_key * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * db + 8 * gq + 4 * half;
        *reinterpret_cast<u32x2_t*>(po + d0) =
            (u32x2_t){pack2<DT>(acc[db][4 * gq + 0] * f, acc[db][4 * gq + 1] * f),
                      pack2<DT>(acc[db][4 * gq + 2] * f, acc[db][4 * gq + 3] * f)};
      }
  }
}

// ---------------------------------------------------------------- dQ

// dQ: one workgroup of 8 waves per 256 query rows of one (batch, head). Each
// wave keeps its 32 rows of Q^T and dO^T in registers as B operands and walks
// the 32-key blocks of the workgroup's key range: S^T = K Q^T and dP^T = V dO^T
// (one query row per lane, so LSE and D are per-lane scalars), dS^T, then
// dQ^T += K^T dS^T with K^T from transposing reads. The two waves of a SIMD
// (w and w + 4, owning adjacent 32-row blocks) alternate in phases separated by
// workgroup barriers: in its matrix phase for block j a wave issues dQ(j - 1),
// S(j) and dP(j) (24 products at d = 128) while its partner forms dS of its own
// block on the vector ALU; the second wave runs one phase behind the first.
//
//   phase   first wave (rows 64p .. 64p+31)    second wave (rows 64p+32 ..)
//   0       S(0), dP(0)                          -
//   2j+1    dS(j)                                dQ(j-1), S(j), dP(j)
//   2j+2    dQ(j), S(j+1), dP(j+1)               dS(j)
//
// 64-key tiles of K and V are staged in LDS three slots deep by the second
// waves: tile t + 3 goes into the slot of tile t in the phase after the second
// waves' dQ(2t + 1) (the slot's last reader), six phases before its first use,
// and each second wave waits for its share of a tile, with a counted vmcnt, at
// the barrier before the phase that first reads it.
constexpr int kDqWaves = 8;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqRowsWG = 32 * kDqWaves;
constexpr int kDqSlots = 3;

template <int DT, int D, bool CAUSAL>
__global__ void __launch_bounds__(kDqThreads, 1)
attn_bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const uint16_t* __restrict__ v, const uint16_t* __restrict__ o,
                   const uint16_t* __restrict__ dout, const float* __restrict__ lse,
                   float* __restrict__ delta, uint16_t* __restrict__ dq, int B, int Hq, int Hkv,
                   int Nq, int Nk, float scale) {
  constexpr int DS = D / 16, DB = D / 32, ROW = D * 2;
  constexpr int TILE = kBwdKT * ROW;
  constexpr int V_AT = kDqSlots * TILE;      // K slots, then V slots
  constexpr int STG_AT = 2 * kDqSlots * TILE;  // then each wave's 32-row staging slot
  constexpr int STG = 32 * ROW;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[STG_AT + kDqWaves * STG];
  static_assert(STG_AT + kDqWaves * STG <= 160 * 1024, "LDS of a gfx950 workgroup");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool second = wave >= kDqWaves / 2;
  const int r32 = lane & 31, half = lane >> 5;
  const int nqt = (Nq + kDqRowsWG - 1) / kDqRowsWG;
  // b * Hq + h and its row block; the causally heaviest (last) blocks of a
  // unit go first.
  int unit, qt;
  bwd_group_order<kDqGroup>(blockIdx.x, B * Hq, nqt, unit, qt);
  if (CAUSAL) qt = nqt - 1 - qt;
  const int b = unit / Hq, h = unit % Hq;
  const int g = h / (Hq / Hkv);
  const int off = Nk - Nq;
  const int q0 = qt * kDqRowsWG;
  const int qw0 = q0 + 32 * (2 * (wave & 3) + (second ? 1 : 0));
  const int my_row = qw0 + r32;  // this lane's query row (column of S^T)
  const int64_t qrow0 = ((int64_t)b * Hq + h) * (int64_t)Nq;
  const int64_t kvoff = ((int64_t)b * Hkv + g) * (int64_t)Nk * D;

  // Keys the workgroup's rows may see: [0, kv_end); tiles of 64 keys, blocks
  // of 32. This wave's rows see blocks [0, nb).
  int kv_end = Nk;
  if (CAUSAL) kv_end = max(0, min(Nk, min(q0 + kDqRowsWG, Nq) - 1 + off + 1));
  const int n_tiles = (kv_end + kBwdKT - 1) / kBwdKT;
  const int n_blocks = 2 * n_tiles;
  int w_end = qw0 < Nq ? Nk : 0;
  if (CAUSAL && qw0 < Nq) w_end = max(0, min(Nk, min(qw0 + 32, Nq) - 1 + off + 1));
  const int nb = __builtin_amdgcn_readfirstlane((w_end + 31) / 32);

  // Tile t of K and V into slot t % 3, issued by the second waves (each moves
  // TILE_LOADS KiB of it).
  constexpr int TILE_LOADS = 2 * (kBwdKT / (64 / (D / 8))) / (kDqWaves / 2);
  auto issue = [&](int t) {
    const int rtid = tid - 64 * (kDqWaves / 2);
    unsigned char* kt = smem + (t % kDqSlots) * TILE;
    stage_rows<D, kBwdKT, kDqWaves / 2>(k + kvoff, t * kBwdKT, Nk, kt, rtid);
    stage_rows<D, kBwdKT, kDqWaves / 2>(v + kvoff, t * kBwdKT, Nk, kt + V_AT, rtid);
  };
  const bool row_ok = my_row < Nq;

  // Q^T and dO^T B operands (lane row r32, chunk half*DS + ds; rows >= Nq
  // zero) and D of the wave's rows. The rows go through LDS: whole 1 KiB row
  // runs per load into the wave's staging slot (Q) and, before any tile is
  // staged, into the tile area (dO), then into registers by conflict-free
  // swizzled reads; O follows into the Q slot. (Loading the operand layout
  // straight from memory makes every load touch 32 rows.)
  const int valid = __builtin_amdgcn_readfirstlane(max(0, min(32, Nq - qw0)));
  unsigned char* stg_q = smem + STG_AT + wave * STG;
  unsigned char* stg_d = smem + wave * STG;
  stage_rows<D, 32, 1>(q + (qrow0 + qw0) * D, 0, valid, stg_q, lane);
  stage_rows<D, 32, 1>(dout + (qrow0 + qw0) * D, 0, valid, stg_d, lane);
  const float lse_row = row_ok ? lse[qrow0 + my_row] : 0.f;
  const int s_off = r32 * ROW;
  u32x4_t qf[DS], dof[DS];
  wait_vmcnt<0>();
  const float l2 = lse_row * kLog2e;
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    const int c16 = ((half * DS + ds) ^ bwd_swz<D>(r32)) << 4;
    qf[ds] = *reinterpret_cast<const u32x4_t*>(stg_q + s_off + c16);
    dof[ds] = *reinterpret_cast<const u32x4_t*>(stg_d + s_off + c16);
  }
  wait_lgkmcnt0();
  stage_rows<D, 32, 1>(o + (qrow0 + qw0) * D, 0, valid, stg_q, lane);
  // Every wave has read its dO rows out of the tile area.
  bare_barrier();
  if (second && n_tiles > 0) issue(0);
  // O has landed (tile 0, issued after it, may not have).
  if (second && n_tiles > 0)
    wait_vmcnt<TILE_LOADS>();
  else
    wait_vmcnt<0>();
  // D of this lane's row, sum_t dO_t O_t: each lane of the pair (l, l ^ 32)
  // sums its half of d; the first-half lane stores D for the dK/dV kernel.
  float dl;
  {
    float acc = 0.f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const u32x4_t ov = *reinterpret_cast<const u32x4_t*>(
          stg_q + s_off + (((half * DS + ds) ^ bwd_swz<D>(r32)) << 4));
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = dot2_acc<DT>(ov[j], dof[ds][j], acc);
    }
    dl = sum_with_partner32(acc);
    if (row_ok && half == 0) delta[qrow0 + my_row] = dl;
  }
  if (second && n_tiles > 1) issue(1);
  const float c = scale * kLog2e;
  f32x16_t dqa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqa[db] = (f32x16_t){};

  // Per-lane LDS byte addresses of the operand reads (as in the dK/dV
  // kernel): K rows and V rows r32 at logical chunk half*DS + ds (two
  // families: the V slots lie beyond the 64 KiB reach of one base), and the
  // transposed K reads of tile_tr (rows 4half + kk, +8; column block db). The
  // slot, the 32-key half and the k-step add compile-time offsets below
  // 64 KiB; the empty asm keeps the compiler from folding them into the
  // addresses.
  uint32_t row_k[DS], row_v[DS], tr_a[DB][2];
  {
    const uint32_t base = lds_addr(smem);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const uint32_t a = base + (uint32_t)(r32 * ROW + (((half * DS + ds) ^ bwd_swz<D>(r32)) << 4));
      row_k[ds] = a;
      row_v[ds] = a + V_AT;
      asm volatile("" : "+v"(row_k[ds]));
      asm volatile("" : "+v"(row_v[ds]));
    }
    const int kk = (lane & 15) >> 2, a4 = lane & 3;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int r = 4 * half + kk + 8 * w;
        const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * a4;
        tr_a[db][w] = base + (uint32_t)(r * ROW + (((col >> 3) ^ bwd_swz<D>(r)) << 4) + (col & 7) * 2);
        asm volatile("" : "+v"(tr_a[db][w]));
      }
  }

  f32x16_t s_, dp_;  // S^T and dP^T of the block between its two phases
  u32x4_t sf[2];     // dS^T of the block, B operands of its two dQ steps
  // Matrix phase: dQ^T += K^T dS^T of block RQ (when HQ; chained per
  // accumulator: product n is d-block n / 2, 16-key step n % 2), then
  // S^T = K Q^T and dP^T = V dO^T of block RS (when HS). Block j is 32-key half
  // j % 2 of tile j / 2 in slot (j / 2) % 3, so R = j % 6 fixes every LDS
  // offset. A operands are read RA products ahead through one ring; with PRE
  // the first RA reads (dQ operands of a block staged long before) were issued
  // during the wave's preceding vector phase.
  constexpr int RA = 4;
  static_assert(2 * DB >= RA, "prefetched reads are all dQ operands");
  u32x4_t ring[RA];
  auto read_dq = [&](auto rq_c, int n) __attribute__((always_inline)) {
    constexpr int RQ = decltype(rq_c)::value;
    const uint32_t o = (RQ / 2) * TILE + 16 * (2 * (RQ % 2) + n % 2) * ROW;
    const u32x2_t lo = lds_read_tr16_staged(lds_ptr<const lds_s16x4_t>(tr_a[n / 2][0] + o));
    const u32x2_t hi = lds_read_tr16_staged(lds_ptr<const lds_s16x4_t>(tr_a[n / 2][1] + o));
    ring[n % RA] = (u32x4_t){lo[0], lo[1], hi[0], hi[1]};
  };
  auto prefetch = [&](auto rq_c) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < RA; ++n) read_dq(rq_c, n);
  };
  auto mphase = [&](auto hq_c, auto hs_c, auto rq_c, auto rs_c, auto pre_c) __attribute__((always_inline)) {
    constexpr bool HQ = decltype(hq_c)::value, HS = decltype(hs_c)::value;
    constexpr bool PRE = decltype(pre_c)::value;
    constexpr int RS = decltype(rs_c)::value;
    constexpr int NQ = HQ ? 2 * DB : 0, NP = NQ + (HS ? 2 * DS : 0);
    static_assert(!PRE || HQ, "prefetch only for dQ products");
    auto read_a = [&](int n) __attribute__((always_inline)) {
      if (n < NQ) {
        read_dq(rq_c, n);
      } else {
        const int p = n - NQ;
        const uint32_t o = (RS / 2) * TILE + 32 * (RS % 2) * ROW;
        ring[n % RA] = lds_read16_staged(
            lds_ptr<const lds_u32x4_t>((p < DS ? row_k[p % DS] : row_v[p % DS]) + o));
      }
    };
    auto product = [&](int n) __attribute__((always_inline)) {
      if (n < NQ) {
        dqa[n / 2] = mfma32x32x16<DT>(ring[n % RA], sf[n % 2], dqa[n / 2]);
      } else {
        const int p = n - NQ;
        if (p < DS)
          s_ = mfma32x32x16<DT>(ring[n % RA], qf[p], p == 0 ? (f32x16_t){} : s_);
        else
          dp_ = mfma32x32x16<DT>(ring[n % RA], dof[p - DS], p == DS ? (f32x16_t){} : dp_);
      }
      if (n + RA < NP) read_a(n + RA);
      __builtin_amdgcn_sched_barrier(0);
    };
    __builtin_amdgcn_s_setprio(1);
    if constexpr (!PRE) {
#pragma unroll
      for (int n = 0; n < RA && n < NP; ++n) read_a(n);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < NP; ++n) product(n);
    __builtin_amdgcn_s_setprio(0);
  };
  constexpr std::true_type yes{};
  constexpr std::false_type no{};
  // dQ(j) alone, the wave's last matrix phase (once per wave: LDS offsets
  // added at run time).
  auto m_dq_any = [&](int j) __attribute__((always_inline)) {
    const uint32_t o0 = (uint32_t)(((j / 2) % kDqSlots) * TILE + 32 * (j % 2) * ROW);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int n = 0; n < 2 * DB; ++n) {
      const uint32_t o = o0 + 16 * (n % 2) * ROW;
      const u32x2_t lo = lds_read_tr16_staged(lds_ptr<const lds_s16x4_t>(tr_a[n / 2][0] + o));
      const u32x2_t hi = lds_read_tr16_staged(lds_ptr<const lds_s16x4_t>(tr_a[n / 2][1] + o));
      dqa[n / 2] = mfma32x32x16<DT>((u32x4_t){lo[0], lo[1], hi[0], hi[1]}, sf[n % 2], dqa[n / 2]);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // dS^T of block j from its S^T and dP^T, packed as the B operands of its
  // two dQ steps; masked where the block straddles this wave's diagonal or a
  // ragged edge.
  auto vphase = [&](int j) __attribute__((always_inline)) {
    const int k0 = 32 * j;
    const bool masked = qw0 + 32 > Nq || k0 + 32 > Nk || (CAUSAL && k0 + 31 > qw0 + off);
    float x[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = fast_exp2(__builtin_fmaf(s_[e], c, -l2));
    if (masked) {
      // Keys k0 + 8(e/4) + 4half + e%4 up to this row's last key stay.
      const int kmax = row_ok ? (CAUSAL ? min(Nk - 1, my_row + off) : Nk - 1) : -1;
      const int lim = kmax - (k0 + 4 * half);
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = 8 * (e >> 2) + (e & 3) <= lim ? x[e] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = x[e] * (dp_[e] - dl);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      sf[u] = (u32x4_t){pack2<DT>(x[8 * u + 0], x[8 * u + 1]), pack2<DT>(x[8 * u + 2], x[8 * u + 3]),
                        pack2<DT>(x[8 * u + 4], x[8 * u + 5]), pack2<DT>(x[8 * u + 6], x[8 * u + 7])};
    __builtin_amdgcn_sched_barrier(0);
  };
  // The second waves' barrier after their matrix phase of block j: for odd j
  // it first waits for their share of tile (j + 1) / 2 (tile (j + 1) / 2 + 1,
  // issued later, may still be in flight).
  auto second_m_barrier = [&](int j) __attribute__((always_inline)) {
    if (j & 1) {
      if ((j + 1) / 2 + 1 < n_tiles)
        phase_barrier<TILE_LOADS>();
      else
        phase_barrier<0>();
    } else {
      bare_barrier();
    }
  };

  // Tile 0 has landed (the second waves' share; each wave's own Q, dO and O
  // loads too); the barrier publishes it.
  if (second && n_tiles > 1)
    phase_barrier<TILE_LOADS>();
  else
    phase_barrier<0>();
  if (n_blocks == 0) {
    // No key for any row of the workgroup: dQ = 0, no further barrier.
  } else if (!second) {
    // Phases M(0) | V(j), M(j + 1) for j = 0 .. n_blocks - 1.
    if (nb > 0) mphase(no, yes, ic<0>{}, ic<0>{}, no);
    bare_barrier();
    int j = 0;
    // Steady state: M(j + 1) does dQ(j), S(j + 1), dP(j + 1); R = (j + 1) % 6.
    auto step = [&](auto r_c) __attribute__((always_inline)) -> bool {
      constexpr int R = decltype(r_c)::value;
      if (j + 1 >= nb) return false;
      prefetch(ic<(R + 5) % 6>{});
      vphase(j);
      bare_barrier();
      mphase(yes, yes, ic<(R + 5) % 6>{}, r_c, yes);
      bare_barrier();
      ++j;
      return true;
    };
    while (step(ic<1>{}) && step(ic<2>{}) && step(ic<3>{}) && step(ic<4>{}) && step(ic<5>{}) &&
           step(ic<0>{})) {
    }
    for (; j < n_blocks; ++j) {
      if (j < nb) vphase(j);
      bare_barrier();
      if (j == nb - 1) m_dq_any(j);
      bare_barrier();
    }
  } else {
    // Phases - | M(j), V(j) for j = 0 .. n_blocks - 1 | M(n_blocks).
    bare_barrier();
    if (nb > 0) mphase(no, yes, ic<0>{}, ic<0>{}, no);
    bare_barrier();
    if (2 < n_tiles) issue(2);
    if (1 < nb) prefetch(ic<0>{});
    if (nb > 0) vphase(0);
    bare_barrier();
    int j = 1;
    // Steady state: M(j) does dQ(j - 1), S(j), dP(j); R = j % 6. V(j) of an
    // even block first issues tile j / 2 + 2.
    auto step = [&](auto r_c) __attribute__((always_inline)) -> bool {
      constexpr int R = decltype(r_c)::value;
      if (j >= nb) return false;
      mphase(yes, yes, ic<(R + 5) % 6>{}, r_c, yes);
      second_m_barrier(j);
      if ((R & 1) == 0 && j / 2 + 2 < n_tiles) issue(j / 2 + 2);
      if (j + 1 < nb) prefetch(r_c);
      vphase(j);
      bare_barrier();
      ++j;
      return true;
    };
    while (step(ic<1>{}) && step(ic<2>{}) && step(ic<3>{}) && step(ic<4>{}) && step(ic<5>{}) &&
           step(ic<0>{})) {
    }
    for (; j < n_blocks; ++j) {
      if (j == nb) m_dq_any(j - 1);
      second_m_barrier(j);
      if ((j & 1) == 0 && j / 2 + 2 < n_tiles) issue(j / 2 + 2);
      bare_barrier();
    }
    if (nb == n_blocks) m_dq_any(n_blocks - 1);
  }

  // dQ = scale * (dQ^T)^T: lane row r32, d = 32db + 8(e/4) + 4half + e%4.
  if (row_ok) {
    uint16_t* pq = dq + (qrow0 + my_row) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * db + 8 * gq + 4 * half;
        *reinterpret_cast<u32x2_t*>(pq + d0) =
            (u32x2_t){pack2<DT>(dqa[db][4 * gq + 0] * scale, dqa[db][4 * gq + 1] * scale),
                      pack2<DT>(dqa[db][4 * gq + 2] * scale, dqa[db][4 * gq + 3] * scale)};
      }
  }
}

// ---------------------------------------------------------------- dQ from a stored dS

// D_i = sum_t dO_it O_it for every row of [rows, D] tensors: each row is summed
// by the D/8 lanes that load its 16-byte chunks, then reduced across them.
// Workgroups of 4 waves take 64 rows (16 per wave).
constexpr int kDeltaRowsWG = 64;

template <int DT, int D>
__global__ void __launch_bounds__(256)
attn_bwd_delta_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                      float* __restrict__ delta, int64_t rows) {
  constexpr int CH = D / 8, RPL = 64 / CH, LOADS = 16 / RPL;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r_wave = (int64_t)blockIdx.x * kDeltaRowsWG + wave * 16;
  const int c = lane % CH;
  u32x4_t ov[LOADS], dv[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int64_t row = r_wave + i * RPL + lane / CH;
    ov[i] = dv[i] = (u32x4_t){0u, 0u, 0u, 0u};
    if (row < rows) {
      ov[i] = *reinterpret_cast<const u32x4_t*>(o + row * D + c * 8);
      dv[i] = *reinterpret_cast<const u32x4_t*>(dout + row * D + c * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = dot2_acc<DT>(ov[i][j], dv[i][j], acc);
#pragma unroll
    for (int m = CH / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    const int64_t row = r_wave + i * RPL + lane / CH;
    if (row < rows && c == 0) delta[row] = acc;
  }
}

// Stages ROWS rows of 128 16-bit values, row r at src + r * stride_bytes (rows
// >= rows_valid read as zero), into an LDS tile laid out like the K tiles of
// width 128 (chunk index XOR bwd_swz<128>). The stored dS^T is read once:
// non-temporal loads keep it from evicting the K rows the row blocks share in
// L2 (6 % of the stored-dS backward on B=4, H=32, N=2048, d=128; storing dS
// non-temporally instead made it 23 % slower).
template <int ROWS, int NW>
__device__ __forceinline__ void stage_rows128_strided(const uint16_t* src, uint32_t stride_bytes,
                                                      int rows_valid, unsigned char* tile,
                                                      int tid) {
  constexpr int CH = 16, RPL = 64 / CH, LOADS = ROWS / RPL;
  static_assert(LOADS % NW == 0, "loads split evenly over the waves");
  const int wave = tid >> 6, lane = tid & 63;
  const int rv = min(rows_valid, ROWS);
  const auto rs = make_rsrc(src, rv > 0 ? (uint32_t)(rv - 1) * stride_bytes + 256u : 0u);
#pragma unroll
  for (int i = 0; i < LOADS / NW; ++i) {
    const int ld = wave * (LOADS / NW) + i;
    const int row = ld * RPL + lane / CH;
    const int pc = lane % CH;
    buf_load16_lds<kNonTemporal>(rs, tile + ld * 1024,
                                 (uint32_t)row * stride_bytes + (uint32_t)((pc ^ bwd_swz<128>(row)) << 4));
  }
}

// dQ = scale * dS K from the dS^T that attn_bwd_dkdv_kernel<..., true> stored:
// one workgroup of 8 waves per 256 query rows of one (batch, head), each wave 32
// rows, walking 64-key tiles of K and of dS^T (the two stored blocks of the
// workgroup's rows: 64 keys x 128 rows, 16 KiB contiguous each) staged in LDS
// three buffers deep, so that two tiles are in flight while one is used (the
// kernel is bound by reading dS). Both operands of dQ^T += K^T dS^T come from
// transposing reads (lane: d index or query row; k-slots: keys), with no
// recomputation of S or dP. On tiles that straddle a wave's causal diagonal the
// dS^T operand is masked to zero past each row's last key (entries the dK/dV
// kernel did not write lie only there).
constexpr int kDqDsWaves = 8;
constexpr int kDqDsRows = 32 * kDqDsWaves;
constexpr int kDqDsThreads = 64 * kDqDsWaves;
constexpr int kDqDsStages = 3;
static_assert(kDqDsRows == 2 * kDsRows, "two stored blocks per tile");

template <int DT, int D, bool CAUSAL>
__global__ void __launch_bounds__(kDqDsThreads, 1)
attn_bwd_dq_ds_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ ds_t,
                      uint16_t* __restrict__ dq, int B, int Hq, int Hkv, int Nq, int Nk,
                      int ds_row_blocks, float scale) {
  constexpr int DB = D / 32, ROW = D * 2;
  constexpr int KTILE = kBwdKT * ROW;
  constexpr int STAGE = KTILE + 2 * kDsBlock;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kDqDsStages * STAGE];
  static_assert(kDqDsStages * STAGE <= 160 * 1024, "LDS of a gfx950 workgroup");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, half = lane >> 5;
  const int nqt = (Nq + kDqDsRows - 1) / kDqDsRows;
  int unit, qt;
  bwd_group_order<kDqDsGroup>(blockIdx.x, B * Hq, nqt, unit, qt);
  if (CAUSAL) qt = nqt - 1 - qt;
  const int b = unit / Hq, h = unit % Hq;
  const int g = h / (Hq / Hkv);
  const int off = Nk - Nq;
  const int q0 = qt * kDqDsRows;
  const int qw0 = q0 + 32 * wave;
  const int my_row = qw0 + r32;
  const int64_t kvoff = ((int64_t)b * Hkv + g) * (int64_t)Nk * D;
  const int nkb = (Nk + kDsKeys - 1) / kDsKeys;
  // The workgroup's first stored block (row block 2 * qt, key tile 0); key tile
  // t is t blocks on, the second row block nkb blocks on.
  const uint16_t* dsh = ds_t + (((int64_t)unit * ds_row_blocks + 2 * qt) * nkb) * (kDsBlock / 2);
  const bool second_block = 2 * qt + 1 < ds_row_blocks;

  f32x16_t dqa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqa[db] = (f32x16_t){};

  int kv_end = Nk;
  if (CAUSAL) kv_end = max(0, min(Nk, min(q0 + kDqDsRows, Nq) - 1 + off + 1));
  const int n_tiles = (kv_end + kBwdKT - 1) / kBwdKT;
  // Loads per wave per tile: K's 1 KiB loads spread over the 8 waves, and 4 of
  // one dS^T block (waves 0-3 the first block, 4-7 the second; an absent second
  // block reads as zeros), so the wait for a tile is a fixed count.
  constexpr int KLOADS = kBwdKT / (64 / (D / 8)) / kDqDsWaves;
  constexpr int TILE_LOADS = KLOADS + kBwdKT / 4 / (kDqDsWaves / 2);
  static_assert(KLOADS >= 1 && TILE_LOADS == KLOADS + 4, "load split");
  auto issue = [&](int t) {
    unsigned char* st = smem + (t % kDqDsStages) * STAGE;
    stage_rows<D, kBwdKT, kDqDsWaves>(k + kvoff, t * kBwdKT, Nk, st, tid);
    const int blk = wave >> 2;
    const uint16_t* src = dsh + ((int64_t)blk * nkb + t) * (kDsBlock / 2);
    const int keys = (blk == 1 && !second_block) ? 0 : Nk - t * kBwdKT;
    stage_rows128_strided<kBwdKT, kDqDsWaves / 2>(src, (uint32_t)kDsRows * 2u, keys,
                                                  st + KTILE + blk * kDsBlock, tid & 255);
  };
  auto step = [&](auto buf_c, int t) {
    constexpr int BUF = decltype(buf_c)::value;
    const int k0 = t * kBwdKT;
    if (CAUSAL && k0 > qw0 + 31 + off) return;
    const bool masked = CAUSAL && k0 + kBwdKT - 1 > qw0 + off;
    const unsigned char* tk = smem + BUF * STAGE;
    const unsigned char* tds = tk + KTILE + (wave >> 2) * kDsBlock;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // lane: query row r32 of this wave; slot m: key k0 + 16ks + 8(m/4) + 4half + m%4
      u32x4_t sb = tile_tr<128>(tds, ks, wave & 3, lane);
      if (masked) {
        const int lim = my_row + off - (k0 + 16 * ks + 4 * half);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int o_lo = 8 * (w >> 1) + 2 * (w & 1);  // key offset of slot 2w
          const uint32_t keep = (o_lo <= lim ? 0x0000ffffu : 0u) | (o_lo + 1 <= lim ? 0xffff0000u : 0u);
          sb[w] &= keep;
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
        dqa[db] = mfma32x32x16<DT>(tile_tr<D>(tk, ks, db, lane), sb, dqa[db]);
    }
  };
  // Start of tile t: this wave's loads of tile t have landed (those of tile
  // t + 1, issued later, may not have); the barrier publishes every wave's and
  // ends all reads of tile t - 1, whose buffer tile t + 2 then takes.
  auto begin_tile = [&](int t) {
    if (t + 1 < n_tiles)
      wait_vmcnt_lgkmcnt0<TILE_LOADS>();
    else
      wait_all_memory();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    if (t + 2 < n_tiles) issue(t + 2);
  };
  if (n_tiles > 0) issue(0);
  if (n_tiles > 1) issue(1);
  for (int t = 0; t < n_tiles; t += kDqDsStages) {
    begin_tile(t);
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < n_tiles) {
      begin_tile(t + 1);
      step(std::integral_constant<int, 1>{}, t + 1);
    }
    if (t + 2 < n_tiles) {
      begin_tile(t + 2);
      step(std::integral_constant<int, 2>{}, t + 2);
    }
  }

  if (my_row < Nq) {
    uint16_t* pq = dq + (((int64_t)b * Hq + h) * (int64_t)Nq + my_row) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * db + 8 * gq + 4 * half;
        *reinterpret_cast<u32x2_t*>(pq + d0) =
            (u32x2_t){pack2<DT>(dqa[db][4 * gq + 0] * scale, dqa[db][4 * gq + 1] * scale),
                      pack2<DT>(dqa[db][4 * gq + 2] * scale, dqa[db][4 * gq + 3] * scale)};
      }
  }
}

// ---------------------------------------------------------------- launch

int64_t bwd_grid_blocks(int B, int Hq, int Hkv, int Nq, int Nk) {
  const int64_t a = (int64_t)B * Hkv * ((Nk + kBwdKeysWG - 1) / kBwdKeysWG);
  const int64_t c = (int64_t)B * Hq * ((Nq + kDqRowsWG - 1) / kDqRowsWG);
  return a > c ? a : c;
}

template <int DT, int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  // dQ first: it also writes D, which the dK/dV kernel reads.
  const int nqt = (a.Nq + kDqRowsWG - 1) / kDqRowsWG;
  const int nkt = (a.Nk + kBwdKeysWG - 1) / kBwdKeysWG;
  MI355_LOG("attn_bwd_dq_kernel<%s,%d,%s> grid=%lld block=%d then attn_bwd_dkdv_kernel grid=%lld "
            "block=%d B=%d Hq=%d Hkv=%d Nq=%d Nk=%d scale=%g delta=%p stream=%p",
            dtype_name(DT), D, CAUSAL ? "causal" : "full", (long long)a.B * a.Hq * nqt,
            kDqThreads, (long long)a.B * a.Hkv * nkt, kDkdvThreads, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
            (double)a.scale, (void*)a.delta, (void*)stream);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<DT, D, CAUSAL>), dim3((unsigned)(a.B * a.Hq * nqt)),
                     dim3(kDqThreads), 0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, (const uint16_t*)a.o, (const uint16_t*)a.dout, a.lse,
                     a.delta, (uint16_t*)a.dq, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DT, D, CAUSAL>), dim3((unsigned)(a.B * a.Hkv * nkt)),
                     dim3(kDkdvThreads), 0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse, a.delta,
                     (uint16_t*)a.dk, (uint16_t*)a.dv, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale,
                     nullptr, 0);
  return hipGetLastError();
}

// ---------------------------------------------------------------- fixed scratch

// attn_bwd_noalloc keeps D (one float per query row) here instead of in a
// caller-provided buffer: callers that cannot allocate (graph capture, tight
// serving loops) get a backward that allocates nothing. Every GPU the library
// runs on holds its own copy (16 MiB) until the process ends; all calls on
// one GPU share it, and the dQ kernel writes every D it holds before the
// dK/dV kernel reads it, so no clearing is needed.
static __device__ __align__(256) float scratch[kBwdScratchFloats];

// This GPU's address of `scratch`, looked up once per device (with that
// device current) on the first call there. The host-side name `scratch` is a
// stand-in for the symbol, never a device address; only the looked-up pointer
// is passed to kernels.
static hipError_t bwd_scratch(float** out) {
  static std::atomic<float*> cached[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  float* p = cached[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (addr == nullptr) return hipErrorInvalidSymbol;
    p = static_cast<float*>(addr);
    cached[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

int64_t bwd_ds_row_blocks(int Nq) { return ((int64_t)Nq + kDsRows - 1) / kDsRows; }

int64_t bwd_ds_bytes_per_head(int Nq, int Nk) {
  return ((int64_t)Nk + kDsKeys - 1) / kDsKeys * bwd_ds_row_blocks(Nq) * kDsBlock;
}

int64_t bwd_ds_grid_blocks(int B, int Hq, int Nq) {
  return ((int64_t)B * Hq * Nq + kDeltaRowsWG - 1) / kDeltaRowsWG;
}

template <int DT, int D, bool CAUSAL>
static hipError_t launch_bwd_ds_t(const BwdArgs& a, hipStream_t stream) {
  // D first, then dK/dV (which reads D and stores dS^T), then dQ from dS^T.
  const int64_t rows = (int64_t)a.B * a.Hq * a.Nq;
  const int nqt2 = (a.Nq + kDqDsRows - 1) / kDqDsRows;
  const int nkt = (a.Nk + kBwdKeysWG - 1) / kBwdKeysWG;
  MI355_LOG("attn_bwd_delta_kernel<%s,%d> grid=%lld block=256, attn_bwd_dkdv_kernel<%s,%d,%s,ds> "
            "grid=%lld block=%d, attn_bwd_dq_ds_kernel grid=%lld block=%d B=%d Hq=%d Hkv=%d "
            "Nq=%d Nk=%d ds_row_blocks=%d scale=%g stream=%p",
            dtype_name(DT), D, (long long)bwd_ds_grid_blocks(a.B, a.Hq, a.Nq), dtype_name(DT), D,
            CAUSAL ? "causal" : "full", (long long)a.B * a.Hkv * nkt, kDkdvThreads,
            (long long)a.B * a.Hq * nqt2, kDqDsThreads, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.ds_row_blocks,
            (double)a.scale, (void*)stream);
  hipLaunchKernelGGL((attn_bwd_delta_kernel<DT, D>),
                     dim3((unsigned)bwd_ds_grid_blocks(a.B, a.Hq, a.Nq)), dim3(256), 0, stream,
                     (const uint16_t*)a.o, (const uint16_t*)a.dout, a.delta, rows);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DT, D, CAUSAL, true>), dim3((unsigned)(a.B * a.Hkv * nkt)),
                     dim3(kDkdvThreads), 0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse, a.delta,
                     (uint16_t*)a.dk, (uint16_t*)a.dv, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale,
                     (uint16_t*)a.ds, a.ds_row_blocks);
  hipLaunchKernelGGL((attn_bwd_dq_ds_kernel<DT, D, CAUSAL>), dim3((unsigned)(a.B * a.Hq * nqt2)),
                     dim3(kDqDsThreads), 0, stream, (const uint16_t*)a.k, (const uint16_t*)a.ds,
                     (uint16_t*)a.dq, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.ds_row_blocks, a.scale);
  return hipGetLastError();
}

hipError_t launch_bwd_ds(const BwdArgs& a, hipStream_t stream) {
#define MI355_BWD_DS_CASE(DTV, DV)                                              \
  if (a.dtype == DTV && a.d == DV) {                                            \
    return a.causal ? launch_bwd_ds_t<DTV, DV, true>(a, stream)                 \
                    : launch_bwd_ds_t<DTV, DV, false>(a, stream);               \
  }
  MI355_BWD_DS_CASE(kBF16, 128)
  MI355_BWD_DS_CASE(kBF16, 64)
  MI355_BWD_DS_CASE(kFP16, 128)
  MI355_BWD_DS_CASE(kFP16, 64)
#undef MI355_BWD_DS_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_noalloc(const BwdArgs& args, hipStream_t stream) {
  BwdArgs a = args;
  hipError_t e = bwd_scratch(&a.delta);
  if (e != hipSuccess) return e;
  return launch_bwd(a, stream);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
#define MI355_BWD_CASE(DTV, DV)                                              \
  if (a.dtype == DTV && a.d == DV) {                                         \
    return a.causal ? launch_bwd_t<DTV, DV, true>(a, stream)                 \
                    : launch_bwd_t<DTV, DV, false>(a, stream);               \
  }
  MI355_BWD_CASE(kBF16, 128)
  MI355_BWD_CASE(kBF16, 64)
  MI355_BWD_CASE(kFP16, 128)
  MI355_BWD_CASE(kFP16, 64)
#undef MI355_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace mi355attn
