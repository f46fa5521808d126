// Attention backward for gfx950: dQ, dK, dV of O = softmax(scale * Q K^T) V
// for an upstream gradient dO.
//
// What is computed: the pages keep only the per-row softmax statistics from
// the forward and recompute the score and probability tiles in the backward
// instead of storing P ("IO-aware tiling strategy in FlashAttention-4", the
// backward-pass paragraph; "Reverse engineering Flash Attention 4's
// proprietary fused attention kernel", point 2).  With the forward's LSE
// (natural log of the softmax denominator) each probability is recomputed
// directly, P_ij = exp(scale * q_i.k_j - LSE_i), and the gradient of the row
// softmax needs one more per-row number, D_i = dO_i . O_i (which equals
// sum_j P_ij dP_ij):
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//     dQ = scale * dS K,  dK = scale * dS^T Q,
// with a K/V head's dK and dV summed over the query heads that share it.
//
// Design (MI355X-first):
//  * bwd_prep_kernel: D and the LSE in log2 units (+inf for rows that see no
//    key, so that their recomputed probabilities are exactly 0), one pass over
//    O and dO.
//  * bwd_dkdv_pair_kernel: one workgroup = 8 waves = 128 keys of one (batch,
//    K/V head), two waves per SIMD sharing 32 keys: one keeps their K
//    fragments and the dV accumulators (S, P, dV += P^T dO), the other their
//    V fragments and the dK accumulators (dP, then dS = P (dP - D) and
//    dK += dS^T Q a step later, with P passed through LDS as fp16).  The
//    workgroup walks every query head of the group and every 64-row query
//    block that can see its keys; Q, dO, LSE and D blocks are copied HBM ->
//    LDS by the buffer unit (buffer_load ... lds) into a ring of three, one
//    block ahead.  The GQA sum stays inside the workgroup, so there are no
//    atomics and the result is deterministic.
//  * bwd_dq_kernel: one workgroup = 4 waves = 128 query rows of one (batch,
//    query head); each wave keeps its rows' Q and dO fragments and fp32 dQ
//    accumulators in registers, and the 64-key K/V tiles stream through
//    double-buffered LDS the same way.  S and dP are recomputed here rather
//    than exchanged between the kernels.
//  * All products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  S
//    and dP come out of the MFMA with one key (dK/dV kernel) or one query row
//    (dQ kernel) per lane column, so their accumulator registers, rounded to
//    bf16, are directly the A operand of the next product (the k-slot order of
//    the accumulator rows is used as the contraction order); the other
//    operand of that product is read column-wise from the row-major LDS tile
//    with the gfx950 transpose read (ds_read_b64_tr_b16).
//  * LDS rows are 256 B with an XOR swizzle of their 16-byte chunks so that
//    both the row reads and the transpose reads spread over the banks.
//  * Both main kernels run two waves per SIMD, so one wave's exponentials and
//    operand reads run beside the other's MFMAs.
//  * blockIdx is remapped so that workgroups reading the same Q/dO (or K/V)
//    run on one XCD and share its L2; causal dQ blocks are dispatched
//    heaviest first.  Packed sequences (PACKED variants) spread the heads of
//    a sequence over the XCDs instead, so that long sequences do not all land
//    on one.
//  * ALIBI variants add the ALiBi bias -slope * |i + Sk - Sq - j| to the
//    exponent of each recomputed probability (the bias does not depend on Q,
//    K or V, so nothing else changes).
#include "gfx950.hpp"
#include "kernels.h"

namespace attn {
namespace {

constexpr int NW = 4;                 // waves per workgroup
constexpr int NT = NW * 64;
constexpr int KV_ROWS = NW * 32;      // keys per dK/dV workgroup
constexpr int QB = 64;                // query rows per step of the dK/dV loop
constexpr int Q_ROWS = NW * 32;       // query rows per dQ workgroup
constexpr int KB = 64;                // keys per step of the dQ loop
constexpr uint32_t kRsrcFlags = 0x00020000;

static_assert(kBwdKvRows == KV_ROWS && kBwdQRows == Q_ROWS, "layout assumed below");

// Sizes that follow from the head dim D (64 or 128) of bf16 rows in LDS.
template <int D>
struct BG {
  static constexpr int RB = 2 * D;        // bytes per row
  static constexpr int NC = D / 8;        // 16-byte chunks per row
  static constexpr int TILE = 64 * RB;    // one 64-row tile
  static constexpr int KS = D / 16;       // MFMA k-steps over d
  static constexpr int NTD = D / 32;      // 32-wide d blocks
  static constexpr int RPI = 1024 / RB;   // rows per 1 KB copy instruction
  static constexpr int CPW = 64 / RPI / NW;   // copy instructions per wave per tile
  static_assert(D == 64 || D == 128, "head dims 64 and 128");
};

// Chunk swizzle of a row: rows r and r + 4k land in different 4-chunk groups
// (16-chunk rows) or chunk pairs (8-chunk rows), and the 4 rows of one
// transpose read in different chunks.
template <int NC>
__device__ __forceinline__ int swz(int r) {
  if constexpr (NC == 8) return ((r & 3) << 1) | ((r >> 2) & 1);
  else return ((r & 3) << 2) | ((r >> 2) & 3);
}
// byte offset of 16-byte chunk c of row `row` in a tile
template <int D>
__device__ __forceinline__ int tile_off(int row, int c) {
  return row * BG<D>::RB + ((c ^ swz<BG<D>::NC>(row & 15)) << 4);
}
// byte offset of element `col` (a multiple of 4) of row `row`
template <int D>
__device__ __forceinline__ int elem_off(int row, int col) {
  return tile_off<D>(row, col >> 3) + ((col & 7) << 1);
}

__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int per = n >> 3;
  return (i < (per << 3)) ? (i & 7) * per + (i >> 3) : i;
}

// vmcnt(0) lgkmcnt(0): this wave's LDS copies have landed and its LDS reads
// are done.
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0x0070); }
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D>
__device__ __forceinline__ bf16x8 lds_row(const char* tile, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(tile + tile_off<D>(row, chunk));
}

// B operand of a product whose contraction runs over tile rows: lane
// (c = lane%32, h = lane/32) needs column `col0 + c` of the 8 rows
// rbase + 4h + {0..3} and rbase + 8 + 4h + {0..3}, in that k-slot order (the
// row order of a 32x32 accumulator's registers 0..7 in a lane half).  Two
// transpose reads: in each 16-lane group lane j gets element j%4 of the
// 4-element row addressed by lane 4e + j/4 (e = 0..3), so lane L of the
// group addresses row rbase + 4h + L/4 at column col0 + 16*((lane/16)%2) +
// 4*(L%4).
template <int D>
__device__ __forceinline__ bf16x8 lds_cols(const char* tile, int rbase, int col0, int lane) {
  const int L = lane & 15;
  const int row = rbase + 4 * (lane >> 5) + (L >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (L & 3);
  const bf16x4 lo = lds_read_tr(tile + elem_off<D>(row, col));
  const bf16x4 hi = lds_read_tr(tile + elem_off<D>(row + 8, col));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// 8 fp32 accumulator values -> bf16 A operand (round to nearest even)
__device__ __forceinline__ bf16x8 to_bf16x8(const float* x) {
  u32x4 u = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
             pack_bf16(x[6], x[7])};
  return __builtin_bit_cast(bf16x8, u);
}

// Asynchronous copy of 16 rows (this wave's share of a 64-row tile) from
// HBM into LDS: each buffer_load_dwordx4 ... lds moves 1 KB (RPI rows), lane i
// landing at byte 16*i, i.e. row +i/NC and physical chunk i%NC, so it fetches
// the logical chunk the swizzle puts there.  Rows past the buffer's range
// read 0.
template <int D>
struct RowCopy {
  static constexpr int RPI = BG<D>::RPI, NC = BG<D>::NC, CPW = BG<D>::CPW;
  uint32_t voff[CPW];
  int row0;
  __device__ void init(int64_t row_stride, int wave, int lane) {
    row0 = 16 * wave;
    const uint32_t ss = (uint32_t)(row_stride * 2);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int row = row0 + RPI * j + lane / NC;
      voff[j] = (uint32_t)row * ss + (uint32_t)(((lane % NC) ^ swz<NC>(row & 15)) << 4);
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, char* tile, uint32_t base) const {
#pragma unroll
    for (int j = 0; j < CPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (ATTN_LDS void*)(tile + (row0 + RPI * j) * BG<D>::RB), 16, voff[j] + base, 0, 0, 0);
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcFlags);
}

// Workgroups are dealt to the 8 XCDs round robin (XCD = i % 8).  Index i of
// a row of B*Hq workgroups goes to K/V head group (i % 8) + 8 * (i / 8 / G),
// query head (i / 8) % G of that group: the G query heads of a group share an
// XCD, consecutive groups (the K/V heads of one sequence) do not.  Needs the
// group count to be a multiple of 8, else i is kept.
__device__ __forceinline__ int spread_groups(int i, int G, int n_groups) {
  if (n_groups & 7) return i;
  const int x = i & 7, j = i >> 3;
  return (x + 8 * (j / G)) * G + (j - (j / G) * G);
}

// One sequence's sizes and offsets: the whole batch entry b, or (packed
// sequences) rows cu_q[b] .. cu_q[b+1]-1 and cu_k[b] .. cu_k[b+1]-1, offsets
// clamped to the packed sizes and lengths to the longest ones.  Row i of query
// head hq has its LSE and workspace values at row0 + hq * hstride + i.
struct SeqView {
  int Sq, Sk;
  int64_t qbase, kbase;   // element offsets of row 0 in q/o/dout/dq and k/v/dk/dv
  int64_t row0, hstride;
};
template <bool PACKED>
__device__ __forceinline__ SeqView seq_view(const BwdArgs& a, int b) {
  SeqView v;
  if (PACKED) {
    const int q_lo = min(max(a.cu_q[b], 0), a.total_q);
    const int q_hi = min(max(a.cu_q[b + 1], q_lo), a.total_q);
    const int k_lo = min(max(a.cu_k[b], 0), a.total_k);
    const int k_hi = min(max(a.cu_k[b + 1], k_lo), a.total_k);
    v.Sq = min(q_hi - q_lo, a.Sq);
    v.Sk = min(k_hi - k_lo, a.Sk);
    v.qbase = (int64_t)q_lo * a.q_ss;
    v.kbase = (int64_t)k_lo * a.k_ss;
    v.row0 = q_lo;
    v.hstride = a.total_q;
  } else {
    v.Sq = a.Sq;
    v.Sk = a.Sk;
    v.qbase = b * a.q_sb;
    v.kbase = b * a.k_sb;
    v.row0 = (int64_t)b * a.Hq * a.Sq;
    v.hstride = a.Sq;
  }
  return v;
}

}  // namespace

// ---- D = rowsum(dO * O) and LSE in log2 units --------------------------------
// D/8 lanes per row, 8 elements per lane (16 rows per workgroup at d = 128,
// 32 at d = 64).
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  constexpr int LPR = D / 8, RPW = 256 / LPR;
  // packed sequences: all total_q rows as one batch entry ([Hq, total_q])
  const int rows = a.cu_q ? a.total_q : a.Sq;
  const int row = blockIdx.x * RPW + threadIdx.x / LPR;
  const int hq = blockIdx.y, b = blockIdx.z;
  const int ch = threadIdx.x % LPR;
  float s = 0.f;
  if (row < rows) {
    const int64_t off = b * a.q_sb + hq * a.q_sh + (int64_t)row * a.q_ss + ch * 8;
    const bf16x8 o8 = *reinterpret_cast<const bf16x8*>(a.o + off);
    const bf16x8 d8 = *reinterpret_cast<const bf16x8*>(a.dout + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf((float)o8[e], (float)d8[e], s);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m, LPR);
  if (ch == 0 && row < rows) {
    const int64_t i = ((int64_t)b * a.Hq + hq) * rows + row;
    a.ws_d[i] = s;
    const float l = a.lse[i];
    a.ws_l[i] = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
}

// Per-lane LDS offsets of the operand reads of a 64-row tile.  The swizzle
// only XORs the 16-byte chunk index with a function of (row % 16), so for rows
// r32 + c (r32 a multiple of 32) and 16-row groups r16 + ... the offsets of
// other k-steps and d blocks follow from one base by an XOR, plus the row
// offset as an immediate:
//   lds_row(tile, r32 + c, 2*ks + h)  = tile + (row ^ (ks << 5)) + r32 * RB
//   lds_cols(tile, r16, 32*n, lane)   = transposed reads at
//                                       tile + (col[x] ^ (n << 6)) + r16 * RB
template <int D>
struct TileAddr {
  int row, col[2];
  __device__ void init(int lane) {
    const int c = lane & 31, h = lane >> 5, L = lane & 15;
    row = tile_off<D>(c, h);
    const int r = 4 * h + (L >> 2);
    const int cc = 16 * ((lane >> 4) & 1) + 4 * (L & 3);
    col[0] = elem_off<D>(r, cc);
    col[1] = elem_off<D>(r + 8, cc);
  }
  __device__ __forceinline__ bf16x8 row_op(const char* tile, int r32, int ks) const {
    return *reinterpret_cast<const bf16x8*>(tile + (row ^ (ks << 5)) + r32 * BG<D>::RB);
  }
  __device__ __forceinline__ bf16x8 col_op(const char* tile, int r16, int n) const {
    const bf16x4 lo = lds_read_tr(tile + (col[0] ^ (n << 6)) + r16 * BG<D>::RB);
    const bf16x4 hi = lds_read_tr(tile + (col[1] ^ (n << 6)) + r16 * BG<D>::RB);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
};

// Walk over the steps of a K/V workgroup: query head hl of the group (local
// index) and query block qb, advanced without divisions.
struct StepPos {
  int hl, qb;
  __device__ __forceinline__ void next(int qb_first, int qb_end) {
    if (++qb == qb_end) {
      qb = qb_first;
      ++hl;
    }
  }
};

// ---- dK, dV with a pair of waves per 32 keys ---------------------------------
// One workgroup = 8 waves = 128 keys of one (batch, K/V head), two waves per
// SIMD.  Waves w and w + 4 (one SIMD) share the keys kw0 .. kw0+31 and split
// the four products of a 64-row query block between them:
//  * the first (role 0) keeps the keys' K fragments and the dV accumulators:
//    S = Q K^T, P = exp2(S*c - L) (masked), P to LDS as fp16, dV += P^T dO;
//  * the second (role 1) keeps the V fragments and the dK accumulators:
//    dP = dO V^T, and one step later (when P of that block is in LDS)
//    dS = P (dP - D), dK += dS^T Q.
// Each wave's VALU work runs beside the other's MFMAs on the shared SIMD, and
// the register budget of two waves per SIMD holds either half (K or V
// fragments, one accumulator set).  Q, dO, L and D blocks go through a ring of
// three LDS buffers (the second role reads block s-1 while block s+1 is
// copied); P goes through two.  One barrier per step.

// Copy of 8 rows (this wave's share of a 64-row tile, 8 waves) from HBM into
// LDS, laid out as RowCopy lays out 16.
template <int D>
struct RowCopy8 {
  static constexpr int RPI = BG<D>::RPI, NC = BG<D>::NC, CPW = 8 / RPI;
  static_assert(CPW >= 1 && CPW * RPI == 8, "8 rows per wave");
  uint32_t voff[CPW];
  int row0;
  __device__ void init(int64_t row_stride, int wave, int lane) {
    row0 = 8 * wave;
    const uint32_t ss = (uint32_t)(row_stride * 2);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int row = row0 + RPI * j + lane / NC;
      voff[j] = (uint32_t)row * ss + (uint32_t)(((lane % NC) ^ swz<NC>(row & 15)) << 4);
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, char* tile, uint32_t base) const {
#pragma unroll
    for (int j = 0; j < CPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (ATTN_LDS void*)(tile + (row0 + RPI * j) * BG<D>::RB), 16, voff[j] + base, 0, 0, 0);
  }
};

template <int D, bool CAUSAL, bool PACKED, bool ALIBI>
__global__ __launch_bounds__(2 * NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_pair_kernel(BwdArgs a) {
  constexpr int TILE = BG<D>::TILE, KS = BG<D>::KS, NTD = BG<D>::NTD;
  constexpr int NB = 3;                         // Q / dO / L / D ring
  constexpr int PSUB = 2 * 64 * 16;             // one sub-block of P: 64 lanes x 32 B
  __shared__ __attribute__((aligned(1024))) char qbuf[NB * TILE];
  __shared__ __attribute__((aligned(1024))) char dobuf[NB * TILE];
  __shared__ __attribute__((aligned(1024))) char pbuf[2 * NW * 2 * PSUB];   // [step&1][pair][sub-block]
  __shared__ __attribute__((aligned(16))) float lbuf[NB * QB];
  __shared__ __attribute__((aligned(16))) float dbuf[NB * QB];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;   // 8 waves
  const int role = wave >> 2, w4 = wave & 3;
  const int c = lane & 31, h = lane >> 5;
  const int n_kb = (a.Sk + KV_ROWS - 1) / KV_ROWS;
  int bg, kb;
  if (PACKED) {
    const int BG_ = a.B * a.Hkv;
    kb = blockIdx.x / BG_;
    bg = blockIdx.x - kb * BG_;
  } else {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    bg = L / n_kb;
    kb = L - bg * n_kb;
  }
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const SeqView sv = seq_view<PACKED>(a, b);
  const int Sq = sv.Sq, Sk = sv.Sk;
  const int k0 = kb * KV_ROWS;
  if (k0 >= Sk) return;                 // whole workgroup: past this sequence's keys
  const int kw0 = k0 + 32 * w4;         // this pair's first key
  const int off = Sk - Sq;

  // K (role 0) or V (role 1) fragments of the pair's keys: B operand of
  // S = Q K^T or dP = dO V^T (lane: key kw0 + c, head-dim slots 16*ks + 8*h)
  bf16x8 kvf[KS];
  {
    const __bf16* src = (role == 0 ? a.k : a.v) + sv.kbase + g * a.k_sh;
    const int key = kw0 + c;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kvf[ks] = key < Sk ? *reinterpret_cast<const bf16x8*>(src + (int64_t)key * a.k_ss + 16 * ks +
                                                            8 * h)
                         : bf16x8{};
  }

  const int qstart = CAUSAL ? max(0, k0 - off) : 0;
  const int qb_first = qstart / QB;
  const int n_qb = (Sq + QB - 1) / QB;
  const int per_head = n_qb - qb_first;
  const int total = a.group * per_head;

  RowCopy8<D> cp;
  cp.init(a.q_ss, wave, lane);
  TileAddr<D> ta;
  ta.init(lane);
  const uint32_t q_bytes = Sq > 0 ? (uint32_t)((int64_t)(Sq - 1) * a.q_ss * 2 + BG<D>::RB) : 0u;
  const uint32_t blk_bytes = (uint32_t)(QB * a.q_ss * 2);
  auto issue = [&](const StepPos& sp, int st) {
    const int hq = g * a.group + sp.hl;
    const int qb = sp.qb;
    const int64_t hoff = sv.qbase + hq * a.q_sh;
    cp.issue(rsrc(a.q + hoff, q_bytes), qbuf + st * TILE, (uint32_t)qb * blk_bytes);
    cp.issue(rsrc(a.dout + hoff, q_bytes), dobuf + st * TILE, (uint32_t)qb * blk_bytes);
    if (wave < 2) {
      const float* src = (wave == 0 ? a.ws_l : a.ws_d) + sv.row0 + hq * sv.hstride;
      float* dst = (wave == 0 ? lbuf : dbuf) + st * QB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(src, (uint32_t)Sq * 4), (ATTN_LDS void*)dst,
                                               4, (uint32_t)(qb * QB + lane) * 4, 0, 0, 0);
    }
  };
  // which 32-row sub-blocks of step s's query block see some of the pair's
  // keys, and whether any of their entries needs the mask
  const int qb_end = qb_first + per_head;
  auto active = [&](int q0, int qs) {
    return kw0 < Sk && !(CAUSAL && kw0 > q0 + 32 * qs + 31 + off);
  };
  auto masked = [&](int q0, int qs) {
    const int r0 = q0 + 32 * qs;
    return (CAUSAL && kw0 + 31 > r0 + off) || (kw0 + 32 > Sk);
  };
  // this lane's 32 bytes of sub-block qs of P in buffer `pb`: two 16-byte
  // halves, each contiguous over the 64 lanes (no bank conflicts)
  auto p_slot = [&](int pb, int qs) { return pbuf + ((pb * NW + w4) * 2 + qs) * PSUB + 16 * lane; };

  f32x16 acc[NTD];                      // dV (role 0) or dK (role 1)
#pragma unroll
  for (int n = 0; n < NTD; ++n) acc[n] = f32x16{};

  // positions of the current step and of the next (the one being copied)
  StepPos cur{0, qb_first}, nxt = cur;
  nxt.next(qb_first, qb_end);
  if (total > 0) issue(cur, 0);
  // The two roles run separate loops (so that neither holds the other's
  // registers) with the same barriers: total + 1 steps, one barrier each.
  if (role == 0) {
    for (int s = 0, st = 0; s <= total; ++s, st = (st == NB - 1) ? 0 : st + 1) {
      wait_all();
      barrier();   // block s's copies are visible; P of step s-2 has been read
      if (s + 1 < total) issue(nxt, st == NB - 1 ? 0 : st + 1);
      if (s >= total) continue;
      const int q0 = cur.qb * QB;
      const float alibi2 = ALIBI ? -a.alibi[g * a.group + cur.hl] * kLog2e : 0.f;
      const float ad0 = (float)(q0 + 4 * h + off - (kw0 + c));
      const char* qt = qbuf + st * TILE;
      const char* dt = dobuf + st * TILE;
      const float* lb = lbuf + st * QB;
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        if (!active(q0, qs)) continue;
        bf16x8 qa[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[ks] = ta.row_op(qt, 32 * qs, ks);
        f32x4 l4[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          l4[q4] = *reinterpret_cast<const f32x4*>(lb + 32 * qs + 8 * q4 + 4 * h);
        f32x16 sacc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sacc = mfma32(qa[ks], kvf[ks], sacc);
        // P = exp2(S*c - L), masked entries 0 (register r: row
        // q0 + 32*qs + 8*(r/4) + 4h + r%4, key kw0 + c)
        const bool msk = masked(q0, qs);
        const int row0 = q0 + 32 * qs + 4 * h, key = kw0 + c;
        float pv[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * q4 + i;
            float e = sacc[r] * a.c - l4[q4][i];
            if (ALIBI)
              e = __builtin_fmaf(alibi2, __builtin_fabsf(ad0 + 32.f * qs + (float)(8 * q4 + i)), e);
            float x = fast_exp2(e);
            if (msk) {
              const int row = row0 + 8 * q4 + i;
              if (key >= Sk || (CAUSAL && key > row + off)) x = 0.f;
            }
            pv[r] = x;
          }
        // P for the partner (fp16: dS = P (dP - D) is rounded to bf16 after,
        // so the fp16 rounding of P is far below the result's precision)
        char* ps = p_slot(s & 1, qs);
        *reinterpret_cast<u32x4*>(ps) = u32x4{pack_f16(pv[0], pv[1]), pack_f16(pv[2], pv[3]),
                                              pack_f16(pv[4], pv[5]), pack_f16(pv[6], pv[7])};
        *reinterpret_cast<u32x4*>(ps + 64 * 16) =
            u32x4{pack_f16(pv[8], pv[9]), pack_f16(pv[10], pv[11]), pack_f16(pv[12], pv[13]),
                  pack_f16(pv[14], pv[15])};
        // dV += P^T dO
        const bf16x8 pa[2] = {to_bf16x8(pv), to_bf16x8(pv + 8)};
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int n = 0; n < NTD; ++n)
            acc[n] = mfma32(pa[t], ta.col_op(dt, 32 * qs + 16 * t, n), acc[n]);
      }
      cur = nxt;
      nxt.next(qb_first, qb_end);
    }
  } else {
    f32x16 dp[2];                       // dP of the previous step's sub-blocks
    dp[0] = f32x16{};
    dp[1] = f32x16{};
    int prev_q0 = 0;
    for (int s = 0, st = 0; s <= total; ++s, st = (st == NB - 1) ? 0 : st + 1) {
      wait_all();
      barrier();   // block s's copies and P of step s-1 are visible
      if (s + 1 < total) issue(nxt, st == NB - 1 ? 0 : st + 1);
      if (s >= 1) {
        // finish step s-1: dS = P (dP - D), dK += dS^T Q
        const int q0 = prev_q0;
        const int stp = st == 0 ? NB - 1 : st - 1;
        const char* qt = qbuf + stp * TILE;
        const float* db = dbuf + stp * QB;
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
          if (!active(q0, qs)) continue;
          const char* ps = p_slot((s - 1) & 1, qs);
          const u32x4 p0 = *reinterpret_cast<const u32x4*>(ps);
          const u32x4 p1 = *reinterpret_cast<const u32x4*>(ps + 64 * 16);
          f32x4 d4[4];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            d4[q4] = *reinterpret_cast<const f32x4*>(db + 32 * qs + 8 * q4 + 4 * h);
          float dsv[16];
#pragma unroll
          for (int r2 = 0; r2 < 8; ++r2) {
            const uint32_t u = r2 < 4 ? p0[r2] : p1[r2 - 4];
            const f16x2 hp = __builtin_bit_cast(f16x2, u);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int r = 2 * r2 + e;
              dsv[r] = (float)hp[e] * (dp[qs][r] - d4[r >> 2][r & 3]);
            }
          }
          const bf16x8 da[2] = {to_bf16x8(dsv), to_bf16x8(dsv + 8)};
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int n = 0; n < NTD; ++n)
              acc[n] = mfma32(da[t], ta.col_op(qt, 32 * qs + 16 * t, n), acc[n]);
        }
      }
      if (s < total) {
        // dP = dO V^T of step s
        const int q0 = cur.qb * QB;
        const char* dt = dobuf + st * TILE;
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
          if (!active(q0, qs)) continue;
          bf16x8 oa[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) oa[ks] = ta.row_op(dt, 32 * qs, ks);
          f32x16 pacc = f32x16{};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) pacc = mfma32(oa[ks], kvf[ks], pacc);
          dp[qs] = pacc;
        }
        prev_q0 = q0;
        cur = nxt;
        nxt.next(qb_first, qb_end);
      }
    }
  }

  // register r of lane (c, h), d block n: key kw0 + 8*(r/4) + 4h + r%4, dim 32n + c
  __bf16* dst = (role == 0 ? a.dv : a.dk) + sv.kbase + g * a.k_sh;
  const float mul = role == 0 ? 1.f : a.scale;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = kw0 + 8 * (r >> 2) + 4 * h + (r & 3);
    if (key < Sk) {
#pragma unroll
      for (int n = 0; n < NTD; ++n) dst[(int64_t)key * a.k_ss + 32 * n + c] = (__bf16)(acc[n][r] * mul);
    }
  }
}

// ---- dQ --------------------------------------------------------------------
// Two workgroups per CU (two waves per SIMD, 64 KB of LDS each): one wave's
// exponentials and operand reads run under the other's MFMAs.
template <int D, bool CAUSAL, bool PACKED, bool ALIBI>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdArgs a) {
  constexpr int TILE = BG<D>::TILE, KS = BG<D>::KS, NTD = BG<D>::NTD;
  __shared__ __attribute__((aligned(1024))) char kbuf[2 * TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf[2 * TILE];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 31, h = lane >> 5;
  const int n_qb = (a.Sq + Q_ROWS - 1) / Q_ROWS;
  const int BH = a.B * a.Hq;
  int bh, qb;
  if (CAUSAL || PACKED) {
    const int row = blockIdx.x / BH;      // heaviest query blocks first
    qb = n_qb - 1 - row;
    // packed sequences: the heads of one sequence spread over the XCDs
    bh = PACKED ? spread_groups(blockIdx.x - row * BH, a.group, a.B * a.Hkv)
                : xcd_remap(blockIdx.x - row * BH, BH);
  } else {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    bh = L / n_qb;
    qb = L - bh * n_qb;
  }
  const int b = bh / a.Hq, hq = bh - b * a.Hq;
  const int g = hq / a.group;
  const SeqView sv = seq_view<PACKED>(a, b);
  const int Sq = sv.Sq, Sk = sv.Sk;
  const int q0 = qb * Q_ROWS;
  if (q0 >= Sq) return;                   // whole workgroup: past this sequence's rows
  const int off = Sk - Sq;
  const int qw0 = q0 + 32 * wave;         // this wave's first row
  const int q = qw0 + c;                  // this lane's row (both halves)

  // Q and dO fragments of the wave's rows: B operand of S^T = K Q^T and of
  // dP^T = V dO^T (lane: row q, head-dim slots 16*ks + 8*h .. +7)
  const int64_t qoff = sv.qbase + hq * a.q_sh;
  bf16x8 qf[KS], df[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (q < Sq) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(a.q + qoff + (int64_t)q * a.q_ss + 16 * ks + 8 * h);
      df[ks] = *reinterpret_cast<const bf16x8*>(a.dout + qoff + (int64_t)q * a.q_ss + 16 * ks + 8 * h);
    } else {
      qf[ks] = bf16x8{};
      df[ks] = bf16x8{};
    }
  }
  const int64_t srow = sv.row0 + hq * sv.hstride;
  const float l2 = q < Sq ? a.ws_l[srow + q] : INFINITY;
  const float drow = q < Sq ? a.ws_d[srow + q] : 0.f;
  const float alibi2 = ALIBI ? -a.alibi[hq] * kLog2e : 0.f;   // -slope * log2(e)

  const int last_row = min(q0 + Q_ROWS, Sq) - 1;
  const int n_keys = CAUSAL ? min(Sk, max(0, last_row + off + 1)) : Sk;
  const int n_kt = (n_keys + KB - 1) / KB;
  const int wave_last = min(qw0 + 31, Sq - 1);

  RowCopy<D> cp;
  cp.init(a.k_ss, wave, lane);
  TileAddr<D> ta;
  ta.init(lane);
  const __bf16* kp = a.k + sv.kbase + g * a.k_sh;
  const __bf16* vp = a.v + sv.kbase + g * a.k_sh;
  const uint32_t k_bytes = Sk > 0 ? (uint32_t)((int64_t)(Sk - 1) * a.k_ss * 2 + BG<D>::RB) : 0u;
  const __amdgpu_buffer_rsrc_t rk = rsrc(kp, k_bytes), rv = rsrc(vp, k_bytes);
  const uint32_t blk_bytes = (uint32_t)(KB * a.k_ss * 2);

  f32x16 dq[NTD];
#pragma unroll
  for (int n = 0; n < NTD; ++n) dq[n] = f32x16{};

  if (n_kt > 0) {
    cp.issue(rk, kbuf, 0);
    cp.issue(rv, vbuf, 0);
  }
  for (int t = 0; t < n_kt; ++t) {
    const int st = t & 1;
    wait_all();
    barrier();
    if (t + 1 < n_kt) {
      cp.issue(rk, kbuf + (st ^ 1) * TILE, (uint32_t)(t + 1) * blk_bytes);
      cp.issue(rv, vbuf + (st ^ 1) * TILE, (uint32_t)(t + 1) * blk_bytes);
    }
    const char* kt = kbuf + st * TILE;
    const char* vt = vbuf + st * TILE;
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      const int kr0 = t * KB + 32 * ks2;
      if (kr0 >= n_keys || qw0 >= Sq) continue;
      if (CAUSAL && kr0 > wave_last + off) continue;   // no row of the wave sees these keys
      const bool mask = (CAUSAL && kr0 + 31 > qw0 + off) || (kr0 + 32 > Sk);
      // S^T[key][q] and dP^T[key][q]: register r of lane (c, h) holds key
      // kr0 + 8*(r/4) + 4h + r%4 against this lane's row q
      // K rows are read as one batch, and the V rows go out before the S^T
      // MFMAs so that they arrive under them
      bf16x8 ka[KS], va[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ka[ks] = ta.row_op(kt, 32 * ks2, ks);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) va[ks] = ta.row_op(vt, 32 * ks2, ks);
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc = mfma32(ka[ks], qf[ks], sacc);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) pacc = mfma32(va[ks], df[ks], pacc);
      float ds[16];
      // ALiBi distance row + off - key of register 0
      const float ad0 = (float)(q + off - kr0 - 4 * h);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = sacc[r] * a.c - l2;
        if (ALIBI)
          e = __builtin_fmaf(alibi2, __builtin_fabsf(ad0 - (float)(8 * (r >> 2) + (r & 3))), e);
        float pv = fast_exp2(e);
        if (mask) {
          const int key = kr0 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key >= Sk || (CAUSAL && key > q + off)) pv = 0.f;
        }
        ds[r] = pv * (pacc[r] - drow);
      }
      // dQ[q][d] += sum_key dS[q][key] K[key][d]
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 da = to_bf16x8(ds + 8 * u);
#pragma unroll
        for (int n = 0; n < NTD; ++n)
          dq[n] = mfma32(da, ta.col_op(kt, 32 * ks2 + 16 * u, n), dq[n]);
      }
    }
  }

  // register r of lane (c, h), d block n: row qw0 + 8*(r/4) + 4h + r%4, dim 32n + c
  __bf16* dqp = a.dq + qoff;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = qw0 + 8 * (r >> 2) + 4 * h + (r & 3);
    if (row < Sq) {
#pragma unroll
      for (int n = 0; n < NTD; ++n) dqp[(int64_t)row * a.q_ss + 32 * n + c] = (__bf16)(dq[n][r] * a.scale);
    }
  }
}

hipError_t launch_backward(const BwdArgs& a, bool causal, hipStream_t stream) {
  const int rows = a.cu_q ? a.total_q : a.Sq;
  const int rpw = a.D == 64 ? 32 : 16;   // rows per workgroup of the row-term kernel
  const int64_t n_prep = ((int64_t)rows + rpw - 1) / rpw;
  const int prep_b = a.cu_q ? 1 : a.B;
  const int64_t g_kv = (int64_t)a.B * a.Hkv * ((a.Sk + KV_ROWS - 1) / KV_ROWS);
  const int64_t g_q = (int64_t)a.B * a.Hq * ((a.Sq + Q_ROWS - 1) / Q_ROWS);
  if (n_prep > 0x7fffffff || a.Hq > 65535 || a.B > 65535 || g_kv > 0x7fffffff ||
      g_q > 0x7fffffff || (a.D != 64 && a.D != 128) || (a.D == 64 && (a.cu_q || a.alibi)))
    return hipErrorInvalidValue;
  const dim3 gp((unsigned)n_prep, a.Hq, prep_b), gk((unsigned)g_kv), gq((unsigned)g_q), bt(NT),
      bt2(2 * NT);
  const bool packed = a.cu_q != nullptr;
  if (a.D == 64) {
    hipLaunchKernelGGL((bwd_prep_kernel<64>), gp, dim3(256), 0, stream, a);
    if (causal) {
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<64, true, false, false>), gk, bt2, 0, stream, a);
      hipLaunchKernelGGL((bwd_dq_kernel<64, true, false, false>), gq, bt, 0, stream, a);
    } else {
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<64, false, false, false>), gk, bt2, 0, stream, a);
      hipLaunchKernelGGL((bwd_dq_kernel<64, false, false, false>), gq, bt, 0, stream, a);
    }
  } else if (packed) {
    hipLaunchKernelGGL((bwd_prep_kernel<128>), gp, dim3(256), 0, stream, a);
    if (causal) {
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<128, true, true, false>), gk, bt2, 0, stream, a);
      hipLaunchKernelGGL((bwd_dq_kernel<128, true, true, false>), gq, bt, 0, stream, a);
    } else {
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<128, false, true, false>), gk, bt2, 0, stream, a);
      hipLaunchKernelGGL((bwd_dq_kernel<128, false, true, false>), gq, bt, 0, stream, a);
    }
  } else if (a.alibi) {
    hipLaunchKernelGGL((bwd_prep_kernel<128>), gp, dim3(256), 0, stream, a);
    if (causal) {
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<128, true, false, true>), gk, bt2, 0, stream, a);
      hipLaunchKernelGGL((bwd_dq_kernel<128, true, false, true>), gq, bt, 0, stream, a);
    } else {
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<128, false, false, true>), gk, bt2, 0, stream, a);
      hipLaunchKernelGGL((bwd_dq_kernel<128, false, false, true>), gq, bt, 0, stream, a);
    }
  } else if (causal) {
    hipLaunchKernelGGL((bwd_prep_kernel<128>), gp, dim3(256), 0, stream, a);
    hipLaunchKernelGGL((bwd_dkdv_pair_kernel<128, true, false, false>), gk, bt2, 0, stream, a);
    hipLaunchKernelGGL((bwd_dq_kernel<128, true, false, false>), gq, bt, 0, stream, a);
  } else {
    hipLaunchKernelGGL((bwd_prep_kernel<128>), gp, dim3(256), 0, stream, a);
    hipLaunchKernelGGL((bwd_dkdv_pair_kernel<128, false, false, false>), gk, bt2, 0, stream, a);
    hipLaunchKernelGGL((bwd_dq_kernel<128, false, false, false>), gq, bt, 0, stream, a);
  }
  return hipGetLastError();
}

// Every kernel variant the launch above uses, instantiated explicitly (the
// host pass otherwise left some of them without their launch stubs).
template __global__ void bwd_prep_kernel<64>(BwdArgs);
template __global__ void bwd_prep_kernel<128>(BwdArgs);
#define ATTN_BWD_VARIANT(D, C, P, A)                                   \
  template __global__ void bwd_dkdv_pair_kernel<D, C, P, A>(BwdArgs); \
  template __global__ void bwd_dq_kernel<D, C, P, A>(BwdArgs);
ATTN_BWD_VARIANT(64, true, false, false)
ATTN_BWD_VARIANT(64, false, false, false)
ATTN_BWD_VARIANT(128, true, true, false)
ATTN_BWD_VARIANT(128, false, true, false)
ATTN_BWD_VARIANT(128, true, false, true)
ATTN_BWD_VARIANT(128, false, false, true)
ATTN_BWD_VARIANT(128, true, false, false)
ATTN_BWD_VARIANT(128, false, false, false)
#undef ATTN_BWD_VARIANT

}  // namespace attn
