// Fused exact attention forward for gfx950: O = softmax(scale * Q K^T) V.
//
// What is computed follows "IO-aware tiling strategy in FlashAttention-4"
// (body): Q is cut into row tiles and K/V into column tiles that are brought
// on chip, the score tile never leaves the chip, and each query row keeps a
// running max m and denominator l that are merged block by block
// (m' = max(m, m_new), l' = l * 2^(m - m') + l_new, with l_new summed against
// m'); the output accumulator is multiplied by the same per-row factor and
// divided by l once, at the end.
//
// Design (MI355X-first; the pages' NVIDIA and gfx942 kernels are prior art):
//  * one workgroup = 8 waves = 256 query rows of one (batch, query head),
//    two waves per SIMD.  Each wave owns 32 rows with its Q fragments and
//    fp32 output accumulators in registers (the MoonMath page's kernel keeps
//    Q and the accumulators in registers too).
//  * The waves form two groups (one wave of each per SIMD) that run the same
//    per-tile sequence half a tile apart, in phases separated by workgroup
//    barriers: while one group issues MFMAs (P.V of the previous tile, then
//    Q.K of this tile) the other runs the softmax of its current tile on the
//    VALU (the MoonMath page's two-group, phase-shifted eight-wave design,
//    re-derived here with both K and V in LDS).  A wave's own independent
//    VALU instructions also issue while its MFMAs execute, which the MFMA
//    phase uses for the V transpose; giving every wave both jobs instead
//    (softmax of tile t between its own Q.K MFMAs of tile t+1) measured
//    slower on this chip, its MFMAs then waiting on their LDS operand reads.
//  * K and V tiles of 64 keys are copied HBM -> LDS by the buffer unit
//    (buffer_load ... lds, 16 B per lane, 256 B per row), double buffered, one
//    tile ahead; keys past Sk fall outside the buffer range and read as zero.
//    Rows are 256 B with an XOR swizzle of their 16-byte chunks so the MFMA
//    operand reads are free of bank conflicts.
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16:
//    the accumulator holds one query row per lane (half of the keys in each
//    lane half), so the row max and sum are in-lane plus one
//    v_permlane32_swap, and the packed probabilities are already the B operand
//    of O^T = V^T P^T.  The V^T operand comes straight from the row-major V
//    tile through the gfx950 LDS transpose read (ds_read_b64_tr_b16).
//  * P.V runs in fp16 (11 significant bits; bf16 keeps 8, too few for the
//    parity bound when a few large V entries nearly cancel): each V tile is
//    converted to fp16 once in LDS by the lanes that copied it, and the
//    denominator sums the same rounded probabilities that multiply V.  A V
//    value outside the fp16 range (or a non-finite input) leaves a non-finite
//    accumulator; the workgroup then redoes its tiles with bf16 P and V,
//    which covers the whole bf16 range.
//  * The rescale of the output accumulator is skipped while the probabilities
//    of a tile, taken against the running max as it stands, sum to at most
//    2^12 per lane: each is then <= 4096, far from the fp16 and fp32 limits,
//    and the quotient O = sum p v / sum p is the same, so the result stays
//    exact.  A row's first tile, or a larger sum, takes the row max and
//    rescales.
//  * Causal: tiles above the diagonal are never loaded, waves whose rows see
//    none of a tile skip its arithmetic, only boundary tiles are masked, the
//    two groups hold interleaved 32-row blocks so they stay balanced on the
//    diagonal, and the heaviest query tiles are dispatched first.
//  * blockIdx is remapped so that workgroups sharing K/V land on one XCD
//    (workgroups are dealt to the 8 XCDs round robin), keeping K/V re-reads in
//    that XCD's L2; causal launches (head count a multiple of 8) also keep the
//    query tiles running at once on an XCD within one or two heads
//    (causal_xcd_order), so the tiles they stream are shared in L2.
//  * Packed sequences of different lengths (cu_q/cu_k offsets): a workgroup
//    reads its sequence's offsets first and returns at once if its query tile
//    lies past the sequence; the heads of one sequence are spread over the
//    XCDs (spread_groups) so the longest sequences do not share one XCD.
//  * ALiBi (ALIBI variants): the linear bias is added to the raw scores at
//    the start of each softmax phase, before the mask and the row max.  The
//    key tiles are taken from the one holding the workgroup's diagonal down
//    to key 0, then upward (causal: the last tile down to the first), so the
//    row max is found on the first tiles and the lazy rescale rarely runs.
#include "gfx950.hpp"
#include "kernels.h"

namespace attn {
namespace {

constexpr int D = kHeadDim;
constexpr int BN = kPrefillBN;
constexpr int BM = kPrefillBM;
constexpr int NW = kPrefillWaves;           // 8
constexpr int NT = NW * 64;                 // 512 threads
constexpr int TILE_BYTES = BN * D * 2;      // 16 KB for one K or V tile
constexpr int ROWS_PER_WAVE_DMA = BN / 4;   // 16 rows of each tile copied per group-1 wave

static_assert(kPrefillRowsPerWave == 32 && NW == 8 && BM == 256, "layout assumed below");

// 4-bit swizzle of a row index: a bijection on 0..15 that sends rows r and
// r+4k to different 4-chunk groups.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// Byte offset of 16-byte chunk c (0..15) of row `row` inside a tile.
__device__ __forceinline__ int tile_off(int row, int c) {
  return row * 256 + ((c ^ swz(row & 15)) << 4);
}

__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int per = n >> 3;
  return (i < (per << 3)) ? (i & 7) * per + (i >> 3) : i;
}

// Workgroups are dealt to the 8 XCDs round robin (XCD = i % 8).  Index i of
// a row of B*Hq workgroups goes to K/V head group (i % 8) + 8 * (i / 8 / G),
// query head (i / 8) % G of that group, so the G query heads of a group share
// an XCD (and its L2) and consecutive groups -- the K/V heads of one
// sequence -- land on different XCDs.  Needs the group count to be a
// multiple of 8, else i is kept.
__device__ __forceinline__ int spread_groups(int i, int G, int n_groups) {
  if (n_groups & 7) return i;
  const int x = i & 7, j = i >> 3;
  return (x + 8 * (j / G)) * G + (j - (j / G) * G);
}

// Asynchronous copy of a wave's 16 rows of one K or V tile from HBM into LDS.
// Each instruction moves 1 KB: lane i lands at byte 16*i, i.e. row +i/16,
// physical chunk i%16, so it fetches the logical chunk that the swizzle puts
// there.  Bytes past the buffer's end (nrec) read as zero.
struct TileLoader {
  u32x4 rk, rv;
  u32x4 rvt;              // prepared fp16 V^T tiles of this (batch, kv head)
  uint32_t voff[4];       // per-lane byte offset, rows 4*j + lane/16 of the wave's 16
  uint32_t tile_bytes;    // BN * row stride in bytes
  int row0;               // first tile row this wave copies
  uint32_t vt_off;        // this wave's quarter of a prepared tile, lane's 16 bytes

  __device__ void init(const __bf16* kp, const __bf16* vp, int64_t k_ss, int Sk, int wave,
                       int lane) {
    wave &= 3;
    const uint32_t ss = (uint32_t)(k_ss * 2);
    const uint32_t nrec = Sk > 0 ? (uint32_t)((int64_t)(Sk - 1) * ss + 256) : 0u;
    rk = buffer_rsrc(kp, nrec);
    rv = buffer_rsrc(vp, nrec);
    tile_bytes = ss * BN;
    row0 = ROWS_PER_WAVE_DMA * wave;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = row0 + 4 * j + (lane >> 4);
      const int c = (lane & 15) ^ swz(row & 15);
      voff[j] = (uint32_t)row * ss + (uint32_t)c * 16;
    }
  }
  __device__ __forceinline__ void issue_k(int tile, char* kt) const {
    const uint32_t base = (uint32_t)tile * tile_bytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_copy16(rk, voff[j] + base, kt + (row0 + 4 * j) * 256);
  }
  __device__ __forceinline__ void issue_v(int tile, char* vt) const {
    const uint32_t base = (uint32_t)tile * tile_bytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_copy16(rv, voff[j] + base, vt + (row0 + 4 * j) * 256);
  }
  // prepared tiles: the byte layout in HBM is the LDS one, so each wave
  // copies its 4 KB quarter of the 16 KB tile as it is
  __device__ void init_vt(const uint8_t* vtp, int n_kt, int wave, int lane) {
    rvt = buffer_rsrc(vtp, (uint32_t)n_kt * (uint32_t)kVtTileBytes);
    vt_off = (uint32_t)(wave & 3) * 4096u + (uint32_t)lane * 16u;
  }
  __device__ __forceinline__ void issue_vt(int tile, char* dst) const {
    const uint32_t base = (uint32_t)tile * (uint32_t)kVtTileBytes + vt_off;
    char* d = dst + (vt_off & ~1023u);
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_copy16(rvt, base + 1024u * j, d + 1024 * j);
  }
};

// s_waitcnt through the intrinsic, so the compiler's own wait tracking knows
// about it: vmcnt(0) (this wave's LDS copies have landed).
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// all but this wave's last n copies have landed (n = 0, 4 or 8: the copies
// of one tile step; vector memory loads complete in order)
__device__ __forceinline__ void wait_copies_but(int n) {
  if (n == 8)
    __builtin_amdgcn_s_waitcnt(0x0F78);
  else if (n == 4)
    __builtin_amdgcn_s_waitcnt(0x0F74);
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);
}
// lgkmcnt(0) only: this wave's LDS writes are done
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier without a hardware memory fence: every cross-wave LDS
// dependency in the loop is ordered by an explicit wait before it.  The empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// V^T tile: the P.V operand of lane (d = 32*db + lane%32, hi = lane/32) for
// k-step kk is the 8 keys 16*kk + {4hi..4hi+3, 8+4hi..8+4hi+3} of row d.
// V^T rows are 128 B (64 keys); the 16-byte chunk 2*kk + hi of row d holds
// exactly those 8 keys in k-slot order, at physical chunk
// (2*kk + hi) ^ ((d >> 1) & 7) so that 16 lanes reading one chunk hit 16
// different banks.
__device__ __forceinline__ int vt_off(int d, int chunk) {
  return d * 128 + ((chunk ^ ((d >> 1) & 7)) << 4);
}

// One wave's share of turning the bf16 V tile (row-major, as copied) into the
// V^T tile: k-step kk = wave%4, i.e. keys 16*kk .. 16*kk+15 -- exactly the 16
// rows this wave copied, so it only has to wait for its own copies -- for all
// four d blocks.
// Everything one wave carries through the tile loop.
struct Wave;
// Everything one wave carries through the tile loop.
struct Wave {
  bf16x8 qf[8];        // Q fragments: B operand of S^T = K Q^T (query = lane%32)
  f32x16 oacc[4];      // O^T accumulators, d blocks of 32
  f32x16 s[2];         // S^T of the current tile, two 32-key blocks
  u32x4 pf[2][2];      // packed probabilities of the current tile (B operand of P.V)
  float m_use;         // running max in log2 units (scale*log2e folded in)
  float lsum;          // this lane's part of the row sum
  int koff[8];         // LDS offsets of the K operand per 16-wide d step
  int vtoff[4];        // LDS offsets of the V^T operand per k-step (d block 0)
  int cvoff[2][4];     // transpose-read offsets into the bf16 V tile per d block
  int first, last;     // the wave's query rows
  int l32, hi;
};

// In two halves (d blocks 2h, 2h+1), each a read step and a write step, so
// that the MFMA wave can spread them between its MFMAs.
struct VTranspose {
  const char* base;    // this wave's 16 rows of the bf16 V tile
  char* vtb;           // the V^T tile
  int woff;
  bf16x8 x[2];
  __device__ __forceinline__ VTranspose(const Wave& w, const char* vb, char* vt, int wave) {
    const int kk = wave & 3;                        // not a compile-time index:
    woff = vt_off(w.l32, 2 * kk + w.hi);            // no indexing of w.vtoff
    base = vb + 16 * kk * 256;
    vtb = vt;
  }
  __device__ __forceinline__ void read(const Wave& w, int h) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bf16x4 lo = lds_read_tr(base + w.cvoff[0][2 * h + j]);
      const bf16x4 up = lds_read_tr(base + w.cvoff[1][2 * h + j]);
      x[j] = bf16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
    }
  }
  template <bool F16>
  __device__ __forceinline__ void write(int h) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 y = __builtin_bit_cast(u32x4, x[j]);
      if (F16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = bf16x2_to_f16x2(y[i]);
      }
      *(u32x4*)(vtb + (2 * h + j) * 32 * 128 + woff) = y;
    }
  }
  template <bool F16>
  __device__ __forceinline__ void all(const Wave& w) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      read(w, h);
      write<F16>(h);
    }
  }
};

struct NoExtra {
  __device__ __forceinline__ void operator()(int, int) const {}
};

// MFMA phase of a wave: S^T = K Q^T for this tile (16 MFMAs), then
// O^T += V^T P^T for the previous tile (16 MFMAs, k-step major so
// consecutive MFMAs feed different accumulators).  The LDS operand reads run
// DEPTH MFMAs ahead of their use (sched_barrier pins that order); the first
// DEPTH reads (K fragments) are issued by the caller before the barrier that
// opens the phase, so the matrix core starts as soon as the phase does.
constexpr int DEPTH = 4;
struct Prefetch {
  bf16x8 fr[DEPTH];
};

__device__ __forceinline__ bf16x8 k_operand(const Wave& w, const char* kt, int j) {
  const int ks = j >> 1, kb = j & 1;
  return *(const bf16x8*)(kt + kb * 32 * 256 + w.koff[ks]);
}
__device__ __forceinline__ bf16x8 vt_operand(const Wave& w, const char* vt, int j) {
  const int kk = j >> 2, db = j & 3;                 // k-step (kb, e) and d block
  return *(const bf16x8*)(vt + db * 32 * 128 + w.vtoff[kk]);
}
// the first DEPTH operands of an MFMA phase that starts with Q.K
__device__ __forceinline__ void prefetch_k(Prefetch& pf, const Wave& w, const char* kt) {
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) pf.fr[i] = k_operand(w, kt, i);
}

template <bool F16, bool QK, bool PV, bool PREFETCHED, class Extra>
__device__ __forceinline__ void mfma_seq(Wave& w, Prefetch& pf, const char* kt,
                                         const char* vt_prev, Extra&& extra) {
  constexpr int NQK = QK ? 16 : 0;
  constexpr int N = NQK + (PV ? 16 : 0);
  auto load = [&](int i) -> bf16x8 {
    return (i < NQK) ? k_operand(w, kt, i) : vt_operand(w, vt_prev, i - NQK);
  };
  auto mma = [&](int i, const bf16x8& f) {
    if (i < NQK) {
      const int ks = i >> 1, kb = i & 1;
      w.s[kb] = mfma32(f, w.qf[ks], w.s[kb]);
    } else {
      const int j = i - NQK, kk = j >> 2, db = j & 3;
      if (F16)
        w.oacc[db] = mfma32(__builtin_bit_cast(f16x8, f),
                            __builtin_bit_cast(f16x8, w.pf[kk >> 1][kk & 1]), w.oacc[db]);
      else
        w.oacc[db] = mfma32(f, __builtin_bit_cast(bf16x8, w.pf[kk >> 1][kk & 1]), w.oacc[db]);
    }
  };
  if (QK) {
    w.s[0] = f32x16{};
    w.s[1] = f32x16{};
  }
  if (!PREFETCHED) {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) pf.fr[i] = load(i);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    mma(i, pf.fr[i % DEPTH]);
    if (i + DEPTH < N) pf.fr[i % DEPTH] = load(i + DEPTH);
    __builtin_amdgcn_sched_barrier(0);
    extra(i, N);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// `extra(i, n)` runs after MFMA i of the n; if the wave has no MFMAs in the
// phase, `alone()` runs instead.
template <bool F16, class Extra, class Alone>
__device__ __forceinline__ void mfma_phase(Wave& w, Prefetch& pf, const char* kt,
                                           const char* vt_prev, bool do_qk, bool do_pv,
                                           bool prefetched, Extra&& extra, Alone&& alone) {
  // The other wave on this SIMD runs its softmax meanwhile; raised priority
  // keeps its VALU stream from delaying this wave's operand reads and MFMA
  // issue (the arbiter otherwise favours the older wave).
  __builtin_amdgcn_s_setprio(3);
  if (do_qk && do_pv) {
    if (prefetched)
      mfma_seq<F16, true, true, true>(w, pf, kt, vt_prev, extra);
    else
      mfma_seq<F16, true, true, false>(w, pf, kt, vt_prev, extra);
  } else if (do_qk) {
    if (prefetched)
      mfma_seq<F16, true, false, true>(w, pf, kt, vt_prev, extra);
    else
      mfma_seq<F16, true, false, false>(w, pf, kt, vt_prev, extra);
  } else if (do_pv) {
    mfma_seq<F16, false, true, false>(w, pf, kt, vt_prev, extra);
  } else {
    alone();
  }
  __builtin_amdgcn_s_setprio(0);
}

// Softmax phase of a wave for the tile whose scores are in w.s.  Fast path:
// probabilities against the current running max, packed for the next MFMA
// phase and summed (rounded values, four independent chains).  Every
// probability is <= this lane's partial tile sum, so if that sum stays below
// 2^12 none of them is near the fp16 limit and the running max may stay as it
// is (the quotient O = sum p v / sum p does not depend on it).  Otherwise (and
// for the first tile of a row) the slow path takes the row max, rescales the
// accumulators and recomputes the tile.
template <bool F16>
__device__ __forceinline__ float probs(Wave& w, float c, float msub) {
  // staged so that each stage is 16-32 independent instructions: the wave
  // runs beside another wave's MFMAs and cannot afford dependency stalls
  float x[32];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) x[16 * kb + r] = __builtin_fmaf(w.s[kb][r], c, -msub);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = fast_exp2(x[i]);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t u[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) u[i] = F16 ? pack_f16(x[2 * i], x[2 * i + 1]) : pack_bf16(x[2 * i], x[2 * i + 1]);
  __builtin_amdgcn_sched_barrier(0);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i & 3] = F16 ? sum2_f16(u[i], acc[i & 3]) : sum2_bf16(u[i], acc[i & 3]);
  // u[4*j .. 4*j+3] hold keys 8*(j) .. of s[kb][8e..8e+7] with j = 2*kb + e
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) w.pf[kb][e][i] = u[4 * (2 * kb + e) + i];
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

template <bool CAUSAL, bool F16, bool ALIBI>
__device__ __forceinline__ void softmax_phase(Wave& w, int kbase, int Sk, int off, float c,
                                              float alibi) {
  if constexpr (ALIBI) {
    // linear bias on the raw scores: alibi * |i + off - j| (alibi = -slope /
    // scale), one subtraction and one fma (|.| as a source modifier) per score
    const float d0 = (float)(w.first + w.l32 + off - kbase - 4 * w.hi);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float key = (float)(kb * 32 + 8 * (r >> 2) + (r & 3));
        w.s[kb][r] = __builtin_fmaf(alibi, __builtin_fabsf(d0 - key), w.s[kb][r]);
      }
  }
  const bool need_mask = (kbase + BN > Sk) || (CAUSAL && kbase + BN - 1 > w.first + off);
  if (need_mask) {
    const int row = w.first + w.l32;
    const int lim = (CAUSAL ? min(Sk - 1, row + off) : Sk - 1) - kbase - 4 * w.hi;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + (r & 3);
        if (key > lim) w.s[kb][r] = -INFINITY;
      }
  }
  float tsum = probs<F16>(w, c, w.m_use);
  const bool ok = (w.m_use != -INFINITY) && (tsum <= 4096.f);
  if (wave_any(!ok)) {
    float mx = w.s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, w.s[kb][r]);
    mx = max_halves(mx);
    const float m_new = fmaxf(w.m_use, mx * c);
    const float alpha = (m_new == w.m_use) ? 1.f : fast_exp2(w.m_use - m_new);
    w.lsum *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) w.oacc[db] *= alpha;
    w.m_use = m_new;
    tsum = probs<F16>(w, c, (m_new == -INFINITY) ? 0.f : m_new);
  }
  w.lsum += tsum;
}

struct Ctx {
  TileLoader ld;
  int n_tiles, Sk, off, wave, lane, group;
  int pivot;     // non-causal ALiBi: the key tile taken first (see tile_loop)
  float c;
  float alibi;   // -slope / scale of this head (ALiBi variants)
};

// The phased tile loop.  Phase 2t: group 0 runs the MFMA phase of tile t
// (Q.K of t, P.V of t-1), group 1 the softmax of tile t-1; phase 2t+1:
// group 0 the softmax of t, group 1 the MFMA phase of t.  The HBM copies are
// issued at the start of the softmax phases, split between the groups so
// that each side carries half of the issue time:
//  * group 1 copies K(t+2) at the start of phase 2t, one tile step ahead, and
//    before the mid barrier waits for K(t+1) (issued in phase 2t-2), so from
//    phase 2t+1 on it is visible to every wave.  K has three buffers: K(t+2)
//    goes to the one last read in phase 2t-1 (K(t-1)'s);
//  * group 0 copies V(t+1) at the start of phase 2t+1 and waits for it at
//    the end of its MFMA phase 2t+2, before the mid barrier of tile t+1.  V
//    has two staging buffers: V(t+1) goes to the one V(t-1) was transposed
//    from in phase 2t-1.
//  * In phase 2t+1 each group-1 wave transposes the 16 rows of V(t) it
//    copied into the V^T buffer last read in phase 2t-1 (V^T(t-2)'s),
//    converting to fp16, with the instructions spread between the MFMAs of
//    its MFMA phase (a wave's independent VALU instructions issue while its
//    own MFMAs execute, so this takes them off the softmax side of phase 2t);
//    V^T(t) is first read in phase 2t+2.
//  * Each group issues the first K-operand reads of its next MFMA phase at
//    the end of its softmax phase, when that K tile is already visible.
template <bool CAUSAL, bool F16, bool ALIBI>
__device__ __forceinline__ void tile_loop(Wave& w, const Ctx& x, char* kbuf, char* vbuf,
                                          char* vtbuf) {
#pragma unroll
  for (int db = 0; db < 4; ++db) w.oacc[db] = f32x16{};
  w.m_use = -INFINITY;
  w.lsum = 0.f;
  const int T = x.n_tiles;
  // Step t of the loop works on key tile key_tile(t).  With an ALiBi bias
  // the tiles go from the pivot (the tile of the diagonal, where the bias of
  // the workgroup's rows is largest) down to key 0, then up from the pivot:
  // the first tile sets the row max and later tiles rarely raise it (the
  // lazy rescale stays on its fast path); in key order the max of a row
  // would grow with nearly every tile up to its diagonal.
  const int pivot = CAUSAL ? T - 1 : x.pivot;
  auto key_tile = [&](int t) { return !ALIBI ? t : t <= pivot ? pivot - t : t; };
  auto visible = [&](int t) {
    return t >= 0 && t < T && w.first <= w.last && (!CAUSAL || key_tile(t) * BN <= w.last + x.off);
  };
  const bool g0 = x.group == 0;
  Prefetch pf;
  auto kslot = [&](int t) { return kbuf + (t % 3) * TILE_BYTES; };
  auto vslot = [&](int t) { return vbuf + (t & 1) * TILE_BYTES; };
  // copy of K(t) (group 1) or V(t) (group 0); returns how many copies were issued
  auto issue_kt = [&](int t) {
    if (t >= T) return 0;
    x.ld.issue_k(key_tile(t), kslot(t));
    return 4;
  };
  auto issue_vt = [&](int t) {
    if (t >= T) return 0;
    x.ld.issue_v(key_tile(t), vslot(t));
    return 4;
  };
  if (g0) {
    issue_vt(0);
    wait_copies();
  } else if (T > 0) {
    issue_kt(0);
    wait_copies_but(issue_kt(1));
  }
  wait_lds();
  barrier();
  bool pre = false;   // this wave holds the first operands of its next MFMA phase
  for (int t = 0; t <= T; ++t) {
    char* kt = kslot(t);                                // K(t)
    char* knext = kslot(t + 1);                         // K(t+1)
    char* vtprev = vtbuf + ((t + 1) & 1) * TILE_BYTES;  // V^T(t-1)
    char* vtcur = vtbuf + (t & 1) * TILE_BYTES;         // V^T(t), written in phase 2t+1
    // ---- phase 2t
    if (g0) {
      mfma_phase<F16>(w, pf, kt, vtprev, visible(t), visible(t - 1), pre, NoExtra{}, [] {});
      pre = false;
      wait_copies();                                    // V(t), copied in phase 2t-1
    } else {
      const int n_new = issue_kt(t + 2);
      if (visible(t - 1)) softmax_phase<CAUSAL, F16, ALIBI>(w, key_tile(t - 1) * BN, x.Sk, x.off,
                                                                   x.c, x.alibi);
      wait_copies_but(n_new);
      pre = visible(t);
      if (pre) prefetch_k(pf, w, kt);                   // K(t) is visible since phase 2t-1
    }
    barrier();   // K(t+1) (group 1) and V(t) (group 0) copies have landed
    // ---- phase 2t+1
    if (g0) {
      issue_vt(t + 1);
      if (visible(t))
        softmax_phase<CAUSAL, F16, ALIBI>(w, key_tile(t) * BN, x.Sk, x.off, x.c, x.alibi);
      pre = visible(t + 1);
      if (pre) prefetch_k(pf, w, knext);                // K(t+1) is visible since the mid barrier
    } else {
      // V(t) -> V^T(t) between the MFMAs (V(t) landed before the mid barrier)
      VTranspose tr(w, vslot(t), vtcur, x.wave);
      const bool tr_now = t < T;
      mfma_phase<F16>(
          w, pf, kt, vtprev, visible(t), visible(t - 1), pre,
          [&](int i, int n) {
            if (!tr_now) return;
            if (i == 1) tr.read(w, 0);
            if (i == n / 4 + 1) tr.write<F16>(0);
            if (i == n / 2) tr.read(w, 1);
            if (i == (3 * n) / 4) tr.write<F16>(1);
          },
          [&] {
            if (tr_now) tr.all<F16>(w);
          });
      pre = false;
      wait_lds();  // the V^T(t) writes are done before they are published
    }
    barrier();
  }
}

// The phased tile loop with prepared fp16 V^T tiles (no transpose): the same
// phases, and both groups run the plain MFMA phase.
//  * group 1 copies K(t+2) at the start of phase 2t and waits for K(t+1)
//    before the mid barrier, as above;
//  * group 0 copies V^T(t+1) at the start of phase 2t+1 and waits for V^T(t)
//    (copied in phase 2t-1) at its end, so that V^T(t) is visible from phase
//    2t+2, where it is first read.  V^T has three buffers: V^T(t+1) goes to
//    V^T(t-2)'s, last read in phase 2t-1.
// The three V^T buffers take the place of the V staging buffers and the
// first V^T buffer of the transposing loop (vtbuf3 = vbuf).
template <bool CAUSAL>
__device__ __forceinline__ void tile_loop_pre(Wave& w, const Ctx& x, char* kbuf, char* vtbuf3) {
#pragma unroll
  for (int db = 0; db < 4; ++db) w.oacc[db] = f32x16{};
  w.m_use = -INFINITY;
  w.lsum = 0.f;
  const int T = x.n_tiles;
  auto visible = [&](int t) {
    return t >= 0 && t < T && w.first <= w.last && (!CAUSAL || t * BN <= w.last + x.off);
  };
  const bool g0 = x.group == 0;
  Prefetch pf;
  auto kslot = [&](int t) { return kbuf + (t % 3) * TILE_BYTES; };
  auto vtslot = [&](int t) { return vtbuf3 + (t % 3) * TILE_BYTES; };
  auto issue_kt = [&](int t) {
    if (t >= T) return 0;
    x.ld.issue_k(t, kslot(t));
    return 4;
  };
  auto issue_vtt = [&](int t) {
    if (t >= T) return 0;
    x.ld.issue_vt(t, vtslot(t));
    return 4;
  };
  if (g0) {
    issue_vtt(0);
  } else if (T > 0) {
    issue_kt(0);
    wait_copies_but(issue_kt(1));
  }
  wait_lds();
  barrier();
  bool pre = false;   // this wave holds the first operands of its next MFMA phase
  for (int t = 0; t <= T; ++t) {
    char* kt = kslot(t);                                // K(t)
    char* knext = kslot(t + 1);                         // K(t+1)
    char* vtprev = vtslot(t + 2);                       // V^T(t-1): slot (t-1) % 3
    // ---- phase 2t
    if (g0) {
      mfma_phase<true>(w, pf, kt, vtprev, visible(t), visible(t - 1), pre, NoExtra{}, [] {});
      pre = false;
    } else {
      const int n_new = issue_kt(t + 2);
      if (visible(t - 1)) softmax_phase<CAUSAL, true, false>(w, (t - 1) * BN, x.Sk, x.off, x.c,
                                                                    0.f);
      wait_copies_but(n_new);
      pre = visible(t);
      if (pre) prefetch_k(pf, w, kt);                   // K(t) is visible since phase 2t-1
    }
    barrier();   // K(t+1) has landed (group 1 waited for it)
    // ---- phase 2t+1
    if (g0) {
      const int n_new = issue_vtt(t + 1);
      if (visible(t)) softmax_phase<CAUSAL, true, false>(w, t * BN, x.Sk, x.off, x.c, 0.f);
      pre = visible(t + 1);
      if (pre) prefetch_k(pf, w, knext);                // K(t+1) is visible since the mid barrier
      wait_copies_but(n_new);                           // V^T(t), copied in phase 2t-1
    } else {
      mfma_phase<true>(w, pf, kt, vtprev, visible(t), visible(t - 1), pre, NoExtra{}, [] {});
      pre = false;
    }
    barrier();
  }
}

__device__ __forceinline__ bool state_finite(const Wave& w) {
  bool ok = __builtin_isfinite(w.lsum);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) ok = ok && __builtin_isfinite(w.oacc[db][r]);
  return ok;
}

template <bool CAUSAL, bool ALIBI, bool PRE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillArgs a) {
  // K (three buffers), V as copied (bf16, two), V^T (fp16, two); with
  // prepared V^T tiles, their three buffers start at vbuf
  __shared__ __attribute__((aligned(1024))) char lds[7 * TILE_BYTES];
  char* const kbuf = lds;
  char* const vbuf = lds + 3 * TILE_BYTES;
  char* const vtbuf = lds + 5 * TILE_BYTES;

  Ctx x;
  const int tid = threadIdx.x;
  x.lane = tid & 63;
  x.wave = tid >> 6;
  x.group = x.wave >> 2;                 // waves 0-3 and 4-7: one of each per SIMD
  Wave w;
  w.l32 = x.lane & 31;
  w.hi = x.lane >> 5;
  const int lane = x.lane;

  // ---- which (batch, head, query tile) this workgroup computes
  const int BH = a.B * a.Hq;
  int bh, qt;
  if (CAUSAL && !a.cu_q && (BH & 7) == 0) {
    causal_xcd_order(blockIdx.x, BH, a.n_qt, bh, qt);
  } else if (CAUSAL || a.cu_q) {
    const int row = blockIdx.x / BH;     // heaviest query tiles first
    qt = a.n_qt - 1 - row;
    // packed sequences of different lengths: the heads of one sequence are
    // spread over the XCDs (a K/V head's query heads kept together), so that
    // no XCD is left with the longest sequences
    bh = a.cu_q ? spread_groups(blockIdx.x - row * BH, a.group, a.B * a.Hkv)
                : xcd_remap(blockIdx.x - row * BH, BH);
  } else {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    bh = L / a.n_qt;
    qt = L - bh * a.n_qt;
  }
  const int b = bh / a.Hq;
  const int hq = bh - b * a.Hq;
  const int hk = hq / a.group;
  // this sequence's rows: the whole [B, ...] batch entry, or (packed
  // sequences) rows cu_q[b] .. cu_q[b+1]-1 of q and cu_k[b] .. cu_k[b+1]-1 of
  // k/v, offsets clamped to the packed sizes
  int Sq = a.Sq, Sk = a.Sk;
  int64_t qbase = b * a.q_sb, kbase = b * a.k_sb;
  int64_t lse_base = (int64_t)(b * a.Hq + hq) * a.Sq;
  if (a.cu_q) {
    const int q_lo = min(max(a.cu_q[b], 0), a.total_q);
    const int q_hi = min(max(a.cu_q[b + 1], q_lo), a.total_q);
    const int k_lo = min(max(a.cu_k[b], 0), a.total_k);
    const int k_hi = min(max(a.cu_k[b + 1], k_lo), a.total_k);
    Sq = min(q_hi - q_lo, a.Sq);         // a.Sq is the longest query length here
    Sk = k_hi - k_lo;
    qbase = (int64_t)q_lo * a.q_ss;
    kbase = (int64_t)k_lo * a.k_ss;
    lse_base = (int64_t)hq * a.total_q + q_lo;
  }
  const int q0 = qt * BM;
  if (q0 >= Sq) return;                  // whole workgroup: past this sequence's rows
  const __bf16* __restrict__ qp = a.q + qbase + hq * a.q_sh;
  const __bf16* kp = a.k + kbase + hk * a.k_sh;
  const __bf16* vp = a.v + kbase + hk * a.k_sh;

  x.off = Sk - Sq;                       // causal: key j visible iff j <= i + off
  x.Sk = Sk;
  x.c = a.c;
  x.alibi = ALIBI ? -a.alibi[hq] * kLog2e / a.c : 0.f;
  const int last_row = min(q0 + BM, Sq) - 1;
  int n_keys = Sk;
  if (CAUSAL) n_keys = min(Sk, max(0, last_row + x.off + 1));
  x.n_tiles = (n_keys + BN - 1) / BN;
  // non-causal: the tile holding the diagonal key (i + off) of the
  // workgroup's middle row (the causal loop takes its last tile)
  const int mid_key = min(q0 + BM / 2, Sq - 1) + x.off;
  x.pivot = min(max(mid_key, 0) / BN, max(x.n_tiles - 1, 0));
  // 32-row blocks interleaved between the groups: SIMD s holds blocks 2s, 2s+1
  const int rb = 2 * (x.wave & 3) + x.group;
  w.first = q0 + 32 * rb;
  w.last = min(w.first + 31, Sq - 1);
  x.ld.init(kp, vp, a.k_ss, Sk, x.wave, lane);
  if (PRE) x.ld.init_vt(a.vt + (int64_t)(b * a.Hkv + hk) * a.n_kt * kVtTileBytes, a.n_kt, x.wave, lane);

  // ---- per-lane LDS offsets
  // K operand (A of S^T): row kb*32 + l32, chunk 2*ks + hi
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) w.koff[ks] = tile_off(w.l32, 2 * ks + w.hi);
  // V^T operand: row d = l32 (+ 32*db as an immediate), chunk 2*kk + hi
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) w.vtoff[kk] = vt_off(w.l32, 2 * kk + w.hi);
  // transpose reads of the bf16 V tile: lane (block beta = lane/16,
  // j = lane%16) addresses row 8*h + 4*hi + j/4 of a 16-key step, columns
  // 32*db + 16*(beta&1) + 4*(j%4); lane j of each 16-lane block receives 4
  // keys of column 32*db + 16*(beta&1) + j.  The swizzle only permutes
  // 16-byte chunks and d block db is chunks 4*db .. 4*db+3, so the offsets of
  // block db differ from block 0's by a lane-dependent XOR: kept per block.
  {
    const int j = lane & 15;
    const int chalf = (lane >> 4) & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * h + 4 * w.hi + (j >> 2);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int col = db * 32 + 16 * chalf + 4 * (j & 3);
        w.cvoff[h][db] = tile_off(r, col >> 3) + (col & 7) * 2;
      }
    }
  }

  // ---- Q fragments: row = query, k-slots = d
  {
    const int row = w.first + w.l32;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (row < Sq)
        w.qf[ks] = *(const bf16x8*)(qp + (int64_t)row * a.q_ss + 16 * ks + 8 * w.hi);
      else
        w.qf[ks] = bf16x8{};
    }
  }

  if (PRE)
    tile_loop_pre<CAUSAL>(w, x, kbuf, vbuf);
  else
    tile_loop<CAUSAL, true, ALIBI>(w, x, kbuf, vbuf, vtbuf);
  // A V value beyond the fp16 range (|v| >= 65520) or a non-finite input
  // shows up as a non-finite accumulator: redo this workgroup with bf16
  // probabilities and bf16 V, which covers the whole bf16 range.
  if (__syncthreads_or(!state_finite(w))) tile_loop<CAUSAL, false, ALIBI>(w, x, kbuf, vbuf, vtbuf);

  // ---- epilogue: O = acc / l (bf16 under the caller's rounding rule) in q's
  // layout; LSE = ln(sum exp)
  const float l = sum_halves(w.lsum);
  const int row = w.first + w.l32;
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  // O goes through LDS (the tile buffers are free: every wave is past the
  // last barrier of the tile loop) so that the global stores write whole
  // 256-byte rows, 16 bytes per lane.  Lane (row l32, half hi) holds
  // d = 32 db + 8 j + 4 hi + e, i.e. 8 bytes of 16-byte chunk 4 db + j of its
  // row; each wave stages its 32 rows (8 KB) with the tile swizzle and reads
  // back only its own rows.
  char* st = (x.wave < 4 ? kbuf : vtbuf) + (x.wave & 3) * 8192;
  with_rounding(a.rounding, [&](auto mode) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 u;
        u[0] = pack_bf16_as<mode()>(w.oacc[db][4 * j + 0] * inv, w.oacc[db][4 * j + 1] * inv);
        u[1] = pack_bf16_as<mode()>(w.oacc[db][4 * j + 2] * inv, w.oacc[db][4 * j + 3] * inv);
        *(u32x2*)(st + tile_off(w.l32, 4 * db + j) + 8 * w.hi) = u;
      }
  });
  wait_lds();
  __bf16* ob = a.o + qbase + hq * a.q_sh;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int rr = 4 * k + (lane >> 4), cc = lane & 15;
    const u32x4 v = *(const u32x4*)(st + tile_off(rr, cc));
    if (w.first + rr < Sq) *(u32x4*)(ob + (int64_t)(w.first + rr) * a.q_ss + 8 * cc) = v;
  }
  if (row < Sq && w.hi == 0) {
    const float lse = (l > 0.f) ? (w.m_use + __log2f(l)) * kLn2 : -INFINITY;
    a.lse[lse_base + row] = lse;
  }
}

// One prepared V^T tile of TK keys per workgroup of 256 threads: the TK x 128
// bf16 V tile (keys past Sk read as zero) is staged in LDS row by row, then
// each thread builds 16-byte chunks of V^T rows -- chunk c of row d holds the
// keys 16(c/2) + {4(c%2) .. +3, 8 + 4(c%2) .. +3}, the k-slots of k-step c/2
// for lane half c%2, as fp16 rounded to nearest even -- and writes them at
// their swizzled place: for TK = 64 the layout of this file's kernel (vt_off,
// 128-byte rows), for TK = 32 that of the GQA kernel (64-byte rows, chunk
// c ^ ((d >> 2) & 3)).  HBM-bound: TK * 256 bytes read and written per tile.
template <int TK>
__global__ __launch_bounds__(256) void prep_v_kernel(PrepVArgs a) {
  constexpr int RS = D + 8;                      // padded LDS row (bf16 elements)
  constexpr int CH = TK / 8;                     // 16-byte chunks per V^T row
  constexpr int PASSES = TK / 16;                // 256 threads x 16 bytes per pass
  __shared__ __attribute__((aligned(16))) __bf16 tile[TK * RS];
  const int64_t id = blockIdx.x;
  const int t = (int)(id % a.n_kt);
  const int64_t bh = id / a.n_kt;
  const int h = (int)(bh % a.Hkv);
  const int b = (int)(bh / a.Hkv);
  const __bf16* vp = a.v + b * a.k_sb + h * a.k_sh;
  const int tid = threadIdx.x;
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    const int r = 16 * pass + (tid >> 4), c = tid & 15;
    const int key = t * TK + r;
    u32x4 val = u32x4{0u, 0u, 0u, 0u};
    if (key < a.Sk) val = *(const u32x4*)(vp + (int64_t)key * a.k_ss + 8 * c);
    *(u32x4*)(tile + r * RS + 8 * c) = val;
  }
  __syncthreads();
  uint8_t* out = a.vt + id * (TK * D * 2);
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    const int idx = 256 * pass + tid;
    const int d = idx / CH, ch = idx % CH;
    const int k0 = 16 * (ch >> 1) + 4 * (ch & 1);
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (float)tile[(k0 + (j < 4 ? j : j + 4)) * RS + d];
    const u32x4 y = u32x4{pack_f16(f[0], f[1]), pack_f16(f[2], f[3]), pack_f16(f[4], f[5]),
                          pack_f16(f[6], f[7])};
    const int off = TK == 64 ? vt_off(d, ch) : d * 64 + ((ch ^ ((d >> 2) & 3)) << 4);
    *(u32x4*)(out + off) = y;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, bool causal, hipStream_t stream) {
  const int64_t grid = (int64_t)a.B * a.Hq * a.n_qt;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidValue;
  if (a.vt) {
    // prepared V^T tiles: dense batches without ALiBi
    if (a.alibi || a.cu_q || a.n_kt != (a.Sk + BN - 1) / BN) return hipErrorInvalidValue;
    if (causal)
      hipLaunchKernelGGL((prefill_kernel<true, false, true>), dim3((unsigned)grid), dim3(NT), 0,
                         stream, a);
    else
      hipLaunchKernelGGL((prefill_kernel<false, false, true>), dim3((unsigned)grid), dim3(NT), 0,
                         stream, a);
  } else if (a.alibi) {
    if (causal)
      hipLaunchKernelGGL((prefill_kernel<true, true, false>), dim3((unsigned)grid), dim3(NT), 0,
                         stream, a);
    else
      hipLaunchKernelGGL((prefill_kernel<false, true, false>), dim3((unsigned)grid), dim3(NT), 0,
                         stream, a);
  } else if (causal) {
    hipLaunchKernelGGL((prefill_kernel<true, false, false>), dim3((unsigned)grid), dim3(NT), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL((prefill_kernel<false, false, false>), dim3((unsigned)grid), dim3(NT), 0,
                       stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_prep_v(const PrepVArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.B * a.Hkv * a.n_kt;
  if (grid <= 0 || grid > 0x7fffffff || (a.tk != BN && a.tk != kPrefillPipeBN) ||
      a.n_kt != (a.Sk + a.tk - 1) / a.tk)
    return hipErrorInvalidValue;
  if (a.tk == BN)
    hipLaunchKernelGGL((prep_v_kernel<BN>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((prep_v_kernel<kPrefillPipeBN>), dim3((unsigned)grid), dim3(256), 0, stream,
                       a);
  return hipGetLastError();
}

}  // namespace attn
