// Attention forward on FP8 (OCP E4M3) Q, K, V for gfx950.
//
// The pages name FP8 inputs only in passing: the FP8 handling of the
// Blackwell kernel falls back to FP16 on ROCm ("Engineering the
// FlashAttention-4 kernel port to ROCm", HIP migration section), and FP8 cuts
// HBM bytes where the hardware has it ("IO-aware tiling strategy in
// FlashAttention-4", monitoring paragraph).  gfx950 has both: the inputs stay
// E4M3 in HBM and in LDS (half the bytes of bf16), Q.K^T runs on the FP8
// matrix core, and V is widened to fp16 for P.V.
//
// What is computed is the online softmax of "IO-aware tiling strategy in
// FlashAttention-4" (body) on the descaled values: S = scale * dq * dk * Q K^T
// (Q, K the E4M3 byte values), O = softmax(S) V * dv.  The products of two
// E4M3 values are exact in fp32 and v_mfma_f32_32x32x64_f8f6f4 accumulates
// them in fp32, so the scores are those of the exactly widened inputs.
// Probabilities are rounded to fp16 for P.V (v_mfma_f32_32x32x16_f16), and
// l sums the same rounded values, as in the bf16 path.
//
// Design: the bf16 kernel's two phase-shifted wave groups (prefill.hip), with
//  * K and V tiles of 64 keys x 128 bytes copied HBM -> LDS by buffer_load
//    ... lds (16 B per lane), rows XOR-swizzled in 16-byte chunks
//    (chunk c of row r stored at c ^ ((r >> 1) & 7)), so that 16 lanes
//    reading one chunk of 16 consecutive rows hit 64 different banks;
//  * S^T = K Q^T on v_mfma_f32_32x32x64_f8f6f4: four MFMAs per 64-key tile
//    (two 32-key blocks x two 64-deep steps) instead of sixteen bf16 ones;
//    the A operand (32 bytes of one key row per lane) comes straight from
//    the fp8 K tile, the B operand (Q) stays in registers.  The score tile
//    has the layout of the bf16 kernel's, so the softmax is the same code;
//  * the V^T tile (fp16) built by the copying wave from the fp8 V rows it
//    copied: ds_read_b64_tr_b8 gives each lane the eight keys of one column
//    in MFMA k-slot order, v_cvt_scalef32_pk_f16_fp8 widens them exactly
//    (scale 1; E4M3 values are all fp16 values), one 16-byte LDS write per
//    lane;
//  * no bf16 rerun: every E4M3 value is finite and within the fp16 range.
//    The E4M3 NaN encoding (s.1111.111) widens to NaN, which then reaches
//    the rows it touches; finite inputs are the contract.
#include "gfx950.hpp"
#include "kernels.h"

namespace attn {
namespace {

constexpr int D = kHeadDim;
constexpr int BN = 64;                      // keys per tile
constexpr int BM = kFp8RowsPerBlock;        // 256 query rows per workgroup
constexpr int NW = 8;
constexpr int NT = NW * 64;
constexpr int ROWB = D;                     // bytes per fp8 K/V row
constexpr int T8 = BN * ROWB;               // 8 KB fp8 tile
constexpr int VT_BYTES = BN * D * 2;        // 16 KB fp16 V^T tile

static_assert(BM == NW * 32, "one 32-row block per wave");

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Byte offset of 16-byte chunk c (0..7) of row r inside an fp8 tile.
__device__ __forceinline__ int t8_off(int r, int c) { return r * ROWB + ((c ^ ((r >> 1) & 7)) << 4); }
// V^T tile: row d (128 bytes = 64 fp16 keys); chunk 2*kk + hi holds the 8 keys
// 16*kk + {4hi..4hi+3, 8+4hi..8+4hi+3} in the MFMA k-slot order of lane half
// hi, stored at chunk ^ ((d >> 1) & 7) (16 lanes reading one chunk of 16
// consecutive rows cover all 64 banks once).
__device__ __forceinline__ int vt_off(int d, int chunk) {
  return d * 128 + ((chunk ^ ((d >> 1) & 7)) << 4);
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // format 0 (E4M3) for both operands, no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// s_waitcnt through the intrinsic so the compiler's own tracking knows it
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_copies_and_lds() { __builtin_amdgcn_s_waitcnt(0x0070); }
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Copy of a copying wave's 16 rows (keys 16*w4 .. 16*w4+15) of one K or V
// tile: two buffer_load_dwordx4 ... lds of 1 KB, lane i of instruction j
// landing at byte 16*i of rows 16*w4 + 8*j .. +7, i.e. row +i/8, physical
// chunk i%8, so it fetches the logical chunk the swizzle puts there.
struct Loader {
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t voff[2];
  uint32_t tile_bytes;     // BN * row stride in bytes
  int row0;

  __device__ void init(const uint8_t* kp, const uint8_t* vp, int64_t k_ss, int Sk, int wave,
                       int lane) {
    const int w4 = wave & 3;
    const uint32_t ss = (uint32_t)k_ss;
    const uint32_t nrec = Sk > 0 ? (uint32_t)((int64_t)(Sk - 1) * ss + ROWB) : 0u;
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)kp, (short)0, (int)nrec, 0x00020000);
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)vp, (short)0, (int)nrec, 0x00020000);
    tile_bytes = ss * BN;
    row0 = 16 * w4;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = row0 + 8 * j + (lane >> 3);
      const int c = (lane & 7) ^ ((row >> 1) & 7);
      voff[j] = (uint32_t)row * ss + (uint32_t)c * 16;
    }
  }
  __device__ __forceinline__ void issue(const __amdgpu_buffer_rsrc_t& r, int tile, char* dst) const {
    const uint32_t base = (uint32_t)tile * tile_bytes;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (ATTN_LDS void*)(dst + (row0 + 8 * j) * ROWB), 16,
                                               voff[j] + base, 0, 0, 0);
  }
  __device__ __forceinline__ void issue_k(int tile, char* kt) const { issue(rk, tile, kt); }
  __device__ __forceinline__ void issue_v(int tile, char* vt) const { issue(rv, tile, vt); }
};

// Everything one wave carries through the tile loop.
struct Wave {
  i32x8 qf[2];         // Q fragments (B operand of S^T = K Q^T): 32 bytes of d per step
  f32x16 oacc[4];      // O^T accumulators, d blocks of 32
  f32x16 s[2];         // S^T of the current tile, two 32-key blocks
  u32x4 pf[2][2];      // packed fp16 probabilities of the current tile
  float m_use;         // running max in log2 units
  float lsum;          // this lane's part of the row sum
  int koff[2][2];      // K operand: [k-step][half of the 32 bytes] byte offsets (row l32)
  int vtoff[4];        // V^T operand offsets per k-step (d block 0)
  int first, last;     // the wave's query rows
  int l32, hi;
};

// One copying wave's share of the V^T tile: keys 16*kk .. 16*kk+15 (the rows
// it copied) for all 128 d, in two halves of 64 d.  Per ds_read_b64_tr_b8,
// in each 16-lane group lane j receives byte j%8 of the 8-byte rows addressed
// by lanes 2e + j/8 (e = 0..7, measured on the device): lane 2e + s addresses
// key 16kk + 4s + e + 4*(e >= 4), d0 .. d0+7, so lane j gets the 8 keys of
// half s = j/8 for column d0 + j%8 in k-slot order.
struct VTranspose8 {
  const char* vb;      // the fp8 V tile
  char* vtb;           // the V^T tile
  int kk, s, d_lane;
  int row_base, sw, gh, g8;
  i32x2 x[2];
  __device__ __forceinline__ VTranspose8(const char* v, char* vt, int wave, int lane) {
    vb = v;
    vtb = vt;
    kk = wave & 3;
    const int j = lane & 15, g = lane >> 4;
    const int e = j >> 1, sp = j & 1;             // this lane addresses key (half sp, slot e)
    const int key = 16 * kk + 4 * sp + e + ((e >= 4) ? 4 : 0);
    row_base = key * ROWB;
    sw = (key >> 1) & 7;
    gh = g >> 1;                                   // d0 = 32*m + 8*g: chunk 2*m + g/2,
    g8 = (g & 1) * 8;                              // byte 8*(g%2) of it
    s = j >> 3;                                    // this lane receives half s
    d_lane = 8 * g + (j & 7);                      // of column 32*m + d_lane
  }
  // address of this lane's 8-byte row for columns 32*m + 8*g .. +7
  __device__ __forceinline__ int addr(int m) const {
    return row_base + (((2 * m + gh) ^ sw) << 4) + g8;
  }
  __device__ __forceinline__ void read(int h) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      x[j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((ATTN_LDS i32x2*)(vb + addr(2 * h + j)));
  }
  __device__ __forceinline__ void write(int h) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int d = 32 * (2 * h + j) + d_lane;
      u32x4 y;
      y[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[j][0], 1.0f, false));
      y[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[j][0], 1.0f, true));
      y[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[j][1], 1.0f, false));
      y[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[j][1], 1.0f, true));
      *(u32x4*)(vtb + vt_off(d, 2 * kk + s)) = y;
    }
  }
  __device__ __forceinline__ void all() {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      read(h);
      write(h);
    }
  }
};

struct NoExtra {
  __device__ __forceinline__ void operator()(int, int) const {}
};

// MFMA operands are read from LDS as 16-byte fragments through one ring of
// DEPTH registers: fragment f < 8 is half f%2 of the K operand of key block
// f/4, 64-deep step (f/2)%2 (32 bytes of key row 32*kb + l32, d = 64*ks +
// 32*hi .. +31); fragment 8 + j is the V^T operand of P.V MFMA j.
constexpr int DEPTH = 4;
struct Prefetch {
  u32x4 fr[DEPTH];
};
__device__ __forceinline__ u32x4 k_frag(const Wave& w, const char* kt, int f) {
  const int kb = f >> 2, ks = (f >> 1) & 1, h = f & 1;
  return *(const u32x4*)(kt + kb * 32 * ROWB + w.koff[ks][h]);
}
__device__ __forceinline__ u32x4 vt_frag(const Wave& w, const char* vt, int j) {
  const int kk = j >> 2, db = j & 3;
  return *(const u32x4*)(vt + db * 32 * 128 + w.vtoff[kk]);
}
// the first DEPTH fragments of an MFMA phase that starts with Q.K, issued by
// the caller before the barrier that opens it
__device__ __forceinline__ void prefetch_k(Prefetch& pf, const Wave& w, const char* kt) {
#pragma unroll
  for (int f = 0; f < DEPTH; ++f) pf.fr[f] = k_frag(w, kt, f);
}

// MFMA phase of a wave: S^T = K Q^T for this tile (4 fp8 MFMAs of two
// fragments each), then O^T += V^T P^T for the previous tile (16 fp16
// MFMAs).  Fragment reads run DEPTH fragments ahead of their MFMAs
// (sched_barrier pins the order).
template <bool QK, bool PV, bool PREFETCHED, class Extra>
__device__ __forceinline__ void mfma_seq(Wave& w, Prefetch& pf, const char* kt,
                                         const char* vt_prev, Extra&& extra) {
  constexpr int NQF = QK ? 8 : 0;                // K fragments
  constexpr int NF = NQF + (PV ? 16 : 0);        // all fragments
  constexpr int NQ = QK ? 4 : 0;                 // Q.K MFMAs
  constexpr int N = NQ + (PV ? 16 : 0);          // all MFMAs
  auto load = [&](int f) -> u32x4 { return (f < NQF) ? k_frag(w, kt, f) : vt_frag(w, vt_prev, f - NQF); };
  if (QK) {
    w.s[0] = f32x16{};
    w.s[1] = f32x16{};
  }
  if (!PREFETCHED) {
#pragma unroll
    for (int f = 0; f < DEPTH; ++f) pf.fr[f] = load(f);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    if (i < NQ) {
      const int kb = i >> 1, ks = i & 1;
      const u32x4 lo = pf.fr[(2 * i) % DEPTH], hi = pf.fr[(2 * i + 1) % DEPTH];
      const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      w.s[kb] = mfma_fp8(a, w.qf[ks], w.s[kb]);
#pragma unroll
      for (int r = 0; r < 2; ++r)
        if (2 * i + r + DEPTH < NF) pf.fr[(2 * i + r) % DEPTH] = load(2 * i + r + DEPTH);
    } else {
      const int j = i - NQ, kk = j >> 2, db = j & 3;
      const int f = NQF + j;
      w.oacc[db] = mfma32(__builtin_bit_cast(f16x8, pf.fr[f % DEPTH]),
                          __builtin_bit_cast(f16x8, w.pf[kk >> 1][kk & 1]), w.oacc[db]);
      if (f + DEPTH < NF) pf.fr[f % DEPTH] = load(f + DEPTH);
    }
    __builtin_amdgcn_sched_barrier(0);
    extra(i, N);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <class Extra, class Alone>
__device__ __forceinline__ void mfma_phase(Wave& w, Prefetch& pf, const char* kt,
                                           const char* vt_prev, bool do_qk, bool do_pv,
                                           bool prefetched, Extra&& extra, Alone&& alone) {
  // raised priority: the other wave of this SIMD runs its softmax meanwhile
  __builtin_amdgcn_s_setprio(3);
  if (do_qk && do_pv) {
    if (prefetched)
      mfma_seq<true, true, true>(w, pf, kt, vt_prev, extra);
    else
      mfma_seq<true, true, false>(w, pf, kt, vt_prev, extra);
  } else if (do_qk) {
    if (prefetched)
      mfma_seq<true, false, true>(w, pf, kt, vt_prev, extra);
    else
      mfma_seq<true, false, false>(w, pf, kt, vt_prev, extra);
  } else if (do_pv) {
    mfma_seq<false, true, false>(w, pf, kt, vt_prev, extra);
  } else {
    alone();
  }
  __builtin_amdgcn_s_setprio(0);
}

// Probabilities of the tile in w.s against the running max (log2 units),
// packed to fp16 for the next MFMA phase; returns this lane's sum of the
// rounded values.
__device__ __forceinline__ float probs(Wave& w, float c, float msub) {
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
  for (int i = 0; i < 16; ++i) u[i] = pack_f16(x[2 * i], x[2 * i + 1]);
  __builtin_amdgcn_sched_barrier(0);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i & 3] = sum2_f16(u[i], acc[i & 3]);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) w.pf[kb][e][i] = u[4 * (2 * kb + e) + i];
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Softmax phase for the tile whose scores are in w.s (keys kbase ..): mask,
// probabilities against the running max while the lane's tile sum stays
// <= 2^12 (every value then far from the fp16 limit; O = sum p v / sum p does
// not depend on the max), else take the row max, rescale and redo the tile.
template <bool CAUSAL>
__device__ __forceinline__ void softmax_phase(Wave& w, int kbase, int Sk, int off, float c) {
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
  float tsum = probs(w, c, w.m_use);
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
    tsum = probs(w, c, (m_new == -INFINITY) ? 0.f : m_new);
  }
  w.lsum += tsum;
}

struct Ctx {
  Loader ld;
  int n_tiles, Sk, off, wave, lane, group;
  float c;
};

// The phased tile loop of the bf16 kernel.  Phase 2t: group 0 runs the MFMA
// phase of tile t (Q.K of t, P.V of t-1), group 1 the softmax of tile t-1;
// phase 2t+1: group 0 the softmax of t, group 1 the MFMA phase of t.
//  * Group 1 copies K(t+1) and V(t) (fp8) at the start of phase 2t (no LDS
//    reads then) and waits for them before the mid barrier.  K(t+1) goes to
//    the K buffer last read in phase 2t-1; the V staging buffer was last read
//    in phase 2t-1.
//  * In phase 2t+1 each group-1 wave builds its 16 keys of V^T(t) (fp16) in
//    the V^T buffer last read in phase 2t-1, between the MFMAs of its MFMA
//    phase; V^T(t) is first read in phase 2t+2.
//  * Each group issues the first K-operand reads of its next MFMA phase at
//    the end of its softmax phase, when that K tile is already visible.
template <bool CAUSAL>
__device__ __forceinline__ void tile_loop(Wave& w, const Ctx& x, char* kbuf, char* vbuf,
                                          char* vtbuf) {
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
  if (T > 0 && !g0) x.ld.issue_k(0, kbuf);
  wait_copies_and_lds();
  barrier();
  bool pre = false;
  for (int t = 0; t <= T; ++t) {
    char* kt = kbuf + (t & 1) * T8;                   // K(t)
    char* knext = kbuf + ((t + 1) & 1) * T8;          // K(t+1)
    char* vtprev = vtbuf + ((t + 1) & 1) * VT_BYTES;  // V^T(t-1)
    char* vtcur = vtbuf + (t & 1) * VT_BYTES;         // V^T(t), built in phase 2t+1
    // ---- phase 2t
    if (g0) {
      mfma_phase(w, pf, kt, vtprev, visible(t), visible(t - 1), pre, NoExtra{}, [] {});
      pre = false;
    } else {
      if (t + 1 < T) x.ld.issue_k(t + 1, knext);
      if (t < T) x.ld.issue_v(t, vbuf);
      if (visible(t - 1)) softmax_phase<CAUSAL>(w, (t - 1) * BN, x.Sk, x.off, x.c);
      wait_copies();
      pre = visible(t);
      if (pre) prefetch_k(pf, w, kt);
    }
    barrier();   // K(t+1), V(t) copies have landed (group 1 waited for them)
    // ---- phase 2t+1
    if (g0) {
      if (visible(t)) softmax_phase<CAUSAL>(w, t * BN, x.Sk, x.off, x.c);
      pre = visible(t + 1);
      if (pre) prefetch_k(pf, w, knext);
    } else {
      VTranspose8 tr(vbuf, vtcur, x.wave, x.lane);
      const bool tr_now = t < T;
      mfma_phase(
          w, pf, kt, vtprev, visible(t), visible(t - 1), pre,
          [&](int i, int n) {
            if (!tr_now) return;
            if (i == 0) tr.read(0);
            if (i == n / 4) tr.write(0);
            if (i == n / 2) tr.read(1);
            if (i == (3 * n) / 4) tr.write(1);
          },
          [&] {
            if (tr_now) tr.all();
          });
      pre = false;
      wait_lds();  // the V^T(t) writes are done before they are published
    }
    barrier();
  }
}

template <bool CAUSAL>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_fp8_kernel(Fp8Args a) {
  // K (fp8, double buffered) at 0, V (fp8, as copied) at 16 KB, V^T (fp16,
  // double buffered) at 32 KB; the epilogue stages O in all 64 KB
  __shared__ __attribute__((aligned(1024))) char smem[64 * 1024];
  char* kbuf = smem;
  char* vbuf = smem + 2 * T8;
  char* vtbuf = smem + 32 * 1024;
  static_assert(2 * T8 + T8 <= 32 * 1024 && 32 * 1024 + 2 * VT_BYTES <= 64 * 1024, "LDS plan");

  Ctx x;
  const int tid = threadIdx.x;
  x.lane = tid & 63;
  // (left a per-lane value on purpose: with the wave index in a scalar
  // register the two groups' branches become scalar branches, and the
  // register allocation of the phase loop then spills heavily)
  x.wave = tid >> 6;
  x.group = x.wave >> 2;                 // waves 0-3 and 4-7: one of each per SIMD
  Wave w;
  w.l32 = x.lane & 31;
  w.hi = x.lane >> 5;
  const int lane = x.lane;

  // ---- which (batch, head, query tile) this workgroup computes
  const int BH = a.B * a.Hq;
  int bh, qt;
  if (CAUSAL && (BH & 7) == 0) {
    causal_xcd_order(blockIdx.x, BH, a.n_qt, bh, qt);
  } else if (CAUSAL) {
    const int row = blockIdx.x / BH;     // heaviest query tiles first
    qt = a.n_qt - 1 - row;
    const int i = blockIdx.x - row * BH, per = BH >> 3;
    bh = (i < (per << 3)) ? (i & 7) * per + (i >> 3) : i;
  } else {
    const int n = gridDim.x, per = n >> 3, i = blockIdx.x;
    const int L = (i < (per << 3)) ? (i & 7) * per + (i >> 3) : i;
    bh = L / a.n_qt;
    qt = L - bh * a.n_qt;
  }
  const int b = bh / a.Hq;
  const int hq = bh - b * a.Hq;
  const int hk = hq / a.group;
  const int Sq = a.Sq, Sk = a.Sk;
  const int q0 = qt * BM;
  const uint8_t* __restrict__ qp = a.q + b * a.q_sb + hq * a.q_sh;
  const uint8_t* kp = a.k + b * a.k_sb + hk * a.k_sh;
  const uint8_t* vp = a.v + b * a.k_sb + hk * a.k_sh;

  x.off = Sk - Sq;                       // causal: key j visible iff j <= i + off
  x.Sk = Sk;
  x.c = a.c;
  const int last_row = min(q0 + BM, Sq) - 1;
  int n_keys = Sk;
  if (CAUSAL) n_keys = min(Sk, max(0, last_row + x.off + 1));
  x.n_tiles = (n_keys + BN - 1) / BN;
  // 32-row blocks interleaved between the groups: SIMD s holds blocks 2s, 2s+1
  const int rb = 2 * (x.wave & 3) + x.group;
  w.first = q0 + 32 * rb;
  w.last = min(w.first + 31, Sq - 1);
  x.ld.init(kp, vp, a.k_ss, Sk, x.wave, lane);

  // ---- per-lane LDS offsets
  // K operand: row l32 of a 32-key block, chunks 4*ks + 2*hi and +1
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int h = 0; h < 2; ++h) w.koff[ks][h] = t8_off(w.l32, 4 * ks + 2 * w.hi + h);
  // V^T operand: row d = l32 (+ 32*db as an immediate), chunk 2*kk + hi
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) w.vtoff[kk] = vt_off(w.l32, 2 * kk + w.hi);

  // ---- Q fragments (E4M3 bytes): query row l32, d = 64*ks + 32*hi .. +31
  {
    const int row = w.first + w.l32;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (row < Sq) {
        const uint8_t* src = qp + (int64_t)row * a.q_ss + 64 * ks + 32 * w.hi;
        const u32x4 lo = *(const u32x4*)src;
        const u32x4 hi = *(const u32x4*)(src + 16);
        w.qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      } else {
        w.qf[ks] = i32x8{};
      }
    }
  }

  tile_loop<CAUSAL>(w, x, kbuf, vbuf, vtbuf);

  // ---- epilogue: O = acc / l * dv (bf16, RTNE) in q's layout;
  // LSE = ln(sum exp).  O is staged through the (then free) LDS so that each
  // global store writes whole 256-byte rows: lane (row l32, half hi) holds
  // d = 32 db + 8 j + 4 hi + e, i.e. 8 bytes of 16-byte chunk 4 db + j of its
  // row; each wave stages its 32 rows (8 KB) and reads back only its own.
  const float l = sum_halves(w.lsum);
  const int row = w.first + w.l32;
  const float inv = (l > 0.f) ? a.out_scale / l : 0.f;
  char* st = smem + x.wave * 8192;
  auto st_off = [](int r, int c) { return r * 256 + ((c ^ (((r & 3) << 2) | ((r >> 2) & 3))) << 4); };
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 u;
      u[0] = pack_bf16(w.oacc[db][4 * j + 0] * inv, w.oacc[db][4 * j + 1] * inv);
      u[1] = pack_bf16(w.oacc[db][4 * j + 2] * inv, w.oacc[db][4 * j + 3] * inv);
      *(u32x2*)(st + st_off(w.l32, 4 * db + j) + 8 * w.hi) = u;
    }
  wait_lds();
  __bf16* ob = a.o + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh;   // q's element strides
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int rr = 4 * k + (lane >> 4), cc = lane & 15;
    const u32x4 v = *(const u32x4*)(st + st_off(rr, cc));
    if (w.first + rr < Sq) *(u32x4*)(ob + (int64_t)(w.first + rr) * a.q_ss + 8 * cc) = v;
  }
  if (row < Sq && w.hi == 0) {
    const float lse = (l > 0.f) ? (w.m_use + __log2f(l)) * kLn2 : -INFINITY;
    a.lse[((int64_t)b * a.Hq + hq) * a.Sq + row] = lse;
  }
}

}  // namespace

hipError_t launch_prefill_fp8(const Fp8Args& a, bool causal, hipStream_t stream) {
  const int64_t n = (int64_t)a.B * a.Hq * a.n_qt;
  if (n <= 0 || n > 0x7fffffff) return hipErrorInvalidValue;
  if (causal)
    hipLaunchKernelGGL(prefill_fp8_kernel<true>, dim3((unsigned)n), dim3(NT), 0, stream, a);
  else
    hipLaunchKernelGGL(prefill_fp8_kernel<false>, dim3((unsigned)n), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
