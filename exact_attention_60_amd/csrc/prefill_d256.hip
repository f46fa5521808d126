// Exact attention forward at head dim 256 for gfx950, software-pipelined
// inside each wave: O = softmax(scale * Q K^T) V.
//
// What is computed follows "IO-aware tiling strategy in FlashAttention-4"
// (body): Q in row tiles, K/V in column tiles brought on chip, the score tile
// never leaving the chip, a running row max m and denominator l merged block
// by block and the output accumulator divided by l once at the end.  Head
// dims other than 128 are what the kernel of "MoonMath AI open-sources a HIP
// attention kernel for AMD MI300X that beats AITER v3" leaves out (scope
// paragraph: head dim fixed at 128).
//
// Design (gfx950):
//  * one workgroup = 4 waves, one per SIMD = 128 query rows of one (batch,
//    query head); a wave owns 32 rows.  At d = 256 the Q fragments (64
//    registers) and the fp32 O^T accumulator (128) alone fill the budget of
//    two waves per SIMD, so the wave takes the whole register file of its
//    SIMD and hides its latencies itself: the iteration for key tile t
//    issues the 16 MFMAs of O^T += V^T(t-1) P(t-1)^T, then the 16 MFMAs of
//    S(t+1) = K(t+1) Q^T, none of which depends on the iteration's VALU work
//    (the softmax of S(t), the conversion of V(t+1)), which sits between
//    them slot by slot.
//  * K and V tiles of 32 keys (rows of 512 bytes, 16 KB per tile) are copied
//    HBM -> LDS by buffer_load ... lds three tiles ahead (a K ring of 4, a V
//    ring of 3), each wave a quarter of the rows; 16-byte chunks are XOR-
//    swizzled by row (conflict-free MFMA operand and transposed reads); keys
//    past Sk fall outside the buffer range and read as zero.
//  * P.V runs in fp16: each wave turns two 32-wide d blocks of V(t+1) into
//    the fp16 V^T tile (ring of 3; row d holds the tile's 32 keys in MFMA
//    k-slot order) by transposed LDS reads (ds_read_b64_tr_b16); a V value
//    beyond the fp16 range or a non-finite input leaves a non-finite
//    accumulator and the workgroup redoes its tiles with bf16 P and V.
//  * With V prepared once per K/V head (prep_v_d256_kernel: fp16 V^T tiles
//    in HBM, laid out as the LDS tile) the copies bring V^T(t+2) into a ring
//    of 4 (V^T(t-1) .. V^T(t+2)) and there is no conversion; the results are
//    bit-identical to the converting path.  With both rings of 4 slots the
//    loop runs four iterations per pass, each with its ring slots fixed at
//    compile time, so that every LDS operand address is a per-lane register
//    plus an instruction offset.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 puts one query row in each lane
//    column, so the probabilities are directly the B operand of the P.V
//    MFMAs and the row sum is in-lane plus one v_permlane32_swap.
//  * Lazy rescale: probabilities are taken against the running max as it
//    stands while a tile's per-lane sum stays <= 2^12; a row's first tile or
//    a larger sum takes the row max and rescales (a slow path that
//    recomputes S(t) from the K tile still in its ring slot).
//  * Causal: tiles past the workgroup's last diagonal are never loaded, only
//    boundary tiles are masked, heaviest query blocks are dispatched first.
//  * LDS: K 4 x 16 KB + V 3 x 16 KB + V^T 3 x 16 KB = 160 KB (prepared: K 4
//    + V^T 4 = 128 KB of the same array), one workgroup per CU.
#include "gfx950.hpp"
#include "kernels.h"

namespace attn {
namespace {

constexpr int D = 256;
constexpr int BN = 32;          // keys per tile
constexpr int NW = 4;           // waves per workgroup, one per SIMD
constexpr int NT = NW * 64;
constexpr int QR = NW * 32;     // query rows per workgroup
constexpr int RB = D * 2;       // bytes per K or V row
constexpr int TB = BN * RB;     // one bf16 K or V tile (16 KB)
constexpr int VTB = D * BN * 2; // one fp16 V^T tile (16 KB)
constexpr int NK = 4;           // K ring: K(t) .. K(t+3)
constexpr int NV = 3;           // V ring: V(t+1) .. V(t+3)
constexpr int NVT = 3;          // V^T ring: V^T(t-1) .. V^T(t+1)
constexpr int NVP = 4;          // prepared V^T ring: V^T(t-1) .. V^T(t+2)
constexpr int AHEAD = 3;        // copies run this many tiles ahead
constexpr int COPIES = 8;       // copy instructions per wave per tile (4 K, 4 V)
constexpr int KS = D / 16;      // k-steps of S^T = K Q^T
constexpr int NDB = D / 32;     // 32-wide d blocks of O^T
static_assert(QR == kPrefillHdRows, "rows per workgroup");
static_assert(NK * TB + NV * TB + NVT * VTB <= 160 * 1024, "LDS plan");
static_assert(NVP * VTB <= NV * TB + NVT * VTB, "prepared V^T ring inside the V and V^T rings");
static_assert(VTB == kVtD256TileBytes && BN == kPrefillD256BN, "prepared tile format");

// 4-bit swizzle of a row index: a bijection on 0..15 that sends rows r and
// r+4k to different 4-chunk groups.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// Byte offset of 16-byte chunk c (0..31) of row `row` of a K or V tile; the
// swizzle changes the low four bits of c.
__device__ __forceinline__ int kv_off(int row, int c) {
  return row * RB + ((c ^ swz(row & 15)) << 4);
}
// V^T tile: row d (64 bytes) holds the 32 keys as 4 chunks; chunk 2*kk + hi
// holds the keys 16*kk + {4hi..4hi+3, 8+4hi..8+4hi+3}, the k-slot order of
// lane half hi in the P.V MFMA of key step kk.  The chunk index is XORed with
// bits 2-3 of d (16 lanes reading one chunk of 16 rows cover 64 banks once).
__device__ __forceinline__ int vt_off(int d, int chunk) {
  return d * 64 + ((chunk ^ ((d >> 2) & 3)) << 4);
}

__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int per = n >> 3;
  return (i < (per << 3)) ? (i & 7) * per + (i >> 3) : i;
}

// s_waitcnt vmcnt(N) lgkmcnt(0) through the intrinsic, so that the
// compiler's own tracking knows it.
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// Pins the instruction order: nothing is moved across it.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// Copies of one K and one V tile: this wave's 8 rows of each, 2 rows per
// 1 KB instruction.  Lane i of instruction j lands at byte 16*i of rows
// 8*wave + 2j, 2j+1, i.e. row + i/32, physical chunk i%32, so it fetches the
// logical chunk the swizzle puts there.  The copies are asm statements that
// the compiler does not track (lds_copy16_at); their completion is ordered by
// vmcnt waits and the workgroup barrier.
struct Loader {
  u32x4 rk, rv;
  uint32_t voff[4];
  uint32_t tile_bytes;
  uint32_t lds_k, lds_v;   // LDS address of this wave's first row in ring slot 0

  __device__ void init(const __bf16* kp, const __bf16* vp, int64_t k_ss, int Sk, int wave,
                       int lane, uint32_t kbuf_lds, uint32_t vbuf_lds) {
    const uint32_t ss = (uint32_t)(k_ss * 2);
    const uint32_t nrec = Sk > 0 ? (uint32_t)((int64_t)(Sk - 1) * ss + RB) : 0u;
    rk = buffer_rsrc(kp, nrec);
    rv = buffer_rsrc(vp, nrec);
    tile_bytes = ss * BN;
    const int row0 = 8 * wave;
    lds_k = kbuf_lds + row0 * RB;
    lds_v = vbuf_lds + row0 * RB;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = row0 + 2 * j + (lane >> 5);
      const int c = (lane & 31) ^ swz(row & 15);
      voff[j] = (uint32_t)row * ss + (uint32_t)c * 16;
    }
  }
  // prepared fp16 V^T tiles (16 KB each, in the LDS layout): each wave copies
  // its contiguous 4 KB quarter as four 1 KB instructions
  u32x4 rvt;
  uint32_t vt_lane;   // this wave's quarter, lane's 16 bytes
  uint32_t lds_vt;    // LDS address of this wave's quarter of prepared ring slot 0
  __device__ void init_vt(const uint8_t* vtp, int n_kt, int wave, int lane, uint32_t vt_lds) {
    rvt = buffer_rsrc(vtp, (uint32_t)n_kt * (uint32_t)VTB);
    vt_lane = (uint32_t)wave * 4096u + (uint32_t)lane * 16u;
    lds_vt = vt_lds + (uint32_t)wave * 4096u;
  }
  // copy instruction `which`: 0..3 rows of K tile `tile` into K ring slot
  // kslot, 4..7 rows of V tile `vtile` into V ring slot vslot (PRE: a quarter
  // of V^T tile `vtile` into prepared ring slot vslot)
  template <bool PRE>
  __device__ __forceinline__ void issue_one(int tile, int kslot, int vtile, int vslot,
                                            int which) const {
    const int j = which & 3;
    if (which < 4) {
      lds_copy16_at(rk, voff[j] + (uint32_t)tile * tile_bytes,
                    lds_k + (uint32_t)(kslot * TB + j * 1024));
    } else if (PRE) {
      lds_copy16_at(rvt, (uint32_t)vtile * (uint32_t)VTB + vt_lane + 1024u * j,
                    lds_vt + (uint32_t)(vslot * VTB + j * 1024));
    } else {
      lds_copy16_at(rv, voff[j] + (uint32_t)vtile * tile_bytes,
                    lds_v + (uint32_t)(vslot * TB + j * 1024));
    }
  }
  __device__ __forceinline__ void issue_k(int tile, int kslot) const {
#pragma unroll
    for (int which = 0; which < 4; ++which) issue_one<false>(tile, kslot, 0, 0, which);
  }
  template <bool PRE>
  __device__ __forceinline__ void issue_v(int vtile, int vslot) const {
#pragma unroll
    for (int which = 4; which < 8; ++which) issue_one<PRE>(0, 0, vtile, vslot, which);
  }
};

struct Wave {
  bf16x8 qf[KS];       // Q fragments: B operand of S^T = K Q^T (row = l32)
  f32x16 o[NDB];       // O^T accumulators per 32-wide d block
  f32x16 s;            // S^T of the current tile
  u32x4 pf[2];         // packed probabilities per 16-key step: B operand of P.V
  float m;             // running row max, log2 units (scale * log2 e folded in)
  float l;             // this lane's part of the row sum
  int koff[KS];        // K operand offsets per k-step
  int vtoff[2];        // V^T operand offsets per key step (d block 0)
  const char* kl[KS];  // K ring slot 0 + koff
  const char* vtl[2];  // prepared V^T ring slot 0 + vtoff
  int cvoff[4][2];     // transposed reads of the bf16 V tile [conversion unit][half]
  int first;           // first query row of the wave
  int l32, hi, wave;
};

struct Ctx {
  Loader ld;
  int T;          // key tiles of this workgroup
  int Sk, off;    // key count; causal offset (key j visible from row i iff j <= i + off)
  int q0;         // first query row of the workgroup
  float c;        // scale * log2(e)
};

// acc *= f for an accumulator that lives in AGPRs: the empty asm statements
// pin it there on both sides of the multiply, so that the compiler moves 16
// values through VGPR temporaries instead of keeping every accumulator in
// VGPRs.
__device__ __forceinline__ void scale_acc(f32x16& acc, float f) {
  asm volatile("" : "+a"(acc));
  acc *= f;
  asm volatile("" : "+a"(acc));
}

// S^T = K Q^T for one key tile (the unpipelined form: prologue, slow path).
__device__ __forceinline__ f32x16 qk_mfmas(const Wave& w, const char* kt) {
  f32x16 s = f32x16{};
#pragma unroll
  for (int k0 = 0; k0 < KS; k0 += 4) {
    bf16x8 a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8*)(kt + w.koff[k0 + i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) s = mfma32(a[i], w.qf[k0 + i], s);
  }
  return s;
}

// O^T += V^T P^T for one key tile (the unpipelined form: the last tile).
template <bool F16>
__device__ __forceinline__ void pv_mfmas(Wave& w, const char* vt) {
#pragma unroll
  for (int f0 = 0; f0 < 16; f0 += 4) {
    bf16x8 a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = f0 + i;
      a[i] = *(const bf16x8*)(vt + (f & 7) * 32 * 64 + w.vtoff[f >> 3]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = f0 + i, n = f & 7, kk = f >> 3;
      if (F16)
        w.o[n] = mfma32(__builtin_bit_cast(f16x8, a[i]), __builtin_bit_cast(f16x8, w.pf[kk]),
                        w.o[n]);
      else
        w.o[n] = mfma32(a[i], __builtin_bit_cast(bf16x8, w.pf[kk]), w.o[n]);
    }
  }
}

// Conversion unit q (0..3) of this wave: d block 2*wave + q/2, key step q%2.
// Two transposed 8-byte reads give lane (l32, hi) the 8 keys of chunk
// 2*(q%2) + hi for d = 32*(2*wave + q/2) + l32; they are widened to fp16 (or
// kept bf16) and written as one 16-byte chunk of the V^T tile.
__device__ __forceinline__ u32x4 conv_join(const bf16x4& lo, const bf16x4& up, bool f16) {
  u32x4 y = __builtin_bit_cast(u32x4, (bf16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2],
                                               up[3]}));
  if (f16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = bf16x2_to_f16x2(y[i]);
  }
  return y;
}
__device__ __forceinline__ int conv_dst(const Wave& w, int q) {
  return (2 * w.wave + (q >> 1)) * 32 * 64 + w.vtoff[q & 1];
}
template <bool F16>
__device__ __forceinline__ void transpose_v(const Wave& w, const char* vb, char* vt) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x4 lo = lds_read_tr(vb + w.cvoff[q][0]);
    const bf16x4 up = lds_read_tr(vb + w.cvoff[q][1]);
    *(u32x4*)(vt + conv_dst(w, q)) = conv_join(lo, up, F16);
  }
}

// Probabilities of the 16 scores against msub, packed into the two key-step
// operands; returns this lane's sum of the rounded values.
template <bool F16>
__device__ __forceinline__ float probs(const f32x16& s, float c, float msub, u32x4& p0,
                                       u32x4& p1) {
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = fast_exp2(__builtin_fmaf(s[r], c, -msub));
  uint32_t u[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    u[i] = F16 ? pack_f16(x[2 * i], x[2 * i + 1]) : pack_bf16(x[2 * i], x[2 * i + 1]);
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    a0 = F16 ? sum2_f16(u[i], a0) : sum2_bf16(u[i], a0);
    a1 = F16 ? sum2_f16(u[i + 1], a1) : sum2_bf16(u[i + 1], a1);
  }
  p0 = u32x4{u[0], u[1], u[2], u[3]};
  p1 = u32x4{u[4], u[5], u[6], u[7]};
  return a0 + a1;
}

// Last visible key of this lane's row relative to the lane's first key of
// the tile at kbase (its scores r hold keys kbase + 8(r/4) + 4hi + r%4).
template <bool CAUSAL>
__device__ __forceinline__ int visible_lim(const Wave& w, const Ctx& x, int kbase) {
  const int row = w.first + w.l32;
  return (CAUSAL ? min(x.Sk - 1, row + x.off) : x.Sk - 1) - kbase - 4 * w.hi;
}

// Slow path for tile t (rare: a row's first tile, or probabilities that
// outgrew the lazy bound): S(t) recomputed from K(t) (still in its ring
// slot), masked, the row max taken, the accumulator and row sum (which hold
// every tile before t) rescaled, the probabilities recomputed.
template <bool CAUSAL, bool F16>
__device__ __forceinline__ float rescale_tile(Wave& w, const Ctx& x, int t, const char* kt) {
  f32x16 s = qk_mfmas(w, kt);
  const int lim = visible_lim<CAUSAL>(w, x, t * BN);
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (8 * (r >> 2) + (r & 3) > lim) s[r] = -INFINITY;
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  mx = max_halves(mx);
  const float m_new = fmaxf(w.m, mx * x.c);
  const float alpha = (m_new == w.m) ? 1.f : fast_exp2(w.m - m_new);
  w.l *= alpha;
#pragma unroll
  for (int n = 0; n < NDB; ++n) scale_acc(w.o[n], alpha);
  w.m = m_new;
  return probs<F16>(s, x.c, (m_new == -INFINITY) ? 0.f : m_new, w.pf[0], w.pf[1]);
}

// One pipelined iteration for key tile t.  On entry S(t) is in w.s, P(t-1) in
// w.pf, and K(t+1), V(t+1), V^T(t-1), V^T(t) are visible in LDS.  The first
// iteration runs P(-1).V^T(-1) on zeros and the last one computes an unused
// S(T) and V^T(T) from the zeros (or unused keys) that the copies past the
// workgroup's tiles deliver, so every iteration is the same instruction
// stream.  Rows past Sq or past a causal diagonal are masked, not skipped.
//
//  group 1, slot j = 0..15: MFMA j of O^T += V^T(t-1) P(t-1)^T (d block j%8,
//    key step j/8); score j of S(t) moved out of the accumulator, masked
//    (MASK), scaled and shifted; the exponential of score j-1; V^T fragments
//    read four slots ahead; copy instruction (j-1)/2 in odd slots (K(t+3),
//    then V(t+3)); conversion units 0 and 1; K fragments of group 2 in
//    slots 12-15.
//  group 2, slot j = 0..15: MFMA j of S(t+1) = K(t+1) Q^T (overwriting the
//    score registers, all read by then); the last exponential; the
//    probabilities packed and summed as they become ready; conversion units
//    2 and 3; K fragments read four slots ahead.
// With prepared tiles (PRE), vbuf is the prepared ring: the copies bring
// V^T(t+2) into its slot (t+2) % 4, the conversion units are left out, and
// S = t % 4 fixes every ring slot at compile time.
template <bool CAUSAL, bool F16, bool MASK, bool PRE, int S>
__device__ __forceinline__ void iteration(Wave& w, const Ctx& x, int t, char* kbuf, char* vbuf,
                                          char* vtbuf) {
  static_assert(!PRE || (S >= 0 && S < NK && NK == NVP), "ring phase of the prepared loop");
  const int lim = MASK ? visible_lim<CAUSAL>(w, x, t * BN) : 0;
  const float c = x.c;
  const int kn = PRE ? (S + 1) % NK : (t + 1) % NK;         // K(t+1)
  const int kcur = PRE ? S : t % NK;                        // K(t), for the slow path
  const int ck = PRE ? (S + AHEAD) % NK : (t + AHEAD) % NK; // K(t+3) copies
  const int vtile = PRE ? t + 2 : t + AHEAD;                // V tile copied here
  const int cv = PRE ? (S + 2) % NVP : (t + AHEAD) % NV;
  const int vp = PRE ? (S + NVP - 1) % NVP : 0;             // prepared V^T(t-1)
  const char* vraw = vbuf + ((t + 1) % NV) * TB;
  const char* vt_prev = vtbuf + ((t + NVT - 1) % NVT) * VTB;
  char* vt_next = vtbuf + ((t + 1) % NVT) * VTB;
  auto kfrag = [&](int ks) { return *(const bf16x8*)(w.kl[ks] + kn * TB); };
  auto pack = [&](float a, float b) -> uint32_t { return F16 ? pack_f16(a, b) : pack_bf16(a, b); };
  auto sum2 = [&](uint32_t u, float acc) -> float {
    return F16 ? sum2_f16(u, acc) : sum2_bf16(u, acc);
  };
  auto score = [&](int r, float nm) -> float {
    // the score registers are MFMA results: the empty asm makes the move to a
    // VGPR happen here, inside the slot
    float sv = w.s[r];
    asm volatile("" : "+v"(sv));
    if (MASK && 8 * (r >> 2) + (r & 3) > lim) sv = -INFINITY;
    return __builtin_fmaf(sv, c, nm);
  };
  auto vt_frag = [&](int f) {
    if (PRE) return *(const bf16x8*)(w.vtl[f >> 3] + vp * VTB + (f & 7) * 32 * 64);
    return *(const bf16x8*)(vt_prev + (f & 7) * 32 * 64 + w.vtoff[f >> 3]);
  };
  float xs[16];
  uint32_t u[8];
  float acc[2] = {0.f, 0.f};
  bf16x8 vf[4], kf[4];
  bf16x4 tr[2];
  u32x4 y = u32x4{};
  // conversion unit q spread over one group: reads in slot 4 (q even) or 10,
  // the widening two slots later, the write one slot after that
  auto conv_step = [&](int j, int q) {
    if (PRE) return;
    if (j == 0) {
      tr[0] = lds_read_tr(vraw + w.cvoff[q][0]);
      tr[1] = lds_read_tr(vraw + w.cvoff[q][1]);
    }
    if (j == 2) y = conv_join(tr[0], tr[1], F16);
    if (j == 3) *(u32x4*)(vt_next + conv_dst(w, q)) = y;
  };

  // ---- group 1: P(t-1).V(t-1) with the scores of S(t)
  fence();
#pragma unroll
  for (int i = 0; i < 4; ++i) vf[i] = vt_frag(i);
  fence();
  const float nm = -w.m;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    {
      const int n = j & 7, kk = j >> 3;
      if (F16)
        w.o[n] = mfma32(__builtin_bit_cast(f16x8, vf[j & 3]), __builtin_bit_cast(f16x8, w.pf[kk]),
                        w.o[n]);
      else
        w.o[n] = mfma32(vf[j & 3], __builtin_bit_cast(bf16x8, w.pf[kk]), w.o[n]);
      if (j + 4 < 16) vf[j & 3] = vt_frag(j + 4);
    }
    if (j & 1) x.ld.issue_one<PRE>(t + AHEAD, ck, vtile, cv, j >> 1);
    if (j >= 12) kf[j - 12] = kfrag(j - 12);
    xs[j] = score(j, nm);
    if (j >= 1) xs[j - 1] = fast_exp2(xs[j - 1]);
    if (j >= 4 && j < 8) conv_step(j - 4, 0);
    if (j >= 10 && j < 14) conv_step(j - 10, 1);
    fence();
  }
  // ---- group 2: S(t+1) = K(t+1) Q^T with the rest of the softmax and of the
  // V(t+1) conversion
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    w.s = mfma32(kf[j & 3], w.qf[j], j == 0 ? f32x16{} : w.s);
    if (j + 4 < 16) kf[j & 3] = kfrag(j + 4);
    if (j == 0) xs[15] = fast_exp2(xs[15]);
    if (j >= 1 && j <= 8) u[j - 1] = pack(xs[2 * (j - 1)], xs[2 * (j - 1) + 1]);
    if (j >= 2 && j <= 9) acc[j & 1] = sum2(u[j - 2], acc[j & 1]);
    if (j >= 4 && j < 8) conv_step(j - 4, 2);
    if (j >= 10 && j < 14) conv_step(j - 10, 3);
    fence();
  }
  w.pf[0] = u32x4{u[0], u[1], u[2], u[3]};
  w.pf[1] = u32x4{u[4], u[5], u[6], u[7]};
  // lazy-rescale check: each lane's tile sum at most 2^12 (so is every
  // probability, far below the fp16 limit) against a finite running max;
  // otherwise (rare) the slow path.  The bf16 redo always takes it: with 8
  // significant bits the dominant probability of a short, peaky row must be
  // exactly 1, not a rounded power of two off a stale max.
  float tsum = acc[0] + acc[1];
  if (!F16 || wave_any(!(w.m != -INFINITY && tsum <= 4096.f)))
    tsum = rescale_tile<CAUSAL, F16>(w, x, t, kbuf + kcur * TB);
  w.l += tsum;
  // tile t+2's copies have landed (t+3's may still be in flight), this wave's
  // V^T writes are done; the barrier publishes both
  wait_vm_lds<COPIES>();
  barrier();
}

// Iterations t .. tend-1.  The prepared loop enters its four-iteration pass
// at the phase t % 4 and then runs whole passes.
template <bool CAUSAL, bool F16, bool MASK, bool PRE>
__device__ __forceinline__ void iterations(Wave& w, const Ctx& x, int& t, int tend, char* kbuf,
                                           char* vbuf, char* vtbuf) {
  if constexpr (PRE) {
    while (t < tend) {
      switch (t & 3) {
        case 0:
          iteration<CAUSAL, F16, MASK, PRE, 0>(w, x, t, kbuf, vbuf, vtbuf);
          if (++t >= tend) break;
          [[fallthrough]];
        case 1:
          iteration<CAUSAL, F16, MASK, PRE, 1>(w, x, t, kbuf, vbuf, vtbuf);
          if (++t >= tend) break;
          [[fallthrough]];
        case 2:
          iteration<CAUSAL, F16, MASK, PRE, 2>(w, x, t, kbuf, vbuf, vtbuf);
          if (++t >= tend) break;
          [[fallthrough]];
        default:
          iteration<CAUSAL, F16, MASK, PRE, 3>(w, x, t, kbuf, vbuf, vtbuf);
          ++t;
      }
    }
  } else {
    for (; t < tend; ++t) iteration<CAUSAL, F16, MASK, PRE, -1>(w, x, t, kbuf, vbuf, vtbuf);
  }
}

template <bool CAUSAL, bool F16, bool PRE = false>
__device__ __forceinline__ void tile_loop(Wave& w, const Ctx& x, char* kbuf, char* vbuf,
                                          char* vtbuf) {
  static_assert(F16 || !PRE, "prepared tiles are fp16");
#pragma unroll
  for (int n = 0; n < NDB; ++n) w.o[n] = f32x16{};
  w.m = -INFINITY;
  w.l = 0.f;
  w.pf[0] = w.pf[1] = u32x4{};
  const int T = x.T;
  if (T <= 0) return;
  // prologue: V^T(-1) (ring slot NVT-1, prepared: NVP-1) zeroed; copies of
  // K(0..2) and V(0..2) (prepared: V^T(0..1)); V^T(0); S(0)
  char* vt_m1 = PRE ? vbuf + (NVP - 1) * VTB : vtbuf + (NVT - 1) * VTB;
#pragma unroll
  for (int i = 0; i < 4; ++i) *(u32x4*)(vt_m1 + 64 * threadIdx.x + 16 * i) = u32x4{};
  if (PRE) {
    x.ld.issue_k(0, 0);
    x.ld.issue_v<true>(0, 0);
    x.ld.issue_k(1, 1);
    x.ld.issue_v<true>(1, 1);
    x.ld.issue_k(2, 2);
    wait_vm_lds<3 * COPIES / 2>();
  } else {
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) {
      x.ld.issue_k(i, i % NK);
      x.ld.issue_v<false>(i, i % NV);
    }
    wait_vm_lds<(AHEAD - 1) * COPIES>();
  }
  barrier();   // tile 0 and the zeros visible
  if (!PRE) transpose_v<F16>(w, vbuf, vtbuf);
  w.s = qk_mfmas(w, kbuf);
  if (PRE)
    wait_vm_lds<COPIES / 2>();
  else
    wait_vm_lds<(AHEAD - 2) * COPIES>();
  barrier();   // tile 1 and V^T(0) visible
  // tiles before the first one that needs a mask for some row of the
  // workgroup (a key past Sk, or past the diagonal of the first row)
  int tm;
  {
    int lo = x.Sk >= BN ? (x.Sk - BN) / BN + 1 : 0;
    if (CAUSAL) {
      const int r = x.q0 + x.off + 1 - BN;
      lo = min(lo, r >= 0 ? r / BN + 1 : 0);
    }
    tm = min(T, lo);
  }
  tm = __builtin_amdgcn_readfirstlane(tm);
  int t = 0;
  iterations<CAUSAL, F16, false, PRE>(w, x, t, tm, kbuf, vbuf, vtbuf);
  iterations<CAUSAL, F16, true, PRE>(w, x, t, T, kbuf, vbuf, vtbuf);
  // drain: P(T-1).V(T-1); then every copy of the ring has landed, so that
  // nothing writes the LDS after the loop (a redo starts its own copies)
  pv_mfmas<F16>(w, PRE ? vbuf + ((T - 1) % NVP) * VTB : vtbuf + ((T - 1) % NVT) * VTB);
  wait_vm_lds<0>();
}

__device__ __forceinline__ bool state_finite(const Wave& w) {
  bool ok = __builtin_isfinite(w.l);
#pragma unroll
  for (int n = 0; n < NDB; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) ok = ok && __builtin_isfinite(w.o[n][r]);
  return ok;
}

// Workgroup-wide OR of pred through four words of the K ring (free once the
// tile loop has drained its copies; the rings take all 160 KB of LDS).
__device__ __forceinline__ bool workgroup_any(bool pred, char* words, int wave) {
  const bool any = wave_any(pred);
  if ((threadIdx.x & 63) == 0) ((int*)words)[wave] = any ? 1 : 0;
  __syncthreads();
  const int* f = (const int*)words;
  const bool r = (f[0] | f[1] | f[2] | f[3]) != 0;
  __syncthreads();   // every wave has read the words before the ring is reused
  return r;
}

template <bool CAUSAL, bool PRE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_d256_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[NK * TB + NV * TB + NVT * VTB];
  char* const kbuf = lds;
  char* const vbuf = lds + NK * TB;
  char* const vtbuf = vbuf + NV * TB;

  Wave w;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  w.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  w.l32 = lane & 31;
  w.hi = lane >> 5;

  // ---- which (batch, query head, 128-row block): heaviest causal blocks
  // first; the heads of one K/V head on one XCD (workgroups are dealt to the
  // 8 XCDs round robin)
  const int n_qb = a.n_qt;
  const int BH = a.B * a.Hq;
  int bh, qb;
  if (CAUSAL) {
    const int row = blockIdx.x / BH;
    qb = n_qb - 1 - row;
    bh = xcd_remap(blockIdx.x - row * BH, BH);
  } else {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    bh = L / n_qb;
    qb = L - bh * n_qb;
  }
  const int b = bh / a.Hq, hq = bh - b * a.Hq;
  const int hk = hq / a.group;
  const int Sq = a.Sq, Sk = a.Sk;
  const __bf16* __restrict__ qp = a.q + b * a.q_sb + hq * a.q_sh;
  const __bf16* kp = a.k + b * a.k_sb + hk * a.k_sh;
  const __bf16* vp = a.v + b * a.k_sb + hk * a.k_sh;

  Ctx x;
  x.off = Sk - Sq;
  x.Sk = Sk;
  x.c = a.c;
  x.q0 = qb * QR;
  const int last_row = min(x.q0 + QR, Sq) - 1;
  int n_keys = Sk;
  if (CAUSAL) n_keys = min(Sk, max(0, last_row + x.off + 1));
  x.T = (n_keys + BN - 1) / BN;
  w.first = x.q0 + 32 * w.wave;
  x.ld.init(kp, vp, a.k_ss, Sk, w.wave, lane,
            __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(ATTN_LDS char*)kbuf),
            __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(ATTN_LDS char*)vbuf));
  if (PRE)
    x.ld.init_vt(a.vt + (int64_t)(b * a.Hkv + hk) * a.n_kt * VTB, a.n_kt, w.wave, lane,
                 __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(ATTN_LDS char*)vbuf));

  // ---- per-lane LDS offsets
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    w.koff[ks] = kv_off(w.l32, 2 * ks + w.hi);
    w.kl[ks] = kbuf + w.koff[ks];
  }
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    w.vtoff[kk] = vt_off(w.l32, 2 * kk + w.hi);
    w.vtl[kk] = vbuf + w.vtoff[kk];
  }
  // transposed reads of the bf16 V tile for conversion unit q (d block
  // 2*wave + q/2, key step q%2): lane (beta = lane/16, j = lane%16)
  // addresses row 16*(q%2) + 8*h + 4*hi + j/4, columns
  // 32*(2*wave + q/2) + 16*(beta&1) + 4*(j%4) .. +3, so that lane j of each
  // 16-lane block receives keys 16*(q%2) + 8*h + 4*hi + 0..3 of column
  // 32*(2*wave + q/2) + 16*(beta&1) + j
  {
    const int j = lane & 15;
    const int chalf = (lane >> 4) & 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = 32 * (2 * w.wave + (q >> 1)) + 16 * chalf + 4 * (j & 3);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 16 * (q & 1) + 8 * h + 4 * w.hi + (j >> 2);
        w.cvoff[q][h] = kv_off(r, col >> 3) + (col & 7) * 2;
      }
    }
  }

  // ---- Q fragments: row = query, k-slots = d
  {
    const int row = w.first + w.l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (row < Sq)
        w.qf[ks] = *(const bf16x8*)(qp + (int64_t)row * a.q_ss + 16 * ks + 8 * w.hi);
      else
        w.qf[ks] = bf16x8{};
    }
  }

  if (PRE)
    tile_loop<CAUSAL, true, true>(w, x, kbuf, vbuf, vtbuf);
  else
    tile_loop<CAUSAL, true>(w, x, kbuf, vbuf, vtbuf);
  // A V value beyond the fp16 range (|v| >= 65520) or a non-finite input
  // shows up as a non-finite accumulator: redo this workgroup with bf16
  // probabilities and bf16 V, which covers the whole bf16 range.
  if (workgroup_any(!state_finite(w), kbuf, w.wave))
    tile_loop<CAUSAL, false>(w, x, kbuf, vbuf, vtbuf);

  // ---- epilogue: O = O^T / l (register r of lane (l32, hi), d block n:
  // d = 32n + 8(r/4) + 4hi + r%4) under the caller's rounding rule;
  // LSE = (m + log2 l) ln 2
  const float L = sum_halves(w.l);
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  const int row = w.first + w.l32;
  if (row < Sq) {
    __bf16* orow = a.o + b * a.q_sb + hq * a.q_sh + (int64_t)row * a.q_ss;
    with_rounding(a.rounding, [&](auto mode) {
#pragma unroll
      for (int n = 0; n < NDB; ++n)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 u;
          u[0] = pack_bf16_as<mode()>(w.o[n][4 * g] * inv, w.o[n][4 * g + 1] * inv);
          u[1] = pack_bf16_as<mode()>(w.o[n][4 * g + 2] * inv, w.o[n][4 * g + 3] * inv);
          *(u32x2*)(orow + 32 * n + 8 * g + 4 * w.hi) = u;
        }
    });
    if (w.hi == 0)
      a.lse[(int64_t)(b * a.Hq + hq) * Sq + row] =
          (L > 0.f) ? (w.m + __log2f(L)) * kLn2 : -INFINITY;
  }
}

// V of one (batch, K/V head) as fp16 V^T tiles of 32 keys for the prepared
// path: tile t (keys 32t .. 32t+31, zeros past Sk) goes to
// vt + ((b * Hkv + h) * n_kt + t) * VTB in exactly the LDS layout that the
// converting path builds (vt_off: row d of 64 bytes, chunk c holding the keys
// 16(c/2) + 4(c%2) + {0..3, 8..11} rounded to fp16, nearest even).  The tile
// goes through LDS as read (rows of bf16 keys) and is written out transposed.
// HBM-bound: 16 KB read and 16 KB written per tile.
__global__ __launch_bounds__(256) void prep_v_d256_kernel(PrepVArgs a) {
  constexpr int RS = D + 8;   // padded LDS row (bf16 elements)
  __shared__ __attribute__((aligned(16))) __bf16 tile[BN * RS];
  const int64_t id = blockIdx.x;
  const int t = (int)(id % a.n_kt);
  const int64_t bh = id / a.n_kt;
  const int h = (int)(bh % a.Hkv);
  const int b = (int)(bh / a.Hkv);
  const __bf16* vp = a.v + b * a.k_sb + h * a.k_sh;
  const int tid = threadIdx.x;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int r = 8 * pass + (tid >> 5), c = tid & 31;
    const int key = t * BN + r;
    u32x4 val = u32x4{0u, 0u, 0u, 0u};
    if (key < a.Sk) val = *(const u32x4*)(vp + (int64_t)key * a.k_ss + 8 * c);
    *(u32x4*)(tile + r * RS + 8 * c) = val;
  }
  __syncthreads();
  uint8_t* out = a.vt + id * VTB;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int idx = 256 * pass + tid;
    const int d = idx >> 2, ch = idx & 3;
    const int k0 = 16 * (ch >> 1) + 4 * (ch & 1);
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (float)tile[(k0 + (j < 4 ? j : j + 4)) * RS + d];
    const u32x4 y = u32x4{pack_f16(f[0], f[1]), pack_f16(f[2], f[3]), pack_f16(f[4], f[5]),
                          pack_f16(f[6], f[7])};
    *(u32x4*)(out + vt_off(d, ch)) = y;
  }
}

}  // namespace

hipError_t launch_prefill_d256(const PrefillArgs& a, bool causal, hipStream_t stream) {
  if (a.cu_q || a.alibi) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)a.B * a.Hq * a.n_qt;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidValue;
  if ((int64_t)a.n_qt * QR < a.Sq) return hipErrorInvalidValue;
  if (a.vt && a.n_kt != (a.Sk + BN - 1) / BN) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), blk(NT);
  if (a.vt) {
    if (causal)
      hipLaunchKernelGGL((prefill_d256_kernel<true, true>), g, blk, 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_d256_kernel<false, true>), g, blk, 0, stream, a);
  } else if (causal) {
    hipLaunchKernelGGL((prefill_d256_kernel<true, false>), g, blk, 0, stream, a);
  } else {
    hipLaunchKernelGGL((prefill_d256_kernel<false, false>), g, blk, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_prep_v_d256(const PrepVArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.B * a.Hkv * a.n_kt;
  if (grid <= 0 || grid > 0x7fffffff || a.tk != BN || a.n_kt != (a.Sk + BN - 1) / BN)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(prep_v_d256_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
