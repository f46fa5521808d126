// Fused exact attention forward for gfx950, software-pipelined inside each
// wave: O = softmax(scale * Q K^T) V.
//
// What is computed follows "IO-aware tiling strategy in FlashAttention-4"
// (body): Q is cut into row tiles and K/V into column tiles that are brought
// on chip, the score tile never leaves the chip, and each query row keeps a
// running max m and denominator l merged block by block (m' = max(m, m_new),
// l' = l * 2^(m - m') + l_new with l_new summed against m'); the output
// accumulator is multiplied by the same per-row factor and divided by l once,
// at the end.
//
// Design (MI355X-first; the pages' NVIDIA and gfx942 kernels are prior art):
//  * one workgroup = 4 waves, one per SIMD, each wave 64 query rows (two
//    32-row MFMA blocks).  A wave owns the whole register file of its SIMD
//    (512 registers: Q fragments and the fp32 O^T accumulators in AGPRs, the
//    score tile, probabilities, operand fragments), so every K or V^T
//    operand read from LDS feeds two MFMAs.
//  * No wave specialisation and no ping-pong between waves: every wave
//    pipelines its own work.  The iteration for key tile t issues the 16
//    MFMAs of O^T += V^T(t-1) P(t-1)^T, then the 16 MFMAs of
//    S(t+1) = K(t+1) Q^T, none of which depends on the iteration's VALU work
//    (the softmax of S(t), the V(t+1) conversion), which is placed between
//    them slot by slot.  A wave's independent VALU instructions issue while
//    its own MFMAs execute; measured on the device, about six VALU issue
//    slots per 32x32x16 MFMA come for free.  With one wave per SIMD every
//    instruction of the wave (VALU, LDS, scalar, waits) shares its issue
//    slots, which is what bounds this design (measured: about 2400 cycles
//    per 32-key tile against 1024 of MFMA).
//  * The 4 waves of a workgroup are 4 query heads of one K/V head over the
//    same 64 rows (GQA/MQA with a group size that is a multiple of 4:
//    "Engineering the FlashAttention-4 kernel port to ROCm", multi-query
//    section, Q:32/KV:8), so each K/V tile is loaded and converted once for
//    all four heads, and causal masking is balanced across the waves.
//  * K and V tiles of 32 keys (8 KB each) are copied HBM -> LDS by the buffer
//    unit (buffer_load ... lds, 16 B per lane, each wave a quarter of the
//    rows, spread over the MFMA slots) into a 4-deep ring, three tiles
//    ahead; keys past Sk fall outside the buffer range and read as zero.
//    Rows are 256 B with an XOR swizzle of their 16-byte chunks
//    (conflict-free MFMA operand reads).
//  * Scores are computed transposed, S^T = K Q^T, on
//    v_mfma_f32_32x32x16_bf16: a lane holds one query row (half of the keys
//    in each lane half), so the row max and sum are in-lane plus one
//    v_permlane32_swap, and the packed probabilities are already the B
//    operand of O^T = V^T P^T.
//  * P.V runs in fp16 (11 significant bits; bf16's 8 are too few for the
//    parity bound when a few large V entries nearly cancel).  Each wave
//    converts one 32-wide d block of the tile: transposed LDS reads
//    (ds_read_b64_tr_b16) of the bf16 V tile, conversion to fp16, one 16-byte
//    LDS write per lane into the V^T tile that the MFMAs read.  A V value
//    outside the fp16 range (or a non-finite input) leaves a non-finite
//    accumulator; the workgroup then redoes its tiles with bf16 P and V.
//  * The output rescale is lazy: probabilities are taken against the running
//    max as it stands while a tile's per-lane sum stays <= 2^12 (each value
//    then far from the fp16 limit, and O = sum p v / sum p unchanged); a
//    row's first tile, or a larger sum, takes the row max and rescales.
//  * One workgroup barrier per tile publishes the copies and the V^T tile
//    (V^T in a ring of 3).
//  * Causal: tiles past the last row's diagonal are never loaded, only
//    boundary tiles are masked (a second loop over the masked tiles at the
//    end), heaviest query tiles are dispatched first.
//  * blockIdx is remapped so that workgroups sharing K/V land on one XCD
//    (workgroups are dealt to the 8 XCDs round robin); causal launches also
//    keep the query tiles running at once on an XCD within one or two heads
//    (causal_xcd_order), so the K/V tiles they stream are shared in L2.
//  * Packed sequences of different lengths (cu_q/cu_k offsets, V converted
//    in the kernel): a workgroup reads its sequence's offsets first and
//    returns at once if its query tile lies past the sequence; head groups
//    are dealt to the XCDs interleaved (every XCD gets a share of each
//    sequence) and each XCD runs the causal order above over its groups.
#include "gfx950.hpp"
#include "kernels.h"

namespace attn {
namespace {

constexpr int D = kHeadDim;       // 128
constexpr int BN = kPrefillPipeBN;   // keys per K/V tile (32)
constexpr int NW = 4;             // waves per workgroup, one per SIMD
constexpr int NT = NW * 64;       // 256 threads
constexpr int TB = BN * 256;      // bytes of one bf16 K or V tile (8 KB)
constexpr int VTB = kVtPipeTileBytes;   // bytes of one V^T tile (8 KB)
constexpr int NBUF = 4;           // K/V copy ring: tiles t+1 .. t+3 resident or in flight
constexpr int AHEAD = NBUF - 1;   // copies run this many tiles ahead
constexpr int COPIES = 4;         // copy instructions per wave per tile
constexpr int NVT = 5;            // V^T ring with prepared tiles: t-1 .. t+3

// 4-bit swizzle of a row index: a bijection on 0..15 that sends rows r and
// r+4k to different 4-chunk groups.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// Byte offset of 16-byte chunk c (0..15) of row `row` in a 256-byte-row tile.
__device__ __forceinline__ int tile_off(int row, int c) {
  return row * 256 + ((c ^ swz(row & 15)) << 4);
}
// V^T tile: row d holds the 32 keys of the tile as 4 chunks of 16 bytes;
// chunk 2*kk + hi holds the 8 keys 16*kk + {4hi..4hi+3, 8+4hi..8+4hi+3} in
// the MFMA k-slot order of lane half hi.  The chunk index is XORed with bits
// 2-3 of d so that 16 lanes reading one chunk of 16 consecutive rows cover
// all 64 banks once.
__device__ __forceinline__ int vt_off(int d, int chunk) {
  return d * 64 + ((chunk ^ ((d >> 2) & 3)) << 4);
}

__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int per = n >> 3;
  return (i < (per << 3)) ? (i & 7) * per + (i >> 3) : i;
}

// s_waitcnt through the intrinsic so the compiler's own tracking knows it.
// vmcnt(N) with lgkmcnt(0): at most N of this wave's copies still in flight
// and its LDS accesses done.
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);
}
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Copies of one K and one V tile: this wave's 8 rows of each (2 x 1 KB per
// tensor).  Lane i of an instruction lands at byte 16*i of a 4-row block,
// i.e. row +i/16, physical chunk i%16, so it fetches the logical chunk the
// swizzle puts there.
struct Loader {
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t voff[2];
  uint32_t tile_bytes;
  int row0;
  uint32_t lds_k, lds_v;   // LDS byte addresses of this wave's first K and V row of ring slot 0
  // prepared fp16 V^T tiles (8 KB, in the LDS layout): each wave copies its
  // contiguous 2 KB quarter as two 1 KB instructions
  u32x4 rvt;
  uint32_t vt_off;         // this wave's quarter, lane's 16 bytes
  uint32_t lds_vt;         // LDS byte address of this wave's quarter of V^T ring slot 0

  __device__ void init_vt(const uint8_t* vtp, int n_kt, int wave, int lane, uint32_t vt_lds) {
    rvt = buffer_rsrc(vtp, (uint32_t)n_kt * (uint32_t)VTB);
    vt_off = (uint32_t)wave * 2048u + (uint32_t)lane * 16u;
    lds_vt = vt_lds + (uint32_t)wave * 2048u;
  }

  __device__ void init(const __bf16* kp, const __bf16* vp, int64_t k_ss, int Sk, int wave,
                       int lane, uint32_t kbuf_lds, uint32_t vbuf_lds) {
    const uint32_t ss = (uint32_t)(k_ss * 2);
    const uint32_t nrec = Sk > 0 ? (uint32_t)((int64_t)(Sk - 1) * ss + 256) : 0u;
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)kp, (short)0, (int)nrec, 0x00020000);
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)vp, (short)0, (int)nrec, 0x00020000);
    tile_bytes = ss * BN;
    row0 = 8 * wave;
    lds_k = kbuf_lds + row0 * 256;
    lds_v = vbuf_lds + row0 * 256;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = row0 + 4 * j + (lane >> 4);
      const int c = (lane & 15) ^ swz(row & 15);
      voff[j] = (uint32_t)row * ss + (uint32_t)c * 16;
    }
  }
  // One of the four copy instructions of a tile (which = 0, 1: K rows;
  // 2, 3: V rows), issued as a plain instruction that the compiler does not
  // track.  The copies write LDS behind the compiler's back on purpose: it
  // would otherwise wait for every copy in flight before each later LDS read
  // (it cannot tell the ring slots apart), stalling the pipeline on the copy
  // latency.  Their completion is ordered explicitly instead: vmcnt waits
  // and the workgroup barrier before any wave reads a slot.  The instruction
  // has no register results (its data goes to LDS); M0 holds the LDS
  // address, written one wait state before the copy reads it (the compiler's
  // hazard tracking does not look inside the asm statement).
  // With prepared tiles (PRE), which = 2, 3 copy this wave's quarter of the
  // V^T tile into V^T ring slot vslot instead of V rows.
  template <bool PRE = false>
  __device__ __forceinline__ void issue_one(int tile, int slot, int which, int vslot = 0) const {
    const uint32_t base = (uint32_t)tile * tile_bytes;
    const int j = which & 1;
    if (PRE && which >= 2) {
      lds_copy16_at(rvt, (uint32_t)tile * (uint32_t)VTB + vt_off + 1024u * j,
                    lds_vt + (uint32_t)(vslot * VTB) + 1024u * j);
      return;
    }
    const uint32_t m0 = (which < 2 ? lds_k : lds_v) + (uint32_t)(slot * TB + 4 * j * 256);
    if (which < 2)
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   : : "s"(m0), "v"(voff[j] + base), "s"(rk) : "memory", "m0");
    else
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   : : "s"(m0), "v"(voff[j] + base), "s"(rv) : "memory", "m0");
  }
  template <bool PRE = false>
  __device__ __forceinline__ void issue(int tile, int slot, int vslot = 0) const {
#pragma unroll
    for (int which = 0; which < 4; ++which) issue_one<PRE>(tile, slot, which, vslot);
  }
};

struct Wave {
  bf16x8 qf[2][8];     // Q fragments per row block: B operand of S^T = K Q^T
  f32x16 o[2][4];      // O^T accumulators [row block][d block]
  f32x16 s[2];         // S^T of the current tile [row block]
  u32x4 pf[2][2];      // packed probabilities [row block][k-step]: B operand of P.V
  float m[2];          // running max per row block, log2 units (scale*log2e folded in)
  float l[2];          // this lane's part of the row sum
  int koff[8];         // K operand offsets per 16-wide d step
  int vtoff[2];        // V^T operand offsets per k-step (d block 0)
  int cvoff[2][2];     // transposed-read offsets into the bf16 V tile [k-step][half]
  int first[2];        // first query row of each row block
  int l32, hi, wave;
};

// Pins the instruction order: nothing is moved across it.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// S^T(rb) = K Q(rb)^T for one key tile: 8 K fragments, each used by both row
// blocks (the unpipelined form, for the prologue and the rescale path).
__device__ __forceinline__ void qk_mfmas(Wave& w, f32x16 (&s)[2], const char* kt) {
  bf16x8 a[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) a[ks] = *(const bf16x8*)(kt + w.koff[ks]);
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    s[0] = mfma32(a[ks], w.qf[0][ks], s[0]);
    s[1] = mfma32(a[ks], w.qf[1][ks], s[1]);
  }
}

// O^T(rb) += V^T P(rb)^T for one key tile, unpipelined (the last tile).
template <bool F16>
__device__ __forceinline__ void pv_mfmas(Wave& w, const char* vt) {
  bf16x8 a[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) a[f] = *(const bf16x8*)(vt + (f & 3) * 32 * 64 + w.vtoff[f >> 2]);
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int kk = f >> 2, db = f & 3;
      if (F16)
        w.o[rb][db] = mfma32(__builtin_bit_cast(f16x8, a[f]), __builtin_bit_cast(f16x8, w.pf[rb][kk]),
                             w.o[rb][db]);
      else
        w.o[rb][db] = mfma32(a[f], __builtin_bit_cast(bf16x8, w.pf[rb][kk]), w.o[rb][db]);
    }
}

// This wave's share of V(t) -> V^T(t): d block `wave`, both k-steps: four
// transposed 8-byte reads per lane, conversion to fp16 (or kept bf16), two
// 16-byte writes (the unpipelined form, for the prologue).
template <bool F16>
__device__ __forceinline__ void transpose_v(const Wave& w, const char* vb, char* vt) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const bf16x4 lo = lds_read_tr(vb + w.cvoff[kk][0]);
    const bf16x4 up = lds_read_tr(vb + w.cvoff[kk][1]);
    u32x4 y = __builtin_bit_cast(u32x4, (bf16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2],
                                                 up[3]}));
    if (F16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = bf16x2_to_f16x2(y[i]);
    }
    *(u32x4*)(vt + w.wave * 32 * 64 + w.vtoff[kk]) = y;
  }
}

// Probabilities of one row block's 16 scores against msub, packed into the
// two k-step operands; returns this lane's sum of the rounded values.
template <bool F16>
__device__ __forceinline__ float probs(const f32x16& s, float c, float msub, u32x4& p0,
                                       u32x4& p1) {
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = __builtin_fmaf(s[r], c, -msub);
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = fast_exp2(x[r]);
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

// Masks one row block's scores of the tile starting at key kbase: keys past
// Sk and, causal, keys past the row's diagonal.
template <bool CAUSAL>
__device__ __forceinline__ void mask_scores(const Wave& w, f32x16& s, int rb, int kbase, int Sk,
                                            int off) {
  const int row = w.first[rb] + w.l32;
  const int lim = (CAUSAL ? min(Sk - 1, row + off) : Sk - 1) - kbase - 4 * w.hi;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = 8 * (r >> 2) + (r & 3);
    if (key > lim) s[r] = -INFINITY;
  }
}
template <bool CAUSAL>
__device__ __forceinline__ bool tile_needs_mask(const Wave& w, int rb, int kbase, int Sk,
                                                int off) {
  return (kbase + BN > Sk) || (CAUSAL && kbase + BN - 1 > w.first[rb] + off);
}

// acc *= f for an accumulator that lives in AGPRs: the empty asm statements
// pin it to the AGPR file on both sides of the multiply, so the compiler
// moves 16 values through VGPR temporaries here instead of keeping every
// accumulator in VGPRs (which do not fit beside the score tiles).
__device__ __forceinline__ void scale_acc(f32x16& acc, float f) {
  asm volatile("" : "+a"(acc));
  acc *= f;
  asm volatile("" : "+a"(acc));
}

struct Ctx {
  Loader ld;
  int T;          // key tiles of this workgroup
  int Sk, off;    // key count; causal offset (key j visible from row i iff j <= i + off)
  float c;        // scale * log2(e)
};

// Slow path for tile t (rare: a row's first tile, or probabilities that
// outgrew the lazy bound): S(t) is recomputed from K(t) (still in its ring
// slot), masked, and each row block that needs it takes the row max,
// rescales its accumulators and row sum (which hold every tile before t) and
// recomputes its probabilities.
template <bool CAUSAL, bool F16>
__device__ __forceinline__ void rescale_tile(Wave& w, const Ctx& x, int t, const char* kt,
                                             bool need0, bool need1, float (&tsum)[2]) {
  f32x16 s[2];
  qk_mfmas(w, s, kt);
  const int kbase = t * BN;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    if (!(rb == 0 ? need0 : need1)) continue;
    if (tile_needs_mask<CAUSAL>(w, rb, kbase, x.Sk, x.off))
      mask_scores<CAUSAL>(w, s[rb], rb, kbase, x.Sk, x.off);
    float mx = s[rb][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[rb][r]);
    mx = max_halves(mx);
    const float m_new = fmaxf(w.m[rb], mx * x.c);
    const float alpha = (m_new == w.m[rb]) ? 1.f : fast_exp2(w.m[rb] - m_new);
    w.l[rb] *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) scale_acc(w.o[rb][db], alpha);
    w.m[rb] = m_new;
    tsum[rb] = probs<F16>(s[rb], x.c, (m_new == -INFINITY) ? 0.f : m_new, w.pf[rb][0],
                          w.pf[rb][1]);
  }
}

// One pipelined iteration for key tile t.  On entry S(t) is in w.s (AGPRs),
// P(t-1) in w.pf, and K(t+1), V(t+1), V^T(t-1), V^T(t) are visible in LDS.
// The first iteration runs P(-1).V^T(-1) on zeros and the last one computes
// an unused S(T) and V^T(T) from the zeros that copies past the keys
// deliver, so every iteration is the same instruction stream; every wave
// runs it whole (rows past Sq or past a causal diagonal are masked, not
// skipped).
//
// The MFMAs of the iteration do not depend on its VALU work, so the two are
// interleaved slot by slot (one MFMA per slot, fences between slots):
//  group 1, slot j = 0..15: MFMA j of O^T += V^T(t-1) P(t-1)^T; scores 2j,
//    2j+1 of S(t) moved out of the AGPRs, scaled and shifted (fma); the
//    exponential of score j;
//    V^T fragments read four slots ahead; the copies of tile t+3 in slots
//    1, 5, 9, 13 (a copy instruction holds up the wave's issue for tens of
//    cycles, which an MFMA in flight hides).
//  group 2, slot j = 0..15: MFMA j of S(t+1) = K(t+1) Q^T (overwriting the
//    score registers, all read by then); the exponential of score 16+j;
//    probabilities packed to fp16 and summed as they become ready; this
//    wave's share of the V(t+1) conversion; K fragments read four slots
//    ahead.
// Score e (0..31) is element e%16 of row block e/16.  MASK (boundary tiles
// only) sets scores past Sk or past a row's diagonal to -inf as they leave
// the AGPRs.  After the slots, the lazy-rescale check; its rare slow path
// recomputes S(t).
// With prepared V^T tiles (PRE) the copies bring V^T(t+3) into a ring of 5
// (V^T(t-1) .. V^T(t+3)) and there is no conversion.
template <bool CAUSAL, bool F16, bool MASK, bool PRE = false>
__device__ __forceinline__ void iteration(Wave& w, const Ctx& x, int t, char* kbuf, char* vbuf,
                                          char* vtbuf) {
  int lim[2] = {0, 0};   // last visible key of this lane's row, relative to its half
  if (MASK) {
    const int kbase = t * BN;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = w.first[rb] + w.l32;
      lim[rb] = (CAUSAL ? min(x.Sk - 1, row + x.off) : x.Sk - 1) - kbase - 4 * w.hi;
    }
  }
  const float c = x.c;
  const int cslot = (t + AHEAD) % NBUF;                // copies of tile t+3 (past the keys: zeros)
  const int vcslot = (t + AHEAD) % NVT;                // PRE: V^T(t+3)
  const char* knext = kbuf + ((t + 1) % NBUF) * TB;
  const char* vraw = vbuf + ((t + 1) % NBUF) * TB;
  const char* vt_prev = PRE ? vtbuf + ((t + NVT - 1) % NVT) * VTB   // V^T(t-1)
                            : vtbuf + ((t + 2) % 3) * VTB;
  char* vt_next = vtbuf + ((t + 1) % 3) * VTB;         // V^T(t+1), converted here
  auto pack = [&](float a, float b) -> uint32_t { return F16 ? pack_f16(a, b) : pack_bf16(a, b); };
  auto sum2 = [&](uint32_t u, float acc) -> float {
    return F16 ? sum2_f16(u, acc) : sum2_bf16(u, acc);
  };
  auto score = [&](int e, float nm) -> float {
    // the score registers are MFMA results in AGPRs: the empty asm makes the
    // move to a VGPR happen here, inside the slot
    float sv = w.s[e >> 4][e & 15];
    asm volatile("" : "+v"(sv));
    if (MASK) {
      const int r = e & 15;
      if (8 * (r >> 2) + (r & 3) > lim[e >> 4]) sv = -INFINITY;
    }
    return __builtin_fmaf(sv, c, nm);
  };
  float xs[32];
  uint32_t u[16];
  float acc[4] = {0.f, 0.f, 0.f, 0.f};   // [row block][chain]
  bf16x8 vf[8], kf[8];
  bf16x4 tr[4];
  u32x4 y[2];

  // ---- group 1: P(t-1).V(t-1) with the scores of S(t)
  fence();
  vf[0] = *(const bf16x8*)(vt_prev + 0 * 32 * 64 + w.vtoff[0]);
  vf[1] = *(const bf16x8*)(vt_prev + 1 * 32 * 64 + w.vtoff[0]);
  fence();
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    {
      const int f = j >> 1, rb = j & 1, kk = f >> 2, db = f & 3;
      if (F16)
        w.o[rb][db] = mfma32(__builtin_bit_cast(f16x8, vf[f]),
                             __builtin_bit_cast(f16x8, w.pf[rb][kk]), w.o[rb][db]);
      else
        w.o[rb][db] = mfma32(vf[f], __builtin_bit_cast(bf16x8, w.pf[rb][kk]), w.o[rb][db]);
      if (rb == 0 && f + 2 < 8)
        vf[f + 2] = *(const bf16x8*)(vt_prev + ((f + 2) & 3) * 32 * 64 + w.vtoff[(f + 2) >> 2]);
    }
    if ((j & 3) == 1) x.ld.issue_one<PRE>(t + AHEAD, cslot, j >> 2, vcslot);
    if (j >= 12) kf[j - 12] = *(const bf16x8*)(knext + w.koff[j - 12]);
    {
      const float nm = -w.m[j >> 3];
      xs[2 * j] = score(2 * j, nm);
      xs[2 * j + 1] = score(2 * j + 1, nm);
    }
    xs[j] = fast_exp2(xs[j]);
    fence();
  }
  // ---- group 2: S(t+1) = K(t+1) Q^T with the rest of the softmax and the
  // V(t+1) conversion
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    {
      const int rb = j & 1, ks = j >> 1;
      w.s[rb] = mfma32(kf[ks], w.qf[rb][ks], ks == 0 ? f32x16{} : w.s[rb]);
      if (rb == 0 && ks + 4 < 8) kf[ks + 4] = *(const bf16x8*)(knext + w.koff[ks + 4]);
    }
    xs[16 + j] = fast_exp2(xs[16 + j]);
    // pairs 0..7 (scores 0..15) are ready from slot 0, pairs 8+q once scores
    // 16+2q, 17+2q are: one pack per slot for the first, one every second
    // slot for the others; each sum one slot after its pack
    if (j < 8) u[j] = pack(xs[2 * j], xs[2 * j + 1]);
    if (j >= 2 && (j & 1) == 0) {
      const int q = (j - 2) >> 1;
      u[8 + q] = pack(xs[16 + 2 * q], xs[17 + 2 * q]);
    }
    if (j >= 1 && j <= 8) acc[(j - 1) & 1] = sum2(u[j - 1], acc[(j - 1) & 1]);
    if (j >= 3 && (j & 1) == 1) {
      const int q = (j - 3) >> 1;
      acc[2 + (q & 1)] = sum2(u[8 + q], acc[2 + (q & 1)]);
    }
    if (!PRE) {
      // conversion of this wave's d block of V(t+1): k-step 0 in slots 0-6,
      // k-step 1 in slots 7-13
      const int h = j < 7 ? 0 : 1, js = j < 7 ? j : j - 7;
      if (js == 0) tr[2 * h] = lds_read_tr(vraw + w.cvoff[h][0]);
      if (js == 1) tr[2 * h + 1] = lds_read_tr(vraw + w.cvoff[h][1]);
      if (js >= 2 && js <= 5) {
        const int q = js - 2;
        if (q == 0)
          y[h] = __builtin_bit_cast(u32x4, (bf16x8{tr[2 * h][0], tr[2 * h][1], tr[2 * h][2],
                                                   tr[2 * h][3], tr[2 * h + 1][0],
                                                   tr[2 * h + 1][1], tr[2 * h + 1][2],
                                                   tr[2 * h + 1][3]}));
        if (F16) y[h][q] = bf16x2_to_f16x2(y[h][q]);
      }
      if (js == 6) *(u32x4*)(vt_next + w.wave * 32 * 64 + w.vtoff[h]) = y[h];
    }
    fence();
  }
  u[15] = pack(xs[30], xs[31]);
  acc[3] = sum2(u[15], acc[3]);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      w.pf[rb][kk] = u32x4{u[8 * rb + 4 * kk], u[8 * rb + 4 * kk + 1], u[8 * rb + 4 * kk + 2],
                           u[8 * rb + 4 * kk + 3]};
  // lazy-rescale check: each lane's tile sum at most 2^12 (so every
  // probability is, far below the fp16 limit) against a finite running max;
  // otherwise (rare) the slow path
  float tsum[2] = {acc[0] + acc[1], acc[2] + acc[3]};
  {
    const bool ok0 = (w.m[0] != -INFINITY) && (tsum[0] <= 4096.f);
    const bool ok1 = (w.m[1] != -INFINITY) && (tsum[1] <= 4096.f);
    if (wave_any(!(ok0 && ok1)))
      rescale_tile<CAUSAL, F16>(w, x, t, kbuf + (t % NBUF) * TB, wave_any(!ok0), wave_any(!ok1),
                                tsum);
  }
  w.l[0] += tsum[0];
  w.l[1] += tsum[1];
  // tile t+2's copies have landed (t+3's may still be in flight), this
  // wave's V^T writes are done; the barrier publishes both
  wait_vm_lds<COPIES>();
  barrier();
}

template <bool CAUSAL, bool F16, bool PRE = false>
__device__ __forceinline__ void tile_loop(Wave& w, const Ctx& x, char* kbuf, char* vbuf,
                                          char* vtbuf) {
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int db = 0; db < 4; ++db) w.o[rb][db] = f32x16{};
    w.m[rb] = -INFINITY;
    w.l[rb] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) w.pf[rb][kk] = u32x4{};
  }
  const int T = x.T;
  if (T <= 0) return;
  // prologue: V^T(-1) (ring slot 2, or 4 with prepared tiles) zeroed, copies
  // of tiles 0 .. AHEAD-1, V^T(0), S(0)
  char* vt_m1 = vtbuf + (PRE ? NVT - 1 : 2) * VTB;
  *(u32x4*)(vt_m1 + 32 * threadIdx.x) = u32x4{};
  *(u32x4*)(vt_m1 + 32 * threadIdx.x + 16) = u32x4{};
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) x.ld.issue<PRE>(i, i, i);
  wait_vm_lds<2 * COPIES>();
  barrier();   // tile 0 and the zeros visible
  if (!PRE) transpose_v<F16>(w, vbuf, vtbuf);
  qk_mfmas(w, w.s, kbuf);
  wait_vm_lds<COPIES>();
  barrier();   // tile 1 and V^T(0) visible
  // tiles before the first one that needs a mask (past Sk or past a row's
  // diagonal), then the masked ones; V^T ring of 3: tile t in slot t % 3
  int tm = T;
  {
    int lo = (x.Sk - BN) / BN + 1;             // first tile with a key past Sk
    if (x.Sk - BN < 0) lo = 0;
    if (CAUSAL) lo = min(lo, max(0, (w.first[0] + x.off + 1 - BN) / BN + 1));
    if (CAUSAL && w.first[0] + x.off + 1 - BN < 0) lo = 0;
    tm = min(T, lo);
  }
  tm = __builtin_amdgcn_readfirstlane(tm);
  int t = 0;
  for (; t < tm; ++t) iteration<CAUSAL, F16, false, PRE>(w, x, t, kbuf, vbuf, vtbuf);
  for (; t < T; ++t) iteration<CAUSAL, F16, true, PRE>(w, x, t, kbuf, vbuf, vtbuf);
  // drain: P(T-1).V(T-1); then the copies of the tiles past the loop (issued
  // by its last iterations) are waited for, so that nothing lands in the
  // rings after this point (the epilogue stages O there, a bf16 redo starts
  // its own copies)
  pv_mfmas<F16>(w, vtbuf + ((T - 1) % (PRE ? NVT : 3)) * VTB);
  wait_vm_lds<0>();
}

__device__ __forceinline__ bool state_finite(const Wave& w) {
  bool ok = __builtin_isfinite(w.l[0]) && __builtin_isfinite(w.l[1]);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) ok = ok && __builtin_isfinite(w.o[rb][db][r]);
  return ok;
}

template <bool CAUSAL, bool PRE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_pipe_kernel(PrefillArgs a) {
  // K ring, V ring (bf16), V^T ring of 3; with prepared V^T tiles their
  // ring of 5 starts at vbuf
  __shared__ __attribute__((aligned(1024))) char lds[2 * NBUF * TB + 3 * VTB];
  static_assert(NVT * VTB <= NBUF * TB + 3 * VTB, "LDS plan");
  char* const kbuf = lds;
  char* const vbuf = lds + NBUF * TB;
  char* const vtbuf = vbuf + NBUF * TB;

  Wave w;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  w.wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  w.l32 = lane & 31;
  w.hi = lane >> 5;

  // ---- which (batch, group of 4 query heads, 64-row query tile) this
  // workgroup computes: wave w takes query head 4*hg + w, the group sharing
  // one K/V head (the group size is a multiple of 4)
  const int NHG = a.Hq / NW;               // groups of 4 query heads per batch entry
  const int NBH = a.B * NHG;
  int bhg, qt;
  if (a.cu_q && (NBH & 7) == 0) {
    // packed sequences: the causal order below over head groups dealt to the
    // XCDs interleaved (XCD x takes groups x, x + 8, ...: every XCD gets a
    // share of each sequence, so none is left with the longest ones), each
    // XCD running 32 query tiles of one group at a time (its K/V in L2)
    int h;
    causal_xcd_order(blockIdx.x, NBH, a.n_qt, h, qt);
    const int hpx = NBH >> 3;
    bhg = (h % hpx) * 8 + h / hpx;
  } else if (a.cu_q) {
    const int row = blockIdx.x / NBH;      // heaviest query tiles first
    qt = a.n_qt - 1 - row;
    bhg = blockIdx.x - row * NBH;
  } else if (CAUSAL && (NBH & 7) == 0) {
    causal_xcd_order(blockIdx.x, NBH, a.n_qt, bhg, qt);
  } else if (CAUSAL) {
    const int row = blockIdx.x / NBH;      // heaviest query tiles first
    qt = a.n_qt - 1 - row;
    bhg = xcd_remap(blockIdx.x - row * NBH, NBH);
  } else {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    bhg = L / a.n_qt;
    qt = L - bhg * a.n_qt;
  }
  const int b = bhg / NHG;
  const int hq = (bhg - b * NHG) * NW + w.wave;   // this wave's query head
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
  const int q0 = qt * 64;
  if (q0 >= Sq) return;                  // whole workgroup: past this sequence's rows
  const __bf16* __restrict__ qp = a.q + qbase + hq * a.q_sh;
  const __bf16* kp = a.k + kbase + hk * a.k_sh;
  const __bf16* vp = a.v + kbase + hk * a.k_sh;

  Ctx x;
  x.off = Sk - Sq;
  x.Sk = Sk;
  x.c = a.c;
  const int last_row = min(q0 + 64, Sq) - 1;
  int n_keys = Sk;
  if (CAUSAL) n_keys = min(Sk, max(0, last_row + x.off + 1));
  x.T = (n_keys + BN - 1) / BN;
  // two 32-row blocks: rows q0 .. q0+31 and q0+32 .. q0+63
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) w.first[rb] = q0 + 32 * rb;
  x.ld.init(kp, vp, a.k_ss, Sk, w.wave, lane,
            __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(ATTN_LDS char*)kbuf),
            __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(ATTN_LDS char*)vbuf));
  if (PRE)
    x.ld.init_vt(a.vt + (int64_t)(b * a.Hkv + hk) * a.n_kt * VTB, a.n_kt, w.wave, lane,
                 __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(ATTN_LDS char*)vbuf));

  // ---- per-lane LDS offsets
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) w.koff[ks] = tile_off(w.l32, 2 * ks + w.hi);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) w.vtoff[kk] = vt_off(w.l32, 2 * kk + w.hi);
  // transposed reads of the bf16 V tile for d block `wave`: lane (beta =
  // lane/16, j = lane%16) addresses row 16*kk + 8*h + 4*hi + j/4, columns
  // 32*wave + 16*(beta&1) + 4*(j%4) .. +3; lane j of each 16-lane block then
  // receives keys 16*kk + 8*h + 4*hi + 0..3 of column 32*wave + 16*(beta&1) + j
  {
    const int j = lane & 15;
    const int chalf = (lane >> 4) & 1;
    const int col = w.wave * 32 + 16 * chalf + 4 * (j & 3);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 16 * kk + 8 * h + 4 * w.hi + (j >> 2);
        w.cvoff[kk][h] = tile_off(r, col >> 3) + (col & 7) * 2;
      }
  }

  // ---- Q fragments: row = query, k-slots = d
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = w.first[rb] + w.l32;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (row < Sq)
        w.qf[rb][ks] = *(const bf16x8*)(qp + (int64_t)row * a.q_ss + 16 * ks + 8 * w.hi);
      else
        w.qf[rb][ks] = bf16x8{};
    }
  }

  if (PRE)
    tile_loop<CAUSAL, true, true>(w, x, kbuf, vbuf, vbuf);
  else
    tile_loop<CAUSAL, true>(w, x, kbuf, vbuf, vtbuf);
  // A V value beyond the fp16 range (|v| >= 65520) or a non-finite input
  // shows up as a non-finite accumulator: redo this workgroup with bf16
  // probabilities and bf16 V, which covers the whole bf16 range.
  if (__syncthreads_or(!state_finite(w))) tile_loop<CAUSAL, false>(w, x, kbuf, vbuf, vtbuf);

  // ---- epilogue: O = acc / l (bf16 under the caller's rounding rule) in q's
  // layout; LSE = ln(sum exp).  O goes through LDS (the K and V rings are
  // free: every wave is past the loop's last barrier) so that each store
  // writes whole 256-byte rows, 16 bytes per lane.  Lane (row l32, half hi)
  // holds d = 32 db + 8 j + 4 hi + e of its row, i.e. 8 bytes of 16-byte
  // chunk 4 db + j; each wave stages its 64 rows (16 KB) and reads back only
  // its own rows.
  __syncthreads();
  char* st = (w.wave < 2 ? kbuf : vbuf) + (w.wave & 1) * 16384;
  float inv[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float l = sum_halves(w.l[rb]);
    w.l[rb] = l;
    inv[rb] = (l > 0.f) ? 1.f / l : 0.f;
  }
  with_rounding(a.rounding, [&](auto mode) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 u;
          u[0] = pack_bf16_as<mode()>(w.o[rb][db][4 * j + 0] * inv[rb],
                                      w.o[rb][db][4 * j + 1] * inv[rb]);
          u[1] = pack_bf16_as<mode()>(w.o[rb][db][4 * j + 2] * inv[rb],
                                      w.o[rb][db][4 * j + 3] * inv[rb]);
          *(u32x2*)(st + tile_off(32 * rb + w.l32, 4 * db + j) + 8 * w.hi) = u;
        }
  });
  wait_vm_lds<0>();
  __bf16* ob = a.o + qbase + hq * a.q_sh;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int rr = 4 * k + (lane >> 4), cc = lane & 15;
    const u32x4 v = *(const u32x4*)(st + tile_off(rr, cc));
    const int row = w.first[rr >> 5] + (rr & 31);
    if (row < Sq) *(u32x4*)(ob + (int64_t)row * a.q_ss + 8 * cc) = v;
  }
  if (w.hi == 0) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = w.first[rb] + w.l32;
      if (row < Sq) {
        const float l = w.l[rb];
        a.lse[lse_base + row] =
            (l > 0.f) ? (w.m[rb] + __log2f(l)) * kLn2 : -INFINITY;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill_pipe(const PrefillArgs& a, bool causal, hipStream_t stream) {
  if ((a.cu_q && a.vt) || a.alibi || a.group % NW) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)a.B * (a.Hq / NW) * a.n_qt;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidValue;
  if (a.vt && a.n_kt != (a.Sk + BN - 1) / BN) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), blk(NT);
  if (a.vt) {
    if (causal)
      hipLaunchKernelGGL((prefill_pipe_kernel<true, true>), g, blk, 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_pipe_kernel<false, true>), g, blk, 0, stream, a);
  } else if (causal) {
    hipLaunchKernelGGL((prefill_pipe_kernel<true, false>), g, blk, 0, stream, a);
  } else {
    hipLaunchKernelGGL((prefill_pipe_kernel<false, false>), g, blk, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attn
