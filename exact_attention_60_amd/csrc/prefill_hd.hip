// Exact attention forward for head dim 64 on gfx950: O = softmax(scale Q K^T) V
// with the same online softmax as the d = 128 kernel ("IO-aware tiling
// strategy in FlashAttention-4", body: Q in row tiles, K/V in column tiles
// brought on chip, a running row max m and denominator l merged block by
// block, the output accumulator rescaled by a per-row factor and divided by
// l once at the end).  Head dims other than 128 are what the MoonMath page's
// kernel leaves out ("MoonMath AI open-sources a HIP attention kernel for AMD
// MI300X that beats AITER v3", scope paragraph: head dim fixed at 128).
//
// Design (gfx950):
//  * one workgroup = 4 waves = 128 query rows of one (batch, query head); a
//    wave owns 32 rows, with its Q fragments and the fp32 O^T accumulator in
//    registers (about 110 VGPRs, so several workgroups share a CU).
//  * K and V tiles of 64 keys (128-byte rows) are copied HBM -> LDS by
//    buffer_load ... lds, double buffered one tile ahead; rows are XOR-swizzled
//    in 16-byte chunks; keys past Sk fall outside the buffer range and read 0.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 puts one query row in each lane
//    column (its 32 keys split over the two lane halves), so the row max and
//    sum are in-lane plus one v_permlane32_swap, the rescale factor is a
//    per-lane scalar for O^T, and the probabilities are directly the B
//    operand of O^T += V^T P^T, whose V^T operand comes from the row-major V
//    tile through ds_read_b64_tr_b16.
//  * P.V runs in fp16 (each wave converts the V rows it copied, in LDS, before
//    the tile's barrier; P rounded to fp16,
//    l summed from the rounded P), as the d = 128 kernel does; a V value
//    beyond the fp16 range or a non-finite input leaves a non-finite
//    accumulator and the workgroup redoes its tiles in bf16.
//  * Causal: tiles past the diagonal are never loaded, waves whose rows see
//    none of a 32-key half skip it, only boundary halves are masked, heaviest
//    query blocks are dispatched first.
#include "gfx950.hpp"
#include "kernels.h"

namespace attn {
namespace {

constexpr int NW = 4;
constexpr int NT = NW * 64;
constexpr int QR = NW * 32;    // query rows per workgroup
static_assert(QR == kPrefillHdRows, "rows per workgroup");

template <int D>
struct Geom {
  static constexpr int KB = D <= 64 ? 64 : 32;   // keys per tile (LDS: 2 stages of K and V)
  static constexpr int RB = D * 2;               // bytes per row
  static constexpr int NC = RB / 16;             // 16-byte chunks per row
  static constexpr int TILE = KB * RB;           // one K or V tile
  static constexpr int KS = D / 16;              // MFMA k-steps over d
  static constexpr int NTD = D / 32;             // 32-wide d blocks of O^T
  static constexpr int RPI = 1024 / RB;          // rows per 1 KB copy instruction
  static constexpr int IPW = KB / RPI / NW;      // copy instructions per wave per tile
  static_assert(IPW >= 1 && IPW * RPI * NW == KB && KB % 32 == 0, "tile layout");
};

// Chunk swizzle of a row: for 8-chunk rows a bijection on rows 0..7 that
// also sends the 4 consecutive rows of a transpose read to 4 different chunk
// pairs; for longer rows the 4-bit version of the same idea.
template <int NC>
__device__ __forceinline__ int hd_swz(int r) {
  if constexpr (NC == 8) return ((r & 3) << 1) | ((r >> 2) & 1);
  else return ((r & 3) << 2) | ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int hd_off(int row, int chunk) {
  return row * Geom<D>::RB + ((chunk ^ hd_swz<Geom<D>::NC>(row & 15)) << 4);
}
template <int D>
__device__ __forceinline__ int hd_elem(int row, int col) {   // col a multiple of 4
  return hd_off<D>(row, col >> 3) + ((col & 7) << 1);
}

__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int per = n >> 3;
  return (i < (per << 3)) ? (i & 7) * per + (i >> 3) : i;
}
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0x0070); }
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D>
struct Copier {
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t voff[Geom<D>::IPW];
  uint32_t tile_bytes;
  int row0;
  __device__ void init(const __bf16* kp, const __bf16* vp, int64_t ss, int Sk, int wave,
                       int lane) {
    constexpr int RPI = Geom<D>::RPI, NC = Geom<D>::NC;
    const uint32_t sb = (uint32_t)(ss * 2);
    const uint32_t nrec = Sk > 0 ? (uint32_t)((int64_t)(Sk - 1) * sb + Geom<D>::RB) : 0u;
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)kp, (short)0, (int)nrec, 0x00020000);
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)vp, (short)0, (int)nrec, 0x00020000);
    tile_bytes = sb * Geom<D>::KB;
    row0 = wave * Geom<D>::IPW * RPI;
#pragma unroll
    for (int j = 0; j < Geom<D>::IPW; ++j) {
      const int row = row0 + j * RPI + lane / NC;
      const int c = (lane % NC) ^ hd_swz<NC>(row & 15);
      voff[j] = (uint32_t)row * sb + (uint32_t)c * 16;
    }
  }
  // prepared fp16 V tiles (the LDS image of a converted tile): this wave's
  // rows are a contiguous IPW KB of the tile
  __amdgpu_buffer_rsrc_t rvt;
  uint32_t vt_lane;
  __device__ void init_vt(const uint8_t* vtp, int n_kt, int wave, int lane) {
    rvt = __builtin_amdgcn_make_buffer_rsrc((void*)vtp, (short)0,
                                            (int)((uint32_t)n_kt * (uint32_t)Geom<D>::TILE),
                                            0x00020000);
    vt_lane = (uint32_t)(wave * Geom<D>::IPW * 1024 + lane * 16);
  }
  // pre: V from the prepared tiles
  __device__ __forceinline__ void issue(int t, char* kt, char* vt, bool pre) const {
    const uint32_t base = (uint32_t)t * tile_bytes;
#pragma unroll
    for (int j = 0; j < Geom<D>::IPW; ++j) {
      const int r = row0 + j * Geom<D>::RPI;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (ATTN_LDS void*)(kt + r * Geom<D>::RB), 16,
                                               voff[j] + base, 0, 0, 0);
      if (pre)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rvt, (ATTN_LDS void*)(vt + r * Geom<D>::RB), 16,
            (uint32_t)t * (uint32_t)Geom<D>::TILE + vt_lane + 1024u * j, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (ATTN_LDS void*)(vt + r * Geom<D>::RB), 16,
                                                 voff[j] + base, 0, 0, 0);
    }
  }
};

template <int D>
struct HdState {
  bf16x8 qf[Geom<D>::KS];       // B operand of S^T = K Q^T (row = lane % 32)
  f32x16 oacc[Geom<D>::NTD];    // O^T, d blocks of 32
  float m;                      // running row max, log2 units (scale*log2e folded in)
  float l;                      // this lane's part of the row sum
};

// The tile loop; F16 selects fp16 (else bf16) for P and V.  Operand
// addresses are per-lane offsets computed once (the second 32-key half of a
// tile, and the rows 16 and 8 further on, keep the same swizzle, so they are
// instruction offsets).  Lazy rescale as in the d = 128 kernels: the
// probabilities are taken against the running max as it stands while a
// lane's sum over the 32 keys stays <= 2^12 (every value then far below the
// fp16 limit, and O = sum p v / sum p does not depend on the max); a row's
// first keys, or a larger sum, take the row max, rescale and recompute.  The
// bf16 redo always takes the row max: with 8 significant bits the dominant
// probability of a short, peaky row must be exactly 1, not a rounded power
// of two off a stale max.
// With prepared tiles (PRE) the V copies bring fp16 rows and there is no
// conversion.  KPRE is the calling kernel's variant: each kernel instantiates
// its own copies of the loop (the host pass of the compiler rejects one
// specialization taking the buffer-descriptor struct from two kernels).
template <int D, bool CAUSAL, bool F16, bool PRE, bool KPRE>
__device__ __forceinline__ void hd_loop(HdState<D>& w, const Copier<D>& cp, char* kbuf,
                                        char* vbuf, int n_kt, int n_keys, int Sk, int Sq, int off,
                                        int qw0, int wave_last, float c, int lane) {
  constexpr bool pre = PRE;
  constexpr int TILE = Geom<D>::TILE, RB = Geom<D>::RB;
  const int cl = lane & 31, h = lane >> 5;
  const int q = qw0 + cl;
  // K operand of k-step ks: key row cl of the half, d = 16ks + 8h .. +7
  int koff[Geom<D>::KS];
#pragma unroll
  for (int ks = 0; ks < Geom<D>::KS; ++ks) koff[ks] = hd_off<D>(cl, 2 * ks + h);
  // V^T operand of d block n (two transposed reads, rows r and r + 8): in
  // each 16-lane group lane L addresses row 4h + L/4 and the 4 columns from
  // 32n + 16 ((lane >> 4) & 1) + 4 (L % 4)
  int voffs[Geom<D>::NTD];
  {
    const int L = lane & 15;
#pragma unroll
    for (int n = 0; n < Geom<D>::NTD; ++n)
      voffs[n] = hd_elem<D>(4 * h + (L >> 2), 32 * n + 16 * ((lane >> 4) & 1) + 4 * (L & 3));
  }
#pragma unroll
  for (int n = 0; n < Geom<D>::NTD; ++n) w.oacc[n] = f32x16{};
  w.m = -INFINITY;
  w.l = 0.f;
  if (n_kt > 0) cp.issue(0, kbuf, vbuf, pre);
  for (int t = 0; t < n_kt; ++t) {
    const int st = t & 1;
    char* kt = kbuf + st * TILE;
    char* vt = vbuf + st * TILE;
    wait_all();    // this wave's copies of tile t have landed
    if constexpr (F16 && !PRE) {
      // bf16 -> fp16 in place for the V rows this wave copied (each lane the
      // 16 bytes its copy instructions wrote), before the barrier publishes
      // the tile; no other wave touches these rows meanwhile
#pragma unroll
      for (int j = 0; j < Geom<D>::IPW; ++j) {
        u32x4* pch = reinterpret_cast<u32x4*>(
            vt + (cp.row0 + j * Geom<D>::RPI) * Geom<D>::RB + 16 * lane);
        u32x4 x = *pch;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = bf16x2_to_f16x2(x[e]);
        *pch = x;
      }
      wait_all();
    }
    barrier();   // tile t is complete for every wave; tile t-1 is no longer read
    if (t + 1 < n_kt) cp.issue(t + 1, kbuf + (st ^ 1) * TILE, vbuf + (st ^ 1) * TILE, pre);
#pragma unroll
    for (int ks2 = 0; ks2 < Geom<D>::KB / 32; ++ks2) {
      const int kr0 = t * Geom<D>::KB + 32 * ks2;
      if (kr0 >= n_keys || qw0 >= Sq) continue;
      if (CAUSAL && kr0 > wave_last + off) continue;   // no row of the wave sees these keys
      const bool mask = (CAUSAL && kr0 + 31 > qw0 + off) || (kr0 + 32 > Sk);
      // S^T[key][q]: register r of lane (cl, h) holds key kr0 + 8*(r/4) + 4h + r%4
      // K rows read four k-steps at a time ahead of their MFMAs
      const char* kh = kt + 32 * ks2 * RB;
      f32x16 s = f32x16{};
#pragma unroll
      for (int k0 = 0; k0 < Geom<D>::KS; k0 += 4) {
        bf16x8 ka[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ka[i] = *reinterpret_cast<const bf16x8*>(kh + koff[k0 + i]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) s = mfma32(ka[i], w.qf[k0 + i], s);
      }
      if (mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kr0 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key >= Sk || (CAUSAL && key > q + off)) s[r] = -INFINITY;
        }
      }
      // probabilities of row q over these 32 keys (16 per lane half) against
      // msub, packed as the B operand of P.V; returns the lane's sum of the
      // rounded values
      uint32_t pk[8];
      auto probs = [&](float msub) {
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p0 = fast_exp2(__builtin_fmaf(s[2 * i], c, -msub));
          const float p1 = fast_exp2(__builtin_fmaf(s[2 * i + 1], c, -msub));
          pk[i] = F16 ? pack_f16(p0, p1) : pack_bf16(p0, p1);
          if (i & 1) t1 = F16 ? sum2_f16(pk[i], t1) : sum2_bf16(pk[i], t1);
          else t0 = F16 ? sum2_f16(pk[i], t0) : sum2_bf16(pk[i], t0);
        }
        return t0 + t1;
      };
      float tsum = F16 ? probs(w.m == -INFINITY ? 0.f : w.m) : 0.f;
      if (!F16 || wave_any(!(w.m != -INFINITY && tsum <= 4096.f))) {
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = max_halves(mx);
        const float m_new = fmaxf(w.m, mx * c);
        const float alpha = (m_new == w.m) ? 1.f : fast_exp2(w.m - m_new);
        w.l *= alpha;
#pragma unroll
        for (int n = 0; n < Geom<D>::NTD; ++n) w.oacc[n] *= alpha;
        w.m = m_new;
        tsum = probs(m_new == -INFINITY ? 0.f : m_new);
      }
      w.l += tsum;
      // O^T[d][q] += sum_key V^T[d][key] P^T[key][q]
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x4 pb = {pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]};
        const char* vr = vt + (32 * ks2 + 16 * u) * RB;
#pragma unroll
        for (int n = 0; n < Geom<D>::NTD; ++n) {
          const bf16x4 lo = lds_read_tr(vr + voffs[n]);
          const bf16x4 hi = lds_read_tr(vr + voffs[n] + 8 * RB);
          const bf16x8 va = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          if constexpr (F16)
            w.oacc[n] = mfma32(__builtin_bit_cast(f16x8, va), __builtin_bit_cast(f16x8, pb),
                               w.oacc[n]);
          else
            w.oacc[n] = mfma32(va, __builtin_bit_cast(bf16x8, pb), w.oacc[n]);
        }
      }
    }
  }
}

template <int D>
__device__ __forceinline__ bool hd_finite(const HdState<D>& w) {
  bool ok = __builtin_isfinite(w.l);
#pragma unroll
  for (int n = 0; n < Geom<D>::NTD; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) ok = ok && __builtin_isfinite(w.oacc[n][r]);
  return ok;
}

// Occupancy at d = 64: four waves per SIMD without the causal mask code (124
// VGPRs), three with it (the mask paths need more registers; four would
// spill).  At d = 256 the Q fragments and O^T alone take 192 registers, and
// the budget of two waves per SIMD spills: one.
template <int D, bool CAUSAL, bool PRE>
__global__ __launch_bounds__(NT)
__attribute__((amdgpu_waves_per_eu(D > 64 ? 1 : (CAUSAL ? 3 : 4), D > 64 ? 1 : 4)))
void prefill_hd_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) char kbuf[2 * Geom<D>::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf[2 * Geom<D>::TILE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cl = lane & 31, h = lane >> 5;
  const int n_qb = a.n_qt;
  const int BH = a.B * a.Hq;
  int bh, qb;
  if (CAUSAL) {
    const int row = blockIdx.x / BH;     // heaviest query blocks first
    qb = n_qb - 1 - row;
    bh = xcd_remap(blockIdx.x - row * BH, BH);
  } else {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    bh = L / n_qb;
    qb = L - bh * n_qb;
  }
  const int b = bh / a.Hq, hq = bh - b * a.Hq;
  const int hk = hq / a.group;
  const int Sq = a.Sq, Sk = a.Sk, off = Sk - Sq;
  const __bf16* qp = a.q + b * a.q_sb + hq * a.q_sh;
  const __bf16* kp = a.k + b * a.k_sb + hk * a.k_sh;
  const __bf16* vp = a.v + b * a.k_sb + hk * a.k_sh;
  const int q0 = qb * QR;
  const int qw0 = q0 + 32 * wave;
  const int q = qw0 + cl;
  const int last_row = min(q0 + QR, Sq) - 1;
  const int n_keys = CAUSAL ? min(Sk, max(0, last_row + off + 1)) : Sk;
  const int n_kt = (n_keys + Geom<D>::KB - 1) / Geom<D>::KB;
  const int wave_last = min(qw0 + 31, Sq - 1);

  HdState<D> w;
#pragma unroll
  for (int ks = 0; ks < Geom<D>::KS; ++ks) {
    if (q < Sq)
      w.qf[ks] = *reinterpret_cast<const bf16x8*>(qp + (int64_t)q * a.q_ss + 16 * ks + 8 * h);
    else
      w.qf[ks] = bf16x8{};
  }
  Copier<D> cp;
  cp.init(kp, vp, a.k_ss, Sk, wave, lane);
  if (PRE) cp.init_vt(a.vt + (int64_t)(b * a.Hkv + hk) * a.n_kt * Geom<D>::TILE, a.n_kt, wave, lane);

  hd_loop<D, CAUSAL, true, PRE, PRE>(w, cp, kbuf, vbuf, n_kt, n_keys, Sk, Sq, off, qw0,
                                     wave_last, a.c, lane);
  if (__syncthreads_or(!hd_finite(w)))
    hd_loop<D, CAUSAL, false, false, PRE>(w, cp, kbuf, vbuf, n_kt, n_keys, Sk, Sq, off, qw0,
                                          wave_last, a.c, lane);

  // epilogue: O = O^T / l in q's layout (register r of lane (cl, h), d block
  // n: d = 32n + 8*(r/4) + 4h + r%4), LSE = (m + log2 l) ln 2
  const float L = sum_halves(w.l);
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  if (q < Sq) {
    __bf16* orow = a.o + b * a.q_sb + hq * a.q_sh + (int64_t)q * a.q_ss;
    with_rounding(a.rounding, [&](auto mode) {
#pragma unroll
      for (int n = 0; n < Geom<D>::NTD; ++n)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 u;
          u[0] = pack_bf16_as<mode()>(w.oacc[n][4 * g] * inv, w.oacc[n][4 * g + 1] * inv);
          u[1] = pack_bf16_as<mode()>(w.oacc[n][4 * g + 2] * inv, w.oacc[n][4 * g + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + 32 * n + 8 * g + 4 * h) = u;
        }
    });
    if (h == 0)
      a.lse[((int64_t)(b * a.Hq + hq)) * Sq + q] = (L > 0.f) ? (w.m + __log2f(L)) * kLn2 : -INFINITY;
  }
}

// V of one (batch, K/V head) as the fp16 tiles of the prepared path: tile t
// (keys 64t .. 64t+63, zeros past Sk) goes to vt + ((b * Hkv + h) * n_kt + t)
// * TILE as exactly the LDS image the converting path builds (rows of 128
// bytes, hd_off's chunk swizzle, each value rounded to fp16, nearest even).
// HBM-bound: 8 KB read and 8 KB written per tile.
__global__ __launch_bounds__(256) void prep_v_d64_kernel(PrepVArgs a) {
  constexpr int D = 64, NC = Geom<D>::NC, TILE = Geom<D>::TILE;
  const int64_t id = blockIdx.x;
  const int t = (int)(id % a.n_kt);
  const int64_t bh = id / a.n_kt;
  const int h = (int)(bh % a.Hkv);
  const int b = (int)(bh / a.Hkv);
  const __bf16* vp = a.v + b * a.k_sb + h * a.k_sh;
  uint8_t* out = a.vt + id * TILE;
#pragma unroll
  for (int pass = 0; pass < TILE / (256 * 16); ++pass) {
    const int idx = 256 * pass + threadIdx.x;
    const int row = idx / NC, c = idx % NC;
    const int key = t * Geom<D>::KB + row;
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    if (key < a.Sk) x = *(const u32x4*)(vp + (int64_t)key * a.k_ss + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = bf16x2_to_f16x2(x[e]);
    *(u32x4*)(out + hd_off<D>(row, c)) = x;
  }
}

}  // namespace

hipError_t launch_prefill_hd(const PrefillArgs& a, bool causal, hipStream_t stream) {
  const int64_t grid = (int64_t)a.B * a.Hq * a.n_qt;
  if (grid <= 0 || grid > 0x7fffffff || a.cu_q || a.alibi) return hipErrorInvalidValue;
  if (a.vt && a.n_kt != (a.Sk + Geom<64>::KB - 1) / Geom<64>::KB) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), bt(NT);
  if (a.vt) {
    if (causal) hipLaunchKernelGGL((prefill_hd_kernel<64, true, true>), g, bt, 0, stream, a);
    else hipLaunchKernelGGL((prefill_hd_kernel<64, false, true>), g, bt, 0, stream, a);
  } else if (causal) {
    hipLaunchKernelGGL((prefill_hd_kernel<64, true, false>), g, bt, 0, stream, a);
  } else {
    hipLaunchKernelGGL((prefill_hd_kernel<64, false, false>), g, bt, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_prep_v_d64(const PrepVArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.B * a.Hkv * a.n_kt;
  if (grid <= 0 || grid > 0x7fffffff || a.tk != Geom<64>::KB ||
      a.n_kt != (a.Sk + Geom<64>::KB - 1) / Geom<64>::KB)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(prep_v_d64_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
