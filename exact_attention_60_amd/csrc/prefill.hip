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
// Design (MI355X-first, not the pages' NVIDIA or gfx942 kernels):
//  * one workgroup = 4 waves = 256 query rows of one (batch, query head);
//    each wave owns 64 rows as two 32-row MFMA blocks, with its Q fragments
//    and fp32 output accumulators in registers (the data placement of the
//    MoonMath page's kernel keeps Q and the accumulators in registers too);
//  * K and V tiles of 64 keys are copied HBM -> LDS directly by the buffer
//    unit (buffer_load ... lds, 16 B per lane, 256 B contiguous per row),
//    double buffered: tile t+1 is in flight while tile t is computed, one
//    barrier per tile.  Both K and V sit in LDS (160 KB per CU on gfx950); rows are 256 B
//    with an XOR swizzle of their 16-byte chunks so that the MFMA operand reads
//    are free of bank conflicts;
//  * scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16:
//    the accumulator then holds one query row per lane (half of the keys in
//    each lane half), so the row max and row sum are in-lane plus one
//    v_permlane32_swap, and the bf16-packed probabilities are already the
//    B operand of O^T = V^T P^T without any data movement;
//  * the V^T operand comes straight from the row-major V tile through the
//    gfx950 LDS transpose read (ds_read_b64_tr_b16);
//  * P.V runs in fp16 (11 significant bits; bf16 keeps 8, too few for the
//    parity bound when a few large V entries nearly cancel): each V tile is
//    converted to fp16 once in LDS, and the denominator sums the same rounded
//    probabilities that multiply V.  A V value outside the fp16 range (or a
//    non-finite input) makes the accumulator non-finite; the workgroup then
//    redoes its tile loop with bf16 P and V, which covers the bf16 range;
//  * the rescale of the output accumulator is skipped while no row max in the
//    wave has grown by more than 2^8 (probabilities stay <= 256, far from fp32
//    or bf16 limits); the result is the same quotient, so it stays exact;
//  * causal: tiles above the diagonal are never loaded, waves whose rows see
//    none of a tile skip its arithmetic, only boundary tiles are masked, and
//    the heaviest query tiles are dispatched first;
//  * blockIdx is remapped so that workgroups sharing K/V land on one XCD
//    (workgroups are dealt to the 8 XCDs round robin), keeping K/V re-reads in
//    that XCD's L2.
#include "gfx950.hpp"
#include "kernels.h"

namespace attn {
namespace {

constexpr int D = kHeadDim;
constexpr int BN = kPrefillBN;
constexpr int BM = kPrefillBM;
constexpr int NT = kPrefillWaves * 64;
constexpr int QB = kPrefillRowsPerWave / 32;
constexpr int TILE_BYTES = BN * D * 2;      // 16 KB for one K or V tile
constexpr float TAU = 8.0f;                 // log2 headroom before a rescale

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

// Asynchronous copy of one K or V tile (64 keys x 256 B) from HBM straight
// into LDS (buffer_load_dwordx4 ... lds): each wave moves 16 rows with four
// instructions of 1 KB; lane i of an instruction lands at byte 16*i of that
// 1 KB, i.e. row +i/16, physical chunk i%16, so it fetches the logical chunk
// that the swizzle places there.  Keys >= Sk are outside the buffer's range
// and read as zeros.
struct TileLoader {
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t voff[4];       // per-lane byte offset of this lane's chunk, row j*4 + lane/16
  uint32_t tile_bytes;    // BN * row stride in bytes
  int lds_row0;           // first tile row this wave fills (16 * wave)

  __device__ void init(const __bf16* kp, const __bf16* vp, int64_t k_ss, int Sk, int wave,
                       int lane) {
    const uint32_t ss = (uint32_t)(k_ss * 2);
    const uint32_t nrec = (uint32_t)((int64_t)(Sk - 1) * ss + 256);
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)kp, (short)0, (int)nrec, 0x00020000);
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)vp, (short)0, (int)nrec, 0x00020000);
    tile_bytes = ss * BN;
    lds_row0 = 16 * wave;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = lds_row0 + 4 * j + (lane >> 4);
      const int c = (lane & 15) ^ swz(row & 15);
      voff[j] = (uint32_t)row * ss + (uint32_t)c * 16;
    }
  }
  __device__ __forceinline__ void issue(int tile, char* kt, char* vt) const {
    const uint32_t base = (uint32_t)tile * tile_bytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lds_off = (lds_row0 + 4 * j) * 256;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (ATTN_LDS void*)(kt + lds_off), 16,
                                               voff[j] + base, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (ATTN_LDS void*)(vt + lds_off), 16,
                                               voff[j] + base, 0, 0, 0);
    }
  }
};

__device__ __forceinline__ void wait_tile_loads() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Converts, in place, the 4 x 16 B of a V tile that this lane's own copy
// instructions brought into LDS from bf16 to fp16 (the lane waited for its
// copies, so the bytes are there; the following barrier publishes them).
__device__ __forceinline__ void convert_v_share(char* vt, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4* p = (u32x4*)(vt + (16 * wave + 4 * j) * 256 + lane * 16);
    u32x4 x = *p;
    u32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = bf16x2_to_f16x2(x[i]);
    *p = y;
  }
}

// Per-wave state of the forward: Q fragments, output accumulators, running
// row max (log2 units) and the lane's partial row sum.
struct WaveState {
  bf16x8 qf[QB][8];
  f32x16 oacc[QB][4];
  float m_use[QB];
  float lsum[QB];
};

// One K/V tile of the online softmax for one wave.  F16: the probabilities
// and the V tile are fp16 for O^T += V^T P^T (V was converted in LDS);
// otherwise both are bf16.
template <bool CAUSAL, bool F16>
__device__ __forceinline__ void tile_step(WaveState& st, const char* kt, const char* vt,
                                          const int (&koff)[8], const int (&voff)[2][4],
                                          int kbase, int w_first, int Sk, int off, float c,
                                          int l32, int hi) {
  // ---- S^T = K Q^T for 64 keys x 64 rows
  f32x16 s[2][QB];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 kf = *(const bf16x8*)(kt + kb * 32 * 256 + koff[ks]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma32(kf, st.qf[qb][ks], s[kb][qb]);
    }
  }
  // ---- mask key tails and the causal diagonal (boundary tiles only)
  const bool need_mask = (kbase + BN > Sk) || (CAUSAL && kbase + BN - 1 > w_first + off);
  if (need_mask) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = w_first + qb * 32 + l32;
      const int lim = (CAUSAL ? min(Sk - 1, row + off) : Sk - 1) - kbase - 4 * hi;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + (r & 3);
          if (key > lim) s[kb][qb][r] = -INFINITY;
        }
    }
  }
  // ---- online softmax; P packed as the B operand of O^T += V^T P^T.  The
  // denominator sums the rounded probabilities, the same weights that
  // multiply V.
  u32x4 pf[QB][2][2];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float mx = s[0][qb][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
    mx = max_halves(mx);
    const float m_tile = mx * c;
    if (wave_any(m_tile > st.m_use[qb] + TAU)) {
      const float m_new = fmaxf(st.m_use[qb], m_tile);
      const float alpha = (m_new == st.m_use[qb]) ? 1.f : fast_exp2(st.m_use[qb] - m_new);
      st.lsum[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) st.oacc[qb][db] *= alpha;
      st.m_use[qb] = m_new;
    }
    const float msub = (st.m_use[qb] == -INFINITY) ? 0.f : st.m_use[qb];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = fast_exp2(__builtin_fmaf(s[kb][qb][8 * e + i], c, -msub));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t u = F16 ? pack_f16(p[2 * i], p[2 * i + 1])
                                 : pack_bf16(p[2 * i], p[2 * i + 1]);
          pf[qb][kb][e][i] = u;
          st.lsum[qb] = F16 ? sum2_f16(u, st.lsum[qb]) : sum2_bf16(u, st.lsum[qb]);
        }
      }
  }
  // ---- O^T += V^T P^T
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const char* base = vt + (kb * 32 + 16 * e) * 256;
        const bf16x4 lo = lds_read_tr(base + voff[0][db]);
        const bf16x4 up = lds_read_tr(base + voff[1][db]);
        const bf16x8 vb = {lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if (F16)
            st.oacc[qb][db] = mfma32(__builtin_bit_cast(f16x8, vb),
                                     __builtin_bit_cast(f16x8, pf[qb][kb][e]), st.oacc[qb][db]);
          else
            st.oacc[qb][db] = mfma32(vb, __builtin_bit_cast(bf16x8, pf[qb][kb][e]),
                                     st.oacc[qb][db]);
        }
      }
  }
}

struct LoopCtx {
  TileLoader ld;
  int koff[8];
  int voff[2][4];
  int n_tiles, w_first, w_last, Sk, off, wave, lane, l32, hi;
  bool w_any;
  float c;
};

// The tile loop of one workgroup: K/V tiles double buffered in kv0/kv1, tile
// t+1 copied while tile t is computed; with F16 each lane converts the V
// bytes it copied to fp16 before the barrier that publishes the tile.
template <bool CAUSAL, bool F16>
__device__ __forceinline__ void tile_loop(WaveState& st, const LoopCtx& x, char* kv0, char* kv1) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < 4; ++db) st.oacc[qb][db] = f32x16{};
    st.m_use[qb] = -INFINITY;
    st.lsum[qb] = 0.f;
  }
  if (x.n_tiles > 0) {
    x.ld.issue(0, kv0, kv0 + TILE_BYTES);
    wait_tile_loads();
    if (F16) convert_v_share(kv0 + TILE_BYTES, x.wave, x.lane);
  }
  __syncthreads();
  auto visible = [&](int kbase) {
    return x.w_any && (!CAUSAL || kbase <= x.w_last + x.off);
  };
  // two tiles per trip so that each buffer index is a compile-time constant
  for (int t = 0; t < x.n_tiles; t += 2) {
    const bool more1 = t + 1 < x.n_tiles;
    if (more1) x.ld.issue(t + 1, kv1, kv1 + TILE_BYTES);
    if (visible(t * BN))
      tile_step<CAUSAL, F16>(st, kv0, kv0 + TILE_BYTES, x.koff, x.voff, t * BN, x.w_first, x.Sk,
                             x.off, x.c, x.l32, x.hi);
    if (more1) {
      wait_tile_loads();
      if (F16) convert_v_share(kv1 + TILE_BYTES, x.wave, x.lane);
    }
    __syncthreads();
    if (!more1) break;
    const bool more2 = t + 2 < x.n_tiles;
    if (more2) x.ld.issue(t + 2, kv0, kv0 + TILE_BYTES);
    if (visible((t + 1) * BN))
      tile_step<CAUSAL, F16>(st, kv1, kv1 + TILE_BYTES, x.koff, x.voff, (t + 1) * BN, x.w_first,
                             x.Sk, x.off, x.c, x.l32, x.hi);
    if (more2) {
      wait_tile_loads();
      if (F16) convert_v_share(kv0 + TILE_BYTES, x.wave, x.lane);
    }
    __syncthreads();
  }
}

__device__ __forceinline__ bool state_finite(const WaveState& st) {
  bool ok = true;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    ok = ok && __builtin_isfinite(st.lsum[qb]);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) ok = ok && __builtin_isfinite(st.oacc[qb][db][r]);
  }
  return ok;
}

template <bool CAUSAL>
__global__ __launch_bounds__(NT, 1) void prefill_kernel(PrefillArgs a) {
  // two K/V buffers as separate arrays so that the copy into one provably
  // does not alias the reads of the other
  __shared__ __attribute__((aligned(1024))) char kv0[2 * TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kv1[2 * TILE_BYTES];

  LoopCtx x;
  const int tid = threadIdx.x;
  x.lane = tid & 63;
  x.wave = tid >> 6;
  x.l32 = x.lane & 31;
  x.hi = x.lane >> 5;
  const int lane = x.lane, hi = x.hi, l32 = x.l32;

  // ---- which (batch, head, query tile) this workgroup computes
  const int BH = a.B * a.Hq;
  int bh, qt;
  if (CAUSAL) {
    const int row = blockIdx.x / BH;            // heaviest query tiles first
    qt = a.n_qt - 1 - row;
    bh = xcd_remap(blockIdx.x - row * BH, BH);
  } else {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    bh = L / a.n_qt;
    qt = L - bh * a.n_qt;
  }
  const int b = bh / a.Hq;
  const int hq = bh - b * a.Hq;
  const int hk = hq / a.group;
  const __bf16* __restrict__ qp = a.q + b * a.q_sb + hq * a.q_sh;
  const __bf16* kp = a.k + b * a.k_sb + hk * a.k_sh;
  const __bf16* vp = a.v + b * a.k_sb + hk * a.k_sh;

  const int q0 = qt * BM;
  x.off = a.Sk - a.Sq;                          // causal: key j visible iff j <= i + off
  x.Sk = a.Sk;
  x.c = a.c;
  const int last_row = min(q0 + BM, a.Sq) - 1;
  int n_keys = a.Sk;
  if (CAUSAL) n_keys = min(a.Sk, max(0, last_row + x.off + 1));
  x.n_tiles = (n_keys + BN - 1) / BN;
  x.w_first = q0 + x.wave * kPrefillRowsPerWave;                  // wave's rows
  x.w_last = min(x.w_first + kPrefillRowsPerWave, a.Sq) - 1;
  x.w_any = x.w_first < a.Sq;
  x.ld.init(kp, vp, a.k_ss, a.Sk, x.wave, lane);

  // ---- per-lane LDS offsets
  // K operand (A of S^T): row kb*32 + l32, chunk 2*ks + hi
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) x.koff[ks] = tile_off(l32, 2 * ks + hi);
  // V^T operand via transpose reads: lane (block beta = lane/16, j = lane%16)
  // addresses row base + 4*hi + j/4, columns db*32 + 16*(beta&1) + 4*(j%4)
  {
    const int j = lane & 15;
    const int chalf = (lane >> 4) & 1;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int r = 8 * w + 4 * hi + (j >> 2);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int col = db * 32 + 16 * chalf + 4 * (j & 3);
        x.voff[w][db] = tile_off(r, col >> 3) + (col & 7) * 2;
      }
    }
  }

  WaveState st;
  // ---- Q fragments (B operand of S^T = K Q^T): row = query, k-slots = d
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = x.w_first + qb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (row < a.Sq)
        st.qf[qb][ks] = *(const bf16x8*)(qp + (int64_t)row * a.q_ss + 16 * ks + 8 * hi);
      else
        st.qf[qb][ks] = bf16x8{};
    }
  }

  tile_loop<CAUSAL, true>(st, x, kv0, kv1);
  // A V value beyond the fp16 range (|v| >= 65520) or a non-finite input
  // shows up as a non-finite accumulator: redo this workgroup with bf16
  // probabilities and bf16 V, which covers the whole bf16 range.
  if (__syncthreads_or(!state_finite(st))) tile_loop<CAUSAL, false>(st, x, kv0, kv1);

  // ---- epilogue: O = acc / l (bf16, RTNE) in q's layout; LSE = ln(sum exp)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = sum_halves(st.lsum[qb]);
    const int row = x.w_first + qb * 32 + l32;
    if (row < a.Sq) {
      const float inv = (l > 0.f) ? 1.f / l : 0.f;
      __bf16* op = a.o + b * a.q_sb + hq * a.q_sh + (int64_t)row * a.q_ss;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 u;
          u[0] = pack_bf16(st.oacc[qb][db][4 * j + 0] * inv, st.oacc[qb][db][4 * j + 1] * inv);
          u[1] = pack_bf16(st.oacc[qb][db][4 * j + 2] * inv, st.oacc[qb][db][4 * j + 3] * inv);
          *(u32x2*)(op + db * 32 + 8 * j + 4 * hi) = u;
        }
      if (hi == 0) {
        const float lse = (l > 0.f) ? (st.m_use[qb] + __log2f(l)) * kLn2 : -INFINITY;
        a.lse[((int64_t)(b * a.Hq + hq)) * a.Sq + row] = lse;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, bool causal, hipStream_t stream) {
  const int64_t grid = (int64_t)a.B * a.Hq * a.n_qt;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidValue;
  if (causal)
    hipLaunchKernelGGL(prefill_kernel<true>, dim3((unsigned)grid), dim3(NT), 0, stream, a);
  else
    hipLaunchKernelGGL(prefill_kernel<false>, dim3((unsigned)grid), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
