// Split-KV paged decode for gfx950: one query row per (sequence, query head)
// against every cached token of a paged KV cache, in two kernels.
//
// The cache layout follows "Engineering the FlashAttention-4 kernel port to
// ROCm: HIP migration and multi-query inference optimisation" (multi-query
// section): 16-token pages listed by an int32 block table, several query heads
// sharing one K/V head (Q:32 / KV:8 there), tokens contiguous along the
// sequence with a stride of head_dim * kv_heads.  The split of the keys with a
// log-sum-exp merge of partial results is the Flash-Decoding style tail split
// of "MoonMath AI open-sources a HIP attention kernel for AMD MI300X that beats
// AITER v3" (third-Q-tile paragraph), generalised from two partial softmaxes to
// any number; within a split the online softmax is the block merge of
// "IO-aware tiling strategy in FlashAttention-4" (body).
//
// decode_split_kernel, grid (splits, Hkv * head_blocks, B), 4 waves:
//   the workgroup covers pages [s*pps, min((s+1)*pps, ceil(len/16))) of one
//   sequence for up to 16 query heads of one K/V head; wave w takes every 4th
//   page.  Per page (16 tokens x 256 B of K and of V for this head):
//     S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K rows straight from global,
//     Q^T in registers, columns = query heads), tokens past the end masked;
//     running max / sum per head (log2 units, rescale skipped while the max
//     grows by less than 2^8);
//     V page converted to fp16 and staged in LDS (rows past the end zeroed,
//     so poisoned cache slots never reach the arithmetic), read back
//     transposed with ds_read_b64_tr_b16, O^T += V^T P^T on
//     v_mfma_f32_16x16x16_f16 with fp16 probabilities (a page holding a V
//     value beyond the fp16 range keeps bf16 for both operands instead).
//   The four waves' states are merged exactly in LDS and the split's
//   normalised fp32 output and natural-log LSE go to the workspace.
// decode_merge_kernel, one wave per (b, query head): LSE = M + ln sum e^(LSE_s-M),
//   O = sum e^(LSE_s - LSE) O_s in split order (deterministic), O to bf16 RTNE.
#include "gfx950.hpp"
#include "kernels.h"

namespace attn {
namespace {

constexpr int D = kHeadDim;
constexpr int NT = kDecodeWaves * 64;
constexpr float TAU = 8.0f;

typedef short i16x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int row_off(int row, int c) {
  return row * 256 + ((c ^ swz(row & 15)) << 4);
}

__device__ __forceinline__ f32x4 mfma16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16_bf16(const u32x2& a, const u32x2& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4v, a),
                                                   __builtin_bit_cast(i16x4v, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16_f16(const u32x2& a, const u32x2& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                               __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// sum / max over the four 16-lane groups (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float xor16(float v) {
  return __shfl_xor(v, 16, 64);
}
__device__ __forceinline__ float max_groups(float v) {
  v = fmaxf(v, xor16(v));
  return max_halves(v);
}
__device__ __forceinline__ float sum_groups(float v) {
  v = v + xor16(v);
  return sum_halves(v);
}

__global__ __launch_bounds__(NT) void decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kDecodeWaves * 16 * D * 4];  // 32 KB
  __shared__ float mbuf[kDecodeWaves][16];
  __shared__ float lbuf[kDecodeWaves][16];

  const int s = blockIdx.x;
  const int g = blockIdx.y / a.n_hb;
  const int hb = blockIdx.y - g * a.n_hb;
  const int b = blockIdx.z;
  const int len = a.lens[b];
  const int np = (len + kPage - 1) / kPage;
  const int p0 = s * a.pps;
  if (p0 >= np) return;  // whole workgroup: uniform exit before any barrier
  const int p1 = min(np, p0 + a.pps);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;   // MFMA column: query head (scores) / token row (K loads)
  const int grp = lane >> 4;   // lane group 0..3

  const int hloc = hb * 16 + col;
  const bool hvalid = hloc < a.G;
  const int hq = g * a.G + hloc;

  // Q^T fragments: B operand of S^T = K Q^T, column = head, k-slots = d
  bf16x8 qf[4];
  {
    const __bf16* qp = a.q + ((int64_t)b * a.Hq + (hvalid ? hq : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[ks] = hvalid ? *(const bf16x8*)(qp + 32 * ks + 8 * grp) : bf16x8{};
  }

  float m_use = -INFINITY;   // per head (column), log2 units
  float lsum = 0.f;          // partial over this lane's tokens
  f32x4 oacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc[i] = f32x4{};

  char* vst = smem + wave * (16 * 256);    // this wave's V page (4 KB)
  // V staging: lane -> token row lane/4, chunks 4*(lane%4) + jj
  const int st_tok = lane >> 2;
  // transpose-read offsets for the A operand of O^T = V^T P^T (16x16x16):
  // lane (block grp, j = col) addresses token 4*grp + j/4, d 16*blk + 4*(j%4)
  int troff[8];
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
    const int d0 = 16 * blk + 4 * (col & 3);
    troff[blk] = row_off(4 * grp + (col >> 2), d0 >> 3) + (d0 & 7) * 2;
  }

  const int32_t* tab = a.table + (int64_t)b * a.max_blocks;
  const float c = a.c;
  for (int p = p0 + wave; p < p1; p += kDecodeWaves) {
    const int64_t phys = tab[p];
    const __bf16* kpg = a.kc + phys * a.page_stride + (int64_t)g * D;
    const __bf16* vpg = a.vc + phys * a.page_stride + (int64_t)g * D;
    const int tok0 = p * kPage;
    // ---- loads: K rows as the A operand (token = col, d = 32ks + 8grp), V rows
    bf16x8 kf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kf[ks] = *(const bf16x8*)(kpg + (int64_t)col * a.token_stride + 32 * ks + 8 * grp);
    u32x4 vr[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      vr[jj] = *(const u32x4*)(vpg + (int64_t)st_tok * a.token_stride + 8 * (4 * (lane & 3) + jj));
    // ---- scores: lane holds head `col`, tokens 4*grp + i
    f32x4 sacc = f32x4{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) sacc = mfma16x32(kf[ks], qf[ks], sacc);
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (tok0 + 4 * grp + i < len) ? sacc[i] : -INFINITY;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = max_groups(mx);
    const float m_tile = mx * c;
    if (wave_any(m_tile > m_use + TAU)) {
      const float m_new = fmaxf(m_use, m_tile);
      const float alpha = (m_new == m_use) ? 1.f : fast_exp2(m_use - m_new);
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) oacc[i] *= alpha;
      m_use = m_new;
    }
    const float msub = (m_use == -INFINITY) ? 0.f : m_use;
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(__builtin_fmaf(sv[i], c, -msub));
    // ---- V page to LDS, rows past the sequence end zeroed.  P.V runs in
    // fp16 (V converted here) unless a V value of this page is beyond the
    // fp16 range, in which case the page uses bf16 P and V.
    const bool tok_ok = tok0 + st_tok < len;
    uint32_t big = 0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if (!tok_ok) vr[jj] = u32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t m = vr[jj][i] & 0x7fff7fffu;
        big |= ((m & 0xffffu) > 0x477fu) | ((m >> 16) > 0x477fu);
      }
    }
    const bool f16_page = !wave_any(big != 0);
    u32x2 pu;
    if (f16_page) {
      pu[0] = pack_f16(pv[0], pv[1]);
      pu[1] = pack_f16(pv[2], pv[3]);
      lsum = sum2_f16(pu[1], sum2_f16(pu[0], lsum));
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[jj][i] = bf16x2_to_f16x2(vr[jj][i]);
    } else {
      pu[0] = pack_bf16(pv[0], pv[1]);
      pu[1] = pack_bf16(pv[2], pv[3]);
      lsum = sum2_bf16(pu[1], sum2_bf16(pu[0], lsum));
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      *(u32x4*)(vst + row_off(st_tok, 4 * (lane & 3) + jj)) = vr[jj];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const u32x2 vf = __builtin_bit_cast(u32x2, lds_read_tr(vst + troff[blk]));
      oacc[blk] = f16_page ? mfma16x16_f16(vf, pu, oacc[blk]) : mfma16x16_bf16(vf, pu, oacc[blk]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the four waves' (m, l, O) in LDS
  const float l_tot = sum_groups(lsum);
  __syncthreads();  // every wave is done with its V page
  float* obuf = (float*)smem;  // [wave][head col][d]
  if (grp == 0) {
    mbuf[wave][col] = m_use;
    lbuf[wave][col] = l_tot;
  }
#pragma unroll
  for (int blk = 0; blk < 8; ++blk)
    *(f32x4*)(obuf + (wave * 16 + col) * D + 16 * blk + 4 * grp) = oacc[blk];
  __syncthreads();

  {
    const int hc = tid >> 4;          // head column 0..15
    const int d0 = (tid & 15) * 8;    // 8 d values
    const int hl = hb * 16 + hc;
    if (hl < a.G) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, mbuf[w][hc]);
      float wt[kDecodeWaves];
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        const float mw = mbuf[w][hc];
        wt[w] = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
        L += wt[w] * lbuf[w][hc];
      }
      const float inv = (L > 0.f) ? 1.f / L : 0.f;
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        const float* src = obuf + (w * 16 + hc) * D + d0;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += wt[w] * src[i];
      }
      const int hqo = g * a.G + hl;
      const int64_t slot = ((int64_t)b * a.Hq + hqo) * a.max_splits + s;
      float* dst = a.ws_o + slot * D + d0;
      *(f32x4*)dst = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
      *(f32x4*)(dst + 4) = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
      if ((tid & 15) == 0)
        a.ws_lse[slot] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -INFINITY;
    }
  }
}

// One wave per (b, query head); lane owns d = 2*lane, 2*lane+1.
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.B * a.Hq) return;
  const int lane = threadIdx.x & 63;
  const int b = wid / a.Hq;
  const int len = a.lens[b];
  const int np = (len + kPage - 1) / kPage;
  const int ns = (np + a.pps - 1) / a.pps;
  const int64_t slot0 = (int64_t)wid * a.max_splits;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.ws_lse[slot0 + s]);
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float ls = a.ws_lse[slot0 + s];
    const float w = (ls == -INFINITY) ? 0.f : fast_exp2((ls - M) * kLog2e);
    const float2 ov = *(const float2*)(a.ws_o + (slot0 + s) * D + 2 * lane);
    L += w;
    o0 += w * ov.x;
    o1 += w * ov.y;
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  *(uint32_t*)(a.o + (int64_t)wid * D + 2 * lane) = pack_bf16(o0 * inv, o1 * inv);
  if (lane == 0) a.lse[wid] = (L > 0.f) ? M + __logf(L) : -INFINITY;
}

}  // namespace

int decode_max_splits(int max_blocks) {
  return (max_blocks + kDecodeMinPagesPerSplit - 1) / kDecodeMinPagesPerSplit;
}

// Pages per split: a power of two >= 8 chosen so that, with sequences about
// half full on average, the grid holds about eight workgroups per CU.
int decode_pages_per_split(int B, int Hkv, int n_hb, int max_blocks, int num_cus) {
  const double est_pages = (double)B * Hkv * n_hb * max_blocks * 0.5;
  const double target_wgs = 8.0 * (num_cus > 0 ? num_cus : 256);
  int pps = kDecodeMinPagesPerSplit;
  while (pps < max_blocks && est_pages / pps > target_wgs) pps *= 2;
  return pps;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const int splits = (a.max_blocks + a.pps - 1) / a.pps;
  if (splits > a.max_splits) return hipErrorInvalidValue;
  dim3 grid1(splits, a.Hkv * a.n_hb, a.B);
  hipLaunchKernelGGL(decode_split_kernel, grid1, dim3(NT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int waves = a.B * a.Hq;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((waves + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
