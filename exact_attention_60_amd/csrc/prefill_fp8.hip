// Attention forward on FP8 (OCP E4M3) Q, K, V for gfx950.
//
// The pages name FP8 inputs only in passing and say that the FP8 handling of
// the Blackwell kernel falls back to FP16 on ROCm ("Engineering the
// FlashAttention-4 kernel port to ROCm", HIP migration section).  Here the
// inputs stay FP8 in HBM (half the bytes of bf16) and are widened to fp16 on
// the way into LDS, exactly: an E4M3 byte s.eeee.mmm placed as the fp16 bit
// pattern s.0eeee.mmm0000000 is the same value times 2^-8 (subnormals
// included), so the widening is two masks and two shifts per pair and needs no
// table.  The 2^-8 of Q and K is folded into the softmax constant, the one of
// V into the output scale, together with the per-tensor descales.  The E4M3
// NaN encoding (s.1111.111) is not recognised: it reads as +-480.
//
// Both products run on v_mfma_f32_32x32x16_f16 with fp32 accumulation, the
// online softmax of "IO-aware tiling strategy in FlashAttention-4" (body),
// probabilities rounded to fp16 for P.V as in the bf16 path.
//
// Workgroup: 4 waves, 128 query rows of one (batch, query head), 32 rows per
// wave; K/V tiles of 64 keys.  Each thread loads its share of tile t+1 from
// HBM into registers while tile t is computed, then widens it into the other
// LDS buffer; one barrier per tile.  LDS tiles (fp16):
//   K:   [64 keys][128 d], 256-byte rows, 16-byte chunk c stored at c ^ (key & 15)
//   V^T: [128 d][64 keys], 128-byte rows, chunk c at c ^ ((d ^ d >> 3) & 7);
//        within each 16-key block the key groups of four are stored in the
//        order 0, 2, 1, 3, which is the order in which the S^T accumulator
//        holds them, so that accumulator registers are directly the P^T operand.
#include "gfx950.hpp"
#include "kernels.h"

namespace attn {
namespace {

constexpr int D = kHeadDim;
constexpr int BM = kFp8RowsPerBlock;   // 128 query rows
constexpr int BN = 64;                 // keys per tile
constexpr int NT = 256;
constexpr int KT_BYTES = BN * D * 2;   // 16 KB
constexpr int BUF_BYTES = 2 * KT_BYTES;

// Two E4M3 bytes (bits 0-7 and 8-15 of x) -> two fp16 holding 2^-8 times
// their values.
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t x) {
  const uint32_t y = (x & 0xFFu) | ((x & 0xFF00u) << 8);
  return ((y & 0x00800080u) << 8) | ((y & 0x007F007Fu) << 7);
}

__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }
__device__ __forceinline__ int perm4(int g) { return ((g & 1) << 1) | (g >> 1); }

struct Raw {
  u32x4 k[2];      // 16 bytes (16 d) of one key, two items
  uint32_t v[2][4];  // 4 bytes (4 d) of four consecutive keys, two items
};

template <bool CAUSAL>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_fp8_kernel(Fp8Args a) {
  __shared__ __attribute__((aligned(1024))) char smem[2][BUF_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // XCD-aware order: consecutive ids go round-robin over the 8 XCDs, so each
  // XCD is given a contiguous range of (batch, head, tile) items
  const int total = (int)gridDim.x;
  int id = (int)blockIdx.x;
  if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
  const int qt = a.n_qt - 1 - id % a.n_qt;   // heaviest causal tiles first
  const int bh = id / a.n_qt;
  const int hq = bh % a.Hq;
  const int b = bh / a.Hq;
  const int g = hq / a.group;

  const uint8_t* qp = a.q + b * a.q_sb + hq * a.q_sh;
  const uint8_t* kp = a.k + b * a.k_sb + g * a.k_sh;
  const uint8_t* vp = a.v + b * a.k_sb + g * a.k_sh;
  const int r0 = qt * BM + wave * 32;   // this wave's first query row
  const int row = r0 + l32;
  const int off = a.Sk - a.Sq;          // causal: key j visible from row i iff j <= i + off

  // keys the workgroup needs
  int n_keys = a.Sk;
  if (CAUSAL) {
    const int last = min(qt * BM + BM - 1, a.Sq - 1);
    n_keys = max(0, min(a.Sk, last + off + 1));
  }
  const int nt = (n_keys + BN - 1) / BN;

  // ---- Q^T operand (B of S^T = K Q^T): lane holds Q[row][16 ks + 8 h .. +7]
  f16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x2 r = {0u, 0u};
    if (row < a.Sq) r = *(const u32x2*)(qp + (int64_t)row * a.q_ss + 16 * ks + 8 * h);
    const u32x4 w = {e4m3x2_to_f16x2(r[0] & 0xFFFFu), e4m3x2_to_f16x2(r[0] >> 16),
                     e4m3x2_to_f16x2(r[1] & 0xFFFFu), e4m3x2_to_f16x2(r[1] >> 16)};
    qf[ks] = __builtin_bit_cast(f16x8, w);
  }

  auto load_raw = [&](Raw& r, int t0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + NT * i;
      const int key = t0 + (idx >> 3);
      r.k[i] = (key < a.Sk) ? *(const u32x4*)(kp + (int64_t)key * a.k_ss + 16 * (idx & 7))
                            : u32x4{0u, 0u, 0u, 0u};
      const int dq = idx & 31, kq = idx >> 5;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kv = t0 + 4 * kq + e;
        r.v[i][e] = (kv < a.Sk) ? *(const uint32_t*)(vp + (int64_t)kv * a.k_ss + 4 * dq) : 0u;
      }
    }
  };
  auto store = [&](const Raw& r, char* buf) {
    char* kt = buf;
    char* vt = buf + KT_BYTES;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + NT * i;
      const int key = idx >> 3, c8 = idx & 7;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t x0 = r.k[i][2 * j], x1 = r.k[i][2 * j + 1];
        const u32x4 w = {e4m3x2_to_f16x2(x0 & 0xFFFFu), e4m3x2_to_f16x2(x0 >> 16),
                         e4m3x2_to_f16x2(x1 & 0xFFFFu), e4m3x2_to_f16x2(x1 >> 16)};
        *(u32x4*)(kt + key * 256 + (((2 * c8 + j) ^ (key & 15)) << 4)) = w;
      }
      const int dq = idx & 31, kq = idx >> 5;
      const int pos = 16 * (kq >> 2) + 4 * perm4(kq & 3);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t sel = 0x0C0C0000u | ((uint32_t)(4 + c) << 8) | (uint32_t)c;
        const uint32_t x01 = __builtin_amdgcn_perm(r.v[i][1], r.v[i][0], sel);
        const uint32_t x23 = __builtin_amdgcn_perm(r.v[i][3], r.v[i][2], sel);
        const u32x2 w = {e4m3x2_to_f16x2(x01), e4m3x2_to_f16x2(x23)};
        const int d = 4 * dq + c;
        *(u32x2*)(vt + d * 128 + (((pos >> 3) ^ vt_swz(d)) << 4) + ((pos & 7) << 1)) = w;
      }
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;   // running max of the scores in log2 units
  float lsum = 0.f;          // this lane's part of the row sum

  Raw raw;
  if (nt > 0) {
    load_raw(raw, 0);
    store(raw, smem[0]);
  }
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int t0 = t * BN;
    const bool more = t + 1 < nt;
    if (more) load_raw(raw, t0 + BN);
    const char* kt = smem[t & 1];
    const char* vt = smem[t & 1] + KT_BYTES;

    // S^T = K Q^T: register r of block kb holds key 32 kb + 8 (r / 4) + 4 h + r % 4
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const int key = 32 * kb + l32;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const f16x8 kf = *(const f16x8*)(kt + key * 256 + (((2 * ks + h) ^ (key & 15)) << 4));
        s[kb] = mfma32(kf, qf[ks], s[kb]);
      }
    }
    // keys past Sk, and past the causal diagonal, are -inf
    const bool tail = t0 + BN > a.Sk;
    const bool diag = CAUSAL && t0 + BN - 1 > r0 + off;
    if (tail || diag) {
      const int lim = CAUSAL ? min(a.Sk - 1, row + off) : a.Sk - 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key > lim) s[kb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = max_halves(mx);
    const float m_new = fmaxf(m_run, mx * a.c);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = (m_run == m_new) ? 1.f : fast_exp2(m_run - m_new);
    m_run = m_new;

    // P (fp16) as the B operand of O^T += V^T P^T, one k-step of 16 keys each
    u32x4 pp[4];
    float ps = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 8 * (st & 1) + 2 * j;
        const float p0 = fast_exp2(fmaf(s[st >> 1][r], a.c, -m_use));
        const float p1 = fast_exp2(fmaf(s[st >> 1][r + 1], a.c, -m_use));
        pp[st][j] = pack_f16(p0, p1);
        ps = sum2_f16(pp[st][j], ps);
      }
    }
    lsum = fmaf(lsum, alpha, ps);
    if (wave_any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const f16x8 pb = __builtin_bit_cast(f16x8, pp[st]);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = 32 * db + l32;
        const f16x8 vf = *(const f16x8*)(vt + d * 128 + (((2 * st + h) ^ vt_swz(d)) << 4));
        oacc[db] = mfma32(vf, pb, oacc[db]);
      }
    }

    if (more) store(raw, smem[(t + 1) & 1]);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l * out_scale (bf16, RTNE); LSE = ln(sum exp)
  const float l_tot = sum_halves(lsum);
  if (row < a.Sq) {
    const float inv = (l_tot > 0.f) ? a.out_scale / l_tot : 0.f;
    __bf16* op = a.o + b * a.q_sb + hq * a.q_sh + (int64_t)row * a.q_ss;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * h;
        const u32x2 w = {pack_bf16(oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv),
                         pack_bf16(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv)};
        *(u32x2*)(op + d) = w;
      }
    if (h == 0)
      a.lse[((int64_t)b * a.Hq + hq) * a.Sq + row] =
          (l_tot > 0.f) ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_prefill_fp8(const Fp8Args& a, bool causal, hipStream_t stream) {
  const int64_t n = (int64_t)a.B * a.Hq * a.n_qt;
  if (n < 1 || n > INT32_MAX) return hipErrorInvalidValue;
  if (causal)
    hipLaunchKernelGGL(prefill_fp8_kernel<true>, dim3((unsigned)n), dim3(NT), 0, stream, a);
  else
    hipLaunchKernelGGL(prefill_fp8_kernel<false>, dim3((unsigned)n), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
