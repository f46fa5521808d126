// Paged decode for gfx950: one query row per (sequence, query head) against
// every cached token of a paged KV cache, in two kernels.
//
// The cache layout follows "Engineering the FlashAttention-4 kernel port to
// ROCm: HIP migration and multi-query inference optimisation" (multi-query
// section): 16-token pages listed by an int32 block table, several query heads
// sharing one K/V head (Q:32 / KV:8 there), tokens contiguous along the
// sequence with a stride of head_dim * kv_heads.  Splitting the keys and
// merging the partial softmaxes through their log-sum-exp is the
// Flash-Decoding style split of "MoonMath AI open-sources a HIP attention
// kernel for AMD MI300X that beats AITER v3" (third-Q-tile paragraph),
// generalised from two partial results to any number; within a part the
// online softmax is the block merge of "IO-aware tiling strategy in
// FlashAttention-4" (body).
//
// decode_partial_kernel: a persistent grid of exactly as many 8-wave
//   workgroups as the GPU holds at once.  Work is laid out as page slots
//   (unit group x, concatenated pages of all sequences), a unit group being
//   eight (K/V head, 16-query-head block) units; the slots are cut into equal
//   chunks of at most 64 pages and workgroup j takes chunks j, j + grid, ...
//   so every CU streams the same number of bytes whatever the lengths.  A
//   chunk is cut further at sequence ends into segments; wave w of the
//   workgroup runs unit 8x + w over the segment's pages (the waves read the
//   same pages of neighbouring heads: whole 16-token pages when Hkv = 8).
//   Per page (16 tokens x 256 B of K and of V for one head):
//     S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K rows straight from global,
//     Q^T in registers, columns = query heads), tokens past the end masked;
//     running max / sum per head (log2 units, rescale skipped while the max
//     grows by less than 2^8);
//     the V page copied into LDS by buffer_load ... lds (rows past the end
//     stored as zeros, so poisoned cache slots never reach the arithmetic),
//     read back transposed with ds_read_b64_tr_b16, converted to fp16, and
//     O^T += V^T P^T on v_mfma_f32_16x16x16_f16 with fp16 probabilities (a
//     page holding a V value beyond the fp16 range keeps bf16 for both).
//   With a cache append, the current token (position len - 1) takes its K row
//   from the new rows instead of the cache (a per-lane load address) and its
//   V row is written over the stale copy in the LDS slot before the page is
//   read back; at the end of that segment the wave of head block 0 stores
//   both rows into the cache slot.  Nothing else in the launch reads that
//   head's bytes of the slot, so no ordering between workgroups is needed.
//   Each segment writes its normalised fp32 output and natural-log LSE per
//   head to the workspace, in the slot of its chunk counted from the first
//   chunk of that (sequence, unit group); the workgroup that holds a
//   sequence's first page also writes how many chunks the sequence spans.
// decode_merge_kernel, one wave per (b, query head): LSE = M + ln sum e^(LSE_s-M),
//   O = sum e^(LSE_s - LSE) O_s in chunk order (deterministic), O to bf16
//   under the caller's rounding rule.
#include "gfx950.hpp"
#include "kernels.h"

namespace attn {
namespace {

constexpr int D = kHeadDim;
constexpr int NT = kDecodeWaves * 64;
constexpr float TAU = 8.0f;
constexpr int kMaxSeqChunks = 1024;   // ceil(65535 / 64) sequence chunks
constexpr int kDecodePrefetch = 1;   // pages in flight beyond the one computed

typedef short i16x4v __attribute__((ext_vector_type(4)));


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

// Sequence length as used: clamped to [0, 16 * max_blocks] so that no block
// table entry past the row is ever read.
__device__ __forceinline__ int seq_len_of(const DecodeArgs& a, int b) {
  return min(max(a.lens[b], 0), a.max_blocks * kPage);
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

// s_waitcnt vmcnt(n) (other counters left alone)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// The four K fragments of a page (d = 32*ks + 8*grp .. +8 of one token row),
// as ordinary loads: the compiler tracks them and waits for them before
// their first use.
__device__ __forceinline__ void load_k(bf16x8 (&kf)[4], const __bf16* row) {
#pragma unroll
  for (int i = 0; i < 4; ++i) kf[i] = *(const bf16x8*)(row + 32 * i);
}
// s_waitcnt vmcnt(N) for the LDS copies of a page: at most N of this wave's
// memory operations still in flight.  The "memory" clobber keeps every
// load and copy issued before it on this side of the wait.
template <int N>
__device__ __forceinline__ void wait_page() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}


// Number of pages of sequence b as used.
__device__ __forceinline__ int seq_pages(const DecodeArgs& a, int b) {
  return (seq_len_of(a, b) + kPage - 1) / kPage;
}

// Inclusive prefix sum over the wave's lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// Cut of the page slots into chunks: W = X * T slots, NC chunks, chunk c
// holding q + 1 slots if c < rem, else q (at most 64, at least 4 unless
// there is a single chunk).  Identical on every workgroup and in the merge.
struct Chunks {
  int64_t T, W, NC, q, rem;
  __device__ Chunks(int64_t T_, int X, int nwg) : T(T_), W((int64_t)X * T_) {
    if (W == 0) { NC = 0; q = 0; rem = 0; return; }
    const int64_t rounds = (W + (int64_t)kDecodeMaxChunkPages * nwg - 1) / ((int64_t)kDecodeMaxChunkPages * nwg);
    NC = min((int64_t)nwg * rounds, W / kDecodeMinChunkPages);
    if (NC < 1) NC = 1;
    q = W / NC;
    rem = W - q * NC;
  }
  __device__ int64_t begin(int64_t c) const { return c * q + min(c, rem); }
  __device__ int64_t chunk_of(int64_t L) const {
    const int64_t big = rem * (q + 1);
    return L < big ? L / (q + 1) : rem + (L - big) / q;
  }
};

// One wave: unit (K/V head, query-head block) over pages [p0, p1) of
// sequence b; writes the normalised partial output and its LSE to `slot`.
__device__ __forceinline__ void run_segment(const DecodeArgs& a, char* va, char* vb, char* vc, int b,
                                            int unit, int p0, int p1, int slot) {
  const int lane = threadIdx.x & 63;
  const int g = unit / a.n_hb;
  const int hb = unit - g * a.n_hb;
  const int len = seq_len_of(a, b);
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

  // LDS layout of a V page slot (4 KB): eight 512-byte d-blocks, block blk
  // holding d = 16*blk .. 16*blk+15 of the 16 tokens as [token][16 d].  A
  // transposed read of one block by the 64 lanes covers its 512 bytes
  // exactly once (no bank conflicts), and the eight blocks differ only by a
  // constant offset.
  // Copy: instruction j moves 1 KB, lane i landing at byte 1024*j + 16*i,
  // i.e. block 2*j + i/32, token (i%32)/2, half i%2 of the block's 32 bytes.
  const uint32_t tsb = (uint32_t)(a.token_stride * 2);   // token stride in bytes
  uint32_t voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    voff[j] = (uint32_t)((lane & 31) >> 1) * tsb + (uint32_t)(2 * j + (lane >> 5)) * 32 +
              (uint32_t)(lane & 1) * 16;
  // transposed read for the A operand of O^T = V^T P^T (16x16x16): lane
  // (group grp, j = col) addresses token 4*grp + j/4, d 16*blk + 4*(j%4)
  const uint32_t tr_lane = (uint32_t)(4 * grp + (col >> 2)) * 32 + (uint32_t)(col & 3) * 8;

  // the segment's block-table entries, one per lane (a segment has at most
  // 64 pages), so that no page waits on a table lookup
  const int32_t tab_lane = (p0 + lane < p1) ? a.table[(int64_t)b * a.max_blocks + p0 + lane] : 0;
  const float c = a.c;
  auto page_of = [&](int p) { return __builtin_amdgcn_readlane(tab_lane, p - p0); };
  // cache append: page pn (-1 if not in this segment), slot sn of the current
  // token; lanes 0..15 hold d = 8*lane .. 8*lane+7 of its K and V rows.  The
  // two loads are issued right after the segment's first page, so the first
  // wait_page (vmcnt(8), only the newest page's eight operations allowed in
  // flight) has completed them before any use.  A table entry outside
  // [0, num_pages) for that page makes the page contribute nothing and
  // suppresses the cache write.
  const int t_new = len - 1;
  const int pn = (a.knew != nullptr && t_new >= 0 && t_new / kPage >= p0 && t_new / kPage < p1)
                     ? t_new / kPage : -1;
  const int sn = t_new & (kPage - 1);
  const int64_t new_row = ((int64_t)b * a.Hkv + g) * D;
  u32x4 kn = u32x4{}, vn = u32x4{};
  auto load_new_rows = [&]() {
    if (pn >= 0 && lane < 16) {
      kn = *(const u32x4*)(a.knew + new_row + 8 * lane);
      vn = *(const u32x4*)(a.vnew + new_row + 8 * lane);
    }
  };
  // tokens of page p that take part: those before the sequence end, none if
  // the table entry is outside [0, num_pages) (then page 0 is addressed and
  // nothing of it is used)
  auto tokens_in = [&](int p) {
    const bool ok = (uint32_t)page_of(p) < (uint32_t)a.num_pages;
    return ok ? min(len - p * kPage, kPage) : 0;
  };

  // Issue page p: K rows into registers as the A operand (token = col,
  // d = 32*ks + 8*grp), V rows into LDS slot `vs`.  V rows past the valid
  // tokens are outside the buffer range of the copy, which stores zeros for
  // them, so poisoned cache slots never reach the arithmetic.
  auto issue_page = [&](bf16x8 (&kf)[4], char* vs, int p) {
    const int e = page_of(p);
    const int64_t phys = ((uint32_t)e < (uint32_t)a.num_pages) ? e : 0;
    const __bf16* kpg = a.kc + phys * a.page_stride + (int64_t)g * D;
    const __bf16* vpg = a.vc + phys * a.page_stride + (int64_t)g * D;
    const __bf16* krow = kpg + (int64_t)col * a.token_stride;
    if (p == pn && col == sn) krow = a.knew + new_row;   // the appended token
    load_k(kf, krow + 8 * grp);
    const int nt = tokens_in(p);
    const uint32_t nrec = nt > 0 ? (uint32_t)(nt - 1) * tsb + 256u : 0u;
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)vpg, (short)0, (int)nrec, 0x00020000);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (ATTN_LDS void*)(vs + j * 1024), 16, voff[j], 0,
                                               0, 0);
  };

  // V^T operands of a page from its LDS slot (ds_read_b64_tr_b16), the eight
  // reads and their wait in one instruction block that the compiler does not
  // track: it would otherwise wait for every LDS copy in flight, the later
  // pages' included.  The page's copies have landed (wait_page) before this
  // runs.
  auto read_v_page = [&](u32x2 (&vf)[8], const char* vs) {
    const uint32_t addr = (uint32_t)(uintptr_t)(const ATTN_LDS char*)vs + tr_lane;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:512\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:1024\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:1536\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:2048\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:2560\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:3072\n\t"
        "ds_read_b64_tr_b16 %7, %8 offset:3584\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(vf[0]), "=&v"(vf[1]), "=&v"(vf[2]), "=&v"(vf[3]), "=&v"(vf[4]), "=&v"(vf[5]),
          "=&v"(vf[6]), "=&v"(vf[7])
        : "v"(addr)
        : "memory");
  };

  auto compute_page = [&](const bf16x8 (&kf)[4], char* vs, int p) {
    const int nt = tokens_in(p);
    // ---- scores: lane holds head `col`, tokens 4*grp + i
    f32x4 sacc = f32x4{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) sacc = mfma16x32(kf[ks], qf[ks], sacc);
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (4 * grp + i < nt) ? sacc[i] : -INFINITY;
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
    // the appended token's V row replaces the stale copy of its slot: the
    // page's copies have landed (wait_page), and a wave's LDS accesses stay in
    // order, so the transposed reads below see it.  Written as an untracked
    // instruction: the compiler would otherwise wait for the next page's LDS
    // copies before it.
    if (p == pn && lane < 16) {
      const uint32_t at = (uint32_t)(uintptr_t)(ATTN_LDS char*)vs + 512 * (lane >> 1) + 32 * sn +
                          16 * (lane & 1);
      asm volatile("ds_write_b128 %0, %1" : : "v"(at), "v"(vn) : "memory");
    }
    // ---- V^T operands from the LDS slot.  P.V runs in fp16 (V converted
    // here) unless a V value of this page is beyond the fp16 range, in which
    // case the page uses bf16 P and V.
    u32x2 vf[8];
    read_v_page(vf, vs);
    uint32_t big = 0;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t m = vf[blk][i] & 0x7fff7fffu;
        big |= ((m & 0xffffu) > 0x477fu) | ((m >> 16) > 0x477fu);
      }
    if (!wave_any(big != 0)) {
      u32x2 pu;
      pu[0] = pack_f16(pv[0], pv[1]);
      pu[1] = pack_f16(pv[2], pv[3]);
      lsum = sum2_f16(pu[1], sum2_f16(pu[0], lsum));
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        vf[blk][0] = bf16x2_to_f16x2(vf[blk][0]);
        vf[blk][1] = bf16x2_to_f16x2(vf[blk][1]);
        oacc[blk] = mfma16x16_f16(vf[blk], pu, oacc[blk]);
      }
    } else {
      // rare: products into a fresh accumulator, added to the running one
      u32x2 pu;
      pu[0] = pack_bf16(pv[0], pv[1]);
      pu[1] = pack_bf16(pv[2], pv[3]);
      lsum = sum2_bf16(pu[1], sum2_bf16(pu[0], lsum));
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) oacc[blk] += mfma16x16_bf16(vf[blk], pu, f32x4{});
    }
  };

  // The wave walks the segment's pages in order with the loads of the next
  // kDecodePrefetch pages in flight while the current page is computed (one
  // register / LDS slot per page, rotated).  The prefetches are issued
  // unconditionally (past the segment's end they re-read its last page) so
  // that each wait is a fixed count: after issuing page p + kDecodePrefetch,
  // the 8 * kDecodePrefetch memory operations of the pages after p may still
  // be outstanding.
  {
    const int plast = p1 - 1;
    int p = p0;
    if constexpr (kDecodePrefetch == 1) {
      bf16x8 ka[4], kb[4];
      issue_page(ka, va, p);
      load_new_rows();
      for (;;) {
        issue_page(kb, vb, min(p + 1, plast));
        wait_page<8>();
        compute_page(ka, va, p);
        if (++p >= p1) break;
        issue_page(ka, va, min(p + 1, plast));
        wait_page<8>();
        compute_page(kb, vb, p);
        if (++p >= p1) break;
      }
    } else {
      bf16x8 ka[4], kb[4], kc[4];
      issue_page(ka, va, p);
      load_new_rows();
      issue_page(kb, vb, min(p + 1, plast));
      for (;;) {
        issue_page(kc, vc, min(p + 2, plast));
        wait_page<16>();
        compute_page(ka, va, p);
        if (++p >= p1) break;
        issue_page(ka, va, min(p + 2, plast));
        wait_page<16>();
        compute_page(kb, vb, p);
        if (++p >= p1) break;
        issue_page(kb, vb, min(p + 2, plast));
        wait_page<16>();
        compute_page(kc, vc, p);
        if (++p >= p1) break;
      }
    }
    wait_vm<0>();   // no copy into LDS may outlive the wave
  }
  // the appended token's rows into the cache (one writer per (b, K/V head))
  if (pn >= 0 && hb == 0 && lane < 16 && (uint32_t)page_of(pn) < (uint32_t)a.num_pages) {
    const int64_t at = (int64_t)page_of(pn) * a.page_stride + (int64_t)sn * a.token_stride +
                       (int64_t)g * D + 8 * lane;
    *(u32x4*)(a.kc_out + at) = kn;
    *(u32x4*)(a.vc_out + at) = vn;
  }

  // ---- the segment's normalised output and natural-log LSE per head.
  // C layout of the 16x16 accumulator: lane column = head, rows 4*grp + i
  // of block blk = d 16*blk + 4*grp + i.
  const float l_tot = sum_groups(lsum);
  if (hvalid) {
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    const int64_t ws = ((int64_t)b * a.Hq + hq) * a.max_splits + slot;
    float* dst = a.ws_o + ws * D + 4 * grp;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) *(f32x4*)(dst + 16 * blk) = oacc[blk] * inv;
    if (grp == 0)
      a.ws_lse[ws] = (l_tot > 0.f) ? (m_use + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_partial_kernel(DecodeArgs a) {
  // V page slots per wave, as separate arrays so that reads of one slot do
  // not wait for copies into another
  __shared__ __attribute__((aligned(1024))) char vslot0[kDecodeWaves][16 * D * 2];
  __shared__ __attribute__((aligned(1024))) char vslot1[kDecodeWaves][16 * D * 2];
  __shared__ __attribute__((aligned(1024))) char vslot2[kDecodePrefetch > 1 ? kDecodeWaves : 1][16 * D * 2];
  // pages per chunk of 64 sequences, then their exclusive prefix sums
  __shared__ int ck_tot[kMaxSeqChunks];
  __shared__ int64_t ck_pre[kMaxSeqChunks + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int nck = (a.B + 63) / 64;

  // ---- page counts of all sequences (every workgroup computes the same)
  for (int k = wave; k < nck; k += kDecodeWaves) {
    const int bb = 64 * k + lane;
    const int t = wave_sum_i(bb < a.B ? seq_pages(a, bb) : 0);
    if (lane == 0) ck_tot[k] = t;
  }
  __syncthreads();
  if (wave == 0) {
    int64_t carry = 0;
    for (int k0 = 0; k0 < nck; k0 += 64) {
      const int t = (k0 + lane < nck) ? ck_tot[k0 + lane] : 0;
      const int incl = wave_incl_scan(t);
      if (k0 + lane < nck) ck_pre[k0 + lane] = carry + incl - t;
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) ck_pre[nck] = carry;
  }
  __syncthreads();

  const int U = a.Hkv * a.n_hb;
  const Chunks ch(ck_pre[nck], a.X, gridDim.x);

  // sequence holding page position r (0 <= r < T) of the concatenated list:
  // binary search over the chunk prefixes, then a scan of that chunk's 64
  // lengths (kept while the search stays in the same chunk)
  int cached_k = -1, np_lane = 0, incl_lane = 0;
  auto find_seq = [&](int64_t r, int& b, int64_t& pre_b, int& np_b) {
    int lo = 0, hi = nck - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ck_pre[mid] <= r) lo = mid; else hi = mid - 1;
    }
    if (lo != cached_k) {
      const int bb = 64 * lo + lane;
      np_lane = bb < a.B ? seq_pages(a, bb) : 0;
      incl_lane = wave_incl_scan(np_lane);
      cached_k = lo;
    }
    const int64_t base = ck_pre[lo];
    const uint64_t m = __builtin_amdgcn_ballot_w64(base + incl_lane > r);
    const int l0 = __builtin_ctzll(m);
    np_b = __builtin_amdgcn_readlane(np_lane, l0);
    pre_b = base + __builtin_amdgcn_readlane(incl_lane, l0) - np_b;
    b = 64 * lo + l0;
  };

  for (int64_t c = blockIdx.x; c < ch.NC; c += gridDim.x) {
    int64_t L = ch.begin(c);
    const int64_t Lend = ch.begin(c + 1);
    while (L < Lend) {
      const int x = (int)(L / ch.T);
      const int64_t r = L - (int64_t)x * ch.T;
      int b, np_b;
      int64_t pre_b;
      find_seq(r, b, pre_b, np_b);
      const int64_t seg_end = min(Lend, (int64_t)x * ch.T + pre_b + np_b);
      const int p0 = (int)(r - pre_b);
      const int p1 = p0 + (int)(seg_end - L);
      const int64_t c_first = ch.chunk_of((int64_t)x * ch.T + pre_b);
      if (p0 == 0 && wave == 0 && lane == 0)
        a.ws_cnt[(int64_t)b * a.X + x] =
            (int)(ch.chunk_of((int64_t)x * ch.T + pre_b + np_b - 1) - c_first + 1);
      const int unit = kDecodeWaves * x + wave;
      const int slot = (int)(c - c_first);
      if (unit < U && slot < a.max_splits) run_segment(a, vslot0[wave], vslot1[wave],
                                                       vslot2[kDecodePrefetch > 1 ? wave : 0],
                                                       b, unit, p0, p1, slot);
      L = seg_end;
    }
  }
}

// One wave per (b, query head); lane owns d = 2*lane, 2*lane+1.  The part
// LSEs are read by the lanes in parallel and reduced across the wave; the
// weighted sum over parts runs in chunk order (deterministic).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return max_halves(v);
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return sum_halves(v);
}

__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  constexpr int C = 16;   // partial outputs loaded per batch
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.B * a.Hq) return;
  const int lane = threadIdx.x & 63;
  const int b = wid / a.Hq;
  const int64_t slot0 = (int64_t)wid * a.max_splits;
  const float* lse_p = a.ws_lse + slot0;
  const float* o_p = a.ws_o + slot0 * D + 2 * lane;
  // The first 64 part LSEs and the first C partial outputs are loaded
  // before the part count is known, so that the common case costs one
  // memory round trip; slots past the count are never used.
  const float lse_first = (lane < a.max_splits) ? lse_p[lane] : -INFINITY;
  float2 ov[C];
#pragma unroll
  for (int i = 0; i < C; ++i)
    ov[i] = (i < a.max_splits) ? *(const float2*)(o_p + (int64_t)i * D) : float2{0.f, 0.f};
  const int hq = wid - b * a.Hq;
  const int G = a.G;
  const int x = ((hq / G) * a.n_hb + (hq % G) / 16) / kDecodeWaves;
  const int cnt = a.ws_cnt[(int64_t)b * a.X + x];
  // a sequence without pages has no parts (and no count written)
  const int ns = seq_pages(a, b) == 0 ? 0 : min(max(cnt, 1), a.max_splits);

  auto lse_at = [&](int s0) {   // this lane's split of the batch s0 .. s0+63
    return (s0 + lane < ns) ? (s0 == 0 ? lse_first : lse_p[s0 + lane]) : -INFINITY;
  };
  float M = lse_at(0);
  for (int s0 = 64; s0 < ns; s0 += 64) M = fmaxf(M, lse_at(s0));
  M = wave_max(M);
  auto weight = [&](float ls) { return (ls == -INFINITY) ? 0.f : fast_exp2((ls - M) * kLog2e); };
  float wl = weight(lse_at(0));   // weight of split `lane`
  float Lp = wl;
  for (int s0 = 64; s0 < ns; s0 += 64) Lp += weight(lse_at(s0));
  const float L = wave_sum(Lp);

  // O = sum_s w_s O_s in split order
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    if (i < ns) {
      const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), i));
      o0 += w * ov[i].x;
      o1 += w * ov[i].y;
    }
  }
  for (int s0 = 0; s0 < ns; s0 += 64) {
    if (s0 > 0) wl = weight(lse_at(s0));
    for (int i0 = (s0 == 0 ? C : 0); i0 < 64 && s0 + i0 < ns; i0 += C) {
#pragma unroll
      for (int i = 0; i < C; ++i)
        if (s0 + i0 + i < ns) ov[i] = *(const float2*)(o_p + (int64_t)(s0 + i0 + i) * D);
#pragma unroll
      for (int i = 0; i < C; ++i) {
        if (s0 + i0 + i < ns) {
          const float w =
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), i0 + i));
          o0 += w * ov[i].x;
          o1 += w * ov[i].y;
        }
      }
    }
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  uint32_t packed;
  with_rounding(a.rounding, [&](auto mode) { packed = pack_bf16_as<mode()>(o0 * inv, o1 * inv); });
  *(uint32_t*)(a.o + (int64_t)wid * D + 2 * lane) = packed;
  if (lane == 0) a.lse[wid] = (L > 0.f) ? M + __logf(L) : -INFINITY;
}


}  // namespace

int decode_max_splits(int max_blocks) {
  return (max_blocks + kDecodeMinChunkPages - 1) / kDecodeMinChunkPages + 1;
}

namespace {
constexpr int kMaxDevices = 64;
int g_wgs_per_cu[kMaxDevices];   // 0 = not yet queried
}

hipError_t launch_decode(DecodeArgs a, int num_cus, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int per_cu = __atomic_load_n(&g_wgs_per_cu[dev], __ATOMIC_ACQUIRE);
  if (per_cu == 0) {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_partial_kernel, NT, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    __atomic_store_n(&g_wgs_per_cu[dev], per_cu, __ATOMIC_RELEASE);
  }
  if (a.B > 64 * kMaxSeqChunks) return hipErrorInvalidValue;
  // exactly one resident workgroup per slot: every CU gets the same share
  a.nwg = per_cu * (num_cus > 0 ? num_cus : 256);
  hipLaunchKernelGGL(decode_partial_kernel, dim3(a.nwg), dim3(NT), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int waves = a.B * a.Hq;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((waves + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
