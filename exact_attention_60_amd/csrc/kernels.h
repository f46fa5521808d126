// Internal interface between the C-ABI host code (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// ---- prefill -------------------------------------------------------------
constexpr int kHeadDim = 128;
constexpr int kPrefillWaves = 8;                      // waves per workgroup (2 per SIMD)
constexpr int kPrefillRowsPerWave = 32;               // one 32-row MFMA block per wave
constexpr int kPrefillBM = kPrefillWaves * kPrefillRowsPerWave;  // 256 query rows
constexpr int kPrefillBN = 64;                        // keys per K/V tile

// Rounding rules of the final fp32 -> bf16 output conversion (the values of
// ATTN_ROUND_* in attn.h): to nearest with ties to even (the hardware
// conversion), to nearest with ties away from zero, toward zero.
enum : int { kRoundRTNE = 0, kRoundRTNA = 1, kRoundRTZ = 2 };

struct PrefillArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  int64_t q_sb, q_sh, q_ss;  // element strides of batch, head, sequence (q and o)
  int64_t k_sb, k_sh, k_ss;  // same for k and v
  int B, Hq, Hkv, Sq, Sk;
  int group;                 // Hq / Hkv
  int n_qt;                  // ceil(Sq / kPrefillBM)
  float c;                   // scale * log2(e)
  int rounding;              // kRoundRTNE / kRoundRTNA / kRoundRTZ for O
  // packed sequences (null cu_q: dense batch): sequence b is rows
  // cu_q[b] .. cu_q[b+1]-1 of q/o and cu_k[b] .. cu_k[b+1]-1 of k/v; Sq is
  // then the longest query length, LSE is [Hq, total_q]
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k;
  // ALiBi slopes [Hq] (null: no bias): -slope * |i + Sk - Sq - j| is added to
  // the scaled scores of query head h
  const float* alibi;
  // V as fp16 V^T tiles written by launch_prep_v (null: the kernel converts
  // and transposes each V tile itself).  Dense batches without ALiBi only;
  // tiles of the kernel's own key count (kPrefillBN, or kPrefillPipeBN for
  // the GQA kernel).
  const uint8_t* vt = nullptr;
  int n_kt = 0;              // tiles per (batch, kv head)
};

hipError_t launch_prefill(const PrefillArgs& a, bool causal, hipStream_t stream);

// V of a dense batch as fp16 V^T tiles for the d = 128 prefill kernel: tile t
// of (batch b, kv head h) -- keys 64t .. 64t+63 (zeros past Sk), all 128 d --
// is kVtTileBytes bytes at vt + ((b * Hkv + h) * n_kt + t) * kVtTileBytes,
// laid out exactly as the kernel's LDS V^T tile (row d of 128 bytes holds the
// 64 keys in MFMA k-slot order, 16-byte chunks swizzled), so that the kernel
// copies it into LDS as it is.  Values are rounded to fp16 (nearest even);
// |v| >= 65520 becomes +-inf, which the kernel meets with its bf16 redo.
// The GQA kernel's tiles (launch_prefill_pipe) hold kPrefillPipeBN keys:
// row d of 64 bytes, 16-byte chunk (2kk + hi) ^ ((d >> 2) & 3).
constexpr int kVtTileBytes = kPrefillBN * kHeadDim * 2;
constexpr int kPrefillPipeBN = 32;
constexpr int kVtPipeTileBytes = kPrefillPipeBN * kHeadDim * 2;
struct PrepVArgs {
  const __bf16* v;
  uint8_t* vt;
  int64_t k_sb, k_sh, k_ss;  // element strides of batch, head, sequence of v
  int B, Hkv, Sk, n_kt;
  int tk;                    // keys per tile: kPrefillBN or kPrefillPipeBN
};
hipError_t launch_prep_v(const PrepVArgs& a, hipStream_t stream);

// Dense d = 128 forward without ALiBi for GQA groups that are a multiple of
// 4, pipelined inside each wave: one wave per SIMD, the 4 waves of a
// workgroup being 4 query heads of one K/V head over the same 64 rows (each
// loaded K/V tile shared by the four).  n_qt = ceil(Sq / kPrefillPipeRows).
constexpr int kPrefillPipeRows = 64;
hipError_t launch_prefill_pipe(const PrefillArgs& a, bool causal, hipStream_t stream);

// ---- FP8 (E4M3) forward ------------------------------------------------------
constexpr int kFp8RowsPerBlock = 256;   // query rows per workgroup

struct Fp8Args {
  const uint8_t* q;          // E4M3 bytes, d = 128 innermost
  const uint8_t* k;
  const uint8_t* v;
  __bf16* o;                 // bf16, q's layout
  float* lse;                // [B, Hq, Sq]
  int64_t q_sb, q_sh, q_ss;  // element strides of batch, head, sequence (q and o)
  int64_t k_sb, k_sh, k_ss;  // same for k and v
  int B, Hq, Hkv, Sq, Sk;
  int group;                 // Hq / Hkv
  int n_qt;                  // ceil(Sq / kFp8RowsPerBlock)
  float c;                   // scale * log2(e) * descale_q * descale_k
  float out_scale;           // descale_v
};

hipError_t launch_prefill_fp8(const Fp8Args& a, bool causal, hipStream_t stream);

// head dims 64 and 256 (dense layouts, no ALiBi): query rows per workgroup
// (n_qt = ceil(Sq / kPrefillHdRows)) and the launches, each optionally on
// prepared tiles.  d = 64: fp16 V tiles of 64 keys (8 KB: the kernel's LDS
// image, rows of 128 bytes, 16-byte chunk c of row r at ((c ^ s(r)) << 4)
// with s(r) = ((r & 3) << 1) | ((r >> 2) & 1)) written by launch_prep_v_d64
// (tk = 64).  d = 256: fp16 V^T tiles of kPrefillD256BN keys written by
// launch_prep_v_d256 (tk = kPrefillD256BN), row d of 64 bytes holding the
// tile's keys in the same chunk order and swizzle as the GQA kernel's tiles,
// kVtD256TileBytes per tile.
constexpr int kPrefillHdRows = 128;
constexpr int kPrefillD256BN = 32;
constexpr int kVtD256TileBytes = kPrefillD256BN * 256 * 2;
hipError_t launch_prefill_hd(const PrefillArgs& a, bool causal, hipStream_t stream);   // d = 64
hipError_t launch_prep_v_d64(const PrepVArgs& a, hipStream_t stream);
hipError_t launch_prefill_d256(const PrefillArgs& a, bool causal, hipStream_t stream);
hipError_t launch_prep_v_d256(const PrepVArgs& a, hipStream_t stream);

// ---- paged decode ----------------------------------------------------------
constexpr int kPage = 16;
constexpr int kDecodeWaves = 8;
constexpr int kDecodeMaxChunkPages = 64;   // one block-table entry per lane
constexpr int kDecodeMinChunkPages = 4;    // bounds the partial results per sequence
constexpr int kDecodeHeadsPerBlock = 16;   // query heads per MFMA column block

struct DecodeArgs {
  const __bf16* q;
  const __bf16* kc;
  const __bf16* vc;
  const int32_t* table;
  const int32_t* lens;
  float* ws_o;     // [B, Hq, max_splits, 128] fp32 normalised partial outputs
  float* ws_lse;   // [B, Hq, max_splits]      fp32 partial LSE (natural log)
  int* ws_cnt;     // [B, X] number of partial results of (sequence, unit group)
  __bf16* o;
  float* lse;
  int B, Hq, Hkv, G, n_hb;   // G = Hq / Hkv, n_hb = ceil(G / 16)
  int X;                     // unit groups: ceil(Hkv * n_hb / 4)
  int max_blocks, max_splits;
  int num_pages;
  int nwg;                   // workgroups of the partial kernel (set at launch)
  int64_t page_stride;       // elements per page: 16 * Hkv * 128
  int64_t token_stride;      // elements per token slot: Hkv * 128
  float c;                   // scale * log2(e)
  int rounding;              // kRoundRTNE / kRoundRTNA / kRoundRTZ for O
  // cache append (null when the call does not append): the current token's
  // K and V rows [B, Hkv, 128], and the caches as writable pointers (the
  // same memory as kc / vc)
  const __bf16* knew;
  const __bf16* vnew;
  __bf16* kc_out;
  __bf16* vc_out;
};

// partial results a (sequence, unit group) can need: ceil(max_blocks / 4) + 1
int decode_max_splits(int max_blocks);
hipError_t launch_decode(DecodeArgs a, int num_cus, hipStream_t stream);

// Scratch of the decode entry point that allocates nothing: a file-scope
// device array of this many bytes per GPU; *ptr is its device address on the
// current device (looked up once per device).
constexpr size_t kDecodeNoAllocScratchBytes = size_t(64) << 20;
hipError_t decode_noalloc_scratch(void** ptr);

// ---- backward ----------------------------------------------------------------
constexpr int kBwdKvRows = 128;   // keys per dK/dV workgroup
constexpr int kBwdQRows = 128;    // query rows per dQ workgroup

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;       // forward output
  const __bf16* dout;    // upstream gradient dO, q's layout
  const float* lse;      // forward LSE [B, Hq, Sq] (natural log)
  __bf16* dq;            // q's layout
  __bf16* dk;            // k's layout
  __bf16* dv;
  float* ws_d;           // [B, Hq, Sq] rowsum(dO * O)
  float* ws_l;           // [B, Hq, Sq] LSE * log2(e), +inf where LSE = -inf
  int64_t q_sb, q_sh, q_ss;  // element strides (q, o, dout, dq)
  int64_t k_sb, k_sh, k_ss;  // element strides (k, v, dk, dv)
  int B, Hq, Hkv, Sq, Sk;
  int group;             // Hq / Hkv
  int D;                 // head dim: 128, or 64 (dense, no ALiBi)
  float c;               // scale * log2(e)
  float scale;
  // packed sequences (null cu_q: dense batch): sequence b is rows
  // cu_q[b] .. cu_q[b+1]-1 of q and cu_k[b] .. cu_k[b+1]-1 of k; Sq and Sk are
  // then the longest lengths, LSE and the workspace [Hq, total_q]
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k;
  const float* alibi;    // ALiBi slopes [Hq] of the forward (null: none; dense only)
};

hipError_t launch_backward(const BwdArgs& a, bool causal, hipStream_t stream);

}  // namespace attn
