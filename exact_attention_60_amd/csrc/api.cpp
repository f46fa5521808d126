// C ABI of the gfx950 attention library: argument checks, launch geometry and
// launches on the caller's stream.  Every check runs before the first HIP
// call, so invalid arguments are reported without touching a device, and the
// library never allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "attn.h"
#include "kernels.h"

static_assert(attn::kRoundRTNE == ATTN_ROUND_RTNE && attn::kRoundRTNA == ATTN_ROUND_RTNA &&
                  attn::kRoundRTZ == ATTN_ROUND_RTZ,
              "kernel rounding codes follow the ABI's");

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];   // 0 unknown, 1 gfx950, -1 unusable
std::atomic<int> g_dev_cus[kMaxDevices];

// Checks once per device that it is a gfx950 and caches its CU count.
int current_device_cus(int* cus) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_DEVICE;
  int st = g_dev_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    st = ok ? 1 : -1;
    g_dev_state[dev].store(st, std::memory_order_release);
  }
  if (st != 1) return ATTN_ERR_DEVICE;
  *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
  return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

bool rounding_ok(int r) { return r == ATTN_ROUND_RTNE || r == ATTN_ROUND_RTNA || r == ATTN_ROUND_RTZ; }

}  // namespace

extern "C" {

int attn_version(void) { return ATTN_VERSION; }

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape (sizes must be >= 1, Hq a multiple of Hkv, within limits)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported argument (head dim 128 everywhere, also 64/256 in attn_fwd[_rounded] and 64 in attn_bwd; page_size 16, layout BSHD/BHSD, scale finite and > 0, causal 0/1, rounding RTNE/RTNA/RTZ)";
    case ATTN_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case ATTN_ERR_DEVICE: return "no usable gfx950 device is current";
    default: return "unknown status";
  }
}

// whether the dense d = 128 forward runs the GQA kernel (groups of 4k query
// heads share each K/V tile; it converts V itself)
static bool uses_pipe(int Hq, int Hkv, int d, bool alibi) {
  return d == attn::kHeadDim && !alibi && (Hq / Hkv) % 4 == 0;
}

static int fwd_call(const void* q, const void* k, const void* v, void* o, float* lse,
                    const float* alibi_slopes, int B, int Hq, int Hkv, int Sq, int Sk, int d,
                    float scale, int causal, int layout, int rounding, void* stream,
                    const void* vt = nullptr) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  // head dim 128 (every variant), or 64 and 256 (dense, no ALiBi)
  const bool hd64 = d == 64 || d == 256;
  if ((d != attn::kHeadDim && !(hd64 && !alibi_slopes)) ||
      (layout != ATTN_BSHD && layout != ATTN_BHSD) || (causal != 0 && causal != 1) ||
      !scale_ok(scale) || !rounding_ok(rounding))
    return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_ALIGN;
  const int64_t D = d;
  attn::PrefillArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  if (layout == ATTN_BSHD) {
    a.q_sb = (int64_t)Sq * Hq * D; a.q_sh = D; a.q_ss = (int64_t)Hq * D;
    a.k_sb = (int64_t)Sk * Hkv * D; a.k_sh = D; a.k_ss = (int64_t)Hkv * D;
  } else {
    a.q_sb = (int64_t)Hq * Sq * D; a.q_sh = (int64_t)Sq * D; a.q_ss = D;
    a.k_sb = (int64_t)Hkv * Sk * D; a.k_sh = (int64_t)Sk * D; a.k_ss = D;
  }
  // K/V of one (batch, kv head) are addressed with 32-bit byte offsets
  if ((int64_t)(Sk - 1) * a.k_ss * 2 + D * 2 > INT32_MAX) return ATTN_ERR_SHAPE;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk;
  a.group = Hq / Hkv;
  // d = 128 without ALiBi and a GQA group that is a multiple of 4: the
  // kernel whose workgroups share each K/V tile among 4 query heads
  const bool pipe = uses_pipe(Hq, Hkv, d, alibi_slopes != nullptr);
  const int rows_per_block = hd64   ? attn::kPrefillHdRows
                             : pipe ? attn::kPrefillPipeRows
                                    : attn::kPrefillBM;
  a.n_qt = (Sq + rows_per_block - 1) / rows_per_block;
  if ((int64_t)B * Hq * a.n_qt > INT32_MAX) return ATTN_ERR_SHAPE;
  a.c = scale * 1.4426950408889634f;
  a.rounding = rounding;
  a.cu_q = nullptr;
  a.cu_k = nullptr;
  a.total_q = a.total_k = 0;
  a.alibi = alibi_slopes;
  const int tk = d == 256 ? attn::kPrefillD256BN : d == 64 ? 64
                 : pipe ? attn::kPrefillPipeBN : attn::kPrefillBN;
  a.vt = static_cast<const uint8_t*>(vt);
  a.n_kt = (Sk + tk - 1) / tk;
  int cus = 0;
  const int ds = current_device_cus(&cus);
  if (ds != ATTN_OK) return ds;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = d == 64    ? attn::launch_prefill_hd(a, causal != 0, st)
                       : d == 256 ? attn::launch_prefill_d256(a, causal != 0, st)
                       : pipe ? attn::launch_prefill_pipe(a, causal != 0, st)
                              : attn::launch_prefill(a, causal != 0, st);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int Hq,
                    int Hkv, int total_q, int total_k, int max_seqlen_q, int d, float scale,
                    int causal, int rounding, void* stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || total_q < 1 || total_k < 1 || max_seqlen_q < 1 ||
      Hq % Hkv != 0)
    return ATTN_ERR_SHAPE;
  if (d != attn::kHeadDim || (causal != 0 && causal != 1) || !scale_ok(scale) ||
      !rounding_ok(rounding))
    return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return ATTN_ERR_ALIGN;
  const int64_t D = attn::kHeadDim;
  attn::PrefillArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  // packed [total, H, 128]: the batch stride is unused (rows come from the offsets)
  a.q_sb = 0; a.q_sh = D; a.q_ss = (int64_t)Hq * D;
  a.k_sb = 0; a.k_sh = D; a.k_ss = (int64_t)Hkv * D;
  // the K/V rows of one sequence are addressed with 32-bit byte offsets
  if ((int64_t)(total_k - 1) * a.k_ss * 2 + 256 > INT32_MAX) return ATTN_ERR_SHAPE;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv;
  a.Sq = max_seqlen_q;
  a.Sk = 0;
  a.group = Hq / Hkv;
  // groups of 4k query heads run the GQA kernel (64-row query tiles of four
  // heads), others the 8-wave kernel (256-row tiles of one head)
  const bool pipe = uses_pipe(Hq, Hkv, d, false);
  const int rows = pipe ? attn::kPrefillPipeRows : attn::kPrefillBM;
  a.n_qt = (max_seqlen_q + rows - 1) / rows;
  if ((int64_t)B * Hq * a.n_qt > INT32_MAX) return ATTN_ERR_SHAPE;
  a.c = scale * 1.4426950408889634f;
  a.rounding = rounding;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  a.alibi = nullptr;
  int cus = 0;
  const int ds = current_device_cus(&cus);
  if (ds != ATTN_OK) return ds;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = pipe ? attn::launch_prefill_pipe(a, causal != 0, st)
                            : attn::launch_prefill(a, causal != 0, st);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// keys per prepared tile: that of the kernel attn_fwd runs for the shape
// keys per prepared tile: the tile size of the kernel that reads them
static int prep_tile_keys(int Hq, int Hkv, int d) {
  if (d == 256) return attn::kPrefillD256BN;
  if (d == 64) return 64;
  return uses_pipe(Hq, Hkv, attn::kHeadDim, false) ? attn::kPrefillPipeBN : attn::kPrefillBN;
}

size_t attn_prep_v_bytes(int B, int Hq, int Hkv, int Sk, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sk < 1 || Hq % Hkv != 0) return 0;
  if (d != attn::kHeadDim && d != 256 && d != 64) return 0;
  const int tk = prep_tile_keys(Hq, Hkv, d);
  const int64_t n_kt = (Sk + tk - 1) / tk;
  return (size_t)B * Hkv * n_kt * tk * d * 2;
}

int attn_prep_v(const void* v, int B, int Hq, int Hkv, int Sk, int d, int layout, void* vt,
                size_t vt_bytes, void* stream) {
  if (!v) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sk < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (layout != ATTN_BSHD && layout != ATTN_BHSD) return ATTN_ERR_UNSUPPORTED;
  const size_t need = attn_prep_v_bytes(B, Hq, Hkv, Sk, d);
  if (need == 0) return ATTN_OK;                     // this shape does not use the tiles
  if (!vt || vt_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned16(v) || !aligned16(vt)) return ATTN_ERR_ALIGN;
  const int64_t D = d;
  attn::PrepVArgs a;
  a.v = static_cast<const __bf16*>(v);
  a.vt = static_cast<uint8_t*>(vt);
  if (layout == ATTN_BSHD) {
    a.k_sb = (int64_t)Sk * Hkv * D; a.k_sh = D; a.k_ss = (int64_t)Hkv * D;
  } else {
    a.k_sb = (int64_t)Hkv * Sk * D; a.k_sh = (int64_t)Sk * D; a.k_ss = D;
  }
  a.B = B; a.Hkv = Hkv; a.Sk = Sk;
  a.tk = prep_tile_keys(Hq, Hkv, d);
  a.n_kt = (Sk + a.tk - 1) / a.tk;
  if ((int64_t)B * Hkv * a.n_kt > INT32_MAX) return ATTN_ERR_SHAPE;
  // one head's tiles are addressed with 32-bit offsets
  if ((int64_t)a.n_kt * a.tk * D * 2 > (int64_t)UINT32_MAX) return ATTN_ERR_SHAPE;
  int cus = 0;
  const int ds = current_device_cus(&cus);
  if (ds != ATTN_OK) return ds;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = d == 256 ? attn::launch_prep_v_d256(a, st)
                       : d == 64  ? attn::launch_prep_v_d64(a, st)
                                  : attn::launch_prep_v(a, st);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_fwd_prepped(const void* q, const void* k, const void* v, const void* vt,
                     size_t vt_bytes, void* o, float* lse, int B, int Hq, int Hkv, int Sq, int Sk,
                     int d, float scale, int causal, int layout, int rounding, void* stream) {
  const size_t need = attn_prep_v_bytes(B, Hq, Hkv, Sk, d);
  if (need != 0) {
    if (!vt) return ATTN_ERR_NULL;
    if (vt_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned16(vt)) return ATTN_ERR_ALIGN;
    const int tk = prep_tile_keys(Hq, Hkv, d);
    if ((int64_t)((Sk + tk - 1) / tk) * tk * d * 2 > (int64_t)UINT32_MAX) return ATTN_ERR_SHAPE;
  }
  return fwd_call(q, k, v, o, lse, nullptr, B, Hq, Hkv, Sq, Sk, d, scale, causal, layout,
                  rounding, stream, need != 0 ? vt : nullptr);
}

int attn_fwd_rounded(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal, int layout,
                     int rounding, void* stream) {
  return fwd_call(q, k, v, o, lse, nullptr, B, Hq, Hkv, Sq, Sk, d, scale, causal, layout,
                  rounding, stream);
}

int attn_fwd_alibi(const void* q, const void* k, const void* v, void* o, float* lse,
                   const float* alibi_slopes, int B, int Hq, int Hkv, int Sq, int Sk, int d,
                   float scale, int causal, int layout, int rounding, void* stream) {
  if (!alibi_slopes) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(alibi_slopes) & 3u) return ATTN_ERR_ALIGN;
  return fwd_call(q, k, v, o, lse, alibi_slopes, B, Hq, Hkv, Sq, Sk, d, scale, causal, layout,
                  rounding, stream);
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
             int Hkv, int Sq, int Sk, int d, float scale, int causal, int layout,
             void* stream) {
  return attn_fwd_rounded(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, scale, causal, layout,
                          ATTN_ROUND_RTNE, stream);
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, float descale_q, float descale_k,
                 float descale_v, void* o, float* lse, int B, int Hq, int Hkv, int Sq, int Sk,
                 int d, float scale, int causal, int layout, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  // the descales and the scale fold into two fp32 constants, which must stay
  // normal, positive and finite
  const double cd = (double)scale * 1.4426950408889634 * (double)descale_q * (double)descale_k;
  const double od = (double)descale_v;
  const bool consts_ok = std::isfinite(cd) && std::isfinite(od) && cd >= 1.2e-38 &&
                         od >= 1.2e-38 && cd <= 3.0e38 && od <= 3.0e38;
  if (d != attn::kHeadDim || (layout != ATTN_BSHD && layout != ATTN_BHSD) ||
      (causal != 0 && causal != 1) || !scale_ok(scale) || !scale_ok(descale_q) ||
      !scale_ok(descale_k) || !scale_ok(descale_v) || !consts_ok)
    return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_ALIGN;
  const int64_t D = d;
  attn::Fp8Args a;
  a.q = static_cast<const uint8_t*>(q);
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  if (layout == ATTN_BSHD) {
    a.q_sb = (int64_t)Sq * Hq * D; a.q_sh = D; a.q_ss = (int64_t)Hq * D;
    a.k_sb = (int64_t)Sk * Hkv * D; a.k_sh = D; a.k_ss = (int64_t)Hkv * D;
  } else {
    a.q_sb = (int64_t)Hq * Sq * D; a.q_sh = (int64_t)Sq * D; a.q_ss = D;
    a.k_sb = (int64_t)Hkv * Sk * D; a.k_sh = (int64_t)Sk * D; a.k_ss = D;
  }
  // K/V of one (batch, kv head) are addressed with 32-bit byte offsets
  if ((int64_t)(Sk - 1) * a.k_ss + D > INT32_MAX) return ATTN_ERR_SHAPE;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk;
  a.group = Hq / Hkv;
  a.n_qt = (Sq + attn::kFp8RowsPerBlock - 1) / attn::kFp8RowsPerBlock;
  if ((int64_t)B * Hq * a.n_qt > INT32_MAX) return ATTN_ERR_SHAPE;
  a.c = (float)cd;
  a.out_scale = (float)od;
  int cus = 0;
  const int ds = current_device_cus(&cus);
  if (ds != ATTN_OK) return ds;
  const hipError_t e = attn::launch_prefill_fp8(a, causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t attn_decode_workspace_bytes(int B, int Hq, int max_blocks_per_seq) {
  if (B < 1 || Hq < 1 || max_blocks_per_seq < 1) return 0;
  const size_t splits = (size_t)attn::decode_max_splits(max_blocks_per_seq);
  // partial outputs and LSEs, then one count per (sequence, unit group) (at
  // most Hq unit groups)
  return (size_t)B * Hq * (splits * (attn::kHeadDim + 1) + 1) * sizeof(float);
}

}  // extern "C"

namespace {

// The decode entry points share this: argument checks, then the launch.
// knew / vnew are null unless the call appends the current token.  noalloc:
// the workspace is the library's own device scratch array (workspace and
// workspace_bytes are ignored); the size limit is checked with the other
// arguments, the array's address looked up after them.
int decode_call(const void* q, const void* knew, const void* vnew, const void* k_cache,
                const void* v_cache, void* kc_out, void* vc_out, const int32_t* block_table,
                const int32_t* seq_lens, void* o, float* lse, int B, int Hq, int Hkv, int d,
                int page_size, int max_blocks_per_seq, int num_pages, float scale, int rounding,
                void* workspace, size_t workspace_bytes, void* stream, bool noalloc = false) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o || !lse) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_blocks_per_seq < 1 || num_pages < 1)
    return ATTN_ERR_SHAPE;
  if (B > 65535 || max_blocks_per_seq > 262140) return ATTN_ERR_SHAPE;
  if (d != attn::kHeadDim || page_size != attn::kPage || !scale_ok(scale) ||
      !rounding_ok(rounding))
    return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(block_table) ||
      !aligned16(seq_lens) || !aligned16(o) || !aligned16(lse) || !aligned16(knew) ||
      !aligned16(vnew))
    return ATTN_ERR_ALIGN;
  const size_t need = attn_decode_workspace_bytes(B, Hq, max_blocks_per_seq);
  if (noalloc) {
    if (need > attn::kDecodeNoAllocScratchBytes) return ATTN_ERR_WORKSPACE;
  } else {
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
  }
  int cus = 0;
  const int ds = current_device_cus(&cus);
  if (ds != ATTN_OK) return ds;
  if (noalloc && attn::decode_noalloc_scratch(&workspace) != hipSuccess) return ATTN_ERR_DEVICE;

  attn::DecodeArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.kc = static_cast<const __bf16*>(k_cache);
  a.vc = static_cast<const __bf16*>(v_cache);
  a.table = block_table;
  a.lens = seq_lens;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.n_hb = (a.G + attn::kDecodeHeadsPerBlock - 1) / attn::kDecodeHeadsPerBlock;
  a.max_blocks = max_blocks_per_seq;
  a.num_pages = num_pages;
  a.X = (Hkv * a.n_hb + attn::kDecodeWaves - 1) / attn::kDecodeWaves;
  a.max_splits = attn::decode_max_splits(max_blocks_per_seq);
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = a.ws_o + (size_t)B * Hq * a.max_splits * attn::kHeadDim;
  a.ws_cnt = reinterpret_cast<int*>(a.ws_lse + (size_t)B * Hq * a.max_splits);
  a.nwg = 0;
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.token_stride = (int64_t)Hkv * attn::kHeadDim;
  a.page_stride = (int64_t)attn::kPage * a.token_stride;
  a.c = scale * 1.4426950408889634f;
  a.rounding = rounding;
  a.knew = static_cast<const __bf16*>(knew);
  a.vnew = static_cast<const __bf16*>(vnew);
  a.kc_out = static_cast<__bf16*>(kc_out);
  a.vc_out = static_cast<__bf16*>(vc_out);
  const hipError_t e = attn::launch_decode(a, cus, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int attn_decode_paged_rounded(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, void* o,
                              float* lse, int B, int Hq, int Hkv, int d, int page_size,
                              int max_blocks_per_seq, int num_pages, float scale, int rounding,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return decode_call(q, nullptr, nullptr, k_cache, v_cache, nullptr, nullptr, block_table,
                     seq_lens, o, lse, B, Hq, Hkv, d, page_size, max_blocks_per_seq, num_pages,
                     scale, rounding, workspace, workspace_bytes, stream);
}

int attn_decode_paged_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                             void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                             void* o, float* lse, int B, int Hq, int Hkv, int d, int page_size,
                             int max_blocks_per_seq, int num_pages, float scale, int rounding,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_new || !v_new) return ATTN_ERR_NULL;
  return decode_call(q, k_new, v_new, k_cache, v_cache, k_cache, v_cache, block_table, seq_lens,
                     o, lse, B, Hq, Hkv, d, page_size, max_blocks_per_seq, num_pages, scale,
                     rounding, workspace, workspace_bytes, stream);
}

int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                      int B, int Hq, int Hkv, int d, int page_size, int max_blocks_per_seq,
                      int num_pages, float scale, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return attn_decode_paged_rounded(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, Hq, Hkv,
                                   d, page_size, max_blocks_per_seq, num_pages, scale,
                                   ATTN_ROUND_RTNE, workspace, workspace_bytes, stream);
}

int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, void* o,
                              float* lse, int B, int Hq, int Hkv, int d, int page_size,
                              int max_blocks_per_seq, int num_pages, float scale, void* stream) {
  return decode_call(q, nullptr, nullptr, k_cache, v_cache, nullptr, nullptr, block_table,
                     seq_lens, o, lse, B, Hq, Hkv, d, page_size, max_blocks_per_seq, num_pages,
                     scale, ATTN_ROUND_RTNE, nullptr, 0, stream, /*noalloc=*/true);
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Sq) {
  if (B < 1 || Hq < 1 || Sq < 1) return 0;
  return (size_t)2 * B * Hq * Sq * sizeof(float);
}

static int bwd_call(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, const float* alibi_slopes,
                    int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                    int layout, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  // head dim 128, or 64 without ALiBi
  if ((d != attn::kHeadDim && !(d == 64 && !alibi_slopes)) ||
      (layout != ATTN_BSHD && layout != ATTN_BHSD) || (causal != 0 && causal != 1) ||
      !scale_ok(scale))
    return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return ATTN_ERR_ALIGN;
  if (B > 65535 || Hq > 65535) return ATTN_ERR_SHAPE;
  const int64_t D = d;
  attn::BwdArgs a;
  if (layout == ATTN_BSHD) {
    a.q_sb = (int64_t)Sq * Hq * D; a.q_sh = D; a.q_ss = (int64_t)Hq * D;
    a.k_sb = (int64_t)Sk * Hkv * D; a.k_sh = D; a.k_ss = (int64_t)Hkv * D;
  } else {
    a.q_sb = (int64_t)Hq * Sq * D; a.q_sh = (int64_t)Sq * D; a.q_ss = D;
    a.k_sb = (int64_t)Hkv * Sk * D; a.k_sh = (int64_t)Sk * D; a.k_ss = D;
  }
  // the rows of one (batch, head) are addressed with 32-bit byte offsets,
  // including the zero-filled rows past the end of a last 64-row block
  if (((int64_t)Sq + 64) * a.q_ss * 2 > INT32_MAX || ((int64_t)Sk + 64) * a.k_ss * 2 > INT32_MAX)
    return ATTN_ERR_SHAPE;
  const size_t need = attn_bwd_workspace_bytes(B, Hq, Sq);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<const __bf16*>(o);
  a.dout = static_cast<const __bf16*>(dout);
  a.lse = lse;
  a.dq = static_cast<__bf16*>(dq);
  a.dk = static_cast<__bf16*>(dk);
  a.dv = static_cast<__bf16*>(dv);
  a.ws_d = static_cast<float*>(workspace);
  a.ws_l = a.ws_d + (size_t)B * Hq * Sq;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk;
  a.group = Hq / Hkv;
  a.D = d;
  a.c = scale * 1.4426950408889634f;
  a.scale = scale;
  a.cu_q = nullptr;
  a.cu_k = nullptr;
  a.total_q = a.total_k = 0;
  a.alibi = alibi_slopes;
  int cus = 0;
  const int ds = current_device_cus(&cus);
  if (ds != ATTN_OK) return ds;
  const hipError_t e = attn::launch_backward(a, causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
             int Sk, int d, float scale, int causal, int layout, void* workspace,
             size_t workspace_bytes, void* stream) {
  return bwd_call(q, k, v, o, lse, dout, dq, dk, dv, nullptr, B, Hq, Hkv, Sq, Sk, d, scale,
                  causal, layout, workspace, workspace_bytes, stream);
}

int attn_bwd_alibi(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, const float* alibi_slopes,
                   int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                   int layout, void* workspace, size_t workspace_bytes, void* stream) {
  if (!alibi_slopes) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(alibi_slopes) & 3u) return ATTN_ERR_ALIGN;
  return bwd_call(q, k, v, o, lse, dout, dq, dk, dv, alibi_slopes, B, Hq, Hkv, Sq, Sk, d, scale,
                  causal, layout, workspace, workspace_bytes, stream);
}

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q,
                    const int32_t* cu_seqlens_k, int B, int Hq, int Hkv, int total_q,
                    int total_k, int max_seqlen_q, int max_seqlen_k, int d, float scale,
                    int causal, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !cu_seqlens_q ||
      !cu_seqlens_k)
    return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || total_q < 1 || total_k < 1 || max_seqlen_q < 1 ||
      max_seqlen_k < 1 || Hq % Hkv != 0)
    return ATTN_ERR_SHAPE;
  if (d != attn::kHeadDim || (causal != 0 && causal != 1) || !scale_ok(scale))
    return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return ATTN_ERR_ALIGN;
  if (Hq > 65535) return ATTN_ERR_SHAPE;
  const int64_t D = attn::kHeadDim;
  attn::BwdArgs a;
  a.q_sb = 0; a.q_sh = D; a.q_ss = (int64_t)Hq * D;
  a.k_sb = 0; a.k_sh = D; a.k_ss = (int64_t)Hkv * D;
  // rows of one sequence are addressed with 32-bit byte offsets, including
  // the zero-filled rows past the end of a last 64-row block
  if (((int64_t)total_q + 64) * a.q_ss * 2 > INT32_MAX ||
      ((int64_t)total_k + 64) * a.k_ss * 2 > INT32_MAX)
    return ATTN_ERR_SHAPE;
  if ((int64_t)B * Hkv * ((max_seqlen_k + attn::kBwdKvRows - 1) / attn::kBwdKvRows) > INT32_MAX ||
      (int64_t)B * Hq * ((max_seqlen_q + attn::kBwdQRows - 1) / attn::kBwdQRows) > INT32_MAX)
    return ATTN_ERR_SHAPE;
  const size_t need = attn_bwd_workspace_bytes(1, Hq, total_q);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<const __bf16*>(o);
  a.dout = static_cast<const __bf16*>(dout);
  a.lse = lse;
  a.dq = static_cast<__bf16*>(dq);
  a.dk = static_cast<__bf16*>(dk);
  a.dv = static_cast<__bf16*>(dv);
  a.ws_d = static_cast<float*>(workspace);
  a.ws_l = a.ws_d + (size_t)Hq * total_q;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv;
  a.Sq = max_seqlen_q;
  a.Sk = max_seqlen_k;
  a.group = Hq / Hkv;
  a.D = attn::kHeadDim;
  a.c = scale * 1.4426950408889634f;
  a.scale = scale;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  a.alibi = nullptr;
  int cus = 0;
  const int ds = current_device_cus(&cus);
  if (ds != ATTN_OK) return ds;
  const hipError_t e = attn::launch_backward(a, causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // extern "C"
