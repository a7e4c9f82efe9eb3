// Host side of the C ABI declared in include/attn.h.
//
// Every argument is validated here, on the host, before any HIP call; an
// unsupported combination returns ATTN_ERR_UNSUPPORTED and nothing runs. The
// anthology-of-the-sota page SOTA-114 ("Cost") names the hazard this avoids:
// fused kernels exist per (mask, dropout, head dim, dtype) combination and a
// silent fallback to a slow path goes unnoticed. This library has no fallback.
#include "../../include/attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "api_internal.hpp"
#include "kernels.hpp"

namespace {

// 0.3.0: Nk is always explicit (no "0 means N" sentinel); zero key rows and
// zero query rows are valid problems; pointers of empty tensors may be NULL.
// 0.4.0: fp8 (e4m3) forward.
// 0.5.0: the backward workspace's two arrays have N rounded up to a multiple
//        of 4 rows per head.
constexpr int32_t kVersion = 500;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(int32_t dt) { return dt == ATTN_F32 ? 4 : (dt == ATTN_E4M3 ? 1 : 2); }

struct Range {
  uintptr_t lo, hi;
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

// Empty ranges (tensors with no elements) overlap nothing.
bool overlap(Range x, Range y) {
  if (x.lo == x.hi || y.lo == y.hi) return false;
  return x.lo < y.hi && y.lo < x.hi;
}

// Rows of K and V.
int32_t key_rows(const attn_params* p) { return p->Nk; }

// A tensor pointer is acceptable if it is 16-byte aligned and non-NULL, or if
// the tensor has no elements (then it is never read or written).
bool ptr_ok(const void* x, size_t bytes) { return bytes == 0 || (x != nullptr && aligned16(x)); }

// Shape/dtype/scalar checks common to every entry point.
attn_status check_params(const attn_params* p) {
  if (p == nullptr) return ATTN_ERR_INVALID_ARG;
  if (p->B < 0 || p->H < 0 || p->N < 0 || p->d < 1) return ATTN_ERR_INVALID_ARG;
  if (p->Nk < 0 || p->window_left < -1 || p->window_right < -1) return ATTN_ERR_INVALID_ARG;
  if (p->dtype != ATTN_F16 && p->dtype != ATTN_BF16 && p->dtype != ATTN_F32 &&
      p->dtype != ATTN_E4M3)
    return ATTN_ERR_INVALID_ARG;
  if (p->out_dtype != ATTN_F16 && p->out_dtype != ATTN_BF16 && p->out_dtype != ATTN_F32 &&
      p->out_dtype != ATTN_E4M3)
    return ATTN_ERR_INVALID_ARG;
  if (p->causal != 0 && p->causal != 1) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(p->scale) || !(p->scale > 0.0f)) return ATTN_ERR_INVALID_ARG;
  if (!(p->dropout_p >= 0.0f && p->dropout_p < 1.0f)) return ATTN_ERR_INVALID_ARG;
  // Element counts: per head N*d must index in 32 bits; the whole tensor must
  // stay far from overflow of 64-bit byte offsets; the grids must fit.
  const long long rows = p->N > key_rows(p) ? p->N : key_rows(p);
  const long long per_head = rows * p->d;
  if (per_head >= (1ll << 31)) return ATTN_ERR_INVALID_ARG;
  const long long heads = (long long)p->B * p->H;
  if (heads >= (1ll << 31)) return ATTN_ERR_INVALID_ARG;
  if ((double)heads * (double)per_head >= 4.0e18) return ATTN_ERR_INVALID_ARG;
  const long long blocks = heads * ((p->N + attn::kFwdBlockQ - 1) / attn::kFwdBlockQ);
  if (blocks + 8 >= (1ll << 31)) return ATTN_ERR_INVALID_ARG;
  const long long key_blocks = heads * ((key_rows(p) + 255) / 256);
  if (key_blocks + 8 >= (1ll << 31)) return ATTN_ERR_INVALID_ARG;
  // Supported kernels (the e4m3 forward is checked by fp8_supported).
  if (p->dtype == ATTN_F32 || p->out_dtype == ATTN_E4M3) return ATTN_ERR_UNSUPPORTED;
  if (p->dtype == ATTN_E4M3) {
    if (p->out_dtype != ATTN_BF16 && p->out_dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
    if (p->d != 128) return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
  }
  if (p->out_dtype != p->dtype && p->out_dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (p->d != 64 && p->d != 128 && p->d != 256) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// The backward has no e4m3 kernels (checked after check_params).
attn_status bwd_supported(const attn_params* p) {
  return p->dtype == ATTN_E4M3 ? ATTN_ERR_UNSUPPORTED : ATTN_OK;
}

// A problem with no query rows, heads or batch entries: nothing to compute and
// no output element to write (call only after check_params has accepted p).
bool is_empty(const attn_params* p) { return p->B == 0 || p->H == 0 || p->N == 0; }

uint32_t drop_threshold(float p) {
  // floor(p * 2^32) is exact in double for a float p in [0, 1).
  return (uint32_t)std::floor((double)p * 4294967296.0);
}

size_t tensor_bytes(const attn_params* p, int32_t dt) {
  return (size_t)p->B * p->H * p->N * p->d * elem_bytes(dt);
}

// K, V, dK, dV: (B, H, Nk, d).
size_t key_tensor_bytes(const attn_params* p, int32_t dt) {
  return (size_t)p->B * p->H * key_rows(p) * p->d * elem_bytes(dt);
}

// The key band [i + lo, i + hi] of query row i that the causal mask and the
// sliding window leave (query i lines up with key i + Nk - N), and the kernel
// mask mode that applies it: kMaskNone when neither mask is set (every key
// below the padding length is visible), kMaskCausal for the plain causal band
// (lo unbounded, hi = 0), kMaskBand otherwise.
int key_band(const attn_params* p, int* lo, int* hi) {
  const long long off = (long long)key_rows(p) - p->N;
  long long l = -attn::kBandInf, h = attn::kBandInf;
  if (p->causal) h = off;
  if (p->window_right >= 0 && off + p->window_right < h) h = off + p->window_right;
  if (p->window_left >= 0) l = off - p->window_left;
  // Beyond +-kBandInf a bound excludes or admits every key of any valid shape
  // alike (|i|, |j| < 2^25 since N*d < 2^31), so clamping changes nothing.
  if (l < -attn::kBandInf) l = -attn::kBandInf;
  if (h > attn::kBandInf) h = attn::kBandInf;
  if (h < -attn::kBandInf) h = -attn::kBandInf;
  if (l > attn::kBandInf) l = attn::kBandInf;
  *lo = (int)l;
  *hi = (int)h;
  if (!(p->causal || p->window_left >= 0 || p->window_right >= 0)) return attn::kMaskNone;
  if (l == -attn::kBandInf && h == 0) return attn::kMaskCausal;
  return attn::kMaskBand;
}

size_t stat_bytes(const attn_params* p) { return (size_t)p->B * p->H * p->N * sizeof(float); }
// Rows per head of the backward's workspace arrays: N rounded up to a
// multiple of 4, so that every group of four rows is one aligned 16-byte load.
int stat_rows(const attn_params* p) { return (p->N + 3) & ~3; }
size_t ws_stat_bytes(const attn_params* p) {
  return (size_t)p->B * p->H * stat_rows(p) * sizeof(float);
}

}  // namespace

extern "C" {

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK: success";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG: invalid argument (pointer, size, scale, p or flag)";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: no kernel for this head dimension / dtype combination";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: backward workspace missing, misaligned or too small";
    case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
    case ATTN_ERR_TOO_LARGE:
      return "ATTN_ERR_TOO_LARGE: the problem needs more than the fixed scratch of the "
             "no-allocation entry point (use attn_bwd with a workspace)";
  }
  return "unknown attn_status";
}

int32_t attn_version(void) { return kVersion; }

attn_status attn_fwd(const attn_params* p, const void* q, const void* k, const void* v,
                     void* o, float* lse, void* stream) {
  attn_status st = check_params(p);
  if (st != ATTN_OK) return st;
  if (is_empty(p)) return ATTN_OK;
  const size_t in_b = tensor_bytes(p, p->dtype);
  const size_t kin_b = key_tensor_bytes(p, p->dtype);
  if (!ptr_ok(q, in_b) || !ptr_ok(k, kin_b) || !ptr_ok(v, kin_b) ||
      !ptr_ok(o, tensor_bytes(p, p->out_dtype)) || !ptr_ok(lse, stat_bytes(p)))
    return ATTN_ERR_INVALID_ARG;
  const Range outs[] = {range_of(o, tensor_bytes(p, p->out_dtype)), range_of(lse, stat_bytes(p))};
  const Range ins[] = {range_of(q, in_b), range_of(k, kin_b), range_of(v, kin_b)};
  if (overlap(outs[0], outs[1])) return ATTN_ERR_INVALID_ARG;
  for (const Range& r : outs)
    for (const Range& x : ins)
      if (overlap(r, x)) return ATTN_ERR_INVALID_ARG;
  if (p->kv_len != nullptr && (reinterpret_cast<uintptr_t>(p->kv_len) & 3u))
    return ATTN_ERR_INVALID_ARG;

  attn::FwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = o;
  a.lse = lse;
  a.kv_len = p->kv_len;
  a.B = p->B;
  a.H = p->H;
  a.N = p->N;
  a.Nk = key_rows(p);
  const int mask = key_band(p, &a.band_lo, &a.band_hi);
  a.nqb = (p->N + attn::kFwdBlockQ - 1) / attn::kFwdBlockQ;
  a.total = p->B * p->H * a.nqb;
  a.per_xcd = (a.total + 7) / 8;
  a.scale = p->scale;
  a.scale_log2 = (float)((double)p->scale * 1.4426950408889634);
  // How far (log2 of probability) a row maximum may exceed the reference
  // before the reference is raised: probabilities up to 2^bits relative to it
  // are formed and rounded into the operand type of the P V product, so the
  // bound is that type's range -- e4m3 holds 448 (2^8 is used), fp16 65504
  // (2^15), bf16 the fp32 exponent range (2^64 leaves the fp32 sums far from
  // overflow). Rounding is relative, so the value does not change accuracy;
  // a larger bound only makes the O rescale rarer.
  const float bits = p->dtype == ATTN_E4M3 ? 8.0f : (p->dtype == ATTN_F16 ? 15.0f : 64.0f);
  a.rescale_thr = bits / a.scale_log2;
  const bool dropout = p->dropout_p > 0.0f;
  a.drop_threshold = drop_threshold(p->dropout_p);
  a.drop_rescale = 1.0f / (1.0f - p->dropout_p);
  a.seed_lo = (uint32_t)(p->seed & 0xFFFFFFFFull);
  a.seed_hi = (uint32_t)(p->seed >> 32);
  const hipError_t e =
      p->dtype == ATTN_E4M3
          ? attn::launch_fwd_fp8(mask, dropout, p->out_dtype == ATTN_F32, a,
                                 static_cast<hipStream_t>(stream))
          : attn::launch_fwd(p->dtype == ATTN_BF16 ? 1 : 0, p->d, mask, dropout,
                             p->out_dtype == ATTN_F32, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t attn_bwd_workspace_bytes(const attn_params* p) {
  if (check_params(p) != ATTN_OK || bwd_supported(p) != ATTN_OK) return 0;
  // Two fp32 (B, H, Np) arrays (Np = N rounded up to a multiple of 4), each
  // rounded up to 256 bytes: D_i = dO_i . O_i and lse_i * log2(e).
  return 2 * ((ws_stat_bytes(p) + 255) & ~size_t(255));
}

// validate_only: run every check except those on the workspace, then return
// without any HIP call.
static attn_status bwd_impl(const attn_params* p, int32_t stage, const void* q, const void* k,
                            const void* v, const void* o, const float* lse, const void* d_o,
                            void* dq, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, void* stream, bool validate_only = false) {
  if (stage < -1 || stage > 2) return ATTN_ERR_INVALID_ARG;
  attn_status st = check_params(p);
  if (st != ATTN_OK) return st;
  st = bwd_supported(p);
  if (st != ATTN_OK) return st;
  // Nothing to write: no heads, or neither query nor key rows. With query rows
  // but no keys, dQ is zero; with keys but no query rows, dK and dV are zero:
  // both are written by the kernels below.
  if (p->B == 0 || p->H == 0 || (p->N == 0 && key_rows(p) == 0)) return ATTN_OK;
  const size_t in_b = tensor_bytes(p, p->dtype);
  const size_t out_b = tensor_bytes(p, p->out_dtype);
  const size_t kin_b = key_tensor_bytes(p, p->dtype);
  const size_t kout_b = key_tensor_bytes(p, p->out_dtype);
  if (!ptr_ok(q, in_b) || !ptr_ok(k, kin_b) || !ptr_ok(v, kin_b) || !ptr_ok(o, out_b) ||
      !ptr_ok(lse, stat_bytes(p)) || !ptr_ok(d_o, in_b) || !ptr_ok(dq, out_b) ||
      !ptr_ok(dk, kout_b) || !ptr_ok(dv, kout_b))
    return ATTN_ERR_INVALID_ARG;
  if (p->kv_len != nullptr && (reinterpret_cast<uintptr_t>(p->kv_len) & 3u))
    return ATTN_ERR_INVALID_ARG;
  const size_t need = validate_only ? 0 : attn_bwd_workspace_bytes(p);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need ||
                   (reinterpret_cast<uintptr_t>(workspace) & 255u)))
    return ATTN_ERR_WORKSPACE;
  const Range outs[] = {range_of(dq, out_b), range_of(dk, kout_b), range_of(dv, kout_b),
                        range_of(workspace, need)};
  const Range ins[] = {range_of(q, in_b), range_of(k, kin_b), range_of(v, kin_b),
                       range_of(o, out_b), range_of(lse, stat_bytes(p)), range_of(d_o, in_b)};
  for (int i = 0; i < 4; ++i) {
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return ATTN_ERR_INVALID_ARG;
    for (const Range& x : ins)
      if (overlap(outs[i], x)) return ATTN_ERR_INVALID_ARG;
  }
  if (validate_only) return ATTN_OK;

  attn::BwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = o;
  a.lse = lse;
  a.d_o = static_cast<const uint16_t*>(d_o);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = static_cast<float*>(workspace);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    ((ws_stat_bytes(p) + 255) & ~size_t(255)));
  a.kv_len = p->kv_len;
  a.B = p->B;
  a.H = p->H;
  a.N = p->N;
  a.Np = stat_rows(p);
  a.Nk = key_rows(p);
  const int mask = key_band(p, &a.band_lo, &a.band_hi);
  a.scale = p->scale;
  a.scale_log2 = (float)((double)p->scale * 1.4426950408889634);
  const bool dropout = p->dropout_p > 0.0f;
  a.drop_threshold = drop_threshold(p->dropout_p);
  a.drop_rescale = 1.0f / (1.0f - p->dropout_p);
  a.seed_lo = (uint32_t)(p->seed & 0xFFFFFFFFull);
  a.seed_hi = (uint32_t)(p->seed >> 32);
  const hipError_t e = attn::launch_bwd(p->dtype == ATTN_BF16 ? 1 : 0, p->d, mask,
                                        dropout, p->out_dtype == ATTN_F32, stage, a,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status attn_bwd(const attn_params* p, const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* d_o, void* dq, void* dk,
                     void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(p, -1, q, k, v, o, lse, d_o, dq, dk, dv, workspace, workspace_bytes, stream);
}

attn_status attn_bwd_stage(const attn_params* p, int32_t stage, const void* q, const void* k,
                           const void* v, const void* o, const float* lse, const void* d_o,
                           void* dq, void* dk, void* dv, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (stage < ATTN_BWD_STAGE_PREPROCESS || stage > ATTN_BWD_STAGE_DQ) return ATTN_ERR_INVALID_ARG;
  return bwd_impl(p, stage, q, k, v, o, lse, d_o, dq, dk, dv, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace attn {

attn_status bwd_validate_without_workspace(const attn_params* p, const void* q, const void* k,
                                           const void* v, const void* o, const float* lse,
                                           const void* d_o, void* dq, void* dk, void* dv) {
  return bwd_impl(p, -1, q, k, v, o, lse, d_o, dq, dk, dv, nullptr, 0, nullptr, true);
}

}  // namespace attn

extern "C" {

attn_status attn_dropout_mask(const attn_params* p, uint8_t* keep, void* stream) {
  attn_status st = check_params(p);
  if (st != ATTN_OK) return st;
  const double cells = (double)p->B * p->H * p->N * (double)key_rows(p);
  if (cells == 0.0) return ATTN_OK;
  if (keep == nullptr || !aligned16(keep)) return ATTN_ERR_INVALID_ARG;
  if (cells >= 9.0e15) return ATTN_ERR_INVALID_ARG;
  attn::MaskArgs a;
  a.keep = keep;
  a.B = p->B;
  a.H = p->H;
  a.N = p->N;
  a.Nk = key_rows(p);
  a.drop_threshold = drop_threshold(p->dropout_p);
  a.seed_lo = (uint32_t)(p->seed & 0xFFFFFFFFull);
  a.seed_hi = (uint32_t)(p->seed >> 32);
  const long long groups = (long long)p->B * p->H * p->N * ((key_rows(p) + 3) / 4);
  if ((groups + 255) / 256 >= (1ll << 31)) return ATTN_ERR_INVALID_ARG;
  const hipError_t e = attn::launch_dropout_mask(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // extern "C"
