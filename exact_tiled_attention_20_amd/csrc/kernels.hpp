// Launch descriptors shared between the host API and the gfx950 kernels.
// Host code fills these after validating the caller's attn_params; kernels
// receive them by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Forward tiling: 4 waves x 32 query rows per workgroup, 64 keys per tile.
constexpr int kFwdBlockQ = 128;
constexpr int kFwdBlockK = 64;
constexpr int kFwdThreads = 256;

// dQ kernel: 4 waves x 32 query rows per workgroup (the dK/dV kernel's shape
// is set next to it).
constexpr int kBwdThreads = 256;

// Banded masks (causal, sliding window, non-square alignment) reach the
// kernels as one key band per query row: key j is visible to query i iff
// i + band_lo <= j <= i + band_hi (and j < the key-padding length). Unbounded
// sides hold -kBandInf / +kBandInf, far enough from 0 that adding any index
// stays inside int32.
constexpr int kBandInf = 1 << 30;

// Mask modes of the kernel instantiations. kMaskCausal is the square causal
// mask (band_lo = -kBandInf, band_hi = 0), compiled with those constants;
// kMaskBand reads both edges from the arguments (sliding windows, causal masks
// on a non-square grid).
constexpr int kMaskNone = 0;
constexpr int kMaskCausal = 1;
constexpr int kMaskBand = 2;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;               // out dtype: 16-bit storage or float
  float* lse;
  const int32_t* kv_len; // device [B] or nullptr
  int B, H, N;           // N: query rows
  int Nk;                // key/value rows
  int band_lo, band_hi;  // visible keys of row i: [i + band_lo, i + band_hi]
  int nqb;               // query blocks per head
  int per_xcd;           // work items per XCD (ceil(total / 8))
  int total;             // B * H * nqb
  float scale;           // softmax scale (fp32)
  float scale_log2;      // scale * log2(e)
  float rescale_thr;     // raise the reference max when a row max exceeds it
                         // by this much (raw q.k units): bits / scale_log2,
                         // bits = 64 (bf16), 15 (fp16), 8 (e4m3)
  uint32_t drop_threshold;  // keep iff draw >= threshold
  float drop_rescale;       // 1 / (1 - p)
  uint32_t seed_lo, seed_hi;
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const void* o;         // out dtype
  const float* lse;
  const uint16_t* d_o;
  void* dq;              // out dtype
  void* dk;
  void* dv;
  float* delta;          // workspace: D_i = dO_i . O_i, (B, H, Np) fp32
  float* lse2;           // workspace: lse_i * log2(e) (+inf where lse_i = -inf), (B, H, Np) fp32
  const int32_t* kv_len;
  int B, H, N;           // N: query rows
  int Np;                // row stride of delta and lse2: N rounded up to a multiple of 4
  int Nk;                // key/value rows
  int band_lo, band_hi;  // as in FwdArgs
  float scale;
  float scale_log2;
  uint32_t drop_threshold;
  float drop_rescale;
  uint32_t seed_lo, seed_hi;
};

struct MaskArgs {
  uint8_t* keep;
  int B, H, N, Nk;
  uint32_t drop_threshold;
  uint32_t seed_lo, seed_hi;
};

// Kernel families. `dtype` is 0 (fp16) or 1 (bf16); `mask` is one of the
// kMask* modes (with kMaskNone every key below the padding length is
// visible); `out_f32` selects float outputs. Each returns hipSuccess or the
// launch error.
hipError_t launch_fwd(int dtype, int d, int mask, bool dropout, bool out_f32,
                      const FwdArgs& a, hipStream_t stream);
// stage: -1 = all three kernels, else 0 (preprocess), 1 (dK/dV), 2 (dQ).
hipError_t launch_bwd(int dtype, int d, int mask, bool dropout, bool out_f32, int stage,
                      const BwdArgs& a, hipStream_t stream);
// The dQ kernel at d = 256 (its own translation unit; called by launch_bwd).
hipError_t launch_bwd_dq256(int dtype, int mask, bool dropout, bool out_f32, const BwdArgs& a,
                            hipStream_t stream);
hipError_t launch_dropout_mask(const MaskArgs& a, hipStream_t stream);
// Forward on e4m3 Q, K, V (d = 128; O in bf16 or float).
hipError_t launch_fwd_fp8(int mask, bool dropout, bool out_f32, const FwdArgs& a,
                          hipStream_t stream);

}  // namespace attn
