// dQ kernel of the attention backward for gfx950 (included by attn_bwd.hip,
// which instantiates it for d <= 128, and by attn_bwd_dq256.hip for d = 256).
//
// With P_ij = exp(scale * Q_i.K_j - lse_i) on visible pairs, Z_ij the dropout
// factor and D_i = dO_i . O_i: dS_ij = P_ij (Z_ij dO_i . V_j - D_i) and
// dQ_i = scale * sum_j dS_ij K_j ("Why FlashAttention Is a Kernel Story",
// section "When it falls down": S and P are rebuilt from the saved
// log-sum-exp, not read back).
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {

constexpr float kLog2e = 1.4426950408889634f;

// dQ. Workgroup: 128 queries of one (b, h); wave w owns 32 query rows. The
// forward's orientation: S^T = K Q^T and dP^T = V dO^T put one query per lane,
// so lse_i and D_i are per-lane scalars, and the packed dS^T registers are the
// B operand of dQ^T += K^T dS^T (K read transposed from LDS). K/V tiles of 64
// keys are copied HBM -> LDS directly; each tile is processed as two 32-key
// halves to keep two waves per SIMD.
// Waves per SIMD the register budget is set for: one at d = 256; three at
// d = 64 (168 registers; 32 KiB of LDS per workgroup) except the unmasked
// dropout instance, which would spill; two otherwise.
template <int D, int MASK, bool DROPOUT>
constexpr int dq_waves_per_simd() {
  return D > 128 ? 1 : (D < 128 && !(DROPOUT && MASK == kMaskNone)) ? 3 : 2;
}

template <typename E, int D, int MASK, bool DROPOUT, bool OUT_F32>
__global__ __launch_bounds__(kBwdThreads)
__attribute__((amdgpu_waves_per_eu(dq_waves_per_simd<D, MASK, DROPOUT>(),
                                   dq_waves_per_simd<D, MASK, DROPOUT>())))
void attn_bwd_dq_kernel(const BwdArgs a) {
  constexpr int BR = 128;
  constexpr int BC = 64;
  constexpr int KK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE_BYTES = BC * D * 2;
  constexpr bool BAND = MASK != kMaskNone;
  constexpr bool LO = MASK == kMaskBand;   // a lower band edge exists

  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE_BYTES];

  const int nqb = (a.N + BR - 1) / BR;
  const WorkItem wi = decode_work_item(blockIdx.x, a.B * a.H, nqb);
  if (!wi.valid) return;
  const int bh = wi.bh;
  const int qblk = BAND ? nqb - 1 - wi.rank : wi.rank;  // heaviest first
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int N = a.N;
  const int q0 = qblk * BR;
  const size_t head = (size_t)bh * (size_t)N * D;
  const size_t khead = (size_t)bh * (size_t)a.Nk * D;
  const uint16_t* __restrict__ Q = a.q + head;
  const uint16_t* __restrict__ K = a.k + khead;
  const uint16_t* __restrict__ V = a.v + khead;
  const uint16_t* __restrict__ dO = a.d_o + head;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  int kv_end = a.Nk;
  if (a.kv_len != nullptr) kv_end = min(max(a.kv_len[b], 0), a.Nk);
  const int band_lo = LO ? a.band_lo : -kBandInf;
  const int band_hi = MASK == kMaskCausal ? 0 : a.band_hi;
  // Key tiles [t0, ntiles) hold every key a row of this block sees.
  int kend = kv_end;
  int t0 = 0;
  if (BAND) {
    kend = min(kend, max(0, min(q0 + BR, N) + band_hi));
    if (LO) t0 = max(0, q0 + band_lo) / BC;
  }
  const int ntiles = (kend + BC - 1) / BC;

  const int wq0 = q0 + 32 * w;
  const int qi = wq0 + l32;
  const bool wave_has_rows = wq0 < N;

  u32x4 qf[KK], of[KK];
  float lse2 = INFINITY, dlt = 0.f;
  {
    const int qr = min(qi, N - 1);
    const uint16_t* qs = Q + (size_t)qr * D + hh * 8;
    const uint16_t* os = dO + (size_t)qr * D + hh * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qf[kk] = *(const u32x4*)(qs + kk * 16);
      of[kk] = *(const u32x4*)(os + kk * 16);
    }
    if (qi < N) {
      const float x = a.lse[(size_t)bh * N + qi];
      lse2 = (x == -INFINITY) ? INFINITY : x * kLog2e;
      dlt = a.delta[(size_t)bh * a.Np + qi];
    }
  }

  char* const kb0 = smem;
  char* const vb0 = smem + 2 * TILE_BYTES;
  TilePairLoader<D, BC, 4> loader;
  loader.init(w, lane);

  int roff[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) roff[kk] = lds_off<D>(l32, (kk * 2 + hh) * 16);
  const int g = lane >> 4;
  const int i16 = lane & 15;
  int toff[2][NDB];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      toff[half][db] = lds_off<D>(4 * hh + (i16 >> 2) + 8 * half,
                                  (32 * db + 16 * (g & 1) + 4 * (i16 & 3)) * 2);

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  const float c2 = a.scale_log2;

  if (ntiles > t0) loader.issue(K, V, t0 * BC, kv_end, kb0, vb0);
  // The loop body is instantiated once per buffer (the loop is unrolled by
  // two), so every LDS address is a per-lane offset plus a constant that the
  // read instructions carry as their immediate offset.
  auto tile_step = [&](int t, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    wait_all_memory();
    __syncthreads();
    // Untracked, so that no LDS read of tile t waits for this prefetch; the
    // wait at the top of the next iteration orders it before its readers.
    if (t + 1 < ntiles) {
      loader.issue_one_untracked(K, (t + 1) * BC, kv_end, kb0 + (buf ^ 1) * TILE_BYTES);
      loader.issue_one_untracked(V, (t + 1) * BC, kv_end, vb0 + (buf ^ 1) * TILE_BYTES);
    }
    const int k0 = t * BC;
    const bool active = wave_has_rows &&
                        (!BAND || (k0 <= wq0 + 31 + band_hi &&
                                   (!LO || k0 + BC - 1 >= wq0 + band_lo)));
    if (!active) return;
    const char* kb = kb0 + buf * TILE_BYTES;
    const char* vb = vb0 + buf * TILE_BYTES;
    const bool need_mask =
        (BAND && (k0 + BC - 1 > wq0 + band_hi || (LO && k0 < wq0 + 31 + band_lo))) ||
        (k0 + BC > kv_end);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      // S^T and dP^T for keys k0 + 32 kb2 .. +32 (lane = query).
      // Without dropout the dP^T chain starts from -D (one value per lane:
      // this lane's query row), so dS^T = P^T dP'^T needs no subtraction.
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = DROPOUT ? 0.f : -dlt;
      }
      const int rbase = kb2 * 32 * D * 2;
      // Interleaved chains: a single dependent MFMA chain cannot issue at
      // the full rate.
      if constexpr (D > 128) {
        // One wave per SIMD: nothing else hides the LDS latency, so the K and
        // V fragments of k-step kk + 1 are read before the MFMAs of step kk.
        u32x4 kf[2], vf[2];
        kf[0] = *(const u32x4*)(kb + rbase + roff[0]);
        vf[0] = *(const u32x4*)(vb + rbase + roff[0]);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          if (kk + 1 < KK) {
            kf[(kk + 1) & 1] = *(const u32x4*)(kb + rbase + roff[kk + 1]);
            vf[(kk + 1) & 1] = *(const u32x4*)(vb + rbase + roff[kk + 1]);
          }
          s = E::mfma(kf[kk & 1], qf[kk], s);
          dp = E::mfma(vf[kk & 1], of[kk], dp);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          s = E::mfma(*(const u32x4*)(kb + rbase + roff[kk]), qf[kk], s);
          dp = E::mfma(*(const u32x4*)(vb + rbase + roff[kk]), of[kk], dp);
        }
      }
      // dS^T = P^T (Z dP^T - D); register r is key k0 + 32kb2 + 8(r/4) + 4hh + r%4.
      // The masked form is a separate instantiation, so the unmasked tiles
      // run branch-free.
      auto grad = [&](auto masked) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int j0 = k0 + kb2 * 32 + 8 * g4 + 4 * hh;
          u32x4 u = u32x4{0, 0, 0, 0};
          if (DROPOUT)
            u = dropout_draws((uint32_t)j0 >> 2, (uint32_t)qi, (uint32_t)h, (uint32_t)b,
                              a.seed_lo, a.seed_hi);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g4 + e;
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c2, -lse2));
            if (decltype(masked)::value) {
              const int jj = j0 + e;
              p = ((BAND && (jj > qi + band_hi || (LO && jj < qi + band_lo))) || jj >= kv_end)
                      ? 0.f : p;
            }
            if (DROPOUT) {
              const float dpz = (u[e] >= a.drop_threshold) ? dp[r] * a.drop_rescale : 0.f;
              s[r] = p * (dpz - dlt);
            } else {
              s[r] = p * dp[r];
            }
          }
        }
      };
      if (need_mask)
        grad(std::true_type());
      else
        grad(std::false_type());
      // dQ^T += K^T dS^T, two 16-key MFMA steps.
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4 sb;
#pragma unroll
        for (int e = 0; e < 4; ++e) sb[e] = E::pack2(s[8 * c + 2 * e], s[8 * c + 2 * e + 1]);
        const int tbase = (kb2 * 2 + c) * 16 * D * 2;
        auto kt = [&](int db) {
          const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(kb, tbase + toff[0][db]));
          const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr16(kb, tbase + toff[1][db]));
          return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        if constexpr (D > 128) {
          u32x4 ktf[2];
          ktf[0] = kt(0);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            if (db + 1 < NDB) ktf[(db + 1) & 1] = kt(db + 1);
            acc[db] = E::mfma(ktf[db & 1], sb, acc[db]);
          }
        } else {
#pragma unroll
          for (int db = 0; db < NDB; ++db) acc[db] = E::mfma(kt(db), sb, acc[db]);
        }
      }
    }
  };
  // Buffers are counted from t0: tile t lives in buffer (t - t0) & 1.
  for (int t = t0; t < ntiles; t += 2) {
    tile_step(t, std::integral_constant<int, 0>());
    if (t + 1 < ntiles) tile_step(t + 1, std::integral_constant<int, 1>());
  }

  if (qi < N) {
    const size_t orow = head + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dcol = 32 * db + 8 * g4 + 4 * hh;
        const float v0 = acc[db][4 * g4 + 0] * a.scale;
        const float v1 = acc[db][4 * g4 + 1] * a.scale;
        const float v2 = acc[db][4 * g4 + 2] * a.scale;
        const float v3 = acc[db][4 * g4 + 3] * a.scale;
        if (OUT_F32) {
          *(f32x4*)((float*)a.dq + orow + dcol) = f32x4{v0, v1, v2, v3};
        } else {
          *(u32x2*)((uint16_t*)a.dq + orow + dcol) = u32x2{E::pack2(v0, v1), E::pack2(v2, v3)};
        }
      }
  }
}

}  // namespace attn
