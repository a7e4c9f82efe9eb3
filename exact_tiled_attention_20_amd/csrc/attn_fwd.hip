// Fused tiled attention forward for gfx950.
//
// Method: "Why FlashAttention Is a Kernel Story", section "Tiling: fitting the
// work inside SRAM" -- keep a block of query rows on chip, stream blocks of K
// and V, update a running row maximum m and denominator l per block (online
// softmax), rescale and accumulate O, and finish with O / l. Only O and the
// row log-sum-exp are written (one natural-log statistic per row instead of
// the page's separate l and m). Mask and dropout are fused into the same pass
// (anthology-of-the-sota SOTA-114, "The general form of the practice above
// it"); the sequence-dimension split of work across workgroups follows the
// same page's note on FlashAttention-2 ("Why this only works as a fused
// kernel").
//
// Mapping to CDNA4:
//   * One workgroup = 4 waves = 128 query rows of one (b, h); each wave owns 32
//     query rows. Q stays in VGPRs as MFMA B operands for the whole pass.
//   * K and V tiles of 64 keys are copied HBM -> LDS directly
//     (global_load_lds_dwordx4), double-buffered, one barrier per tile, in a
//     chunk-swizzled row-major layout. K is read by rows; V is read with
//     ds_read_b64_tr_b16, so no transpose is stored.
//   * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16): each
//     lane then owns one query row, so the running max, the denominator and the
//     O rescale factor are per-lane scalars; the row maximum needs a single
//     exchange between the two 32-lane halves.
//   * O^T = V^T P^T: the fp32 score registers, rounded to the input dtype, are
//     already the MFMA B operand (the key order inside a 16-key step is
//     permuted consistently on the V side by the transpose reads).
//   * Work items are dealt out so that all query blocks of one head run on the
//     same XCD (workgroup ids are dispatched round-robin over the 8 XCDs), which
//     keeps that head's K/V re-reads in one L2; under a causal mask the
//     heaviest (last) query blocks of all of an XCD's heads start first.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {

template <typename E, int D, bool CAUSAL, bool DROPOUT, bool OUT_F32>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const FwdArgs a) {
  constexpr int BR = kFwdBlockQ;
  constexpr int BC = kFwdBlockK;
  constexpr int KK = D / 16;            // MFMA k-steps over the head dimension
  constexpr int NDB = D / 32;           // 32-row blocks of O^T
  constexpr int NKB = BC / 32;          // 32-key blocks of S^T per tile
  constexpr int NC16 = BC / 16;         // 16-key MFMA steps of the PV product
  constexpr int TILE_BYTES = BC * D * 2;

  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE_BYTES];

  const WorkItem wi = decode_work_item(blockIdx.x, a.B * a.H, a.nqb);
  if (!wi.valid) return;
  const int bh = wi.bh;
  const int qb = CAUSAL ? a.nqb - 1 - wi.rank : wi.rank;  // heaviest first
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int N = a.N;
  const int q0 = qb * BR;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Q = a.q + head;
  const uint16_t* __restrict__ K = a.k + head;
  const uint16_t* __restrict__ V = a.v + head;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  int kv_end = N;
  if (a.kv_len != nullptr) kv_end = min(max(a.kv_len[b], 0), N);
  int kend = kv_end;
  if (CAUSAL) kend = min(kend, q0 + BR);
  const int ntiles = (kend + BC - 1) / BC;

  const int wq0 = q0 + w * 32;          // first query row of this wave
  const int qi = wq0 + l32;             // this lane's query row
  const bool wave_has_rows = wq0 < N;

  // Q fragments: lane holds Q[qi][16*kk + 8*hh .. +8] for every k-step.
  u32x4 qf[KK];
  {
    const int qrow = min(qi, N - 1);
    const uint16_t* src = Q + (size_t)qrow * D + hh * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const u32x4*)(src + kk * 16);
  }

  char* const kb0 = smem;
  char* const vb0 = smem + 2 * TILE_BYTES;

  // K/V tiles are copied HBM -> LDS directly, in the swizzled layout.
  TilePairLoader<D, BC, 4> loader;
  loader.init(w, lane);
  // The copies are issued untracked: the compiler would otherwise make the
  // first LDS read after them wait for their completion, which would serialise
  // the prefetch of tile t+1 with the PV product of tile t. The wait at the
  // top of each iteration orders them before every read of their buffer.
  auto issue_tile = [&](int t, int buf) {
    loader.issue_one_untracked(K, t * BC, kv_end, kb0 + buf * TILE_BYTES);
    loader.issue_one_untracked(V, t * BC, kv_end, vb0 + buf * TILE_BYTES);
  };

  // Loop-invariant LDS offsets. The swizzle depends only on the low four row
  // bits, so moving by 32 K rows or 16 V rows is a plain byte offset.
  int koff[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) koff[kk] = lds_off<D>(l32, (kk * 2 + hh) * 16);
  const int g = lane >> 4;
  const int i16 = lane & 15;
  int voff[2][NDB];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      voff[half][db] = lds_off<D>(4 * hh + (i16 >> 2) + 8 * half,
                                  (32 * db + 16 * (g & 1) + 4 * (i16 & 3)) * 2);

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  // m_ref: reference maximum (raw q.k units) that the exponentials are taken
  // against. It is raised only when a tile's row maximum exceeds it by more
  // than 2^8 in probability, so the O rescale runs rarely; O and l always
  // share the same reference, which keeps O / l exact.
  float m_ref = -INFINITY;
  // This half-lane's share of the running denominator, twice: l sums the fp32
  // probabilities (it defines lse); lr sums the same probabilities rounded to
  // the MFMA operand type (it normalises O, so a row dominated by one key
  // reproduces that key's value row without a normalisation gap).
  float l = 0.f;
  float lr = 0.f;
  const float c2 = a.scale_log2;
  const float thr = a.rescale_thr;

  if (ntiles > 0) issue_tile(0, 0);

  // The loop body is instantiated once per buffer (the loop is unrolled by
  // two), so every LDS address is a per-lane offset plus a constant that the
  // read instructions carry as their immediate offset.
  auto tile_step = [&](int t, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    // Tile t has landed in LDS once every wave's copies are complete.
    wait_all_memory();
    __syncthreads();
    const bool more = (t + 1) < ntiles;
    // Buffer buf^1 was last read in iteration t-1, which every wave has left.
    if (more) issue_tile(t + 1, buf ^ 1);
    const int k0 = t * BC;
    const bool active = wave_has_rows && (!CAUSAL || k0 <= wq0 + 31);
    if (active) {
      const char* kb = kb0 + buf * TILE_BYTES;
      const char* vb = vb0 + buf * TILE_BYTES;
      // S^T = K Q^T, 32 keys x 32 queries per block.
      // The NKB accumulator chains are interleaved step by step: a single
      // chain of dependent MFMAs cannot issue at the full rate.
      f32x16 s[NKB];
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb2][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2)
          s[kb2] = E::mfma(*(const u32x4*)(kb + kb2 * 32 * D * 2 + koff[kk]), qf[kk], s[kb2]);
      // Mask: causal diagonal tiles, the ragged tail and key padding.
      const bool need_mask = (CAUSAL && (k0 + BC - 1 > wq0)) || (k0 + BC > kv_end);
      if (need_mask) {
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = k0 + kb2 * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool dead = (CAUSAL && j > qi) || (j >= kv_end);
            if (dead) s[kb2][r] = -INFINITY;
          }
      }
      // Online softmax (log2 domain for v_exp_f32).
      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb2][r]);
      mx = halves_max(mx);
      const bool raise = mx > m_ref + thr;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float alpha = raise ? __builtin_amdgcn_exp2f((m_ref - mx) * c2) : 1.f;
        if (raise) m_ref = mx;
        l *= alpha;
        lr *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      }
      const float mb = (m_ref == -INFINITY) ? 0.f : m_ref * c2;
      float rs = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb2][r], c2, -mb));
          rs += p;
          s[kb2][r] = p;
        }
      l += rs;
      // P^T as MFMA B operands: 16 keys per step, 8 per lane.
      u32x4 pf[NC16];
      float rr_sum = 0.f;
#pragma unroll
      for (int c = 0; c < NC16; ++c) {
        const int kb2 = c >> 1;
        const int rr = (c & 1) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pf[c][e] = E::pack2(s[kb2][rr + 2 * e], s[kb2][rr + 2 * e + 1]);
          rr_sum = E::add_pair(pf[c][e], rr_sum);
        }
      }
      lr += rr_sum;
      if (DROPOUT) {
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int j0 = k0 + kb2 * 32 + 8 * g4 + 4 * hh;
            const u32x4 u = dropout_draws((uint32_t)j0 >> 2, (uint32_t)qi, (uint32_t)h,
                                          (uint32_t)b, a.seed_lo, a.seed_hi);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (u[e] < a.drop_threshold) s[kb2][4 * g4 + e] = 0.f;
          }
#pragma unroll
        for (int c = 0; c < NC16; ++c) {
          const int kb2 = c >> 1;
          const int rr = (c & 1) * 8;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pf[c][e] = E::pack2(s[kb2][rr + 2 * e], s[kb2][rr + 2 * e + 1]);
        }
      }
      // O^T += V^T P^T. Lane (group g = lane/16, i = lane%16) addresses row
      // 16c + 4hh + i/4 (+8) and columns 32db + 16(g&1) + 4(i&3) .. +4.
#pragma unroll
      for (int c = 0; c < NC16; ++c) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x2 lo = __builtin_bit_cast(
              u32x2, lds_read_tr16(vb, c * 16 * D * 2 + voff[0][db]));
          const u32x2 hi = __builtin_bit_cast(
              u32x2, lds_read_tr16(vb, c * 16 * D * 2 + voff[1][db]));
          acc[db] = E::mfma(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[c], acc[db]);
        }
      }
    }
  };
  for (int t = 0; t < ntiles; t += 2) {
    tile_step(t, std::integral_constant<int, 0>());
    if (t + 1 < ntiles) tile_step(t + 1, std::integral_constant<int, 1>());
  }

  // Epilogue: O = O_acc / lr (times 1/(1-p) under dropout), lse = m + ln l.
  const float lt = halves_sum(l);
  const float lrt = halves_sum(lr);
  if (qi < N) {
    float inv = (lrt > 0.f) ? (1.f / lrt) : 0.f;
    if (DROPOUT) inv *= a.drop_rescale;
    const size_t orow = head + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dcol = 32 * db + 8 * g4 + 4 * hh;
        const float v0 = acc[db][4 * g4 + 0] * inv;
        const float v1 = acc[db][4 * g4 + 1] * inv;
        const float v2 = acc[db][4 * g4 + 2] * inv;
        const float v3 = acc[db][4 * g4 + 3] * inv;
        if (OUT_F32) {
          float* o = (float*)a.o + orow + dcol;
          *(f32x4*)o = f32x4{v0, v1, v2, v3};
        } else {
          uint16_t* o = (uint16_t*)a.o + orow + dcol;
          *(u32x2*)o = u32x2{E::pack2(v0, v1), E::pack2(v2, v3)};
        }
      }
    if (hh == 0) {
      a.lse[(size_t)bh * N + qi] = (lt > 0.f) ? (a.scale * m_ref + logf(lt)) : -INFINITY;
    }
  }
}

template <typename E, int D, bool CAUSAL, bool DROPOUT, bool OUT_F32>
static hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  const dim3 grid(a.per_xcd * 8);
  hipLaunchKernelGGL((attn_fwd_kernel<E, D, CAUSAL, DROPOUT, OUT_F32>), grid,
                     dim3(kFwdThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t launch_d(bool causal, bool dropout, bool out_f32, const FwdArgs& a,
                           hipStream_t s) {
  if (causal) {
    if (dropout) return out_f32 ? launch_one<E, D, true, true, true>(a, s)
                                : launch_one<E, D, true, true, false>(a, s);
    return out_f32 ? launch_one<E, D, true, false, true>(a, s)
                   : launch_one<E, D, true, false, false>(a, s);
  }
  if (dropout) return out_f32 ? launch_one<E, D, false, true, true>(a, s)
                              : launch_one<E, D, false, true, false>(a, s);
  return out_f32 ? launch_one<E, D, false, false, true>(a, s)
                 : launch_one<E, D, false, false, false>(a, s);
}

hipError_t launch_fwd(int dtype, int d, bool causal, bool dropout, bool out_f32,
                      const FwdArgs& a, hipStream_t stream) {
  if (dtype == 1) {
    if (d == 128) return launch_d<Elem<bf16_t>, 128>(causal, dropout, out_f32, a, stream);
    return launch_d<Elem<bf16_t>, 64>(causal, dropout, out_f32, a, stream);
  }
  if (d == 128) return launch_d<Elem<f16_t>, 128>(causal, dropout, out_f32, a, stream);
  return launch_d<Elem<f16_t>, 64>(causal, dropout, out_f32, a, stream);
}

}  // namespace attn
