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
// note on FlashAttention-2 in "Why FlashAttention Is a Kernel Story", section
// "Why this only works as a fused kernel".
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
//   * Banded masks -- causal, sliding window, and the bottom-right alignment of
//     a non-square Q x K grid (the variants named in the page's section "When
//     it falls down") -- arrive as one key band [i + band_lo, i + band_hi] per
//     query row i. A workgroup visits only the K/V tiles that meet the band of
//     one of its rows; tiles that cross a band edge are masked element-wise.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {

// Waves per SIMD the register budget is set for: one at d = 256; three at
// d = 64 without dropout or a two-sided band (those instances fit in 168
// registers, and the small grids of d = 64 layers then stay resident in one
// round of three 32 KiB-LDS workgroups per CU); two otherwise.
template <int D, int MASK, bool DROPOUT>
constexpr int fwd_waves_per_simd() {
  return D > 128 ? 1 : (D < 128 && !DROPOUT && MASK != kMaskBand) ? 3 : 2;
}

template <typename E, int D, int MASK, bool DROPOUT, bool OUT_F32>
__global__ __launch_bounds__(kFwdThreads)
__attribute__((amdgpu_waves_per_eu(fwd_waves_per_simd<D, MASK, DROPOUT>(),
                                   fwd_waves_per_simd<D, MASK, DROPOUT>())))
void attn_fwd_kernel(const FwdArgs a) {
  constexpr int BR = kFwdBlockQ;
  constexpr int BC = kFwdBlockK;
  constexpr int KK = D / 16;            // MFMA k-steps over the head dimension
  constexpr int NDB = D / 32;           // 32-row blocks of O^T
  constexpr int NKB = BC / 32;          // 32-key blocks of S^T per tile
  constexpr int NC16 = BC / 16;         // 16-key MFMA steps of the PV product
  constexpr int TILE_BYTES = BC * D * 2;
  constexpr bool BAND = MASK != kMaskNone;
  constexpr bool LO = MASK == kMaskBand;   // a lower band edge exists

  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE_BYTES];

  const WorkItem wi = decode_work_item(blockIdx.x, a.B * a.H, a.nqb);
  if (!wi.valid) return;
  const int bh = wi.bh;
  const int qb = BAND ? a.nqb - 1 - wi.rank : wi.rank;  // heaviest first
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int N = a.N;
  const int q0 = qb * BR;
  const size_t head = (size_t)bh * (size_t)N * D;
  const size_t khead = (size_t)bh * (size_t)a.Nk * D;
  const uint16_t* __restrict__ Q = a.q + head;
  const uint16_t* __restrict__ K = a.k + khead;
  const uint16_t* __restrict__ V = a.v + khead;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  int kv_end = a.Nk;
  if (a.kv_len != nullptr) kv_end = min(max(a.kv_len[b], 0), a.Nk);
  const int band_lo = LO ? a.band_lo : -kBandInf;
  const int band_hi = MASK == kMaskCausal ? 0 : a.band_hi;
  // Tiles [t0, ntiles) hold every key visible to a row of this block: from the
  // first row's lower band edge to the last row's upper band edge.
  int kend = kv_end;
  int t0 = 0;
  if (BAND) {
    kend = min(kend, max(0, min(q0 + BR, N) + band_hi));
    if (LO) t0 = max(0, q0 + band_lo) / BC;
  }
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

  // K/V tiles are copied HBM -> LDS directly, in the swizzled layout. The
  // copies are issued untracked: the compiler would otherwise make the first
  // LDS read after them wait for their completion, which would serialise the
  // prefetch with the products of the current tile. The wait at the top of
  // each iteration orders them before every read of their buffer.
  TilePairLoader<D, BC, 4> loader;
  loader.init(w, lane);

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
  // than the operand type's range allows (2^64 in probability for bf16, 2^15
  // for fp16), so the O rescale runs rarely even when the scores spread widely;
  // O and l always share the same reference, which keeps O / l exact.
  float m_ref = -INFINITY;
  // This half-lane's share of the running denominator, twice: l sums the fp32
  // probabilities (it defines lse); lr sums the same probabilities rounded to
  // the MFMA operand type (it normalises O, so a row dominated by one key
  // reproduces that key's value row without a normalisation gap).
  float l = 0.f;
  float lr = 0.f;
  const float c2 = a.scale_log2;
  const float thr = a.rescale_thr;

  // Tiles this wave computes: under a band a wave stops after the tile that
  // holds its last row's upper band edge (it keeps meeting the barriers).
  // Every wave starts at the block's first tile; keys below a wave's own
  // lower band edge are masked.
  int ntiles_w = wave_has_rows ? ntiles : 0;
  if (BAND) {
    const int last_key = wq0 + 31 + band_hi;
    ntiles_w = last_key < 0 ? 0 : min(ntiles_w, last_key / BC + 1);
  }

  // Scores of one tile: S^T = K Q^T, 32 keys x 32 queries per block. The
  // NKB accumulator chains are interleaved step by step: a single chain of
  // dependent MFMAs cannot issue at the full rate. The K fragments of step
  // kk + 1 are read from LDS before the MFMAs of step kk, in program order
  // ahead of before_step (which may issue tile copies: the copies are inline
  // assembly that no memory access moves across), so the MFMAs do not wait
  // for their operands' LDS latency. after_step runs VALU work of the
  // caller's between the steps' MFMAs.
  auto scores = [&](const char* kb, f32x16 (&s)[NKB], auto&& before_step,
                    auto&& after_step) {
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb2][r] = 0.f;
    if constexpr (DROPOUT) {
      // The dropout instances keep the operand reads beside their MFMAs:
      // the Philox state leaves no registers for a second fragment set.
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        before_step(kk);
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2)
          s[kb2] = E::mfma(*(const u32x4*)(kb + kb2 * 32 * D * 2 + koff[kk]), qf[kk], s[kb2]);
        after_step(kk);
      }
    } else {
      u32x4 kf[2][NKB];
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2)
        kf[0][kb2] = *(const u32x4*)(kb + kb2 * 32 * D * 2 + koff[0]);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) {
#pragma unroll
          for (int kb2 = 0; kb2 < NKB; ++kb2)
            kf[(kk + 1) & 1][kb2] = *(const u32x4*)(kb + kb2 * 32 * D * 2 + koff[kk + 1]);
        }
        before_step(kk);
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2) s[kb2] = E::mfma(kf[kk & 1][kb2], qf[kk], s[kb2]);
        after_step(kk);
      }
    }
  };
  auto no_hook = [](int) {};
  // Mask (band edges, the ragged tail, key padding) of the tile starting at
  // key k0, and the row maximum of a tile.
  auto mask = [&](f32x16 (&s)[NKB], int k0) {
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = k0 + kb2 * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        const bool dead =
            (BAND && (j > qi + band_hi || (LO && j < qi + band_lo))) || (j >= kv_end);
        if (dead) s[kb2][r] = -INFINITY;
      }
  };
  auto row_max = [&](const f32x16 (&s)[NKB]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb2][r]);
    return halves_max(mx);
  };
  auto need_mask = [&](int k0) {
    return (BAND && (k0 + BC - 1 > wq0 + band_hi || (LO && k0 < wq0 + 31 + band_lo))) ||
           (k0 + BC > kv_end);
  };
  // Online softmax, lazy form: the reference is raised only when the tile's
  // row maximum exceeds it by more than the threshold.
  auto rescale = [&](float mx) {
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
  };

  // Scores of tile t (raw q.k) live in ss[(t - t0) & 1]: iteration t reads
  // one set and fills the other, so no copy is needed between iterations.
  // Buffers are counted from the block's first tile t0 the same way.
  f32x16 ss[2][NKB];
  if (ntiles > t0) {
    loader.issue_one_untracked(K, t0 * BC, kv_end, kb0);
    loader.issue_one_untracked(V, t0 * BC, kv_end, vb0);
    wait_all_memory();
    __syncthreads();
    if (t0 + 1 < ntiles) loader.issue_one_untracked(K, (t0 + 1) * BC, kv_end, kb0 + TILE_BYTES);
    if (ntiles_w > t0) {
      scores(kb0, ss[0], no_hook, no_hook);
      if (need_mask(t0 * BC)) mask(ss[0], t0 * BC);
      rescale(row_max(ss[0]));
    }
  }

  // Iteration t: P(t) = exp(S(t) - m) times V(t). The MFMAs of
  // S(t+1) = K(t+1) Q^T run beside the exponentials of tile t, and the row
  // maximum of tile t+1 (with the reference update it triggers) beside the PV
  // MFMAs. K(t) and V(t) live in buffer (t - t0) & 1 of their region; K runs
  // one tile ahead of V. After a wave's last tile the scores of the next one are formed
  // from whatever that buffer holds and discarded, which keeps the body one
  // straight-line block.
  // With SPREAD the copies of K(t+2) and V(t+1) (both full tiles) are issued
  // one slice per k-step of the S(t+1) product instead of all at once: a burst
  // of tile copies from every wave of the CU stalls each wave at the issue.
  constexpr int SPW = TilePairLoader<D, BC, 4>::SPW;
  auto body = [&](int t, auto buf_c, auto spread_c) {
    constexpr int buf = decltype(buf_c)::value;
    constexpr bool SPREAD = decltype(spread_c)::value;
    f32x16 (&sc)[NKB] = ss[buf];
    f32x16 (&sn)[NKB] = ss[buf ^ 1];
    const int k0 = t * BC;
    const char* kbn = kb0 + (buf ^ 1) * TILE_BYTES;
    const char* vb = vb0 + buf * TILE_BYTES;
    // Probabilities of tile t (log2 domain for v_exp_f32), in key order, PER
    // per group; each adjacent pair is rounded into the MFMA B operand of the
    // PV product as soon as it exists. l sums the fp32 probabilities, lr the
    // rounded ones. (Placing the groups between the k-steps of S(t+1) was
    // measured slower than running them after the S(t+1) MFMAs.)
    const float mb = (m_ref == -INFINITY) ? 0.f : m_ref * c2;
    float rs = 0.f;
    float rr_sum = 0.f;
    u32x4 pf[NC16];
    constexpr int PER = NKB * 16 / KK;
    auto exps = [&](int kk) {
#pragma unroll
      for (int u = 0; u < PER; u += 2) {
        const int e = kk * PER + u;
        const int kb2 = e >> 4;
        const int r = e & 15;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb2][r], c2, -mb));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb2][r + 1], c2, -mb));
        rs += p0;
        rs += p1;
        sc[kb2][r] = p0;
        sc[kb2][r + 1] = p1;
        const int c = kb2 * 2 + (r >> 3);
        const int ee = (r & 7) >> 1;
        pf[c][ee] = E::pack2(p0, p1);
        rr_sum = E::add_pair(pf[c][ee], rr_sum);
      }
    };
    scores(kbn, sn, [&](int kk) {
      if constexpr (SPREAD) {
        constexpr int per = KK / (2 * SPW) > 0 ? KK / (2 * SPW) : 1;
        if (kk % per == 0 && kk / per < 2 * SPW) {
          const int i = kk / per;
          if (i < SPW)
            loader.issue_slice_full(K, (t + 2) * BC, kb0 + buf * TILE_BYTES, i);
          else
            loader.issue_slice_full(V, (t + 1) * BC, vb0 + (buf ^ 1) * TILE_BYTES, i - SPW);
        }
      }
    }, no_hook);
    if constexpr (DROPOUT) {
      // One pass of exponentials, then one of packing: the order that keeps
      // the dropout instances' registers lowest.
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb2][r], c2, -mb));
          rs += p;
          sc[kb2][r] = p;
        }
#pragma unroll
      for (int c = 0; c < NC16; ++c) {
        const int kb2 = c >> 1;
        const int rr = (c & 1) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pf[c][e] = E::pack2(sc[kb2][rr + 2 * e], sc[kb2][rr + 2 * e + 1]);
          rr_sum = E::add_pair(pf[c][e], rr_sum);
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) exps(kk);
    }
    l += rs;
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
            if (u[e] < a.drop_threshold) sc[kb2][4 * g4 + e] = 0.f;
        }
#pragma unroll
      for (int c = 0; c < NC16; ++c) {
        const int kb2 = c >> 1;
        const int rr = (c & 1) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pf[c][e] = E::pack2(sc[kb2][rr + 2 * e], sc[kb2][rr + 2 * e + 1]);
      }
    }
    // O^T += V^T P^T. Lane (group g = lane/16, i = lane%16) addresses row
    // 16c + 4hh + i/4 (+8) and columns 32db + 16(g&1) + 4(i&3) .. +4. The V
    // fragment of the next MFMA is read before the current one is issued.
    auto vfrag = [&](int i) {
      const int c = i / NDB;
      const int db = i % NDB;
      const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(vb, c * 16 * D * 2 + voff[0][db]));
      const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr16(vb, c * 16 * D * 2 + voff[1][db]));
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    if constexpr (DROPOUT) {
#pragma unroll
      for (int i = 0; i < NC16 * NDB; ++i) acc[i % NDB] = E::mfma(vfrag(i), pf[i / NDB], acc[i % NDB]);
    } else {
      u32x4 vf[2];
      vf[0] = vfrag(0);
#pragma unroll
      for (int i = 0; i < NC16 * NDB; ++i) {
        if (i + 1 < NC16 * NDB) vf[(i + 1) & 1] = vfrag(i + 1);
        acc[i % NDB] = E::mfma(vf[i & 1], pf[i / NDB], acc[i % NDB]);
      }
    }
    // Maximum of tile t+1 beside the PV MFMAs; a tile that needs a mask is
    // masked afterwards and its maximum taken again. After a wave's last tile
    // the next scores are not real.
    float mx = row_max(sn);
    if (need_mask(k0 + BC)) {
      mask(sn, k0 + BC);
      mx = row_max(sn);
    }
    if (t + 1 < ntiles_w) rescale(mx);
  };

  // The loop body is instantiated once per buffer (the loop is unrolled by
  // two), so every LDS address is a per-lane offset plus a constant that the
  // read instructions carry as their immediate offset.
  auto tile_step = [&](int t, auto buf_c, auto spread_c) {
    constexpr int buf = decltype(buf_c)::value;
    constexpr bool SPREAD = decltype(spread_c)::value;
    // K(t+1) and V(t) have landed once every wave's copies are complete.
    wait_all_memory();
    __syncthreads();
    // K(t) was last read in iteration t-1 and V(t-1) there too, which every
    // wave has left.
    if constexpr (!SPREAD) {
      if (t + 2 < ntiles)
        loader.issue_one_untracked(K, (t + 2) * BC, kv_end, kb0 + buf * TILE_BYTES);
      if (t + 1 < ntiles)
        loader.issue_one_untracked(V, (t + 1) * BC, kv_end, vb0 + (buf ^ 1) * TILE_BYTES);
    }
    if (t < ntiles_w) {
      body(t, buf_c, spread_c);
    } else if constexpr (SPREAD) {
      loader.issue_one_untracked(K, (t + 2) * BC, kv_end, kb0 + buf * TILE_BYTES);
      loader.issue_one_untracked(V, (t + 1) * BC, kv_end, vb0 + (buf ^ 1) * TILE_BYTES);
    }
  };
  // Iterations t < tsp copy two full tiles (K(t+2) and V(t+1)) and spread
  // them; the last few iterations copy the possibly partial tail at the top.
  const int tsp = max(0, min(ntiles - 2, kv_end / BC - 2));
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  int t = t0;
  for (; t + 1 < tsp; t += 2) {
    tile_step(t, C0(), std::true_type());
    tile_step(t + 1, C1(), std::true_type());
  }
  // t - t0 is even here.
  for (; t < ntiles; t += 2) {
    tile_step(t, C0(), std::false_type());
    if (t + 1 < ntiles) tile_step(t + 1, C1(), std::false_type());
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

template <typename E, int D, int MASK, bool DROPOUT, bool OUT_F32>
static hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  const dim3 grid(a.per_xcd * 8);
  hipLaunchKernelGGL((attn_fwd_kernel<E, D, MASK, DROPOUT, OUT_F32>), grid,
                     dim3(kFwdThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename E, int D, int MASK>
static hipError_t launch_m(bool dropout, bool out_f32, const FwdArgs& a, hipStream_t s) {
  if (dropout) return out_f32 ? launch_one<E, D, MASK, true, true>(a, s)
                              : launch_one<E, D, MASK, true, false>(a, s);
  return out_f32 ? launch_one<E, D, MASK, false, true>(a, s)
                 : launch_one<E, D, MASK, false, false>(a, s);
}

template <typename E, int D>
static hipError_t launch_d(int mask, bool dropout, bool out_f32, const FwdArgs& a,
                           hipStream_t s) {
  if (mask == kMaskCausal) return launch_m<E, D, kMaskCausal>(dropout, out_f32, a, s);
  if (mask == kMaskBand) return launch_m<E, D, kMaskBand>(dropout, out_f32, a, s);
  return launch_m<E, D, kMaskNone>(dropout, out_f32, a, s);
}

hipError_t launch_fwd(int dtype, int d, int mask, bool dropout, bool out_f32,
                      const FwdArgs& a, hipStream_t stream) {
  if (dtype == 1) {
    if (d == 256) return launch_d<Elem<bf16_t>, 256>(mask, dropout, out_f32, a, stream);
    if (d == 128) return launch_d<Elem<bf16_t>, 128>(mask, dropout, out_f32, a, stream);
    return launch_d<Elem<bf16_t>, 64>(mask, dropout, out_f32, a, stream);
  }
  if (d == 256) return launch_d<Elem<f16_t>, 256>(mask, dropout, out_f32, a, stream);
  if (d == 128) return launch_d<Elem<f16_t>, 128>(mask, dropout, out_f32, a, stream);
  return launch_d<Elem<f16_t>, 64>(mask, dropout, out_f32, a, stream);
}

}  // namespace attn
