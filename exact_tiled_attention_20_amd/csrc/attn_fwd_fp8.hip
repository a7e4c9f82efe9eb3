// Fused tiled attention forward on fp8 (OCP E4M3) Q, K, V for gfx950.
//
// The method is the one of attn_fwd.hip ("Why FlashAttention Is a Kernel
// Story", section "Tiling: fitting the work inside SRAM": a block of query rows
// stays on chip, K/V tiles stream through, a running maximum and denominator
// are updated per tile, O is rescaled and accumulated, only O and the
// log-sum-exp are written). The same page's section "When it falls down" names
// FP8 score tiles as a variant that needs care with precision; here both
// products run on the fp8 matrix cores (v_mfma_f32_32x32x64_f8f6f4, twice the
// bf16 rate) with fp32 accumulation:
//   * S^T = K Q^T from e4m3 K and Q: products of two e4m3 values are exact in
//     fp32, so the scores carry no fp8 error.
//   * P is rounded to e4m3 before O^T += V^T P^T. It is rounded relative to the
//     running reference maximum (at most 2^8, so it never overflows e4m3), and
//     O is normalised by the fp32 sum of the unrounded probabilities, which
//     also defines the log-sum-exp.
//
// Mapping (head dimension 128):
//   * One workgroup = 4 waves x 32 query rows; two waves per SIMD. Q stays in
//     VGPRs: for k-step ks (64 bytes of d) lane l holds bytes 32hh .. 32hh+31
//     of that step of query row l%32 (hh = l/32), the MFMA B operand.
//   * K and V tiles of 64 keys x 128 bytes are copied HBM -> LDS directly,
//     double-buffered, K one tile ahead of V. A row's 16-byte chunk c is stored
//     at chunk position c ^ s(row), s = bits 1..3 of the row with the lower two
//     exchanged: the K row reads (16 rows of 128 bytes per 256-byte bank sweep,
//     one chunk each) and the transposed V reads (32 lanes of 8 bytes per sweep,
//     8 keys, chunks 2db and 2db + 1) both touch every bank once. With s = bits
//     1..3 unpermuted, the two 16-lane halves of a V read met in the same banks.
//   * The MFMA pairs byte t of lane l in A with byte t of lane l in B (rows and
//     columns l%32); any assignment of the 64 k indices to (hh, t) works if A
//     and B share it. The S^T accumulator holds, in lane l (query l%32) and
//     register r of key block kb, key 32kb + 8(r/4) + 4hh + r%4; rounded to
//     e4m3 in that order (byte t = 16kb + r) the 32 probabilities of a lane
//     are exactly its B operand of one 64-key PV step, with key(t, hh) =
//     32(t/16) + 8((t%16)/4) + 4hh + t%4. The V^T operand (lane = d column)
//     must then hold V[key(t, hh)][d] in byte t: four ds_read_b64_tr_b8 reads
//     (8 keys each) gather it. Within a 16-lane group, lane i of such a read
//     receives byte i%8 of the 8-byte chunks addressed by lanes i/8, i/8 + 2,
//     .., i/8 + 14, in that order, so addressing lane L points at key
//     key(8m + L/2, hh) and columns 32db + 16G + 8(L%2) .. +8 (G = which 16
//     lanes of the 32, m = which read).
//   * Masks, dropout (Philox4x32-10, one call per query row and 4 keys), the
//     XCD-local work order and the lazy reference follow attn_fwd.hip.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kF8D = 128;           // head dimension
constexpr int kF8Row = kF8D;        // bytes per K/V row
constexpr int kF8BC = 64;           // keys per tile
constexpr int kF8Tile = kF8BC * kF8Row;  // 8 KiB

// Chunk position of 16-byte chunk c of tile row `row` (an involution in c).
__device__ __forceinline__ int f8_chunk(int row, int c) {
  const int j = (row >> 1) & 7;
  return c ^ ((j & 4) | ((j & 1) << 1) | ((j >> 1) & 1));
}

// C = A B + C on e4m3 operands (format code 0 for both; no block scaling).
__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Four floats rounded to e4m3 (nearest, ties to even), packed low byte first.
__device__ __forceinline__ int pack4_e4m3(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}

// Copies of 64-row x 128-byte tiles, 4 waves sharing the work: a 1 KiB slice
// is 8 rows; wave w fills slices 2w and 2w+1 of a tile, lane l the chunk
// position l%8 of row l/8 of its slice. Rows at or past `valid` repeat row
// valid-1 (finite data that the mask removes).
struct F8TileLoader {
  uint32_t goff[2];
  int grow[2];
  int wave;
  __device__ __forceinline__ void init(int w, int lane) {
    wave = w;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      grow[u] = (2 * w + u) * 8 + lane / 8;
      const int pos = lane % 8;
      // Chunk position pos of row grow holds source chunk pos ^ swizzle.
      goff[u] = (uint32_t)(grow[u] * kF8Row + (f8_chunk(grow[u], pos) << 4));
    }
  }
  __device__ __forceinline__ void issue(const uint8_t* A, int row0, int valid, char* lds) const {
    const char* at = (const char*)A + (size_t)row0 * kF8Row;
    const bool partial = row0 + kF8BC > valid;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t off = goff[u];
      if (partial && row0 + grow[u] >= valid)
        off += (uint32_t)((valid - 1 - row0 - grow[u]) * kF8Row);
      load_lds16_untracked(at, off, lds + (wave * 2 + u) * 1024);
    }
  }
};

}  // namespace

template <int MASK, bool DROPOUT, bool OUT_F32>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_fp8_kernel(const FwdArgs a) {
  constexpr int D = kF8D;
  constexpr int BR = kFwdBlockQ;
  constexpr int BC = kF8BC;
  constexpr int NKS = D / 64;          // MFMA k-steps of S (64 bytes of d each)
  constexpr int NDB = D / 32;          // 32-row blocks of O^T
  constexpr int NKB = BC / 32;         // 32-key blocks of S^T per tile
  constexpr int TILE = kF8Tile;
  constexpr bool BAND = MASK != kMaskNone;
  constexpr bool LO = MASK == kMaskBand;

  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];
  char* const kb0 = smem;
  char* const vb0 = smem + 2 * TILE;

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
  const uint8_t* __restrict__ Q = (const uint8_t*)a.q + head;
  const uint8_t* __restrict__ K = (const uint8_t*)a.k + khead;
  const uint8_t* __restrict__ V = (const uint8_t*)a.v + khead;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  int kv_end = a.Nk;
  if (a.kv_len != nullptr) kv_end = min(max(a.kv_len[b], 0), a.Nk);
  const int band_lo = LO ? a.band_lo : -kBandInf;
  const int band_hi = MASK == kMaskCausal ? 0 : a.band_hi;
  int kend = kv_end;
  int t0 = 0;
  if (BAND) {
    kend = min(kend, max(0, min(q0 + BR, N) + band_hi));
    if (LO) t0 = max(0, q0 + band_lo) / BC;
  }
  const int ntiles = (kend + BC - 1) / BC;

  const int wq0 = q0 + w * 32;
  const int qi = wq0 + l32;
  const bool wave_has_rows = wq0 < N;

  // Q: B operand of step ks, bytes 64ks + 32hh .. +32 of row qi.
  i32x8 qf[NKS];
  {
    const uint8_t* src = Q + (size_t)min(qi, N - 1) * D + hh * 32;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const u32x4 lo = *(const u32x4*)(src + ks * 64);
      const u32x4 hi = *(const u32x4*)(src + ks * 64 + 16);
      qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }

  F8TileLoader loader;
  loader.init(w, lane);

  // K row reads: key 32kb + l32, chunks 4ks + 2hh and 4ks + 2hh + 1. The
  // swizzle depends on row bits 1..3 only, so the second key block is a
  // constant 32 rows away.
  int koff[NKS][2];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      koff[ks][e] = l32 * kF8Row + (f8_chunk(l32, 4 * ks + 2 * hh + e) << 4);
  // V transposed reads: read m, addressing lane L = lane % 16 of group G.
  int voff[4][NDB];
  {
    const int L = lane & 15;
    const int G = (lane >> 4) & 1;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int key = 16 * m + 8 * (L >> 3) + 4 * hh + ((L >> 1) & 3);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        voff[m][db] = key * kF8Row + (f8_chunk(key, 2 * db + G) << 4) + 8 * (L & 1);
    }
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m_ref = -INFINITY;   // reference maximum (raw q.k units)
  float l = 0.f;             // this half-lane's share of the fp32 denominator
  const float c2 = a.scale_log2;
  const float thr = a.rescale_thr;

  int ntiles_w = wave_has_rows ? ntiles : 0;
  if (BAND) {
    const int last_key = wq0 + 31 + band_hi;
    ntiles_w = last_key < 0 ? 0 : min(ntiles_w, last_key / BC + 1);
  }

  auto scores = [&](const char* kb, f32x16 (&s)[NKB]) {
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb2][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) {
        const char* row = kb + kb2 * 32 * kF8Row;
        const u32x4 lo = *(const u32x4*)(row + koff[ks][0]);
        const u32x4 hi = *(const u32x4*)(row + koff[ks][1]);
        const i32x8 kf = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        s[kb2] = mfma_f8(kf, qf[ks], s[kb2]);
      }
  };
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
  auto rescale = [&](float mx) {
    const bool raise = mx > m_ref + thr;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float alpha = raise ? __builtin_amdgcn_exp2f((m_ref - mx) * c2) : 1.f;
      if (raise) m_ref = mx;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }
  };

  f32x16 ss[2][NKB];
  if (ntiles > t0) {
    loader.issue(K, t0 * BC, kv_end, kb0);
    loader.issue(V, t0 * BC, kv_end, vb0);
    wait_all_memory();
    __syncthreads();
    if (t0 + 1 < ntiles) loader.issue(K, (t0 + 1) * BC, kv_end, kb0 + TILE);
    if (ntiles_w > t0) {
      scores(kb0, ss[0]);
      if (need_mask(t0 * BC)) mask(ss[0], t0 * BC);
      rescale(row_max(ss[0]));
    }
  }

  // Iteration t: P(t) = exp(S(t) - m) rounded to e4m3, times V(t); beside it
  // the scores of tile t+1 from K(t+1), and their maximum. K(t) and V(t) live
  // in buffer (t - t0) & 1 of their region; K runs one tile ahead of V. After
  // a wave's last tile the next scores come from a stale buffer and are
  // discarded.
  auto body = [&](int t, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    f32x16 (&sc)[NKB] = ss[buf];
    f32x16 (&sn)[NKB] = ss[buf ^ 1];
    const int k0 = t * BC;
    const char* kbn = kb0 + (buf ^ 1) * TILE;
    const char* vb = vb0 + buf * TILE;
    scores(kbn, sn);
    const float mb = (m_ref == -INFINITY) ? 0.f : m_ref * c2;
    float rs = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb2][r], c2, -mb));
        rs += p;
        sc[kb2][r] = p;
      }
    l += rs;
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
    }
    // B operand of the PV step: byte t = 16 kb2 + r.
    i32x8 pb;
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) {
      const int kb2 = wd >> 2;
      const int r0 = 4 * (wd & 3);
      pb[wd] = pack4_e4m3(sc[kb2][r0], sc[kb2][r0 + 1], sc[kb2][r0 + 2], sc[kb2][r0 + 3]);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      i32x8 vf;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vb + voff[m][db]));
        vf[2 * m] = x[0];
        vf[2 * m + 1] = x[1];
      }
      acc[db] = mfma_f8(vf, pb, acc[db]);
    }
    float mx = row_max(sn);
    if (need_mask(k0 + BC)) {
      mask(sn, k0 + BC);
      mx = row_max(sn);
    }
    if (t + 1 < ntiles_w) rescale(mx);
  };
  auto tile_step = [&](int t, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    wait_all_memory();
    __syncthreads();
    if (t + 2 < ntiles) loader.issue(K, (t + 2) * BC, kv_end, kb0 + buf * TILE);
    if (t + 1 < ntiles) loader.issue(V, (t + 1) * BC, kv_end, vb0 + (buf ^ 1) * TILE);
    if (t < ntiles_w) body(t, buf_c);
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  for (int t = t0; t < ntiles; t += 2) {
    tile_step(t, C0());
    if (t + 1 < ntiles) tile_step(t + 1, C1());
  }

  // O = O_acc / l (times 1/(1-p) under dropout), lse = m + ln l.
  const float lt = halves_sum(l);
  if (qi < N) {
    float inv = (lt > 0.f) ? (1.f / lt) : 0.f;
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
          *(f32x4*)((float*)a.o + orow + dcol) = f32x4{v0, v1, v2, v3};
        } else {
          *(u32x2*)((uint16_t*)a.o + orow + dcol) =
              u32x2{Elem<bf16_t>::pack2(v0, v1), Elem<bf16_t>::pack2(v2, v3)};
        }
      }
    if (hh == 0)
      a.lse[(size_t)bh * N + qi] = (lt > 0.f) ? (a.scale * m_ref + logf(lt)) : -INFINITY;
  }
}

template <int MASK, bool DROPOUT, bool OUT_F32>
static hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<MASK, DROPOUT, OUT_F32>), dim3(a.per_xcd * 8),
                     dim3(kFwdThreads), 0, stream, a);
  return hipGetLastError();
}

template <int MASK>
static hipError_t launch_m(bool dropout, bool out_f32, const FwdArgs& a, hipStream_t s) {
  if (dropout) return out_f32 ? launch_one<MASK, true, true>(a, s)
                              : launch_one<MASK, true, false>(a, s);
  return out_f32 ? launch_one<MASK, false, true>(a, s) : launch_one<MASK, false, false>(a, s);
}

hipError_t launch_fwd_fp8(int mask, bool dropout, bool out_f32, const FwdArgs& a,
                          hipStream_t stream) {
  if (mask == kMaskCausal) return launch_m<kMaskCausal>(dropout, out_f32, a, stream);
  if (mask == kMaskBand) return launch_m<kMaskBand>(dropout, out_f32, a, stream);
  return launch_m<kMaskNone>(dropout, out_f32, a, stream);
}

}  // namespace attn
