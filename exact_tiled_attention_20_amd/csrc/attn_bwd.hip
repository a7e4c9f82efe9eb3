// Fused attention backward for gfx950, recomputing scores from the saved
// log-sum-exp ("Why FlashAttention Is a Kernel Story", section "When it falls
// down", backward pass: S and P are not stored by the forward and are rebuilt
// from the output and the log-sum-exp).
//
// With P_ij = exp(scale * Q_i.K_j - lse_i) on visible pairs, Z_ij the dropout
// factor (keep / (1-p), or 1), and D_i = dO_i . O_i:
//     dV_j = sum_i P_ij Z_ij dO_i
//     dP_ij = Z_ij dO_i . V_j,   dS_ij = P_ij (dP_ij - D_i)
//     dK_j = scale * sum_i dS_ij Q_i,   dQ_i = scale * sum_j dS_ij K_j
//
// Three kernels on the caller's stream:
//   1. preprocess: D_i for every row (HBM-bound, 16 lanes per row).
//   2. dK/dV: one workgroup per 256 keys at d = 128 (8 waves x 32 keys, two
//      waves per SIMD; 128 keys and 4 waves at d = 64 and d = 256). K and V
//      rows stay in LDS for the whole pass; Q and dO stream
//      through LDS in tiles of 32 queries; lse and D come from L2 into
//      registers, one tile ahead. Scores are computed as S = Q K^T so that each lane owns one
//      key and the query index runs along the accumulator registers: the fp32
//      registers of P and dS, rounded to the input dtype, are then directly the
//      A operands of dV = P^T dO and dK = dS^T Q, and dO and Q are fed as B
//      operands by ds_read_b64_tr_b16 from their row-major LDS tiles.
//   3. dQ (attn_bwd_dq.hpp; the d = 256 instances in attn_bwd_dq256.hip): one
//      workgroup per 128 queries (4 waves x 32 queries), the forward's
//      orientation (S^T = K Q^T, one query per lane) plus dP^T = V dO^T; dQ^T =
//      K^T dS^T reads K transposed from LDS. Deterministic: no atomics.
// Banded masks (causal, sliding window, non-square alignment) arrive as the key
// band [i + band_lo, i + band_hi] of query row i, as in the forward: the dK/dV
// kernel visits only the query tiles whose rows see one of its keys, the dQ
// kernel only the key tiles its rows see.
#include <type_traits>

#include "attn_bwd_dq.hpp"
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {

template <bool OUT_F32, typename E>
__device__ __forceinline__ float load_out(const void* p, size_t idx) {
  if (OUT_F32) return ((const float*)p)[idx];
  return E::to_float(((const uint16_t*)p)[idx]);
}

// ---------------------------------------------------------------------------
// D_i = sum_c dO[i][c] * O[i][c], and lse_i in log2 units (the form the
// dK/dV kernel subtracts from its exponents; +inf for a row without visible
// keys, so that its probabilities come out 0). D/8 lanes per row, 8 elements
// per lane. Both arrays have Np rows per head (N rounded up to a multiple of
// 4); the rows past N hold D = 0 and lse = +inf (finite products, zero
// probabilities), so that the dK/dV kernel reads every group of four rows as
// one aligned 16-byte load.
template <typename E, int D, bool OUT_F32>
__global__ __launch_bounds__(256) void attn_bwd_preprocess_kernel(const BwdArgs a) {
  constexpr int LPR = D / 8;  // lanes per row
  const long long rows = (long long)a.B * a.H * a.Np;
  const long long row = ((long long)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int part = threadIdx.x % LPR;
  const long long bh = row / a.Np;
  const int i = (int)(row - bh * a.Np);
  const long long src = bh * a.N + i;  // the row in (B, H, N) arrays
  const bool real = row < rows && i < a.N;
  float acc = 0.f;
  if (real) {
    const size_t base = (size_t)src * D + part * 8;
    const u32x4 g = *(const u32x4*)(a.d_o + base);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float g0 = E::to_float((uint16_t)(g[e] & 0xFFFF));
      const float g1 = E::to_float((uint16_t)(g[e] >> 16));
      acc = __builtin_fmaf(g0, load_out<OUT_F32, E>(a.o, base + 2 * e), acc);
      acc = __builtin_fmaf(g1, load_out<OUT_F32, E>(a.o, base + 2 * e + 1), acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) {
    a.delta[row] = acc;
    const float x = real ? a.lse[src] : -INFINITY;
    a.lse2[row] = (x == -INFINITY) ? INFINITY : x * kLog2e;
  }
}

// Dropout draws in the dK/dV kernel. A lane there holds one key j and 16 query
// rows; the draws of keys 4t..4t+3 for one row come from one Philox4x32-10
// call, and the four lanes of a quad hold those four keys. Each lane makes the
// calls for 4 of the 16 rows and a 4 x 4 transpose across the quad hands every
// lane its own word of all of them: one call per (row, 4-key group), as in the
// forward, instead of one per element.
//
// Lane u of each quad holds x[w] = M[u][w]; returns y with y[g] = M[g][u]. Two
// butterfly stages: exchange with lane u^1 (DPP quad_perm 1,0,3,2), then with
// lane u^2 (quad_perm 2,3,0,1). b and c are bits 0 and 1 of u.
__device__ __forceinline__ u32x4 quad_transpose4(u32x4 x, bool b, bool c) {
  const uint32_t s0 = b ? x[0] : x[1];
  const uint32_t s1 = b ? x[2] : x[3];
  const uint32_t k0 = b ? x[1] : x[0];
  const uint32_t k1 = b ? x[3] : x[2];
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s0, 0xB1, 0xF, 0xF, true);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0xB1, 0xF, 0xF, true);
  // After stage 1 lane u holds M[g][w] for g in {u, u^1} and w in {b, b + 2}:
  // y<g&1><w>>1> = (g&1 == b) ? kept : received. Stage 2 keeps w>>1 == c.
  const uint32_t y00 = b ? r0 : k0, y01 = b ? r1 : k1;
  const uint32_t y10 = b ? k0 : r0, y11 = b ? k1 : r1;
  const uint32_t send0 = c ? y00 : y01, send1 = c ? y10 : y11;
  const uint32_t keep0 = c ? y01 : y00, keep1 = c ? y11 : y10;
  const uint32_t recv0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)send0, 0x4E, 0xF, 0xF, true);
  const uint32_t recv1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)send1, 0x4E, 0xF, 0xF, true);
  u32x4 y;
  y[0] = c ? recv0 : keep0;
  y[1] = c ? recv1 : keep1;
  y[2] = c ? keep0 : recv0;
  y[3] = c ? keep1 : recv1;
  return y;
}

// ---------------------------------------------------------------------------
// dK, dV. Workgroup at d = 128: 8 waves x 32 keys = 256 keys of one (b, h),
// two waves per SIMD. The workgroup's K and V rows stay in LDS for the whole
// pass; Q and dO tiles of 32 query rows stream HBM -> LDS directly,
// double-buffered (for d = 128 that fills the 160 KiB of LDS exactly); lse and
// D of the tile's rows are read from L2 into registers one tile ahead (at d =
// 256, with single-buffered tiles, at the top of their own tile).
constexpr int kDkdvWaves = 8;
// d = 64: 4 waves (128 keys, 48 KiB of LDS), so two workgroups share a CU and
// the short grids of d = 64 layers (a few key blocks per head) spread over
// twice as many workgroups. d = 256: 4 waves (128 keys, 128 KiB of K/V rows)
// at one wave per SIMD, and a single Q tile and dO tile of 16 KiB each:
// 160 KiB of LDS in all.
template <int D>
constexpr int dkdv_waves() { return D == 128 ? kDkdvWaves : 4; }

template <typename E, int D, int MASK, bool DROPOUT, bool OUT_F32>
__global__ __launch_bounds__(64 * dkdv_waves<D>())
__attribute__((amdgpu_waves_per_eu(D > 128 ? 1 : 2, D > 128 ? 1 : 2)))
void attn_bwd_dkdv_kernel(const BwdArgs a) {
  constexpr int NW = dkdv_waves<D>();
  constexpr bool DBUF = D <= 128;      // double-buffered Q / dO tiles
  constexpr int BKW = 32 * NW;         // keys per workgroup
  constexpr int BQ = 32;               // query rows per tile
  constexpr int KK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE_BYTES = BQ * D * 2;
  constexpr int KV_BYTES = BKW * D * 2;
  constexpr int QW = (TILE_BYTES / 1024 < NW) ? TILE_BYTES / 1024 : NW;  // waves that load a tile
  constexpr bool BAND = MASK != kMaskNone;
  constexpr bool LO = MASK == kMaskBand;   // a lower band edge exists

  // LDS: the Q and dO tiles first (within reach of the 16-bit immediate
  // offset of LDS reads), then one block per wave holding that wave's 32 K
  // rows followed by its 32 V rows, so both are addressed from one per-lane
  // base.
  constexpr int KV_WAVE = 32 * D * 2;            // K (or V) rows of one wave
  constexpr int NBUF = DBUF ? 2 : 1;
  __shared__ __attribute__((aligned(1024))) char smem[2 * NBUF * TILE_BYTES + 2 * KV_BYTES];
  char* const qb0 = smem;                        // [NBUF] Q tiles
  char* const ob0 = smem + NBUF * TILE_BYTES;    // [NBUF] dO tiles
  constexpr int KVB = 2 * NBUF * TILE_BYTES;     // byte offset of the per-wave K/V blocks

  const int nkb = (a.Nk + BKW - 1) / BKW;
  const WorkItem wi = decode_work_item(blockIdx.x, a.B * a.H, nkb);
  if (!wi.valid) return;
  const int bh = wi.bh;
  const int kblk = wi.rank;            // ascending: heaviest first under causal
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int N = a.N;
  const size_t head = (size_t)bh * (size_t)N * D;
  const size_t khead = (size_t)bh * (size_t)a.Nk * D;
  const uint16_t* __restrict__ Q = a.q + head;
  const uint16_t* __restrict__ K = a.k + khead;
  const uint16_t* __restrict__ V = a.v + khead;
  const uint16_t* __restrict__ dO = a.d_o + head;
  const float* __restrict__ LSE = a.lse2 + (size_t)bh * a.Np;  // lse * log2(e)
  const float* __restrict__ DEL = a.delta + (size_t)bh * a.Np;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int k0 = kblk * BKW;
  const int kw = k0 + 32 * w;
  const int j = kw + l32;              // this lane's key

  int kv_end = a.Nk;
  if (a.kv_len != nullptr) kv_end = min(max(a.kv_len[b], 0), a.Nk);
  const int band_lo = LO ? a.band_lo : -kBandInf;
  const int band_hi = MASK == kMaskCausal ? 0 : a.band_hi;

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }

  if (k0 < kv_end) {
    const bool key_tail = kw + 32 > kv_end;
    const bool wave_has_keys = kw < kv_end;
    // Query tiles [qt0, nqt) hold every row that sees one of this block's
    // keys: row i sees key j only if j - band_hi <= i <= j - band_lo.
    int qt0 = 0;
    int nqt = (N + BQ - 1) / BQ;
    if (BAND) {
      // Rounded down to an even tile (one extra, fully skipped tile at most):
      // with an even start the loop unrolled by two fits the register budget.
      qt0 = MASK == kMaskCausal ? k0 / BQ : (max(0, k0 - band_hi) / BQ) & ~1;
      if (LO) {
        const int last_row = k0 + BKW - 1 - band_lo;
        nqt = last_row < 0 ? 0 : min(nqt, last_row / BQ + 1);
      }
    }
    // No query row sees these keys (or there are no query rows): dK = dV = 0,
    // and no copy is issued that the workgroup would never wait for.
    if (qt0 >= nqt) goto write_out;
    {
      // Wave w's slices of the 256-row K/V block are exactly its own 32 keys.
      TilePairLoader<D, BKW, NW> kvload;
      static_assert(TilePairLoader<D, BKW, NW>::SPW * 1024 == KV_WAVE, "one block per wave");
      kvload.init(w, lane);
      char* const mine = smem + KVB + w * 2 * KV_WAVE;
      kvload.issue_local(K, V, k0, kv_end, mine, mine + KV_WAVE);
    }
    TilePairLoader<D, BQ, QW> loader;
    if (w < QW) loader.init(w, lane);
    auto issue_tile = [&](int t, int buf) {
      if ((DBUF && QW == NW) || w < QW)
        loader.issue(Q, dO, t * BQ, N, qb0 + buf * TILE_BYTES, ob0 + buf * TILE_BYTES);
    };

    int roff[KK];     // row-read offsets (A operands and the K/V B operands)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) roff[kk] = lds_off<D>(l32, (kk * 2 + hh) * 16);
    int kvoff[KK];    // the same reads in this wave's K block (V: + KV_WAVE)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) kvoff[kk] = KVB + w * 2 * KV_WAVE + roff[kk];
    const int g = lane >> 4;
    const int i16 = lane & 15;
    int toff[2][NDB];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        toff[half][db] = lds_off<D>(4 * hh + (i16 >> 2) + 8 * half,
                                    (32 * db + 16 * (g & 1) + 4 * (i16 & 3)) * 2);
    const float c2 = a.scale_log2;

    if (qt0 < nqt) issue_tile(qt0, 0);
    // lse (in log2 units) and D of this lane's 16 query rows of tile t, rows
    // t BQ + 8 g4 + 4 hh + e. With double-buffered tiles they are loaded one
    // tile ahead, at the end of the previous tile's work: loaded at the top of
    // their own tile, their L2 latency, and with it the wait for the copy of
    // the next Q / dO tile issued in between (vector-memory operations
    // complete in issue order), fell between the S / dP products and the
    // gradient. The workspace rows are padded to a multiple of 4 (the padding
    // holds finite values), so a group of four rows is always one aligned
    // 16-byte load, clamped into the padded range for the tail tile.
    f32x4 lsn[4], dln[4];
    auto load_rows = [&](int t) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int q4 = min(t * BQ + 8 * g4 + 4 * hh, a.Np - 4);
        lsn[g4] = *(const f32x4*)(LSE + q4);
        dln[g4] = *(const f32x4*)(DEL + q4);
      }
    };
    // The waits below count vector-memory operations: per tile a wave issues
    // exactly the two slices of the next tile's copy, then, at the end, the
    // eight row loads of the next tile.
    static_assert(!DBUF || (QW == NW && TilePairLoader<D, BQ, QW>::SPW == 1),
                  "one Q and one dO slice per wave and tile");
    if constexpr (DBUF) load_rows(qt0);
    // Unrolled by two (one instantiation per buffer), so LDS addresses carry
    // the buffer offset as an immediate.
    auto tile_step = [&](int t, auto buf_c) {
      constexpr int buf = DBUF ? decltype(buf_c)::value : 0;
      if constexpr (DBUF) {
        // Everything but this tile's eight row loads has completed (among it
        // the copy of this tile); then the copy of the next tile is issued
        // (the last tile copies itself again into the idle buffer, so that
        // every tile issues the same operations).
        wait_vm_lgkm0<8>();
        barrier_only();
        issue_tile(min(t + 1, nqt - 1), buf ^ 1);
      } else {
        wait_all_memory();
        __syncthreads();
      }
      const int qbase = t * BQ;
      const bool active = wave_has_keys &&
                          (!BAND || (qbase + 31 >= kw - band_hi &&
                                     (!LO || qbase <= kw + 31 - band_lo)));
      if (!active) {
        if constexpr (DBUF) load_rows(min(t + 1, nqt - 1));
        return;
      }
      const char* qb = qb0 + buf * TILE_BYTES;
      const char* ob = ob0 + buf * TILE_BYTES;

      f32x4 ls4[4], dl4[4];
      if constexpr (DBUF) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          ls4[g4] = lsn[g4];
          dl4[g4] = dln[g4];
        }
      } else {
        // Vector loads only where the rows are 16-byte aligned (N % 4 == 0).
        const bool vec_rows = (N & 3) == 0;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int q4 = qbase + 8 * g4 + 4 * hh;
          if (vec_rows && q4 + 3 < N) {
            ls4[g4] = *(const f32x4*)(LSE + q4);
            dl4[g4] = *(const f32x4*)(DEL + q4);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int qc = min(q4 + e, N - 1);
              ls4[g4][e] = LSE[qc];
              dl4[g4][e] = DEL[qc];
            }
          }
        }
      }

      // S = Q K^T and dP = dO V^T (32 queries x 32 keys), lane = key.
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
      if constexpr (D > 128) {
        // One wave per SIMD: nothing else hides the LDS latency, so each
        // k-step's four fragments are read one step ahead.
        u32x4 fq[2], fo[2], fk[2], fv[2];
        auto rd = [&](int kk, int i) {
          fq[i] = *(const u32x4*)(qb + roff[kk]);
          fo[i] = *(const u32x4*)(ob + roff[kk]);
          fk[i] = *(const u32x4*)(smem + kvoff[kk]);
          fv[i] = *(const u32x4*)(smem + kvoff[kk] + KV_WAVE);
        };
        rd(0, 0);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          if (kk + 1 < KK) rd(kk + 1, (kk + 1) & 1);
          s = E::mfma(fq[kk & 1], fk[kk & 1], s);
          dp = E::mfma(fo[kk & 1], fv[kk & 1], dp);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          s = E::mfma(*(const u32x4*)(qb + roff[kk]), *(const u32x4*)(smem + kvoff[kk]), s);
          dp = E::mfma(*(const u32x4*)(ob + roff[kk]),
                       *(const u32x4*)(smem + kvoff[kk] + KV_WAVE), dp);
        }
      }

      // The row loads are complete once only the two copy slices issued at
      // the top may still be outstanding.
      if constexpr (DBUF) wait_vm<2>();
      // P (masked), dropout, dS; packed as MFMA A operands for 16-query steps.
      // Register r holds query qbase + 8(r/4) + 4hh + r%4.
      const bool need_mask =
          (BAND && (qbase + band_hi < kw + 31 || (LO && qbase + 31 + band_lo > kw))) || key_tail ||
          (qbase + 32 > N);
      auto grad = [&](u32x4 (&pa)[2], u32x4 (&sa)[2], auto masked) {
        f32x16 pz, ds;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // This lane's dropout words for rows qbase + 8 g4 + 4 hh + e,
          // g4 = 0..3: the lane at quad position u draws row g4 = u, the
          // transpose distributes the words.
          u32x4 zw = u32x4{0, 0, 0, 0};
          if (DROPOUT) {
            const u32x4 mine = dropout_draws(
                (uint32_t)j >> 2, (uint32_t)(qbase + 8 * (lane & 3) + 4 * hh + e), (uint32_t)h,
                (uint32_t)b, a.seed_lo, a.seed_hi);
            zw = quad_transpose4(mine, (lane & 1) != 0, (lane & 2) != 0);
          }
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int r = 4 * g4 + e;
            const int qi = qbase + 8 * g4 + 4 * hh + e;
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c2, -ls4[g4][e]));
            if (decltype(masked)::value) {
              const bool dead = (BAND & ((j > qi + band_hi) | (LO & (j < qi + band_lo)))) |
                                (j >= kv_end) | (qi >= N);
              p = dead ? 0.f : p;
            }
            const float z = DROPOUT ? ((zw[g4] >= a.drop_threshold) ? a.drop_rescale : 0.f) : 1.f;
            pz[r] = p * z;
            ds[r] = p * (dp[r] * z - dl4[g4][e]);
          }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pa[c][e] = E::pack2(pz[8 * c + 2 * e], pz[8 * c + 2 * e + 1]);
            sa[c][e] = E::pack2(ds[8 * c + 2 * e], ds[8 * c + 2 * e + 1]);
          }
      };
      u32x4 pa[2], sa[2];
      if (need_mask)
        grad(pa, sa, std::true_type());
      else
        grad(pa, sa, std::false_type());

      // dV += (P Z)^T dO and dK += dS^T Q with dO, Q read transposed.
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int tbase = 16 * c * D * 2;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x2 olo = __builtin_bit_cast(u32x2, lds_read_tr16(ob, tbase + toff[0][db]));
          const u32x2 ohi = __builtin_bit_cast(u32x2, lds_read_tr16(ob, tbase + toff[1][db]));
          const u32x2 qlo = __builtin_bit_cast(u32x2, lds_read_tr16(qb, tbase + toff[0][db]));
          const u32x2 qhi = __builtin_bit_cast(u32x2, lds_read_tr16(qb, tbase + toff[1][db]));
          dv[db] = E::mfma(pa[c], u32x4{olo[0], olo[1], ohi[0], ohi[1]}, dv[db]);
          dk[db] = E::mfma(sa[c], u32x4{qlo[0], qlo[1], qhi[0], qhi[1]}, dk[db]);
        }
      }
      if constexpr (DBUF) load_rows(min(t + 1, nqt - 1));
    };
    if constexpr (DBUF) {
      for (int t = qt0; t < nqt; t += 2) {
        tile_step(t, std::integral_constant<int, 0>());
        if (t + 1 < nqt) tile_step(t + 1, std::integral_constant<int, 1>());
      }
      wait_all_memory();  // the last tile's redundant copy and row loads
    } else {
      // One buffer: the next tile is copied once every wave has read this
      // one (waves that skip a tile still meet both barriers).
      for (int t = qt0; t < nqt; ++t) {
        tile_step(t, std::integral_constant<int, 0>());
        __syncthreads();
        if (t + 1 < nqt) issue_tile(t + 1, 0);
      }
    }
  }

write_out:
  // Write dK (times scale) and dV: lane holds column 32db + l32 of key rows
  // kw + 8(r/4) + 4hh + r%4.
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (key < a.Nk) {
        const size_t idx = khead + (size_t)key * D + 32 * db + l32;
        const float gk = dk[db][r] * a.scale;
        const float gv = dv[db][r];
        if (OUT_F32) {
          ((float*)a.dk)[idx] = gk;
          ((float*)a.dv)[idx] = gv;
        } else {
          ((typename E::scalar*)a.dk)[idx] = (typename E::scalar)gk;
          ((typename E::scalar*)a.dv)[idx] = (typename E::scalar)gv;
        }
      }
    }
}

template <typename E, int D, int MASK, bool DROPOUT, bool OUT_F32>
static hipError_t launch_all(int stage, const BwdArgs& a, hipStream_t stream) {
  // A kernel with no work item is not launched (a zero-sized grid is a launch
  // error): no query rows leave only dK = dV = 0 to write, no key rows only
  // dQ = 0.
  hipError_t e = hipSuccess;
  if ((stage < 0 || stage == 0) && a.N > 0) {
    const long long rows = (long long)a.B * a.H * a.Np;
    const long long threads = rows * (D / 8);
    hipLaunchKernelGGL((attn_bwd_preprocess_kernel<E, D, OUT_F32>),
                       dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((stage < 0 || stage == 1) && a.Nk > 0) {
    constexpr int NW = dkdv_waves<D>();
    const int nkb = (a.Nk + 32 * NW - 1) / (32 * NW);
    const int tk = a.B * a.H * nkb;
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<E, D, MASK, DROPOUT, OUT_F32>),
                       dim3(((tk + 7) / 8) * 8), dim3(64 * NW), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((stage < 0 || stage == 2) && a.N > 0) {
    if constexpr (D > 128) {
      // Built in its own translation unit with other code-generation flags.
      e = launch_bwd_dq256(std::is_same<E, Elem<bf16_t>>::value ? 1 : 0, MASK, DROPOUT, OUT_F32,
                           a, stream);
    } else {
      const int nqb = (a.N + 127) / 128;
      const int tq = a.B * a.H * nqb;
      hipLaunchKernelGGL((attn_bwd_dq_kernel<E, D, MASK, DROPOUT, OUT_F32>),
                         dim3(((tq + 7) / 8) * 8), dim3(kBwdThreads), 0, stream, a);
      e = hipGetLastError();
    }
  }
  return e;
}

template <typename E, int D, int MASK>
static hipError_t launch_m(bool dropout, bool out_f32, int st, const BwdArgs& a, hipStream_t s) {
  if (dropout) return out_f32 ? launch_all<E, D, MASK, true, true>(st, a, s)
                              : launch_all<E, D, MASK, true, false>(st, a, s);
  return out_f32 ? launch_all<E, D, MASK, false, true>(st, a, s)
                 : launch_all<E, D, MASK, false, false>(st, a, s);
}

template <typename E, int D>
static hipError_t launch_d(int mask, bool dropout, bool out_f32, int st, const BwdArgs& a,
                           hipStream_t s) {
  if (mask == kMaskCausal) return launch_m<E, D, kMaskCausal>(dropout, out_f32, st, a, s);
  if (mask == kMaskBand) return launch_m<E, D, kMaskBand>(dropout, out_f32, st, a, s);
  return launch_m<E, D, kMaskNone>(dropout, out_f32, st, a, s);
}

hipError_t launch_bwd(int dtype, int d, int mask, bool dropout, bool out_f32, int stage,
                      const BwdArgs& a, hipStream_t stream) {
  if (dtype == 1) {
    if (d == 256) return launch_d<Elem<bf16_t>, 256>(mask, dropout, out_f32, stage, a, stream);
    if (d == 128) return launch_d<Elem<bf16_t>, 128>(mask, dropout, out_f32, stage, a, stream);
    return launch_d<Elem<bf16_t>, 64>(mask, dropout, out_f32, stage, a, stream);
  }
  if (d == 256) return launch_d<Elem<f16_t>, 256>(mask, dropout, out_f32, stage, a, stream);
  if (d == 128) return launch_d<Elem<f16_t>, 128>(mask, dropout, out_f32, stage, a, stream);
  return launch_d<Elem<f16_t>, 64>(mask, dropout, out_f32, stage, a, stream);
}

}  // namespace attn
