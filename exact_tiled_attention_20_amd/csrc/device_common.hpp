// Device-side building blocks shared by the gfx950 attention kernels.
//
// Everything here is written for CDNA4 (gfx950) wave64 execution:
//   * MFMA wrappers for v_mfma_f32_32x32x16_{bf16,f16}. Lane layouts (checked
//     on the device): A operand, lane l holds A[l%32][8*(l/32) .. +8];
//     B operand, lane l holds B[8*(l/32) .. +8][l%32]; the 32x32 fp32 result
//     is spread so that lane l holds column l%32 and, in register r, row
//     8*(r/4) + 4*(l/32) + r%4.
//   * ds_read_b64_tr_b16 (LDS transpose read): within each group of 16 lanes,
//     lane i receives element (i%4) of the 4-element rows addressed by lanes
//     i/4, i/4+4, i/4+8, i/4+12 of its group.
//   * Philox4x32-10 written from its published definition (Salmon, Moraes,
//     Dror, Shaw, SC'11).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Storage element tags. Both are 16-bit in memory.
struct bf16_t {};
struct f16_t {};

template <typename E> struct Elem;
template <> struct Elem<bf16_t> {
  typedef bf16x8 vec8;
  typedef __bf16 scalar;
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Round-to-nearest-even pack of two floats into one dword (lo, hi):
  // a single v_cvt_pk_bf16_f32.
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
  }
  static __device__ __forceinline__ float to_float(uint16_t x) {
    return __uint_as_float((uint32_t)x << 16);
  }
  // acc + lo + hi of a packed pair (v_dot2c_f32_bf16 against (1, 1)).
  static __device__ __forceinline__ float add_pair(uint32_t packed, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
  }
};
template <> struct Elem<f16_t> {
  typedef f16x8 vec8;
  typedef _Float16 scalar;
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // v_cvt_pk_f16_f32 (round to nearest even).
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
  }
  static __device__ __forceinline__ float to_float(uint16_t x) {
    return (float)__builtin_bit_cast(_Float16, x);
  }
  // acc + lo + hi of a packed pair (v_dot2c_f32_f16 against (1, 1)).
  static __device__ __forceinline__ float add_pair(uint32_t packed, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), one, acc, false);
  }
};

// ---------------------------------------------------------------------------
// Philox4x32-10 (SC'11): two multiplier rounds per step, Weyl key schedule.
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    // One 32x32 -> 64-bit multiply per product (v_mad_u64_u32) gives both
    // halves the round needs.
    const uint64_t p0 = (uint64_t)kPhiloxM0 * c[0];
    const uint64_t p1 = (uint64_t)kPhiloxM1 * c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    u32x4 n;
    n[0] = hi1 ^ c[1] ^ k0;
    n[1] = lo1;
    n[2] = hi0 ^ c[3] ^ k1;
    n[3] = lo0;
    c = n;
  }
  return c;
}

// Draws for keys 4t..4t+3 of query i in head (b, h): counter (t, i, h, b).
__device__ __forceinline__ u32x4 dropout_draws(uint32_t t, uint32_t i, uint32_t h,
                                               uint32_t b, uint32_t k0, uint32_t k1) {
  u32x4 c;
  c[0] = t;
  c[1] = i;
  c[2] = h;
  c[3] = b;
  return philox4x32_10(c, k0, k1);
}

// ---------------------------------------------------------------------------
// LDS tile layout. A tile is ROWS x D 16-bit elements, one row per key (or per
// query), D*2 bytes per row. Tiles are read two ways:
//   * row reads (MFMA A operands): 32 consecutive rows, one 16-byte chunk each;
//   * transpose reads (ds_read_b64_tr_b16): per 32 lanes, 4 consecutive rows
//     (starting at a multiple of 4) x 64 contiguous bytes.
// The 16-byte chunk index is XORed with a row-dependent mask whose two high
// bits rotate the 64-byte segment with row%4 and whose two low bits take the
// next row bits, so both patterns touch every bank once per 256 bytes.
template <int D>
__device__ __forceinline__ int lds_swz(int row) {
  // d = 256 rows span two 256-byte bank rounds; the bank group of a chunk is
  // its index mod 16, so the d = 128 mask (4 bits) serves both.
  if (D >= 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

template <int D>
__device__ __forceinline__ int lds_off(int row, int byte_in_row) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row: 16 (D=128) or 8 (D=64)
  const int chunk = (byte_in_row >> 4) ^ lds_swz<D>(row);
  return row * (D * 2) + ((chunk & (CPR - 1)) << 4) + (byte_in_row & 15);
}

// Direct HBM -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane l
// writes LDS bytes [lds_base + 16 l, +16). lds_base must be wave-uniform.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
__device__ __forceinline__ void load_lds16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds_base, 16, 0, 0);
}

// Copies ROWS x D tiles of two row-major (rows, D) arrays A and B from HBM into
// LDS in the lds_off layout, NWAVES waves sharing the work: each wave fills
// SPW slices of 1 KiB per tile; within a slice lane l fills LDS chunk l, which
// holds logical chunk (l % CPR) ^ swizzle(row) of tile row slice*RPS + l/CPR.
// Rows at or past `valid` repeat row valid-1 (finite data the caller masks).
// The same 16-byte copy written as inline assembly: base is wave-uniform,
// voff is this lane's byte offset, lds_base the wave-uniform destination.
// Writing M0 needs one wait state before the copy reads it. M0 is declared as
// an output of the statement, so the compiler knows its value changed (M0 is
// a reserved register and cannot appear in a clobber list). The copy counts
// against vmcnt like any vector load.
__device__ __forceinline__ void load_lds16_untracked(const void* base, uint32_t voff,
                                                     void* lds_base) {
  const uint32_t m0v = (uint32_t)(uintptr_t)(lds_void_t*)lds_base;
  uint32_t m0_out;
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      : "={m0}"(m0_out)
      : "v"(voff), "s"(base), "s"(m0v)
      : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (they complete in issue order); LDS and export counters are not waited on.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int D, int ROWS, int NWAVES>
struct TilePairLoader {
  static constexpr int CPR = D / 8;
  static constexpr int TILE_BYTES = ROWS * D * 2;
  static constexpr int RPS = 1024 / (D * 2);
  static constexpr int SPW = TILE_BYTES / 1024 / NWAVES;
  static_assert(SPW >= 1 && SPW * NWAVES * 1024 == TILE_BYTES, "tile does not split evenly");
  uint32_t goff[SPW];
  int grow[SPW];
  int wave;

  __device__ __forceinline__ void init(int w, int lane) {
    wave = w;
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      grow[u] = (w * SPW + u) * RPS + lane / CPR;
      goff[u] = (uint32_t)(grow[u] * D * 2 + (((lane % CPR) ^ lds_swz<D>(grow[u])) << 4));
    }
  }
  // Tile rows [row0, row0 + ROWS) of one array into lds, issued so that the
  // compiler does not track the copy: no wait for it is inserted before later
  // LDS reads, and the caller orders every read of the destination after
  // wait_vm() and a barrier.
  __device__ __forceinline__ void issue_one_untracked(const uint16_t* A, int row0, int valid,
                                                      char* lds) const {
    const char* at = (const char*)A + (size_t)row0 * D * 2;
    if (row0 + ROWS <= valid) {  // full tile (wave-uniform branch)
#pragma unroll
      for (int u = 0; u < SPW; ++u)
        load_lds16_untracked(at, goff[u], lds + (wave * SPW + u) * 1024);
      return;
    }
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      uint32_t off = goff[u];
      if (row0 + grow[u] >= valid) off += (uint32_t)((valid - 1 - row0 - grow[u]) * D * 2);
      load_lds16_untracked(at, off, lds + (wave * SPW + u) * 1024);
    }
  }
  // Slice u of a full tile (every row below `valid`), untracked like
  // issue_one_untracked: lets a caller spread one tile's copies over a stretch
  // of other work.
  __device__ __forceinline__ void issue_slice_full(const uint16_t* A, int row0, char* lds,
                                                   int u) const {
    const char* at = (const char*)A + (size_t)row0 * D * 2;
    load_lds16_untracked(at, goff[u], lds + (wave * SPW + u) * 1024);
  }
  // Tile rows [row0, row0 + ROWS) of one array into lds.
  __device__ __forceinline__ void issue_one(const uint16_t* A, int row0, int valid,
                                            char* lds) const {
    const char* at = (const char*)A + (size_t)row0 * D * 2;
    const bool partial = row0 + ROWS > valid;
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      uint32_t off = goff[u];
      if (partial && row0 + grow[u] >= valid)
        off += (uint32_t)((valid - 1 - row0 - grow[u]) * D * 2);
      load_lds16(at + off, lds + (wave * SPW + u) * 1024);
    }
  }
  // Like issue(), but slice u of this wave goes to lds_a / lds_b + u * 1024:
  // the caller passes this wave's own destination blocks.
  __device__ __forceinline__ void issue_local(const uint16_t* A, const uint16_t* B, int row0,
                                              int valid, char* lds_a, char* lds_b) const {
    const char* at = (const char*)A + (size_t)row0 * D * 2;
    const char* bt = (const char*)B + (size_t)row0 * D * 2;
    const bool partial = row0 + ROWS > valid;
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      uint32_t off = goff[u];
      if (partial && row0 + grow[u] >= valid)
        off += (uint32_t)((valid - 1 - row0 - grow[u]) * D * 2);
      load_lds16(at + off, lds_a + u * 1024);
      load_lds16(bt + off, lds_b + u * 1024);
    }
  }
  // Tile rows [row0, row0 + ROWS) of A and B into lds_a / lds_b.
  __device__ __forceinline__ void issue(const uint16_t* A, const uint16_t* B, int row0,
                                        int valid, char* lds_a, char* lds_b) const {
    const char* at = (const char*)A + (size_t)row0 * D * 2;
    const char* bt = (const char*)B + (size_t)row0 * D * 2;
    const bool partial = row0 + ROWS > valid;
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      uint32_t off = goff[u];
      if (partial && row0 + grow[u] >= valid)
        off += (uint32_t)((valid - 1 - row0 - grow[u]) * D * 2);
      const int dst = (wave * SPW + u) * 1024;
      load_lds16(at + off, lds_a + dst);
      load_lds16(bt + off, lds_b + dst);
    }
  }
};

// Work decomposition over the 8 XCDs. Workgroup id g runs on XCD g % 8, and
// each XCD has its own L2, so every (b, h) head is kept on one XCD, where its
// K/V re-reads stay in that L2. Within an XCD the block rank varies slowest
// when the heads split evenly over the XCDs: the heaviest block of every head
// starts before any lighter one, which keeps the tail of a causal launch
// short. Otherwise each XCD takes a consecutive range of (head, rank) items.
// The grid is 8 * ceil(heads * nblk / 8) workgroups.
struct WorkItem {
  int bh;    // b * H + h
  int rank;  // 0 = first block to start
  bool valid;
};
__device__ __forceinline__ WorkItem decode_work_item(int bid, int heads, int nblk) {
  const int x = bid & 7;
  const int i = bid >> 3;
  if ((heads & 7) == 0) {
    const int hpx = heads >> 3;
    const int rank = i / hpx;
    return {x * hpx + (i - rank * hpx), rank, rank < nblk};
  }
  const int total = heads * nblk;
  const int item = x * ((total + 7) / 8) + i;
  const int bh = item / nblk;
  return {bh, item - bh * nblk, item < total};
}

// Wait until at most N vector-memory operations of this wave are outstanding
// and every LDS / scalar-memory operation has completed.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Workgroup execution barrier that waits for no outstanding memory operation.
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// 4-byte variant: lane l writes LDS bytes [lds_base + 4 l, +4).
__device__ __forceinline__ void load_lds4(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds_base, 4, 0, 0);
}

// Wait until every outstanding memory operation of this wave has completed,
// including HBM -> LDS copies (which count as vector-memory loads).
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds_base, int byte_off) {
  const char* p = (const char*)lds_base + byte_off;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

__device__ __forceinline__ float wave_swap_halves(float x) {
  // Exchange with the lane 32 positions away (lanes 0..31 <-> 32..63).
  return __shfl_xor(x, 32, 64);
}

// max / sum of x over lanes l and l^32 with one v_permlane32_swap: the swap
// returns (x of the upper half in the lower lanes, x of the lower half in the
// upper lanes) beside the untouched copies, so combining the pair gives the
// two-lane result in every lane.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace attn
