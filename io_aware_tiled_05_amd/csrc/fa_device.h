// fa_device.h — gfx950 device helpers shared by the attention kernels.
//
// Matrix-core (MFMA) operand layouts used throughout, for
// v_mfma_f32_16x16x32_{bf16,f16} on a 64-lane wavefront, with lane = 16*g + n
// (n = lane & 15, g = lane >> 4):
//   A operand (16 x 32, row-major M x K): lane holds row n, k = 8g .. 8g+7
//   B operand (32 x 16, K x N):           lane holds col n, k = 8g .. 8g+7
//   C/D accumulator (16 x 16):            lane holds col n, rows 4g .. 4g+3
// The order of the 32 k values inside one instruction does not change the
// result as long as A and B use the same order, which the kernels exploit to
// feed an accumulator straight back in as the next operand.
//
// ds_read_b64_tr_b16 (LDS transpose read) on gfx950: inside each group of 16
// lanes, lane s supplies the address of 4 consecutive 16-bit elements; lane j
// of the group receives element (j % 4) of lanes 4i + j/4, i = 0..3.  If lane
// s points at row r0 + s/4, columns c0 + 4(s%4) .. +3 of a row-major tile,
// lane j therefore receives column c0 + j of rows r0 .. r0+3: a 4 x 16 block
// read column-wise.  This gives the k-contiguous operand for contractions
// over the row index of a row-major tile (V in P·V, dO in dV, Q in dK, K in
// dQ) without a transposing store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element-type traits: 16-bit storage type, MFMA operand vector, rounding.
template <typename T> struct Elt;

template <> struct Elt<__bf16> {
  typedef bf16x8 vec8;
  static __device__ __forceinline__ f32x4 mfma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mfma32(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // round-to-nearest-even conversion of two floats into one packed dword
  // (one v_cvt_pk_bf16_f32)
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    const f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  // acc + lo(p) + hi(p) (v_dot2c_f32_bf16 against 1.0, 1.0)
  static __device__ __forceinline__ float sum2(uint32_t p, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), one, acc, false);
  }
};

template <> struct Elt<_Float16> {
  typedef f16x8 vec8;
  static __device__ __forceinline__ f32x4 mfma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mfma32(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    const f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  static __device__ __forceinline__ float sum2(uint32_t p, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p), one, acc, false);
  }
};

template <typename T>
__device__ __forceinline__ typename Elt<T>::vec8 as_vec8(u32x4 u) {
  return __builtin_bit_cast(typename Elt<T>::vec8, u);
}

// Four floats (an accumulator quarter) -> four 16-bit values in two dwords.
template <typename T>
__device__ __forceinline__ u32x2 pack4(f32x4 x) {
  u32x2 r;
  r.x = Elt<T>::pack2(x[0], x[1]);
  r.y = Elt<T>::pack2(x[2], x[3]);
  return r;
}

// Eight floats (two accumulator quarters) -> one 16-bit MFMA operand.
template <typename T>
__device__ __forceinline__ typename Elt<T>::vec8 pack8(f32x4 lo, f32x4 hi) {
  u32x4 r;
  r.x = Elt<T>::pack2(lo[0], lo[1]);
  r.y = Elt<T>::pack2(lo[2], lo[3]);
  r.z = Elt<T>::pack2(hi[0], hi[1]);
  r.w = Elt<T>::pack2(hi[2], hi[3]);
  return as_vec8<T>(r);
}

// x - round16(x): the part of x a 16-bit operand loses.  pack8 of x plus
// pack8 of the residual carries x to about 16 significant bits through two
// MFMAs (used where a bf16-rounded operand would eat the error budget).
template <typename T>
__device__ __forceinline__ f32x4 residual16(f32x4 x) {
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = x[i] - (float)(T)x[i];
  return r;
}

// 16 bytes (columns col .. col+7) of row `row` of a tensor with nrows >= 1
// rows of stride rs elements; zero for row >= nrows.  The load is issued
// for every lane (from the last row where row >= nrows) and the zero is a
// select, so a run of these loads is straight-line code: a branch around
// each load makes the compiler wait for the loads before it at the join,
// which serialises their latencies in the kernels' prologues.
__device__ __forceinline__ u32x4 ldg16_row(const uint16_t* base, int row, int64_t rs, int col,
                                           int nrows) {
  const int r = row < nrows ? row : nrows - 1;
  const u32x4 v = *reinterpret_cast<const u32x4*>(base + (int64_t)r * rs + col);
  const u32x4 z = {0u, 0u, 0u, 0u};
  return row < nrows ? v : z;
}

// The same without the zero: rows >= nrows read a copy of the last row.
// For operands whose rows past the end reach only outputs that are never
// stored (the queries of the forward), this leaves the load's destination
// free of a select, so the compiler can issue a run of them back to back
// even where registers are scarce (with the select it reuses one
// destination and waits for each load in turn).
__device__ __forceinline__ u32x4 ldg16_clamp(const uint16_t* base, int row, int64_t rs, int col,
                                             int nrows) {
  const int r = row < nrows ? row : nrows - 1;
  return *reinterpret_cast<const u32x4*>(base + (int64_t)r * rs + col);
}

// element i of a float array of n >= 1 elements, `other` for i >= n (a
// select after an unconditional load, as above)
__device__ __forceinline__ float ldg_f32(const float* a, int i, int n, float other) {
  const float v = a[i < n ? i : n - 1];
  return i < n ? v : other;
}

__device__ __forceinline__ u32x4 lds16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void sts16(uint16_t* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// Transpose read of 4 16-bit elements (see the header comment).
__device__ __forceinline__ u32x2 lds_tr4(const uint16_t* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

template <typename T>
__device__ __forceinline__ typename Elt<T>::vec8 join8(u32x2 lo, u32x2 hi) {
  u32x4 r = {lo.x, lo.y, hi.x, hi.y};
  return as_vec8<T>(r);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

__device__ __forceinline__ float fast_log2(float x) {
  return __builtin_amdgcn_logf(x);   // v_log_f32 (base 2)
}

// max / sum over the four 16-lane groups that share a column n
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float group_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// XOR swizzle of the 16-byte chunks of an LDS tile row (r = tile row,
// CPR = 16-byte chunks per row: 4, 8, 12, 16 for d = 32, 64, 96, 128).
// Element (r, c) of a [rows][D] tile lives at r*D + ((c/8) ^ swz(r))*8 + c%8.
// The permutation makes both read patterns of a tile conflict-free on the
// 64 LDS banks (16 chunk-wide bank groups): the row-wise 16-byte reads of 16
// consecutive rows (one chunk column) and the transpose reads of 4
// consecutive rows x an aligned group of 4 chunks.  For 4- and 12-chunk rows
// the 4 rows r, r+4, r+8, r+12 share a bank group, and swz = (r/4) mod 4
// (below 4, so a chunk stays inside its aligned group of 4) separates them;
// 4 consecutive rows then already fall in 4 different bank groups.
template <int CPR>
__host__ __device__ __forceinline__ int swz(int r) {
  static_assert(CPR == 4 || CPR == 8 || CPR == 12 || CPR == 16, "d must be 32, 64, 96 or 128");
  if (CPR == 8)  // bit-reversed (r >> 1) & 7
    return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
  if (CPR == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (r >> 2) & 3;
}

template <int D>
__host__ __device__ __forceinline__ int tile_off(int r, int c) {
  return r * D + (((c >> 3) ^ swz<D / 8>(r)) << 3) + (c & 7);
}

// Element offset, relative to row0 * rs, that a copy lane reads for the
// chunk at offset `off` = r * rs + (chunk column) of tile row r, in a matrix
// of row stride rs, when rows at or past `nrows` re-read row nrows - 1.
// Signed: row0 itself may lie past nrows - 1 (the second half of the last
// 128-row block of a block-sparse list), and the result is then negative.
// The row read is min(row0 + r, nrows - 1).
__host__ __device__ inline int64_t clamped_chunk_offset(uint32_t off, int r, int64_t rs, int row0,
                                                        int nrows) {
  const int last = nrows - 1 - row0;  // last valid row, relative to row0
  return r <= last ? (int64_t)off : (int64_t)off - (int64_t)(r - last) * rs;
}

// Copies rows [row0, row0 + ROWS) of a row-major 16-bit matrix with D
// elements per row and a row stride of rs elements (rs = D when the rows
// are packed; a multiple of 8) into a swizzled LDS tile with direct
// global->LDS loads (no VGPR staging).  NW waves share the copy: 16-byte
// slot s of the tile (slot = 64 * instruction + lane) receives row s / CPR,
// chunk (s % CPR) ^ swz(row).  The per-lane element offsets are
// tile-invariant and computed once for the row stride given at
// construction; a copy is then one load per instruction from a
// wave-uniform base.  A copy from a matrix of another row stride (copy_rs)
// adjusts the offsets on the way, a few instructions per chunk.  Rows at or
// past `nrows` re-read row nrows-1 (their contents are never used
// unmasked).  Completion is tracked by vmcnt.
template <int D, int ROWS, int NW>
struct TileCopy {
  static constexpr int CPR = D / 8;
  static constexpr int ITER = ROWS * CPR / (64 * NW);
  static_assert(ITER * 64 * NW == ROWS * CPR, "tile must split evenly over the waves");
  uint32_t off[ITER];  // element offset of this lane's chunk from the tile's first row
  int wave, lane;
  int64_t rs;

  __device__ __forceinline__ TileCopy(int wave_, int lane_, int64_t rs_)
      : wave(wave_), lane(lane_), rs(rs_) {
#pragma unroll
    for (int j = 0; j < ITER; ++j) {
      const int s = (j * NW + wave) * 64 + lane;
      const int r = s / CPR, c = (s % CPR) ^ swz<CPR>(r);
      off[j] = (uint32_t)(r * rs + c * 8);
    }
  }

  __device__ __forceinline__ void operator()(const uint16_t* g, int row0, int nrows,
                                             uint16_t* lds) const {
    copy_rs(g, rs, row0, nrows, lds);
  }

  // the same from a matrix of row stride rsm
  __device__ __forceinline__ void copy_rs(const uint16_t* g, int64_t rsm, int row0, int nrows,
                                          uint16_t* lds) const {
    const uint16_t* base = g + (int64_t)row0 * rsm;
    if (row0 + ROWS <= nrows && rsm == rs) {
#pragma unroll
      for (int j = 0; j < ITER; ++j)
        __builtin_amdgcn_global_load_lds(base + off[j], lds + (j * NW + wave) * 512, 16, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < ITER; ++j) {
        const int r = ((j * NW + wave) * 64 + lane) / CPR;
        const uint32_t o = (uint32_t)((int64_t)off[j] + r * (rsm - rs));  // r * rsm + chunk
        __builtin_amdgcn_global_load_lds(base + clamped_chunk_offset(o, r, rsm, row0, nrows),
                                         lds + (j * NW + wave) * 512, 16, 0, 0);
      }
    }
  }
};

// OR of v over the four lanes of a quad (lanes 4q .. 4q + 3), in every lane
// of it: two DPP quad permutations, swapping neighbours and then pairs.
// Every lane of the wave must be active.
__device__ inline uint32_t quad_or(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  return v;
}

// OR of v over the 8 lanes that differ from this one in lane bits 0, 1 and
// 3 (inside one row of 16): the two quad swaps, then row_ror:8, which
// brings lane i ^ 8 of the row.  Every lane of the wave must be active.
__device__ inline uint32_t or8_bits013(uint32_t v) {
  v = quad_or(v);
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
  return v;
}

// a ^ b ^ c; on the device one v_bitop3_b32 (gfx950's three-input bitwise
// operation, 0x96 being the truth table of the three-way xor)
__host__ __device__ inline uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
#else
  return a ^ b ^ c;
#endif
}

// Philox4x32-10, the counter-based generator of J. K. Salmon, M. A. Moraes,
// R. O. Dror and D. E. Shaw ("Parallel random numbers: as easy as 1, 2,
// 3", SC 2011): ten rounds, each multiplying counter words 0 and 2 by the
// round multipliers into 64-bit products and forming (hi1 ^ c1 ^ k0, lo1,
// hi0 ^ c3 ^ k1, lo0); the key is bumped by the Weyl increments between
// rounds.  Four 32-bit outputs per counter.
__host__ __device__ inline void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                         uint32_t c3, uint32_t k0, uint32_t k1,
                                         uint32_t (&w)[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
    const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  w[0] = c0;
  w[1] = c1;
  w[2] = c2;
  w[3] = c3;
}

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }
__device__ __forceinline__ float pos_inf() { return __builtin_huge_valf(); }

// Workgroup id -> (tile rank, head index).  Workgroups are dispatched round
// robin over the 8 XCDs (each with its own L2); when the head count is a
// multiple of 8 every tile of one head is placed on the same XCD so that the
// head's K/V (or Q/dO) stream is shared through that XCD's L2.  Tile rank 0
// is dispatched first.
//
// `period` > 0 is the number of compute units that take one workgroup each
// per dispatch round (per XCD when heads are grouped by XCD): a CU receives
// the workgroups period apart, so with ranks in plain order one CU gets the
// longest tile of every round.  Reversing the order in every other round
// ("snake") gives each CU a long and a short tile in turn, which balances
// causal work whose length falls with the rank.
// Reverses slot order inside every odd round of `period` slots; a partial
// last round is reversed within its own length, so the map is a permutation
// of [0, total).
__host__ __device__ inline int snake(int slot, int period, int total) {
  if (period <= 0) return slot;
  const int round = slot / period, pos = slot - round * period, first = round * period;
  if ((round & 1) == 0) return slot;
  const int len = total - first < period ? total - first : period;
  return first + (len - 1 - pos);
}

// ntiles tiles per head, nheads heads, grid = ntiles * nheads workgroups.
__host__ __device__ inline void map_workgroup(int id, int ntiles, int nheads, int period,
                                              int* rank, int* head) {
  if ((nheads & 7) == 0) {
    const int xcd = id & 7, hpx = nheads >> 3;
    const int slot = snake(id >> 3, period, ntiles * hpx);
    *rank = slot / hpx;
    *head = xcd + 8 * (slot % hpx);
  } else {
    const int slot = snake(id, period, ntiles * nheads);
    *rank = slot / nheads;
    *head = slot % nheads;
  }
}

}  // namespace fa
