// LDS tile helpers shared by the backward and decode kernels: row-major
// tiles of 16-bit rows copied from HBM by buffer_load ... lds, read back as
// MFMA row fragments or, through the transposing LDS read, as fragments of
// the transposed tile.
#pragma once

#include "attn_fwd_kernels.h"

namespace mi_attn {
namespace {

// ----------------------------------------------------------------------------
// LDS tiles of the backward and decode kernels.  A tile is `ROWS` rows of D
// 16-bit elements, row-major, with the 16-byte chunks of row r XOR-swizzled
// by TSwz<D>::f(r).  The tiles are read both ways: as row fragments (one
// 16-byte chunk of 16 different rows per LDS cycle: the swizzle must map
// those rows to 16 different bank quads, i.e. be a bijection of the row
// bits that the row stride leaves inside one 256-byte bank line) and through
// the transposing read (four consecutive rows per read: their chunks must
// fall in four different 4-chunk groups, which VSwz's high bits give).  The
// low two bits, XOR-ed with (r >> 2) & 3, complete the bijection without
// changing the 4-chunk group, so both reads are free of bank conflicts.
// ----------------------------------------------------------------------------
template <int D>
struct TSwz {
  __device__ static int f(int row) { return VSwz<D>::f(row) | ((row >> 2) & 3); }
};

// Per-lane byte offsets (from the tile's first row in global memory) of the
// chunks this thread copies, for LOADS copies of NT x 16 bytes (NT threads
// copy the tile together).
template <int D, int LOADS, int NT = kThreads>
__device__ __forceinline__ void tile_offsets(uint32_t (&off)[LOADS], int64_t st_b, int tid) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int pos = i * NT + tid;
    const int row = pos / CPR;
    const int c = (pos % CPR) ^ TSwz<D>::f(row);
    off[i] = (uint32_t)(row * st_b + c * 16);
  }
}

// Copy `rows` rows of a [tokens, D] tensor view (first row at `base`, token
// stride st_b bytes) into the tile at `dst`; tile rows at or past `rows` read
// as zeros (rows <= 0: the whole tile is zero).
template <int D, int LOADS, int NT = kThreads>
__device__ __forceinline__ void load_tile(const char* base, int64_t st_b, int rows, lds_char* dst,
                                          const uint32_t* off, int wave) {
  const uint32_t bytes = rows > 0 ? (uint32_t)((rows - 1) * st_b + D * 2) : 0u;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(uniform_ptr(base), bytes);
#pragma unroll
  for (int i = 0; i < LOADS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + wave * 1024 + i * NT * 16),
                                             16, off[i], 0, 0, 0);
}

// 8 consecutive elements of tile row `row` starting at column 16 ks + 8 hf
// (an MFMA operand row fragment).
template <int D>
__device__ __forceinline__ u32x4_t row_frag(const lds_char* tile, int row, int ks, int hf) {
  const int c = (2 * ks + hf) ^ TSwz<D>::f(row);
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(tile + row * (D * 2) + c * 16);
}

// Transposed fragment: rows 16 ks + {0..3, 8..11} + 4 hf of column
// 32 db + lane % 32, through two ds_read_b64_tr_b16 (the A operand of a
// product whose reduction runs over the tile's rows).
template <int D>
__device__ __forceinline__ u32x4_t tr_frag(const lds_char* tile, int ks, int db, int lane) {
  const int hf = lane >> 5;
  const int key_lane = 4 * hf + ((lane & 15) >> 2);
  const int chunk_lane = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int byte_lane = (lane & 1) * 8;
  u32x4_t r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 16 * ks + 8 * h + key_lane;
    const int c = (4 * db + chunk_lane) ^ TSwz<D>::f(row);
    const v4i16_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16_t*)(tile + row * (D * 2) + c * 16 + byte_lane));
    const u32x2_t xw = __builtin_bit_cast(u32x2_t, x);
    r[2 * h] = xw[0];
    r[2 * h + 1] = xw[1];
  }
  return r;
}

// B-operand fragment of k-step kk (16 rows of the accumulator's M axis) from
// a 32x32 fp32 accumulator block: the lane's entries 8 kk .. 8 kk + 7, i.e.
// M rows 16 kk + {0..3, 8..11} + 4 hf, rounded to T (RNE).
template <typename T>
__device__ __forceinline__ u32x4_t pack_b(const f32x16_t& x, int kk) {
  u32x4_t r;
#pragma unroll
  for (int w = 0; w < 4; ++w) r[w] = Elem<T>::pack(x[8 * kk + 2 * w], x[8 * kk + 2 * w + 1]);
  return r;
}

}  // namespace
}  // namespace mi_attn
