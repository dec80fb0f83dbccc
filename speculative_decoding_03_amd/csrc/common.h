// Shared device helpers for the CDNA4 (gfx950) kernels of libspecdec.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specdec {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;
constexpr int TILE_N = 16;       // rows of W (output features) per packed tile
constexpr int TILE_K = 32;       // reduction elements per packed tile
constexpr int TILE_ELEMS = 512;  // 16 x 32
constexpr int LANE_ELEMS = 8;    // elements each lane holds of a tile

// Storage element type tags.
struct bf16_t { uint16_t v; };

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16 with the gfx950 conversion instruction (round to nearest even; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 values -> packed bf16 pair (lo in bits 0-15), one conversion instruction.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  const f2_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, b2_t));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
  static __device__ __forceinline__ float to_f32(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(p->v); }
  static __device__ __forceinline__ void store(bf16_t* p, float v) { p->v = f32_to_bf16(v); }
};

// Offset (in elements) of logical element (n, k) of a packed [N][Kd] matrix.
// Tile (n/16, k/32) is 512 contiguous elements; inside it lane = ((k%32)/8)*16 + n%16 holds
// elements k%8 = 0..7, which is the operand layout of the 16x16x32 bf16 MFMA.
__host__ __device__ __forceinline__ size_t packed_offset(int n, int k, int nkb) {
  const size_t tile = (size_t)(n >> 4) * (size_t)nkb + (size_t)(k >> 5);
  const int lane = (((k & 31) >> 3) << 4) | (n & 15);
  return tile * TILE_ELEMS + (size_t)lane * LANE_ELEMS + (k & 7);
}

// The 4-bit block weight format (one fp16 step per 32 reduction elements, 4-bit codes, weight =
// step * (code - 8)): a 16-row tile and a group of 128 reduction elements take Q4_BLOCK_BYTES,
// the codes first (lane kg*16 + r: 16 bytes, dword kb holding the 8 codes of row r at
// k = kb*32 + kg*8 + 0..7: elements 0, 2, 4, 6 in bits 0-15, 1, 3, 5, 7 in bits 16-31, four bits
// each from the lowest), then row r's four steps at Q4_CODE_BYTES + 8r.  Blocks are stored tile
// by tile, each tile's k-groups in order.
constexpr int Q4_GROUP_K = 128;
constexpr int Q4_CODE_BYTES = 1024;
constexpr int Q4_BLOCK_BYTES = 1152;

__host__ __device__ inline size_t q4_block_offset(int n, int k, int nkb) {
  return ((size_t)(n >> 4) * (size_t)(nkb >> 2) + (size_t)(k >> 7)) * Q4_BLOCK_BYTES;
}

// Weights (n, k0 .. k0+7) of a 4-bit block matrix as fp32 (exact: an fp16 step times a small
// integer), k0 a multiple of 8.
__device__ __forceinline__ void q4_run8(const uint8_t* W, int n, int k0, int nkb, float (&v)[8]) {
  const uint8_t* blk = W + q4_block_offset(n, k0, nkb);
  const int kb = (k0 >> 5) & 3, kg = (k0 >> 3) & 3, r = n & 15;
  const uint32_t c = *reinterpret_cast<const uint32_t*>(blk + (kg * 16 + r) * 16 + kb * 4);
  const uint16_t h = *reinterpret_cast<const uint16_t*>(blk + Q4_CODE_BYTES + r * 8 + kb * 2);
  const float d = (float)__builtin_bit_cast(_Float16, h);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = d * (float)((int)((c >> ((e & 1) * 16 + (e >> 1) * 4)) & 15u) - 8);
}

// Device-scope fences / atomics for the split-K "last arriver" reduction.
__device__ __forceinline__ void fence_device() { __threadfence(); }

__device__ __forceinline__ int atomic_inc_device(int* p) {
  return __hip_atomic_fetch_add(p, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void atomic_store_zero(int* p) {
  __hip_atomic_store(p, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lowest-index-wins argmax combine on (value, index) pairs.
__device__ __forceinline__ void argmax_combine(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

// Lane exchange inside each row of 16 lanes (DPP): quad permutations and the row mirrors.
enum : int { DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140 };
template <int CTRL> __device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL> __device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// Sum over each row of 16 lanes, in VALU lane exchanges: pairs, quads, half rows, rows.  Every
// step adds two equal-sized groups symmetrically, so all 16 lanes end with the same bits.
__device__ __forceinline__ float sum16(float v) {
  v += dpp_f32<DPP_XOR1>(v);
  v += dpp_f32<DPP_XOR2>(v);
  v += dpp_f32<DPP_HALF_MIRROR>(v);
  v += dpp_f32<DPP_MIRROR>(v);
  return v;
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp_f32<DPP_XOR1>(v));
  v = fmaxf(v, dpp_f32<DPP_XOR2>(v));
  v = fmaxf(v, dpp_f32<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f32<DPP_MIRROR>(v));
  return v;
}

// Rows of 16 lanes combined on the gfx950 row-swap instructions: after a swap the pair holds both
// rows' values in every lane, in the same order, so all lanes keep identical bits.
__device__ __forceinline__ float wave_sum(float v) {
  v = sum16(v);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// (max, lowest index) over each row of 16 lanes, in the same exchange pattern as sum16.
__device__ __forceinline__ void argmax16(float& v, int& i) {
  argmax_combine(v, i, dpp_f32<DPP_XOR1>(v), dpp_i32<DPP_XOR1>(i));
  argmax_combine(v, i, dpp_f32<DPP_XOR2>(v), dpp_i32<DPP_XOR2>(i));
  argmax_combine(v, i, dpp_f32<DPP_HALF_MIRROR>(v), dpp_i32<DPP_HALF_MIRROR>(i));
  argmax_combine(v, i, dpp_f32<DPP_MIRROR>(v), dpp_i32<DPP_MIRROR>(i));
}

// (max, lowest index) over the wave; every lane ends with the same pair.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax16(v, i);
  auto rv = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  auto ri = __builtin_amdgcn_permlane16_swap((unsigned)i, (unsigned)i, false, false);
  v = __uint_as_float(rv[0]);
  i = (int)ri[0];
  argmax_combine(v, i, __uint_as_float(rv[1]), (int)ri[1]);
  rv = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  ri = __builtin_amdgcn_permlane32_swap((unsigned)i, (unsigned)i, false, false);
  v = __uint_as_float(rv[0]);
  i = (int)ri[0];
  argmax_combine(v, i, __uint_as_float(rv[1]), (int)ri[1]);
}

__device__ __forceinline__ float wave_max(float v) {
  v = max16(v);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Activation layout for at most 4 rows ("quad"): the reduction axis in blocks of 128 (four
// k-blocks of 32), 512 elements per block; element (r, k) sits in lane kg*16 + j*4 + r of its
// block, 8 consecutive elements per lane (kg = (k % 32) / 8, j = (k / 32) % 4).  One wave load
// of a block holds four k-blocks; the operand fragment of k-block j (lane kg*16 + r holding row
// r) is the block shifted down by 4j lanes within each row of 16 lanes.
__host__ __device__ inline size_t qx_offset(int r, int k) {
  return (size_t)(k >> 7) * 512 + (size_t)(((((k >> 3) & 3) << 4) + (((k >> 5) & 3) << 2) + r) << 3) +
         (size_t)(k & 7);
}
// element (r, k) of an activation matrix with row stride ld, row-major or quad
__host__ __device__ inline size_t x_offset(int qx, int r, int k, int ld) {
  return qx ? qx_offset(r, k) : (size_t)r * ld + k;
}

// One lane's share of a 16x32 MFMA operand tile: 8 consecutive reduction elements of one row.
template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
  u32x4 v;
};
template <> struct Frag<float> {
  u32x4 v[2];
};

template <typename T>
__device__ __forceinline__ void zero_frag(Frag<T>& f) {
  if constexpr (sizeof(T) == 2) {
    f.v = u32x4{0, 0, 0, 0};
  } else {
    f.v[0] = u32x4{0, 0, 0, 0};
    f.v[1] = u32x4{0, 0, 0, 0};
  }
}

// 8 fp32 values -> fragment of the storage type (bf16: round to nearest even).
template <typename T>
__device__ __forceinline__ void to_frag(Frag<T>& f, const float (&y)[8]) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = f32x2_to_bf16x2(y[2 * i], y[2 * i + 1]);
    f.v = u32x4{w[0], w[1], w[2], w[3]};
  } else {
    f.v[0] = u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                   __float_as_uint(y[3])};
    f.v[1] = u32x4{__float_as_uint(y[4]), __float_as_uint(y[5]), __float_as_uint(y[6]),
                   __float_as_uint(y[7])};
  }
}

// 16-byte (bf16) / 32-byte (fp32) fragment load of 8 consecutive elements.
template <typename T>
__device__ __forceinline__ void load_frag(Frag<T>& f, const T* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  if constexpr (sizeof(T) == 2) {
    f.v = *q;
  } else {
    f.v[0] = q[0];
    f.v[1] = q[1];
  }
}

// The 8 values of a fragment as fp32.
template <typename T>
__device__ __forceinline__ void frag_values(const Frag<T>& f, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(f.v[i] << 16);
      v[2 * i + 1] = __uint_as_float(f.v[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(f.v[0][i]);
      v[4 + i] = __uint_as_float(f.v[1][i]);
    }
  }
}

// acc += A (16 rows x 32, lanes as Frag) . B^T (16 cols x 32): C[i][j], lane l holds rows
// (l/16)*4 + 0..3 of column l%16.
template <typename T>
__device__ __forceinline__ f32x4 mma(const Frag<T>& a, const Frag<T>& b, f32x4 acc) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                   __builtin_bit_cast(bf16x8, b.v), acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v[h][e]),
                                                   __uint_as_float(b.v[h][e]), acc, 0, 0, 0);
    return acc;
  }
}

// Error word bits raised by kernels (sticky until cleared by the host).
enum : int { ERRBIT_CAPACITY = 1, ERRBIT_NAN = 2, ERRBIT_TOKEN = 4 };

__device__ __forceinline__ void raise_error(int* err, int bit) {
  if (err) __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace specdec
