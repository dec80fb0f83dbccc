// Device-side seeded fills for synthetic workloads (weights, KV caches, hidden states).
//
// Same counter-based generator as workloads/synth.py: element i of the stream with key k is the
// (i+1)-th SplitMix64 output of state k (Steele, Lea and Flood, OOPSLA 2014; Stafford's Mix13
// finaliser).  value = float32(2*u24 - (2^24-1)) * scale, u24 = top 24 bits; bf16 tensors round
// that fp32 value to nearest-even.  4-bit tensors are drawn as codes and steps (workloads/synth.py
// describes both).  Holds no part of the decoding method.
#include <hip/hip_runtime.h>
#include <stdint.h>

// every product is rounded to fp32 on its own, as on the host (no fused multiply-add)
#pragma clang fp contract(off)

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float value_at(uint64_t key, uint64_t idx, float scale) {
  const uint64_t z = mix64(key + (idx + 1ull) * 0x9E3779B97F4A7C15ull);
  const int odd = (int)((z >> 40) * 2ull) - ((1 << 24) - 1);
  return (float)odd * scale;
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__global__ void fill_uniform(void* dst, int64_t n, int bf16, uint64_t key, int64_t start,
                             float scale) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float v = value_at(key, (uint64_t)(start + i), scale);
    if (bf16) reinterpret_cast<uint16_t*>(dst)[i] = to_bf16(v);
    else reinterpret_cast<float*>(dst)[i] = v;
  }
}

// 4-bit tensors as drawn: code i = top 4 bits of element start_q + i of stream key_q; step j =
// fp16(float32(u23 + 2^23) * scale), u23 the top 23 bits of element start_d + j of stream key_d.
__global__ void fill_q4(uint8_t* codes, int64_t n_codes, uint16_t* steps, int64_t n_steps,
                        uint64_t key_q, int64_t start_q, uint64_t key_d, int64_t start_d,
                        float scale) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_codes; i += stride) {
    const uint64_t z = mix64(key_q + ((uint64_t)(start_q + i) + 1ull) * 0x9E3779B97F4A7C15ull);
    codes[i] = (uint8_t)(z >> 60);
  }
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_steps; i += stride) {
    const uint64_t z = mix64(key_d + ((uint64_t)(start_d + i) + 1ull) * 0x9E3779B97F4A7C15ull);
    float v = (float)((uint32_t)(z >> 41) + 8388608u) * scale;
    // the product is rounded to fp32 before the fp16 conversion (the host's two roundings); the
    // empty asm keeps the compiler from fusing both into one mixed-precision multiply
    asm volatile("" : "+v"(v));
    steps[i] = __builtin_bit_cast(uint16_t, (_Float16)v);
  }
}

// KV cache: K [L][Bc][Hkv][max_ctx][hd], V transposed [L][Bc][Hkv][hd][max_ctx].  Positions
// [0, ctx) of sequences [0, Bl) get the logical element (((l*Bl + b)*Hkv + g)*ctx + pos)*hd + c.
__global__ void fill_kv(void* dst, int L, int Bl, int Bc, int Hkv, int ctx, int max_ctx, int hd,
                        int bf16, uint64_t key, float scale, int transposed) {
  const int64_t n = (int64_t)L * Bl * Hkv * ctx * hd;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = i;
    const int c = (int)(r % hd); r /= hd;
    const int pos = (int)(r % ctx); r /= ctx;
    const int g = (int)(r % Hkv); r /= Hkv;
    const int b = (int)(r % Bl); r /= Bl;
    const int l = (int)r;
    const int64_t head = ((int64_t)l * Bc + b) * Hkv + g;
    const int64_t o = transposed ? (head * hd + c) * max_ctx + pos : (head * max_ctx + pos) * hd + c;
    const float v = value_at(key, (uint64_t)i, scale);
    if (bf16) reinterpret_cast<uint16_t*>(dst)[o] = to_bf16(v);
    else reinterpret_cast<float*>(dst)[o] = v;
  }
}

// Streaming-read ceiling (a measurement, not part of the method): n_wg workgroups of 8 waves read
// a buffer once, each wave a contiguous run of per_wave16 16-byte units with non-temporal loads,
// 8 in flight per lane (the access pattern of a weight stream).  The loaded words are folded into
// one value that is stored only if it equals a constant, so the reads are not removed.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(512) stream_read(const u32x4_t* __restrict__ p, int64_t per_wave16,
                                                   unsigned* sink) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const u32x4_t* base = p + ((int64_t)blockIdx.x * 8 + w) * per_wave16;
  unsigned acc = 0;
  for (int64_t i = 0; i + 64 * 8 <= per_wave16; i += 64 * 8) {
    u32x4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(base + i + j * 64 + lane);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j].x ^ v[j].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

int grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (int)(b < 65536 ? (b > 0 ? b : 1) : 65536);
}

}  // namespace

extern "C" {

int synth_fill_uniform(void* dst, int64_t n, int bf16, uint64_t key, int64_t start, float scale,
                       void* stream) {
  if (!dst || n < 0) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(fill_uniform, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, dst, n,
                     bf16, key, start, scale);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int synth_fill_q4(void* codes, int64_t n_codes, void* steps, int64_t n_steps, uint64_t key_q,
                  int64_t start_q, uint64_t key_d, int64_t start_d, float scale, void* stream) {
  if (!codes || !steps || n_codes < 0 || n_steps < 0) return -1;
  const int64_t n = n_codes > n_steps ? n_codes : n_steps;
  if (n == 0) return 0;
  hipLaunchKernelGGL(fill_q4, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)codes, n_codes, (uint16_t*)steps, n_steps, key_q, start_q, key_d,
                     start_d, scale);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int synth_fill_kv(void* dst, int L, int Bl, int Bc, int Hkv, int ctx, int max_ctx, int hd,
                  int bf16, uint64_t key, float scale, int transposed, void* stream) {
  if (!dst || ctx > max_ctx || Bl > Bc) return -1;
  const int64_t n = (int64_t)L * Bl * Hkv * ctx * hd;
  if (n == 0) return 0;
  hipLaunchKernelGGL(fill_kv, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, dst, L, Bl,
                     Bc, Hkv, ctx, max_ctx, hd, bf16, key, scale, transposed);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Reads n_wg * 8 * per_wave16 16-byte units of src (per_wave16 a multiple of 512).
int synth_stream_read(const void* src, int64_t per_wave16, int n_wg, void* sink, void* stream) {
  if (!src || !sink || n_wg < 1 || per_wave16 < 512 || per_wave16 % 512) return -1;
  hipLaunchKernelGGL(stream_read, dim3(n_wg), dim3(512), 0, (hipStream_t)stream,
                     (const u32x4_t*)src, per_wave16, (unsigned*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
