// Grouped-query attention over the contiguous KV cache, for the K+1 verify rows (causal among
// the new rows, full over the committed prefix) and for the drafter's cross-attention into the
// target's cache (keys [0, len), no cache of its own).
//
// Grid: (chunk, kv head, sequence).  A workgroup loads one chunk of `chunk` keys of one KV head
// once and serves every query vector that reads that head: all rows x all query heads of the
// group.  Per chunk it writes the running max, the sum of exponentials and the unnormalised
// value sum; the last chunk to arrive combines them in chunk order.  Chunk boundaries sit at
// fixed absolute positions and every reduction has a fixed order, so a row's output does not
// depend on how many other rows are in the call.

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace specdec {

namespace {

constexpr int RB = 16;                 // query vectors per pass
constexpr int LDS_F = RB * 256;        // floats per LDS buffer
constexpr int COMB_LDS = LDS_F;        // (query vector, chunk) pairs per combine pass

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <typename T>
__global__ void __launch_bounds__(256) attn_kernel(AttnArgs a) {
  const int chunk = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wid = t >> 6;
  const int G = a.hq / a.hkv;
  const int Rall = a.R * G;
  const int CH = a.chunk;
  const int hd = a.hd;
  const int len = a.len[b];
  const int end_max = len + a.R - 1 + a.key_off;  // keys [0, end_max) are read by some row
  if (end_max > a.max_ctx || len < 0) {
    if (chunk == 0 && g == 0 && t == 0) raise_error(a.err, ERRBIT_CAPACITY);
    return;
  }
  const int n_act = (end_max + CH - 1) / CH;
  if (n_act == 0) {
    // no visible key (drafter before any context): the attention output is defined as zero
    if (chunk == 0) {
      for (int idx = t; idx < Rall * hd; idx += 256) {
        const int qv = idx / hd, d = idx - (idx / hd) * hd;
        const int row = qv / G, h = g * G + (qv - (qv / G) * G);
        Elem<T>::store(reinterpret_cast<T*>(a.out) + ((size_t)b * a.R + row) * (a.hq * hd) + h * hd + d, 0.f);
      }
    }
    return;
  }
  if (chunk >= n_act) return;

  __shared__ float qs[LDS_F];   // query block; combine: l_c
  __shared__ float sc[LDS_F];   // scores / probabilities; value-part reduction; combine: weights
  __shared__ float ms[RB], ls[RB];
  __shared__ float lsum[RB];
  __shared__ int last_flag;
  float* ored = sc;

  const T* Kc = reinterpret_cast<const T*>(a.kcache) + (size_t)b * a.cache_b_stride +
                (size_t)g * a.max_ctx * hd;
  const T* Vc = reinterpret_cast<const T*>(a.vcache) + (size_t)b * a.cache_b_stride +
                (size_t)g * a.max_ctx * hd;
  const int TPK = 256 / CH;      // threads per key in the score phase
  const int kk = t / TPK;        // key within chunk
  const int part = t - kk * TPK;
  const int dpt = hd / TPK;      // dims per thread (multiple of 8)
  const int j = chunk * CH + kk; // absolute key position
  const int KP = hd <= 256 ? max(1, 256 / hd) : 1;  // key parts in the value phase
  const int dv = t % hd;
  const int kp = t / hd;
  const int keys_per_kp = CH / KP;
  float* part_base = a.part + (((size_t)b * a.hkv + g) * a.n_chunks + chunk) * (size_t)Rall * (hd + 2);

  for (int r0 = 0; r0 < Rall; r0 += RB) {
    const int nr = min(RB, Rall - r0);
    // stage the block's query vectors
    for (int idx = t; idx < nr * hd; idx += 256) {
      const int r = idx / hd, d = idx - (idx / hd) * hd;
      const int qv = r0 + r;
      const int row = qv / G, h = g * G + (qv - (qv / G) * G);
      qs[r * hd + d] = a.q[(((size_t)b * a.R + row) * a.hq + h) * hd + d];
    }
    __syncthreads();
    // scores
    float s[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) s[r] = 0.f;
    if (j < end_max) {
      const T* kp_ = Kc + (size_t)j * hd + part * dpt;
      for (int d0 = 0; d0 < dpt; d0 += 8) {
        float kv[8];
        load8<T>(kp_ + d0, kv);
        const int dd = part * dpt + d0;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          if (r < nr) {
            const float4 qa = *reinterpret_cast<const float4*>(&qs[r * hd + dd]);
            const float4 qb = *reinterpret_cast<const float4*>(&qs[r * hd + dd + 4]);
            float acc = s[r];
            acc = fmaf(qa.x, kv[0], acc); acc = fmaf(qa.y, kv[1], acc);
            acc = fmaf(qa.z, kv[2], acc); acc = fmaf(qa.w, kv[3], acc);
            acc = fmaf(qb.x, kv[4], acc); acc = fmaf(qb.y, kv[5], acc);
            acc = fmaf(qb.z, kv[6], acc); acc = fmaf(qb.w, kv[7], acc);
            s[r] = acc;
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      for (int o = 1; o < TPK; o <<= 1) s[r] += __shfl_xor(s[r], o, WAVE);
    }
    if (part == 0) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (r < nr) {
          const int row = (r0 + r) / G;
          const int kend = len + row + a.key_off;
          sc[r * CH + kk] = (j < kend) ? s[r] * a.scale : -INFINITY;
        }
      }
    }
    __syncthreads();
    // softmax statistics per query vector (one wave per vector, fixed lane order)
    for (int r = wid; r < nr; r += 4) {
      float mx = -INFINITY;
      for (int k = lane; k < CH; k += WAVE) mx = fmaxf(mx, sc[r * CH + k]);
      mx = wave_max(mx);
      float sum = 0.f;
      for (int k = lane; k < CH; k += WAVE) {
        const float v = sc[r * CH + k];
        const float p = (mx == -INFINITY) ? 0.f : expf(v - mx);
        sc[r * CH + k] = p;
        sum += p;
      }
      sum = wave_sum(sum);
      if (lane == 0) { ms[r] = mx; ls[r] = sum; }
    }
    __syncthreads();
    // value accumulation
    float o[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) o[r] = 0.f;
    if (kp < KP && t < KP * hd) {
      const int k0 = kp * keys_per_kp;
      const int kmax = min(k0 + keys_per_kp, end_max - chunk * CH);
      for (int k = k0; k < kmax; ++k) {
        const float v = Elem<T>::load(Vc + (size_t)(chunk * CH + k) * hd + dv);
#pragma unroll
        for (int r = 0; r < RB; ++r)
          if (r < nr) o[r] = fmaf(sc[r * CH + k], v, o[r]);
      }
    }
    if (KP > 1) {
      __syncthreads();
      if (kp < KP && t < KP * hd) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
          if (r < nr) ored[(kp * RB + r) * hd + dv] = o[r];
      }
      __syncthreads();
      if (t < hd) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          if (r < nr) {
            float acc = ored[r * hd + t];
            for (int p = 1; p < KP; ++p) acc += ored[(p * RB + r) * hd + t];
            o[r] = acc;
          }
        }
      }
    }
    if (t < hd) {
#pragma unroll
      for (int r = 0; r < RB; ++r)
        if (r < nr) part_base[(size_t)(r0 + r) * (hd + 2) + t] = o[r];
    }
    if (t < nr) {
      part_base[(size_t)(r0 + t) * (hd + 2) + hd] = ms[t];
      part_base[(size_t)(r0 + t) * (hd + 2) + hd + 1] = ls[t];
    }
    __syncthreads();
  }

  // last chunk to arrive combines
  fence_device();
  __syncthreads();
  if (t == 0) {
    const int old = atomic_inc_device(a.cnt + b * a.hkv + g);
    last_flag = (old == n_act - 1);
  }
  __syncthreads();
  if (!last_flag) return;
  fence_device();
  float* w = sc;  // reuse: weights [qv][chunk]
  const float* pbase = a.part + ((size_t)b * a.hkv + g) * a.n_chunks * (size_t)Rall * (hd + 2);
  const size_t cstride = (size_t)Rall * (hd + 2);
  const int QB = max(1, min(min(Rall, RB), COMB_LDS / n_act));
  for (int q0 = 0; q0 < Rall; q0 += QB) {
    const int nq = min(QB, Rall - q0);
    for (int idx = t; idx < nq * n_act; idx += 256) {
      const int qi = idx / n_act, c = idx - (idx / n_act) * n_act;
      const float* p = pbase + c * cstride + (size_t)(q0 + qi) * (hd + 2) + hd;
      w[qi * n_act + c] = __builtin_nontemporal_load(p);   // m_c
      qs[qi * n_act + c] = __builtin_nontemporal_load(p + 1);  // l_c
    }
    __syncthreads();
    if (t < nq) {
      float M = -INFINITY;
      for (int c = 0; c < n_act; ++c) M = fmaxf(M, w[t * n_act + c]);
      float L = 0.f;
      for (int c = 0; c < n_act; ++c) {
        const float mc = w[t * n_act + c];
        const float e = (mc == -INFINITY) ? 0.f : expf(mc - M);
        w[t * n_act + c] = e;
        L += qs[t * n_act + c] * e;
      }
      lsum[t] = L;
    }
    __syncthreads();
    for (int idx = t; idx < nq * hd; idx += 256) {
      const int qi = idx / hd, d = idx - (idx / hd) * hd;
      float acc = 0.f;
      for (int c = 0; c < n_act; ++c)
        acc += w[qi * n_act + c] * __builtin_nontemporal_load(pbase + c * cstride + (size_t)(q0 + qi) * (hd + 2) + d);
      const float val = acc / lsum[qi];
      const int qv = q0 + qi;
      const int row = qv / G, h = g * G + (qv - (qv / G) * G);
      Elem<T>::store(reinterpret_cast<T*>(a.out) + ((size_t)b * a.R + row) * (a.hq * hd) + h * hd + d, val);
    }
    __syncthreads();
  }
  if (t == 0) atomic_store_zero(a.cnt + b * a.hkv + g);
}

}  // namespace

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.n_chunks, a.hkv, a.B), block(256);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(attn_kernel<bf16_t>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(attn_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace specdec
